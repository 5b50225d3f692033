"""The method's scalars, by name (the vocabulary of the pages' review of the
Mega-mHC integration: hc_norm_eps, rmsnorm_eps, hc_post_scale,
sinkhorn_eps)."""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Params:
    hc_norm_eps: float = 1e-6
    rmsnorm_eps: float = 1e-6
    hc_post_scale: float = 2.0
    sinkhorn_eps: float = 1e-6
    sinkhorn_iters: int = 20

    def as_kwargs(self) -> dict:
        return dataclasses.asdict(self)
