"""libmhc: the mHC hyper-connection hot path on MI355X (gfx950).

The compute lives in the HIP shared library ``libmhc.so`` built from
``csrc/``; this package loads it lazily (importing the package never needs a
GPU) and exposes thin bindings with the library's names.
"""
