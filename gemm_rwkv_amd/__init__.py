"""gemm_rwkv_amd: quantized-weight GEMV/GEMM for RWKV-7 projections on MI355X.

The compute lives in the HIP library ``librq.so`` (C ABI declared in
``include/rq.h``); ``gemm_rwkv_amd.rq`` is the thin ctypes binding that the
tests and the benchmark call.  ``gemm_rwkv_amd.synth`` draws the seeded
synthetic inputs and holds no arithmetic of the method.  Importing the package
does not load the library; the first call through ``gemm_rwkv_amd.rq`` does,
and fails loudly if it is missing.
"""
