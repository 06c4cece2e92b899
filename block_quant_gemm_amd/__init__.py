"""MX-FP8 block quantization and (grouped) GEMM for AMD MI355X (gfx950).

The compute path is the HIP library ``libmxq.so`` (sources in ``csrc/``,
C declarations in ``include/mxq.h``); :mod:`block_quant_gemm_amd.mxq` is a
thin ctypes binding over it.  :mod:`block_quant_gemm_amd.workloads` draws the
seeded synthetic inputs.
"""
