"""CPU oracle for MX-FP8 block quantization, per-tensor FP8 quantization and
the (grouped) GEMMs they feed.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP
library: its arithmetic is plain NumPy in float64 and exact integer/bit
operations, written from the pages' definitions, slow on purpose.

Sources (cited by page title and section):

* [HP329] "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" (mindspore/hyper-parallel
  issue #329): §3 format table (E4M3 data, E8M0 scale, 1x32/32x1 blocks,
  scale from the current input), §3.2 (current scaling: the FP32 scale is
  the tensor's amax over the format's largest value when amax is finite and
  non-zero, and 1 otherwise), §8 direction
  table, §13.4 matmul / grouped-matmul interface.
* [FPBLOG] "Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度":
  §二.1 bit fields and the general value formula, §二.2 format table and the
  E4M3 (fn) and BF16 notes, §五 FP32 accumulation, §七.2 per-tensor scaling,
  §八.3 kernel-difference rules, §九.1 bit-pattern examples.
* [TTNPU] "低精度训练特性（MXFP8 / HiFloat8）" (torchtitan-npu): MX block size
  32, one shared scale per 32 elements; grouped MX quant for wgrad.

Readings taken where the pages are silent (each is also listed with the test
that pins it):

* Shared exponent of an MX block: ``e = floor(log2(amax)) - 8`` where 8 is the
  exponent of E4M3's largest value (448 = 1.75 * 2^8), clamped below at -127;
  an all-zero block takes -127.  This is the OCP Microscaling convention.
* E8M0 is a biased exponent with bias 127 (the FP32 bias); 0xFF is NaN.
* Rounding to E4M3 is round-to-nearest-even; magnitudes >= 448 saturate to 448.
* A block holding NaN or Inf gets scale 0xFF and every code 0x7F.
* Per-tensor quantization divides in FP32: ``q = E4M3(fp32(x) / s)``.

Parity status: every public function here is pinned by ``tests/test_oracle_*``;
no function is "parity unpinned".
"""

from . import codec, mx, per_tensor, gemm  # noqa: F401
