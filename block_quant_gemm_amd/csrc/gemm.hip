// MX-FP8 GEMM kernels for gfx950 (dense, grouped variable-M, grouped
// variable-K) on the block-scaled FP8 MFMA, with their C-ABI launchers.
//
// Method: "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" §8 (forward, dgrad and
// wgrad are one quantized matmul each on the copy blocked along the
// contraction dim), §5.2 and §13.4 (grouped matmul over per-expert token
// groups); "Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度" §五
// (FP32 accumulation, one rounding to BF16 at the end).
//
// Tiling.  A workgroup of 512 lanes (8 wavefronts, two per SIMD) computes a
// 256 x 256 output tile; each wavefront owns 128 x 64 = 4 x 2 MFMA tiles of
// 32 x 32 (128 FP32 accumulators per lane).  The K loop steps 64 codes (two
// 32-blocks, one MFMA deep) at a time; operand tiles go from HBM straight
// into LDS with buffer_load_dwordx4 ... lds (no register staging) in stages
// of two k-steps (128-byte row pieces) through a 2-slot ring.  The two
// wavefronts of a SIMD ping-pong: one multiplies while the other reads its
// next fragments from LDS.  Rows and K positions outside the operand read as
// zero through the buffer descriptor's range check.  Dense GEMMs too small to
// fill the CUs with 256-row tiles use 128-row tiles (each wavefront 64 x 64,
// the same k loop with half the matrix work per stage; the A stage's upper
// half then holds zeros).
//
// Matrix instruction.  v_mfma_scale_f32_32x32x64_f8f6f4 takes, per lane l,
// 32 codes of row l%32: bytes 0-15 are k = 16h .. 16h+15 and bytes 16-31 are
// k = 32+16h .. 47+16h of the 64-wide step, h = l/32; the lane with h = 0
// supplies the E8M0 scale of k 0..31 and the lane with h = 1 that of k 32..63,
// selected from a 32-bit register by op_sel.  Each lane therefore loads, per
// operand row it serves and step, the one scale byte of its half.  The B tile
// is the instruction's first operand, so each lane's accumulators hold 4
// consecutive output columns of one output row.

#include "common.h"

#include <type_traits>
#include <utility>

namespace mxq {

constexpr int TM = 256, TN = 256;
constexpr int TK = 64;                            // k-step: one MFMA deep
constexpr int TS = 128;                           // stage: two k-steps, 128-byte row segments
constexpr int kThreads = 512;                     // 8 wavefronts, 2 per SIMD
constexpr int kSlots = 2;                         // LDS ring of stages
constexpr int kStage = TM * TS;                   // bytes per operand per stage (32 KB)
constexpr int kCStride = TN * 2 + 16;             // LDS row stride of the staged BF16 tile
constexpr int kSmem = kSlots * 2 * kStage > TM * kCStride ? kSlots * 2 * kStage : TM * kCStride;
// M tiles per rasterization group: dense GEMMs walk N with 8 M-tiles (each
// XCD takes a contiguous run of tiles); grouped variable-M GEMMs with 4,
// dispatched in plain order so that all XCDs work on neighbouring tiles
// (measured on the expert-layer shapes: the shared last-level cache then
// serves the panels every XCD reads).
constexpr int kGroupMDense = 8;
constexpr int kGroupMVarM = 4;
constexpr int kMaxGroups = 256;

// Compile-time loops: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, B + I>{}), ...);
}
template <int B, int E, class F>
__device__ __forceinline__ void static_for_range(F&& f) {
  static_for_seq<B>(f, std::make_integer_sequence<int, E - B>{});
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_range<0, N>(f); }

enum GemmKind { kDense = 0, kVarM = 1, kVarK = 2 };

// Buffer descriptor for gfx9: 48-bit base, stride 0, num_records bytes (range
// checked: loads at or past it read 0), data format word 0x00020000.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((a >> 32) & 0xFFFFu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// Asynchronous loads straight into LDS (issued as inline assembly: the
// compiler does not track them; the k loop's explicit vmcnt waits and
// barriers order them; nothing else in these kernels uses m0).  16 bytes per
// lane to m0 + 16*lane, or one byte per
// lane zero-extended to m0 + 4*lane.
// m0 and the descriptor are wave-uniform; readfirstlane puts them in SGPRs.
__device__ __forceinline__ i32x4 uniform(i32x4 r) {
  i32x4 u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}
__device__ __forceinline__ void dma_b128(i32x4 r, uint32_t m0, uint32_t off) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void dma_b32(i32x4 r, uint32_t m0, uint32_t off) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void dma_b8(i32x4 r, uint32_t m0, uint32_t off) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_ubyte %1, %2, 0 offen lds"
               :: "s"(m), "v"(off), "s"(r) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// LDS offset of 16-byte chunk c (0..7) of tile row r in a stage: rows are
// 128 B; chunks are XOR-swizzled with bits 1-3 of the row, so 16 consecutive
// rows read at one chunk index (the 16 lanes the LDS serves per clock for
// 16-byte reads) cover all 16 16-byte slots of the 256-byte bank line.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * TS + ((c ^ swz(r)) << 4); }

struct GemmArgs {
  const uint8_t* a; const uint8_t* as; int64_t lda, ldsa;
  const uint8_t* b; const uint8_t* bs; int64_t ldb, ldsb;
  int64_t b_estride, bs_estride;                    // per-group B strides (variable M)
  const float* pta; const float* ptb;               // per-tensor scales (variable M: per group)
  const int64_t* offsets; int32_t E;
  int64_t M, N, K;
  void* c; int64_t ldc;
  uint32_t tiles_n;                                 // output tiles along N
  uint32_t nblocks;                                 // grid size (for the XCD remap)
  uint32_t rows128;                                 // dense: 128-row tiles (k_gemm_rows128)
  // SwiGLU epilogue (variable M): h = silu(gate) * up of the gate/up product,
  // written as its MX row copy and grouped column copy.
  int64_t F;                                        // h columns (gate rows per expert)
  uint8_t* hq; uint8_t* hs; int64_t ldhq, ldhs;     // row copy [M, F], scales [M, F/32]
  uint8_t* hqT; uint8_t* hsT; int64_t ldhqT, ldhsT; // column copy [F, hcap], scales
  int64_t hcap;                                     // columns of the column copy
  int64_t* poff;                                    // padded offsets out [E+1], or null
  uint32_t* camax;                                  // per-tensor dense: max |C| out, or null
  // per-group-scaled SwiGLU product: h in BF16 and each group's max |h|
  uint16_t* h; int64_t ldh;
  uint32_t* hamax;                                  // [E] FP32 bit patterns (atomic max)
};

// One operand of a workgroup: codes and scales as buffer resources whose
// offset 0 is the tile's first row at the start of the contraction range.
struct OpTile {
  i32x4 q, s;
  uint32_t ld, lds;
  uint32_t smis;                                    // scale base misalignment (0..3 bytes
                                                    // or, for scale windows, 0..15)
  int rows;                                         // valid rows in this tile (<= 256)
};

// `windows`: scales are read in 16-byte windows (row strides are multiples of
// 16, so every row has the same misalignment); the descriptor starts at the
// 16-byte boundary at or below the tile's first scale and its range is rounded
// up to whole windows, which never crosses a page the valid bytes are not in.
__device__ __forceinline__ OpTile op_tile(const uint8_t* q, const uint8_t* s, int64_t ld,
                                          int64_t lds, int64_t row0, int64_t k0, int64_t rows,
                                          int64_t kdim, bool scales, bool windows) {
  OpTile t;
  const int r = rows > TM ? TM : (rows < 0 ? 0 : (int)rows);
  t.rows = r;
  t.ld = (uint32_t)ld;
  t.lds = (uint32_t)lds;
  const uint8_t* qb = q + row0 * ld + k0;
  // valid bytes: r rows of ld bytes, the last one only up to kdim
  const uint32_t qbytes = r > 0 ? (uint32_t)((r - 1) * ld + kdim) : 0;
  t.q = make_rsrc(qb, qbytes);
  if (scales) {
    const uint8_t* sb = s + row0 * lds + (k0 >> 5);
    const uintptr_t a = reinterpret_cast<uintptr_t>(sb);
    const uintptr_t align = windows ? 15 : 3;
    t.smis = (uint32_t)(a & align);
    const uint8_t* sba = reinterpret_cast<const uint8_t*>(a & ~align);
    uint32_t sbytes = r > 0 ? (uint32_t)((r - 1) * lds + t.smis + ((kdim + 31) >> 5)) : 0;
    if (windows) sbytes = (sbytes + 15) & ~15u;
    t.s = make_rsrc(sba, sbytes);
  } else {
    t.smis = 0;
    t.s = t.q;
  }
  return t;
}

// Per-lane load offsets of one operand, computed once per workgroup.
// Codes: wavefront w fills row groups g = 4w .. 4w+3 (8 rows of 128 B, 1 KB
// each) of the operand's LDS stage slot; lane i lands at byte 16 i of a
// group, i.e. row i/8 and 16-byte slot i%8, which must hold chunk
// (i%8) ^ swz(row); swz(8g + i/8) = 4 (g%2) + i/16, so the chunk depends on
// the lane and the parity of j.
// Scales (byte path): entry e = 64 w + i of the operand's 512 scale entries
// per k-step is block e%2 of the step for tile row e/2.
struct LaneOffsets {
  uint32_t q[4];            // row * ld + chunk * 16 (0x80000000 for rows past the tile)
  uint32_t kc0;             // chunk * 16 for even j (odd j: kc0 ^ 64)
  uint32_t s;               // smis + row * lds + blk of the lane's scale entry
  uint32_t sblk;            // blk (0 or 1) of the lane's scale entry
};

__device__ __forceinline__ LaneOffsets lane_offsets(const OpTile& t) {
  LaneOffsets o;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane >> 3, slot = lane & 7;
  o.kc0 = (uint32_t)((slot ^ (rsub >> 1)) * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (w * 4 + j) * 8 + rsub;
    const uint32_t kc = o.kc0 ^ ((j & 1) * 64);     // == ((slot ^ swz(row)) * 16)
    o.q[j] = row < t.rows ? (uint32_t)(row * t.ld) + kc : 0x80000000u;
  }
  const int e = w * 64 + lane;
  o.s = t.smis + (uint32_t)((e >> 1) * t.lds) + (uint32_t)(e & 1);
  o.sblk = (uint32_t)(e & 1);
  return o;
}

// SwiGLU product (gate/up weight of one expert: gate rows [0, F), up rows
// [F, 2F)).  The B stage holds, in LDS row R, for the 64-row block p = R/64,
// gate row hc0 + 32p + R%32 when R%64 < 32 and the up row F + hc0 + 32p +
// R%32 otherwise, hc0 being the tile's first h column: each wavefront's 64
// accumulator columns are then 32 gate columns and the 32 up columns of the
// same h columns.  -1 marks rows past F.
__device__ __forceinline__ int64_t gu_row(int R, int64_t hc0, int64_t F) {
  const int64_t hc = hc0 + 32 * (R >> 6) + (R & 31);
  if (hc >= F) return -1;
  return (R & 32) ? F + hc : hc;
}

// Offset that reads zeros through any descriptor of this file: past every
// range (ranges stay below 2^30), also after a k offset below 2^31 is added.
constexpr uint32_t kDeadRow = 0x40000000u;

// A whole expert's gate/up weight as one operand (2F rows from row 0); rows
// are picked per lane with gu_row.
__device__ __forceinline__ OpTile op_expert(const uint8_t* q, const uint8_t* s, int64_t ld,
                                            int64_t lds, int64_t rows, int64_t kdim,
                                            bool windows) {
  OpTile t;
  t.rows = 0;
  t.ld = (uint32_t)ld;
  t.lds = (uint32_t)lds;
  t.q = make_rsrc(q, rows > 0 ? (uint32_t)((rows - 1) * ld + kdim) : 0);
  const uintptr_t a = reinterpret_cast<uintptr_t>(s);
  const uintptr_t align = windows ? 15 : 3;
  t.smis = (uint32_t)(a & align);
  uint32_t sbytes = rows > 0 ? (uint32_t)((rows - 1) * lds + t.smis + ((kdim + 31) >> 5)) : 0;
  if (windows) sbytes = (sbytes + 15) & ~15u;
  t.s = make_rsrc(reinterpret_cast<const uint8_t*>(a & ~align), sbytes);
  return t;
}

// lane_offsets for the SwiGLU product's B operand (rows through gu_row).
__device__ __forceinline__ LaneOffsets lane_offsets_gu(const OpTile& t, int64_t hc0, int64_t F) {
  LaneOffsets o;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane >> 3, slot = lane & 7;
  o.kc0 = (uint32_t)((slot ^ (rsub >> 1)) * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t gr = gu_row((w * 4 + j) * 8 + rsub, hc0, F);
    const uint32_t kc = o.kc0 ^ ((j & 1) * 64);
    o.q[j] = gr >= 0 ? (uint32_t)(gr * t.ld) + kc : kDeadRow;
  }
  const int e = w * 64 + lane;
  const int64_t gr = gu_row(e >> 1, hc0, F);
  o.s = gr >= 0 ? t.smis + (uint32_t)(gr * t.lds) + (uint32_t)(e & 1) : kDeadRow;
  o.sblk = (uint32_t)(e & 1);
  return o;
}

// silu(x) = x / (1 + e^-x) in FP32, e^-x = 2^(-x log2 e) on the hardware
// exponential; for x below about -88 it is +inf and the result -0.
__device__ __forceinline__ float silu_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// MX block of 32 FP32 values: E8M0 code from the largest magnitude (sign
// cleared, integer order: NaN above Inf above finite values; code = exponent
// field - 8 clamped at 0, 0xFF for NaN/Inf) and the 32 E4M3 codes packed
// into 8 dwords (all 0x7F for a NaN/Inf block).
__device__ __forceinline__ uint32_t mx_block_f32(const float (&v)[32], uint32_t (&out)[8]) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t m = __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu;
    am = am > m ? am : m;
  }
  const uint32_t E = am >> 23;
  const uint32_t code = am >= 0x7F800000u ? 0xFFu : (E > 8u ? E - 8u : 0u);
  const float inv = mx_inv_scale(code == 0xFFu ? 127u : code);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t w = cvt2_e4m3_sat<false>(v[4 * d] * inv, v[4 * d + 1] * inv, 0u);
    w = cvt2_e4m3_sat<true>(v[4 * d + 2] * inv, v[4 * d + 3] * inv, w);
    out[d] = code == 0xFFu ? 0x7F7F7F7Fu : w;
  }
  return code;
}

// E8M0 code c as the FP32 scale operand of the scaled conversions, which
// take its exponent field: 2^(c - 127); 0xFF (a NaN block) turns every
// converted value into NaN.
__device__ __forceinline__ float e8m0_f32(uint32_t c) { return __builtin_bit_cast(float, c << 23); }

// Eight E4M3 codes (bytes of w0, then w1) times 2^(c - 127) as BF16, element
// i from byte i.  Exact while the product is a normal or subnormal BF16
// value with its bits intact: scale codes 3..246.
__device__ __forceinline__ bf16x8 widen8_bf16(uint32_t w0, uint32_t w1, float s) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, s, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, s, true);
  const bf16x4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const bf16x4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The MFMA operand of tile row r for one k-step: 16-byte chunks c0 and c1.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* l, int r, int c0, int c1) {
  const uint4 x = *reinterpret_cast<const uint4*>(l + lds_off(r, c0));
  const uint4 y = *reinterpret_cast<const uint4*>(l + lds_off(r, c1));
  i32x8 f;
  f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
  f[4] = y.x; f[5] = y.y; f[6] = y.z; f[7] = y.w;
  return f;
}

template <int OUT>
__device__ __forceinline__ void store4(void* c, int64_t ldc, int64_t m, int64_t n, int64_t N,
                                       float v0, float v1, float v2, float v3) {
  if (OUT == MXQ_OUT_FP32) {
    float* p = static_cast<float*>(c) + m * ldc + n;
    if (n + 3 < N && ((reinterpret_cast<uintptr_t>(p) & 15) == 0)) {
      *reinterpret_cast<float4*>(p) = make_float4(v0, v1, v2, v3);
    } else {
      if (n < N) p[0] = v0;
      if (n + 1 < N) p[1] = v1;
      if (n + 2 < N) p[2] = v2;
      if (n + 3 < N) p[3] = v3;
    }
  } else {
    __bf16* p = static_cast<__bf16*>(c) + m * ldc + n;
    if (n + 3 < N && ((reinterpret_cast<uintptr_t>(p) & 7) == 0)) {
      *reinterpret_cast<uint2*>(p) = make_uint2(bf16x2_bits(v0, v1), bf16x2_bits(v2, v3));
    } else {
      const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
      if (n < N) p[0] = b0;
      if (n + 1 < N) p[1] = b1;
      if (n + 2 < N) p[2] = b2;
      if (n + 3 < N) p[3] = b3;
    }
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous run of tile indices so tiles sharing operand panels share an L2.
// Used for dense GEMMs.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
  const uint32_t X = 8, per = n / X, rem = n % X;
  const uint32_t x = bid % X, i = bid / X;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

// Tile index -> (tm, tn): groups of G M-tiles walk N together, so the tiles
// in flight read a few A panels and a few B panels.
template <int kGroupM>
__device__ __forceinline__ void raster(uint32_t tile, uint32_t tiles_m, uint32_t tiles_n,
                                       uint32_t& tm, uint32_t& tn) {
  const uint32_t per_group = kGroupM * tiles_n;
  const uint32_t grp = tile / per_group, in = tile % per_group;
  const uint32_t first = grp * kGroupM;
  const uint32_t gm = tiles_m - first < (uint32_t)kGroupM ? tiles_m - first : (uint32_t)kGroupM;
  tm = first + in % gm;
  tn = in / gm;
}

// Per-group tile prefix for variable M, computed by wavefront 0 into LDS:
// s_start[g] = first M-tile index of group g; s_off[g] = clamped offsets.
__device__ void group_table(const int64_t* offsets, int E, int64_t M, int64_t* s_off,
                            int32_t* s_start) {
  const int t = threadIdx.x;
  for (int g = t; g <= E; g += blockDim.x) {
    const int64_t o = offsets[g];
    s_off[g] = o < 0 ? 0 : (o > M ? M : o);
  }
  __syncthreads();
  if (t < 64) {
    int32_t carry = 0;
    if (t == 0) s_start[0] = 0;
    for (int base = 0; base < E; base += 64) {
      const int g = base + t;
      int32_t cnt = 0;
      if (g < E) {
        const int64_t d = s_off[g + 1] - s_off[g];
        cnt = d > 0 ? (int32_t)((d + TM - 1) / TM) : 0;
      }
      int32_t v = cnt;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        const int32_t u = __shfl_up(v, sh, 64);
        if (t >= sh) v += u;
      }
      if (g < E) s_start[g + 1] = carry + v;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
}

// Weight-gradient tile order: the experts by padded token count, largest
// first, so the longest tiles start first whatever the routing's expert order.
// Counts are ranked by binade (the bit length of count / 32, so within a
// factor of 2), ties by index; experts already in that order keep it.
// Wavefront 0 checks the order with one ballot per 64 experts, else ranks them
// with one ballot per binade present.  s_off receives the offsets rounded down
// to 32 and clamped to [0, cap] (as the tiles read them) and s_perm[r] the
// expert of rank r; the ranks form a permutation whatever the offsets hold.
__device__ void expert_order(const int64_t* offsets, int E, int64_t cap, int64_t* s_off,
                             int32_t* s_perm) {
  const int t = threadIdx.x;
  for (int e = t; e <= E; e += blockDim.x) {
    const int64_t o = offsets[e] & ~31LL;
    s_off[e] = o < 0 ? 0 : (o > cap ? cap : o);
  }
  __syncthreads();
  if (t < 64) {
    constexpr int R = kMaxGroups / 64;              // rounds of 64 experts
    const int rounds = (E + 63) / 64;
    int bin[R];                                     // -1 past E
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int e = c * 64 + t;
      int b = -1;
      if (e < E) {
        const int64_t d = s_off[e + 1] - s_off[e];
        const uint64_t u = d > 0 ? (uint64_t)d >> 5 : 0;
        b = u ? 64 - __builtin_clzll(u) : 0;
      }
      bin[c] = b;
    }
    // in order already: binades non-increasing with the index
    bool sorted = true;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      if (c < rounds) {
        int nxt = __shfl_down(bin[c], 1, 64);       // expert e + 1
        const int first_next = c + 1 < R ? __shfl(bin[c + 1 < R ? c + 1 : c], 0, 64) : -1;
        if (t == 63) nxt = first_next;              // lane 63: the next round's first
        if (__ballot(bin[c] >= 0 && nxt > bin[c]) != 0) sorted = false;
      }
    }
    if (sorted) {
      for (int e = t; e < E; e += 64) s_perm[e] = e;
    } else {
      // rank = experts in higher binades + experts of the same binade with a
      // lower index (earlier rounds, then lower lanes of this round), over the
      // binades present only
      int bhi = -1, blo = 64;
#pragma unroll
      for (int c = 0; c < R; ++c)
        if (bin[c] >= 0) {
          bhi = bhi > bin[c] ? bhi : bin[c];
          blo = blo < bin[c] ? blo : bin[c];
        }
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) {
        const int ohi = __shfl_xor(bhi, sh, 64), olo = __shfl_xor(blo, sh, 64);
        bhi = bhi > ohi ? bhi : ohi;
        blo = blo < olo ? blo : olo;
      }
      bhi = __builtin_amdgcn_readfirstlane(bhi);
      blo = __builtin_amdgcn_readfirstlane(blo);
      int above = 0, rank[R];
#pragma unroll
      for (int c = 0; c < R; ++c) rank[c] = 0;
      for (int b = bhi; b >= blo; --b) {
        int before = 0;
#pragma unroll
        for (int c = 0; c < R; ++c) {
          if (c < rounds) {
            const uint64_t m = __ballot(bin[c] == b);
            if (bin[c] == b) rank[c] = above + before + __builtin_popcountll(m & ((1ull << t) - 1ull));
            before += __builtin_popcountll(m);
          }
        }
        above += before;
      }
#pragma unroll
      for (int c = 0; c < R; ++c)
        if (bin[c] >= 0) s_perm[rank[c]] = c * 64 + t;
    }
  }
  __syncthreads();
}

// Vector-memory instructions a wavefront issues per stage: 4 + 4 tile loads,
// plus 2 + 2 scale-byte loads for MX scales read byte by byte.
template <bool SBYTES>
constexpr int vmem_per_stage() { return SBYTES ? 12 : 8; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N (split field bits 3:0 and 15:14), expcnt and
  // lgkmcnt left at their "don't wait" maxima.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Scale windows: 3-slot ring of [A, B][256 rows][16 bytes] (16 blocks of 32,
// i.e. 8 k-steps, per row).
constexpr int kWinSlots = 3;
constexpr int kWinBytes = 2 * TM * 16;

// Blockwise FP32 scales: per stage (= one 128-wide block of the contraction)
// 256 A-row scales and the tile's two B block-row scales, [slot][A 256 | B 64].
constexpr int kBlkScaleWords = 320;

// SW: MX scales read in 16-byte windows (row strides multiples of 16);
// otherwise byte by byte (any stride).  PT: per-tensor scaled (no block scales).
// SWI: the SwiGLU product (variable M, MX): B is an expert's gate/up weight
// read through gu_row, and the epilogue writes h's MX copies.
// BLK: blockwise FP32 scales (dense only): 1x128 blocks of A, 128x128 blocks
// of B; each k-step's product is formed with unit scales and promoted into
// the FP32 accumulators times its blocks' two scales.
// XA: exact products (MXQ_ACC_FP32): each 32-block of codes is widened to
// BF16 with its E8M0 scale folded in (exact for scale codes 3..246, which
// every finite BF16 block yields unless its largest magnitude is below
// 2^-116), and multiplied on the BF16 matrix instruction, whose products are
// exact and whose sums are FP32-accurate.
template <int KIND, bool PT, int OUT, bool SW, bool SWI, bool BLK, bool XA = false, int MI = 4>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
  static_assert(MI == 4 || (MI == 2 && !SWI && !BLK), "row tiles per wavefront");
  constexpr int TMR = MI * 64;                      // tile rows (256, or 128)
  constexpr int RW = MI * 32;                       // rows per wavefront
  constexpr int DPM = 4 / MI;                       // stage loads issued per MFMA
  static_assert(!SWI || (KIND == kVarM && OUT == MXQ_OUT_BF16), "SwiGLU product kind");
  static_assert(!BLK || (KIND == kDense && !PT && !SW && !SWI), "blockwise kind");
  static_assert(!XA || (!SWI && !BLK), "exact-product kind");
  constexpr bool SBYTES = !PT && !SW && !BLK;       // per-step scale-byte loads
  constexpr bool SWIN = !PT && SW && !BLK;          // scale windows
  // [slot][A, B] stages; after the k loop, the staged BF16 output tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
  // byte path: [slot][k-step][A, B][row][blk] as dwords;
  // windows: [wslot][A, B][row][16 B]
  __shared__ __attribute__((aligned(16)))
  uint32_t ssc[SBYTES ? kSlots * 2 * 2 * 2 * TM
                      : (SWIN ? kWinSlots * kWinBytes / 4 : (BLK ? kSlots * kBlkScaleWords : 1))];
  __shared__ int64_t s_off[KIND == kVarM || KIND == kVarK ? kMaxGroups + 1 : 1];
  __shared__ int32_t s_perm[KIND == kVarK ? kMaxGroups : 1];
  __shared__ int32_t s_start[KIND == kVarM ? kMaxGroups + 1 : 1];
  __shared__ uint32_t s_cmax[KIND == kDense && PT ? kThreads / 64 : 1];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: scalar branches
  // Wavefronts w and w + 4 share a SIMD.  Group grp = w / 4 owns output
  // columns [128 grp, 128 grp + 128) of the tile; within it wavefront w
  // computes rows [128 wm, +128) x columns [bn, bn + 64).
  const int grp = wave >> 2, qw = wave & 3;
  const int wm = qw >> 1;
  const int bn = grp * 128 + (qw & 1) * 64;
  const int r32 = lane & 31, half = lane >> 5;

  // ---- map the workgroup to (group, m0, n0) ----
  int64_t m0 = 0, n0 = 0, kdim = g.K, c_rows = 0;
  void* cbase = g.c;
  int group = 0;                                    // the tile's group (variable M, K)
  OpTile A, B;
  if (KIND == kDense) {
    const uint32_t tiles_m = (uint32_t)((g.M + TMR - 1) / TMR);
    uint32_t tm, tn;
    raster<kGroupMDense>(xcd_remap(blockIdx.x, g.nblocks), tiles_m, g.tiles_n, tm, tn);
    m0 = (int64_t)tm * TMR;
    n0 = (int64_t)tn * TN;
    c_rows = g.M - m0;
    if (c_rows > TMR) c_rows = TMR;
    A = op_tile(g.a, g.as, g.lda, g.ldsa, m0, 0, c_rows, kdim, !PT && !BLK, SW);
    B = op_tile(g.b, g.bs, g.ldb, g.ldsb, n0, 0, g.N - n0, kdim, !PT && !BLK, SW);
  } else if (KIND == kVarM) {
    group_table(g.offsets, g.E, g.M, s_off, s_start);
    if (SWI && blockIdx.x == 0 && wave == 0 && g.poff) {
      // padded offsets of the column copy: each group rounded up to 32 rows
      int64_t carry = 0;
      if (lane == 0) g.poff[0] = 0;
      for (int base = 0; base < g.E; base += 64) {
        const int gi = base + lane;
        int64_t v = 0;
        if (gi < g.E) {
          const int64_t d = s_off[gi + 1] - s_off[gi];
          v = d > 0 ? (d + 31) & ~31LL : 0;
        }
#pragma unroll
        for (int sh = 1; sh < 64; sh <<= 1) {
          const int64_t u = __shfl_up(v, sh, 64);
          if (lane >= sh) v += u;
        }
        if (gi < g.E) g.poff[gi + 1] = carry + v;
        carry += __shfl(v, 63, 64);
      }
    }
    const uint32_t tiles_m = (uint32_t)s_start[g.E];  // data-dependent M-tile count
    const uint32_t tile = blockIdx.x;
    if (tile >= tiles_m * g.tiles_n) return;          // surplus workgroup
    uint32_t tm, tn;
    raster<kGroupMVarM>(tile, tiles_m, g.tiles_n, tm, tn);
    int lo = 0, hi = g.E - 1;                         // group e: s_start[e] <= tm < s_start[e+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= (int32_t)tm) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    group = e;
    m0 = s_off[e] + (int64_t)(tm - s_start[e]) * TM;
    n0 = (int64_t)tn * TN;
    c_rows = s_off[e + 1] - m0;
    A = op_tile(g.a, g.as, g.lda, g.ldsa, m0, 0, c_rows, kdim, !PT, SW);
    if (SWI)
      B = op_expert(g.b + (int64_t)e * g.b_estride,
                    PT ? nullptr : g.bs + (int64_t)e * g.bs_estride, g.ldb, g.ldsb, 2 * g.F,
                    kdim, SW);
    else
      B = op_tile(g.b + (int64_t)e * g.b_estride,
                  PT ? nullptr : g.bs + (int64_t)e * g.bs_estride, g.ldb, g.ldsb, n0, 0,
                  g.N - n0, kdim, !PT, SW);
  } else {
    // variable K: tile = (e, tm over rows of A = dW rows, tn over rows of B =
    // dW cols).  Work per tile is proportional to the group's tokens, so the
    // experts go largest first (expert_order) and the dispatch follows that
    // tile order, except that within each block of 64 workgroups (8 per XCD,
    // dispatched round-robin) workgroup 64q + 8r + x takes tile 64q + 8x + r:
    // 8 consecutive tiles, which share an A panel, then run on one XCD and
    // share its L2.
    uint32_t tile = blockIdx.x;
    if ((tile | 63u) < g.nblocks) tile = (tile & ~63u) | ((tile & 7u) << 3) | ((tile >> 3) & 7u);
    const uint32_t tn = tile % g.tiles_n, tmg = tile / g.tiles_n;
    const uint32_t tiles_m = (uint32_t)((g.M + TM - 1) / TM);
    // g.K holds the token capacity; padded offsets are multiples of 32, and
    // rounding down keeps every access inside [0, capacity) even for
    // malformed offsets.
    expert_order(g.offsets, g.E, g.K & ~31LL, s_off, s_perm);
    const int e = __builtin_amdgcn_readfirstlane(s_perm[tmg / tiles_m]);
    m0 = (int64_t)(tmg % tiles_m) * TM;
    n0 = (int64_t)tn * TN;
    const int64_t lo_t = s_off[e], hi_t = s_off[e + 1];
    kdim = hi_t > lo_t ? hi_t - lo_t : 0;
    c_rows = g.M - m0;
    group = e;
    A = op_tile(g.a, g.as, g.lda, g.ldsa, m0, lo_t, c_rows, kdim, !PT, SW);
    B = op_tile(g.b, g.bs, g.ldb, g.ldsb, n0, lo_t, g.N - n0, kdim, !PT, SW);
    cbase = static_cast<uint8_t*>(g.c) + (int64_t)e * g.M * g.ldc * (OUT == MXQ_OUT_FP32 ? 4 : 2);
  }

  // Blockwise scale descriptors: the tile's A rows and B block rows (FP32,
  // row strides ldsa / ldsb in floats).
  i32x4 sdA = make_rsrc(g.c, 0), sdB = sdA;
  if constexpr (BLK) {
    const int64_t ra = c_rows < TM ? c_rows : TM;
    const int64_t nbr = (g.N - n0 + 127) / 128 < 2 ? (g.N - n0 + 127) / 128 : 2;
    const int64_t kb = kdim / 128;
    sdA = make_rsrc(g.as + m0 * g.ldsa * 4, (uint32_t)(((ra - 1) * g.ldsa + kb) * 4));
    sdB = make_rsrc(g.bs + (n0 / 128) * g.ldsb * 4, (uint32_t)(((nbr - 1) * g.ldsb + kb) * 4));
  }

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // kdim < 2^31 (the launchers check that a tile's byte offsets fit in 32 bits)
  const uint32_t kdim32 = (uint32_t)kdim;
  const int32_t nsteps = (int32_t)((kdim + TK - 1) / TK);
  const LaneOffsets oA = lane_offsets(A);
  const LaneOffsets oB = SWI ? lane_offsets_gu(B, n0 / 2, g.F) : lane_offsets(B);
  const i32x4 none = make_rsrc(g.c, 0);              // zero range: loads read 0
  const uint32_t lds_codes = lds_addr(smem), lds_scales = lds_addr(ssc);

  const int32_t nstages = (nsteps + 1) / 2;
  // This wavefront's share of the loads of stage u (k-steps 2u, 2u+1) into
  // ring slot u % kSlots.  Dead stages load through the zero-range
  // descriptor.  Only the last stage can be partial: its chunks and scale
  // blocks past kdim load nothing (zero codes, scale code 0 = 2^-127,
  // finite), so they add exact zeros.
  // Code load d (0..7) of this wavefront's share of stage u: row group j = d/2
  // of operand d%2.
  auto stage_dma = [&](int32_t u, int d) {
    const bool live = u < nstages;
    const int j = d >> 1, op = d & 1;
    const i32x4 q = uniform(live ? (op ? B.q : A.q) : none);
    const uint32_t kb = (uint32_t)u * TS;
    const uint32_t slot = (uint32_t)(u & (kSlots - 1));
    const uint32_t kc = oA.kc0 ^ ((j & 1) * 64);
    uint32_t off = kb + kc < kdim32 ? (op ? oB.q[j] : oA.q[j]) + kb : 0x80000000u;
    asm volatile("" : "+v"(off));                   // select the offset, not the load
    dma_b128(q, lds_codes + (slot * 2 + op) * kStage + wave * 4 * 1024 + j * 1024, off);
  };
  auto issue_stage_scales = [&](int32_t u) {
    const bool live = u < nstages;
    const uint32_t slot = (uint32_t)(u & (kSlots - 1));
    if constexpr (BLK) {
      // waves 0-3: one A-row scale per lane; waves 4-7: the two B block rows
      // (lanes alternate between them; the copies land on the same words)
      const uint32_t base = lds_scales + slot * kBlkScaleWords * 4;
      if (wave < 4) {
        const i32x4 d = uniform(live ? sdA : none);
        dma_b32(d, base + wave * 64 * 4,
                (uint32_t)(((int64_t)(wave * 64 + lane) * g.ldsa + u) * 4));
      } else {
        const i32x4 d = uniform(live ? sdB : none);
        dma_b32(d, base + 256 * 4, (uint32_t)(((int64_t)(lane & 1) * g.ldsb + u) * 4));
      }
    }
    if (SBYTES) {
      const i32x4 sa = uniform(live ? A.s : none), sb = uniform(live ? B.s : none);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t st = 2 * (uint32_t)u + ks;
        uint32_t soff = (2 * st + oA.sblk) * 32 < kdim32 ? 2 * st : 0x80000000u;
        asm volatile("" : "+v"(soff));
        const uint32_t sbase = lds_scales + (slot * 2 + ks) * 2 * 2 * TM * 4 + wave * 64 * 4;
        dma_b8(sa, sbase, oA.s + soff);
        dma_b8(sb, sbase + 2 * TM * 4, oB.s + soff);
      }
    }
  };
  auto issue_stage = [&](int32_t u) {
#pragma unroll
    for (int d = 0; d < 8; ++d) stage_dma(u, d);
    issue_stage_scales(u);
  };
  // Scale windows: wavefront w loads rows [64 (w%4), +64) of operand w/4;
  // window j of a row holds its scale bytes [16 j - smis, 16 j + 16 - smis)
  // of the contraction range, in ring slot j % kWinSlots.  Steps 8p .. 8p+7
  // read windows p and p+1; window p+2 is loaded during step 8p+1, into the
  // slot of window p-1.
  const uint32_t lds_win = lds_scales;
  const int wop = wave >> 2;
  uint32_t win_off = (uint32_t)(((wave & 3) * 64 + lane) * (wop ? B.lds : A.lds));
  if (SWI && wop) {
    const int64_t gr = gu_row((wave & 3) * 64 + lane, n0 / 2, g.F);
    win_off = gr >= 0 ? (uint32_t)(gr * B.lds) : kDeadRow;
  }
  const uint32_t nblk = (kdim32 + 31) >> 5;
  // Only windows holding a block of the range are loaded (the others go
  // through the zero-range descriptor): with an empty range the scale
  // pointers may be null.
  auto issue_window = [&](int32_t j) {
    const bool live = nblk > 0 && 16 * (uint32_t)j < nblk + (wop ? B.smis : A.smis);
    const i32x4 d = uniform(live ? (wop ? B.s : A.s) : none);
    const uint32_t slot = (uint32_t)(j % kWinSlots);
    dma_b128(d, lds_win + (slot * 2 + wop) * (kWinBytes / 2) + (wave & 3) * 64 * 16,
             win_off + (uint32_t)(16 * j));
  };

  // Fragments and scales of one k-step for this wavefront's 128 x 64 tile.
  // sa / sb: the scale code each lane passes to the FP8 instruction (block
  // `half` of the step); with XA, sa / sb hold block 0 and sa1 / sb1 block 1.
  struct Frags {
    i32x8 a[MI], b[2];
    uint32_t sa[MI], sb[2];
    uint32_t sa1[MI], sb1[2];
  };
  auto read = [&](int32_t s, Frags& f) {
    const uint32_t slot = (uint32_t)((s >> 1) & (kSlots - 1));
    const int ks = (int)(s & 1);
    const uint8_t* lA = smem + slot * 2 * kStage;
    const uint8_t* lB = lA + kStage;
    const int c0 = ks * 4 + half, c1 = c0 + 2;
#pragma unroll
    for (int i = 0; i < MI; ++i) f.a[i] = read_frag(lA, wm * RW + i * 32 + r32, c0, c1);
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[j] = read_frag(lB, bn + j * 32 + r32, c0, c1);
    if (BLK) {
      const uint32_t* sc = ssc + slot * kBlkScaleWords;
#pragma unroll
      for (int i = 0; i < MI; ++i) f.sa[i] = sc[wm * RW + i * 32 + r32];
      f.sb[0] = f.sb[1] = sc[256 + (bn >> 7)];
    } else if (PT) {
#pragma unroll
      for (int i = 0; i < MI; ++i) f.sa[i] = f.sa1[i] = 127u;
#pragma unroll
      for (int j = 0; j < 2; ++j) f.sb[j] = f.sb1[j] = 127u;
    } else if (SBYTES) {
      const uint32_t* sc = ssc + (slot * 2 + ks) * 2 * 2 * TM;
      const int h0 = XA ? 0 : half;
#pragma unroll
      for (int i = 0; i < MI; ++i) f.sa[i] = sc[(wm * RW + i * 32 + r32) * 2 + h0];
#pragma unroll
      for (int j = 0; j < 2; ++j) f.sb[j] = sc[2 * TM + (bn + j * 32 + r32) * 2 + h0];
      if (XA) {
#pragma unroll
        for (int i = 0; i < MI; ++i) f.sa1[i] = sc[(wm * RW + i * 32 + r32) * 2 + 1];
#pragma unroll
        for (int j = 0; j < 2; ++j) f.sb1[j] = sc[2 * TM + (bn + j * 32 + r32) * 2 + 1];
      }
    } else {
      // block 2s + half of row r: window (smis + 2s + half) / 16 relative to
      // the tile, byte (smis + 2s + half) % 16; blocks past the range read as
      // scale code 0 (their codes are zero).
      const int32_t p = s >> 3;
      const uint32_t ps0 = (uint32_t)(p % kWinSlots), ps1 = ps0 == kWinSlots - 1 ? 0 : ps0 + 1;
      auto window_codes = [&](int hb, uint32_t (&sa)[MI], uint32_t (&sb)[2]) {
        const uint32_t u = (uint32_t)(2 * (s & 7) + hb);
        const bool valid = 2 * (uint32_t)s + hb < nblk;
        const uint32_t ta = A.smis + u, tb = B.smis + u;
        const uint8_t* wA = reinterpret_cast<const uint8_t*>(ssc) +
                            (ta >> 4 ? ps1 : ps0) * kWinBytes + (ta & 15) + (wm * RW + r32) * 16;
        const uint8_t* wB = reinterpret_cast<const uint8_t*>(ssc) +
                            (tb >> 4 ? ps1 : ps0) * kWinBytes + kWinBytes / 2 + (tb & 15) +
                            (bn + r32) * 16;
        const uint32_t keep = valid ? 0xFFu : 0u;   // a mask, so the loads stay unconditional
#pragma unroll
        for (int i = 0; i < MI; ++i) sa[i] = (uint32_t)wA[i * 32 * 16] & keep;
#pragma unroll
        for (int j = 0; j < 2; ++j) sb[j] = (uint32_t)wB[j * 32 * 16] & keep;
      };
      window_codes(XA ? 0 : half, f.sa, f.sb);
      if (XA) window_codes(1, f.sa1, f.sb1);
    }
  };
  // The 8 MFMAs of one k-step; with ISSUE, this wavefront's share of stage
  // u's loads goes in between them (one load after each MFMA, so the loads
  // issue while the matrix core is busy).
  // The asm statements pin the MFMAs inside the compute phase: the operands
  // are "produced" after the phase's opening barrier and the accumulators
  // "consumed" before its closing one.
  auto mma = [&](Frags& f, auto issue_tag, int32_t u) {
    constexpr bool ISSUE = decltype(issue_tag)::value;
    if constexpr (MI == 4)
      asm volatile("" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]),
                   "+v"(f.b[1]), "+v"(f.sa[0]), "+v"(f.sa[1]), "+v"(f.sa[2]), "+v"(f.sa[3]),
                   "+v"(f.sb[0]), "+v"(f.sb[1]));
    else
      asm volatile("" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.sa[0]),
                   "+v"(f.sa[1]), "+v"(f.sb[0]), "+v"(f.sb[1]));
    if constexpr (BLK) {
      // Promotion: each product starts from zero with unit scales, and is
      // added to the accumulators times sa[row] * sb one MFMA later, so the
      // adds of one pair overlap the matrix unit's work on the next.
      float sab[4];
      const float sbv = __builtin_bit_cast(float, f.sb[0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sab[i] = __builtin_bit_cast(float, f.sa[i]) * sbv;
      const f32x16 zero = {};
      f32x16 tp[2];
      static_for<8>([&](auto k) {
        constexpr int K = decltype(k)::value, i = K / 2, j = K % 2;
        tp[K & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], zero, 0, 0, 0,
                                                                    127, 0, 127);
        if constexpr (K > 0) {
          constexpr int P = K - 1, pi = P / 2, pj = P % 2;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            acc[pi][pj][v] = __builtin_fmaf(tp[P & 1][v], sab[pi], acc[pi][pj][v]);
        }
        if constexpr (ISSUE) stage_dma(u, K);
        __builtin_amdgcn_sched_barrier(0);
      });
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[3][1][v] = __builtin_fmaf(tp[1][v], sab[3], acc[3][1][v]);
    } else if constexpr (XA) {
      if constexpr (MI == 4)
        asm volatile("" : "+v"(f.sa1[0]), "+v"(f.sa1[1]), "+v"(f.sa1[2]), "+v"(f.sa1[3]),
                     "+v"(f.sb1[0]), "+v"(f.sb1[1]));
      else
        asm volatile("" : "+v"(f.sa1[0]), "+v"(f.sa1[1]), "+v"(f.sb1[0]), "+v"(f.sb1[1]));
      // Block HB of the step is dwords 4 HB .. 4 HB + 3 of every fragment (16
      // codes per lane); each BF16 instruction takes 8 of them per lane, the
      // same k positions for A and B.  One 32-block at a time keeps the
      // widened operands within the register budget.
      static_for<2>([&](auto hbc) {
        constexpr int HB = decltype(hbc)::value;
        bf16x8 bw[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float sc = e8m0_f32(HB ? f.sb1[j] : f.sb[j]);
          bw[j][0] = widen8_bf16(f.b[j][4 * HB], f.b[j][4 * HB + 1], sc);
          bw[j][1] = widen8_bf16(f.b[j][4 * HB + 2], f.b[j][4 * HB + 3], sc);
        }
        static_for<MI>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          const float sc = e8m0_f32(HB ? f.sa1[I] : f.sa[I]);
          const bf16x8 a0 = widen8_bf16(f.a[I][4 * HB], f.a[I][4 * HB + 1], sc);
          const bf16x8 a1 = widen8_bf16(f.a[I][4 * HB + 2], f.a[I][4 * HB + 3], sc);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[j][0], a0, acc[I][j], 0, 0, 0);
            acc[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[j][1], a1, acc[I][j], 0, 0, 0);
          }
          if constexpr (ISSUE)
            static_for<DPM>([&](auto dd) { stage_dma(u, HB * 4 + I * DPM + decltype(dd)::value); });
        });
      });
    } else {
    static_for<2 * MI>([&](auto k) {
      constexpr int K = decltype(k)::value, i = K / 2, j = K % 2;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.b[j], f.a[i], acc[i][j], 0, 0, 0, (int)f.sb[j], 0, (int)f.sa[i]);
      if constexpr (ISSUE)
        static_for<DPM>([&](auto dd) { stage_dma(u, K * DPM + decltype(dd)::value); });
      __builtin_amdgcn_sched_barrier(0);
    });
    }
    if constexpr (ISSUE) issue_stage_scales(u);
    if constexpr (MI == 4)
      asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]),
                   "+v"(acc[2][0]), "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1]));
    else
      asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));
  };
  // Barrier that nothing is scheduled across; `fence` also completes this
  // wavefront's LDS reads first.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto bare_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  static_assert(kSlots == 2, "slot reuse below assumes a 2-slot ring");
  constexpr int VS = BLK ? 9 : vmem_per_stage<SBYTES>();

  // Ping-pong.  Each k-step s is a memory phase (read step s's fragments
  // from LDS) and a compute phase (8 MFMAs), separated by workgroup
  // barriers.  Group 1 runs one phase behind group 0, so on every SIMD one
  // wavefront multiplies while the other reads LDS.  Phase numbers: group 0
  // reads step s in phase 2s-1 and multiplies it in phase 2s; group 1 one
  // phase later.  Stage t (steps 2t, 2t+1) is read in phases 4t-1 .. 4t+2.
  // Stage t+1 is loaded by group 0 during its compute phase of step 2t
  // (phase 4t) and by group 1 during that of step 2t-1 (phase 4t-1), into
  // the slot of stage t-1 (last read in phase 4t-2), interleaved with the
  // MFMAs; group 0 waits for its share at the end of its compute phase of
  // step 2t+1, group 1 at the end of its memory phase of step 2t+1 (both
  // phase 4t+2), so the stage is visible when first read (phase 4t+3).
  // Stages past the end load zeros into free slots; an odd step count runs
  // one extra step on zero codes.  Scale window p+2 is loaded at steps 8p+1
  // (group 1) and 8p+2 (group 0), into the slot of window p-1 (last read at
  // step 8p-1), and first read at step 8p+8.
  using On = std::true_type;
  using Off = std::false_type;
  if (SWIN) {
    issue_window(0);
    issue_window(1);
  }
  issue_stage(0);
  if (grp == 1) {
    issue_stage(1);                                 // group 0 loads its share at step 0
    wait_vmcnt<VS>();                               // windows 0, 1 and stage 0 landed
  } else {
    wait_vmcnt<0>();
  }
  barrier();
  Frags f;
  if (grp == 0) {
    for (int32_t t = 0; t < nstages; ++t) {
      read(2 * t, f);
      barrier();
      mma(f, On{}, t + 1);
      if (SWIN && (t & 3) == 1) issue_window((t >> 2) + 2);
      barrier();
      read(2 * t + 1, f);
      barrier();
      mma(f, Off{}, 0);
      wait_vmcnt<0>();
      barrier();
    }
    bare_barrier();
  } else {
    bare_barrier();
    for (int32_t t = 0; t < nstages; ++t) {
      read(2 * t, f);
      barrier();
      mma(f, Off{}, 0);
      barrier();
      read(2 * t + 1, f);
      wait_vmcnt<0>();
      barrier();
      mma(f, On{}, t + 2);
      if (SWIN && (t & 3) == 0) issue_window((t >> 2) + 2);
      barrier();
    }
  }
  // Drain the trailing (zero-range) loads before the LDS goes away.
  wait_vmcnt<0>();

  if constexpr (SWI) {
    // ---- SwiGLU epilogue: acc[i][0] holds the gate and acc[i][1] the up
    // values of h columns hb + 8*(v/4) + 4*(lane/32) + v%4 of the tile (hb =
    // bn/2), rows wm*128 + i*32 + lane%32.
    const int64_t F = g.F;
    const int64_t hct = n0 / 2;                     // the tile's first h column
    const int rows_t = c_rows < TM ? (int)c_rows : TM;
    const int hb = bn / 2;
    if constexpr (PT) {
      // per-group scales: the products are scale_a[e] * scale_b[e] * sums
      const float mul = g.pta[group] * g.ptb[group];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] *= mul;
    }
    barrier();                                      // the k loop's LDS reads are done
    if (cbase) {
      // The gate/up product in BF16 (gate columns to [hct, +128), up columns
      // to [F + hct, +128)), staged as [256 rows][128 gate | 128 up], stored
      // non-temporally like the plain product's output.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ml = wm * 128 + i * 32 + r32, cl = hb + q * 8 + half * 4;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x16& v = acc[i][j];
            *reinterpret_cast<uint2*>(smem + ml * kCStride + (j * 128 + cl) * 2) =
                make_uint2(bf16x2_bits(v[4 * q], v[4 * q + 1]), bf16x2_bits(v[4 * q + 2], v[4 * q + 3]));
          }
        }
      barrier();
      const int rsub = lane >> 5, col = lane & 31;
      const int64_t hc = hct + (col & 15) * 8;
      const int64_t gcol = ((col >> 4) ? F : 0) + hc;
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int row = wave * 32 + it * 2 + rsub;
        if (row < rows_t && hc < F) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(smem + row * kCStride + col * 16);
          __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(
              static_cast<uint8_t*>(cbase) + (m0 + row) * g.ldc * 2 + gcol * 2));
        }
      }
      barrier();
    }
    if constexpr (PT) {
      // h in BF16 (the per-group quantizer's input), staged as [256 rows][128
      // columns], and the group's largest |h| as an FP32 bit pattern
      // (magnitudes order as integers; NaN above Inf above finite values).
      u16x2 am2 = __builtin_bit_cast(u16x2, 0u);    // largest |h| bit patterns, per half
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ml = wm * 128 + i * 32 + r32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float hv[4];
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) hv[e4] = silu_f32(acc[i][0][4 * q + e4]) * acc[i][1][4 * q + e4];
          const uint2 u = make_uint2(bf16x2_bits(hv[0], hv[1]), bf16x2_bits(hv[2], hv[3]));
          const bool live = ml < rows_t && hct + hb + q * 8 + half * 4 < F;
          if (live) {
            am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(u16x2, u.x & 0x7FFF7FFFu));
            am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(u16x2, u.y & 0x7FFF7FFFu));
          }
          *reinterpret_cast<uint2*>(smem + ml * kCStride + (hb + q * 8 + half * 4) * 2) = u;
        }
      }
      uint32_t am = am2.x > am2.y ? am2.x : am2.y;
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)am, sh, 64);
        am = am > o ? am : o;
      }
      __shared__ uint32_t s_am[kThreads / 64];
      if (lane == 0) s_am[wave] = am;
      barrier();
      const int rsub = lane >> 4, col = lane & 15;
      const int64_t hc = hct + col * 8;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = wave * 32 + it * 4 + rsub;
        if (row < rows_t && hc < F) {
          const uint4 v = *reinterpret_cast<const uint4*>(smem + row * kCStride + col * 16);
          *reinterpret_cast<uint4*>(g.h + (m0 + row) * g.ldh + hc) = v;
        }
      }
      // One atomic per tile, last, so that nothing waits for it (a workgroup
      // barrier would first complete its round trip to the contended address).
      if (t == 0) {
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) am = am > s_am[w] ? am : s_am[w];
        if (am != 0u)
          __hip_atomic_fetch_max(g.hamax + group, am << 16, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    } else {
    // h in FP32, staged as [256 rows][128 columns] (rows of kCStride bytes);
    // rows past the group are zero: the column copy's padding.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ml = wm * 128 + i * 32 + r32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 hv;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          hv[e4] = ml < rows_t ? silu_f32(acc[i][0][4 * q + e4]) * acc[i][1][4 * q + e4] : 0.0f;
        *reinterpret_cast<f32x4*>(smem + ml * kCStride + (hb + q * 8 + half * 4) * 4) = hv;
      }
    }
    barrier();
    // Row copy: (row, 32-column block) items, two per lane.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int item = t + kThreads * k;
      const int row = item >> 2, blk = item & 3;
      float v[32];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(smem + row * kCStride + blk * 128 + c * 16);
        v[4 * c] = x[0]; v[4 * c + 1] = x[1]; v[4 * c + 2] = x[2]; v[4 * c + 3] = x[3];
      }
      uint32_t w[8];
      const uint32_t code = mx_block_f32(v, w);
      const int64_t hc = hct + blk * 32;
      if (row < rows_t && hc < F) {
        uint8_t* d = g.hq + (m0 + row) * g.ldhq + hc;
        *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(d + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        g.hs[(m0 + row) * g.ldhs + (hc >> 5)] = (uint8_t)code;
      }
    }
    // Column copy: (column, 32-row block) items, two per lane, at the
    // group's padded position.
    int64_t pe = 0;
    for (int gi = lane; gi < group; gi += 64) {
      const int64_t d = s_off[gi + 1] - s_off[gi];
      pe += d > 0 ? (d + 31) & ~31LL : 0;
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) pe += __shfl_xor(pe, sh, 64);
    const int64_t pbase = pe + (m0 - s_off[group]);
    const int rows_p = (rows_t + 31) & ~31;
    const float* hst = reinterpret_cast<const float*>(smem);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int item = t + kThreads * k;
      const int col = item & 127, blk = item >> 7;
      float v[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) v[r] = hst[(blk * 32 + r) * (kCStride / 4) + col];
      uint32_t w[8];
      const uint32_t code = mx_block_f32(v, w);
      const int64_t hc = hct + col, pcol = pbase + blk * 32;
      if (blk * 32 < rows_p && hc < F && pcol + 32 <= g.hcap) {
        uint8_t* d = g.hqT + hc * g.ldhqT + pcol;
        *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(d + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        g.hsT[hc * g.ldhsT + (pcol >> 5)] = (uint8_t)code;
      }
    }
    return;
    }
  }

  // ---- epilogue: acc[i][j] holds C[m = wm*128 + i*32 + lane%32]
  //                [n = bn + j*32 + 8*(v/4) + 4*(lane/32) + v%4]
  float mul = 1.0f;
  if (PT) mul = g.pta[group] * g.ptb[group];
  const int64_t c_cols = g.N - n0;                  // valid columns (may exceed TN)
  // Per-tensor dense product with camax: the largest |C| of the tile's valid
  // outputs as stored, kept as an FP32 bit pattern with the sign cleared
  // (patterns order as magnitudes; NaN above Inf above finite values) and
  // merged by one atomic max per workgroup after its stores (one per
  // wavefront queues up at the single address: 20% on the dense FFN GEMM).  Scaling by
  // |mul| and rounding (to FP32, then to BF16) are monotonic, so that is the
  // largest accumulator magnitude scaled and rounded once.  Accumulators of
  // rows and columns past the output are exact zeros (zero codes), but
  // partial tiles mask them anyway.
  uint32_t camax = 0;
  if constexpr (KIND == kDense && PT) {
    if (g.camax) {
      if (c_rows >= TMR && c_cols >= TN) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              // through a float: a bit_cast of a vector element lvalue reads element 0
              const float x = acc[i][j][v];
              const uint32_t m = __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu;
              camax = camax > m ? camax : m;
            }
      } else {
        const int cr = (int)(c_rows < TMR ? c_rows : TMR), cc = (int)(c_cols < TN ? c_cols : TN);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const bool rok = wm * RW + i * 32 + r32 < cr;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int nl = bn + j * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
              const float x = acc[i][j][v];
              const uint32_t m = rok && nl < cc ? __builtin_bit_cast(uint32_t, x) & 0x7FFFFFFFu : 0u;
              camax = camax > m ? camax : m;
            }
        }
      }
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)camax, sh, 64);
        camax = camax > o ? camax : o;
      }
      const float f = __builtin_bit_cast(float, camax) * __builtin_fabsf(mul);
      camax = (OUT == MXQ_OUT_BF16 ? bf16x2_bits(f, 0.0f) << 16 : __builtin_bit_cast(uint32_t, f)) &
              0x7FFFFFFFu;
      if (lane == 0) s_cmax[wave] = camax;          // read after the epilogue's next barrier
    }
  }
  auto merge_camax = [&]() {
    if constexpr (KIND == kDense && PT) {
      if (g.camax && t == 0) {
        uint32_t m = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) m = m > s_cmax[w] ? m : s_cmax[w];
        if (m != 0u) __hip_atomic_fetch_max(g.camax, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  // Staged when the tile's valid columns are whole 16-byte chunks: a full
  // tile, or a partial one of an output whose width is a multiple of 8.
  const bool staged = OUT == MXQ_OUT_BF16 && (c_cols >= TN || (g.N & 7) == 0) &&
                      (g.ldc & 7) == 0 && (reinterpret_cast<uintptr_t>(cbase) & 15) == 0;
  if (staged) {
    // BF16 tile: round into LDS (rows of kCStride bytes; the 16
    // bytes of padding spread 16 consecutive rows over the banks), then store
    // whole rows, 16 bytes per lane, two 512-byte rows per instruction.  The
    // stores are non-temporal: the output is not read again by this kernel,
    // and kept out of the caches it leaves them to the operand panels.
    barrier();                                      // every wave's loads drained
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ml = wm * RW + i * 32 + r32, nl = bn + j * 32 + q * 8 + half * 4;
          const f32x16& v = acc[i][j];
          *reinterpret_cast<uint2*>(smem + ml * kCStride + nl * 2) =
              make_uint2(bf16x2_bits(v[4 * q] * mul, v[4 * q + 1] * mul),
                         bf16x2_bits(v[4 * q + 2] * mul, v[4 * q + 3] * mul));
        }
    barrier();
    const int rsub = lane >> 5, col = lane & 31;
#pragma unroll
    for (int it = 0; it < TMR / 16; ++it) {
      const int row = wave * (TMR / 8) + it * 2 + rsub;
      if (row < c_rows && col * 8 < c_cols) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(smem + row * kCStride + col * 16);
        __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(static_cast<uint8_t*>(cbase) +
                                    (m0 + row) * g.ldc * 2 + n0 * 2 + col * 16));
      }
    }
    merge_camax();
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t ml = wm * RW + i * 32 + r32;
    if (ml >= c_rows) continue;
    const int64_t m = m0 + ml;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + bn + j * 32 + q * 8 + half * 4;
        store4<OUT>(cbase, g.ldc, m, n, g.N, acc[i][j][4 * q] * mul,
                    acc[i][j][4 * q + 1] * mul, acc[i][j][4 * q + 2] * mul,
                    acc[i][j][4 * q + 3] * mul);
      }
    }
  }
  if constexpr (KIND == kDense && PT) {
    if (g.camax) barrier();                         // every wavefront's s_cmax written
  }
  merge_camax();
}

template <int KIND, bool PT, int OUT, bool SW, bool XA>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmArgs g) {
  gemm_body<KIND, PT, OUT, SW, false, false, XA>(g);
}

// Dense GEMMs with few tiles: 128-row tiles (each wavefront 64 x 64).
template <bool PT, int OUT, bool SW, bool XA>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_rows128(GemmArgs g) {
  gemm_body<kDense, PT, OUT, SW, false, false, XA, 2>(g);
}

template <bool SW>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_swiglu(GemmArgs g) {
  gemm_body<kVarM, false, MXQ_OUT_BF16, SW, true, false>(g);
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_swiglu_pg(GemmArgs g) {
  gemm_body<kVarM, true, MXQ_OUT_BF16, false, true, false>(g);
}

template <int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_blockwise(GemmArgs g) {
  gemm_body<kDense, false, OUT, false, false, true>(g);
}

__global__ void k_clear_u32(uint32_t* p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace mxq

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

using namespace mxq;

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <int KIND, bool PT, bool SW, bool XA>
static void launch_kernel(const GemmArgs& g, uint32_t blocks, int out, hipStream_t stream) {
  if (KIND == kDense && g.rows128) {
    if (out == MXQ_OUT_BF16)
      hipLaunchKernelGGL((k_gemm_rows128<PT, MXQ_OUT_BF16, SW, XA>), dim3(blocks),
                         dim3(kThreads), 0, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_rows128<PT, MXQ_OUT_FP32, SW, XA>), dim3(blocks),
                         dim3(kThreads), 0, stream, g);
  } else if (out == MXQ_OUT_BF16)
    hipLaunchKernelGGL((k_gemm<KIND, PT, MXQ_OUT_BF16, SW, XA>), dim3(blocks), dim3(kThreads), 0,
                       stream, g);
  else
    hipLaunchKernelGGL((k_gemm<KIND, PT, MXQ_OUT_FP32, SW, XA>), dim3(blocks), dim3(kThreads), 0,
                       stream, g);
}

template <int KIND, bool PT, bool SW>
static void launch_accum(const GemmArgs& g, uint32_t blocks, int out, int accum,
                         hipStream_t stream) {
  if (accum == MXQ_ACC_FP32)
    launch_kernel<KIND, PT, SW, true>(g, blocks, out, stream);
  else
    launch_kernel<KIND, PT, SW, false>(g, blocks, out, stream);
}

// A dense GEMM whose 256-row tiles would fill at most half the CUs runs on
// 128-row tiles (twice the workgroups, each with half the matrix work).
// Measured on MI355X: 1024 x 2048 x 2048 23.0 -> 18.8 us, 4096 x 2048 x 2048
// 25.6 -> 23.5 us; with more tiles than CUs the 256-row tiles are faster
// (4096 x 2816 x 2048: 176 tiles, 28.6 against 40.9 us).
constexpr int64_t kRows128MaxTiles = 128;
static uint32_t rows128(int64_t M, uint32_t tiles_n) {
  return sat_mul(sat_add(M, TM - 1) / TM, tiles_n) <= kRows128MaxTiles ? 1u : 0u;
}

// Scale windows need both operands' scale row strides to be multiples of 16.
template <int KIND, bool PT>
static int launch_gemm(GemmArgs& g, int64_t blocks, int out, int accum, hipStream_t stream) {
  if (blocks == 0) return MXQ_OK;
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  g.nblocks = (uint32_t)blocks;
  if constexpr (PT)
    launch_accum<KIND, PT, false>(g, (uint32_t)blocks, out, accum, stream);
  else if (g.ldsa % 16 == 0 && g.ldsb % 16 == 0)
    launch_accum<KIND, PT, true>(g, (uint32_t)blocks, out, accum, stream);
  else
    launch_accum<KIND, PT, false>(g, (uint32_t)blocks, out, accum, stream);
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

// Largest size or stride any GEMM accepts (2^39: far past any tensor that
// fits in memory; it keeps tile counts and byte offsets of the checks in range).
constexpr int64_t kMaxDim = int64_t(1) << 39;

static int check_common(int64_t M, int64_t N, int64_t K, int64_t ldc, int out, int accum) {
  if (M < 0 || N < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || ldc > kMaxDim) return MXQ_ERR_SHAPE;
  if (out != MXQ_OUT_BF16 && out != MXQ_OUT_FP32) return MXQ_ERR_ARG;
  if (accum != MXQ_ACC_MFMA_FP8 && accum != MXQ_ACC_FP32) return MXQ_ERR_ARG;
  if (ldc < N) return MXQ_ERR_SHAPE;
  return MXQ_OK;
}

// Buffer offsets are 32-bit: one tile of rows must fit.
static bool fits32(int64_t ld, int64_t K) {
  return sat_add(sat_mul(ld, TM + 1), K) < 0x7FFFFFFFLL;
}

// Tiles of `n` rows (an upper bound for sizes near the int64 limit, which the
// size checks reject anyway).
static int64_t tiles_of(int64_t n, int64_t t) { return sat_add(n, t - 1) / t; }

static int check_operand(const uint8_t* q, const void* s, int64_t ld, int64_t lds, int64_t K,
                         bool mx) {
  if (!q || !s) return MXQ_ERR_NULL;
  if (ld < K || (mx && lds < K / 32)) return MXQ_ERR_SHAPE;
  if (!fits32(ld, K) || (mx && !fits32(lds, K / 32))) return MXQ_ERR_SHAPE;
  if (ld % 16 != 0 || !aligned(q, 16)) return MXQ_ERR_ALIGN;
  if (!mx && !aligned(s, 4)) return MXQ_ERR_ALIGN;
  return MXQ_OK;
}

static GemmArgs make_args(const uint8_t* a, const uint8_t* as, int64_t lda, int64_t ldsa,
                          const uint8_t* b, const uint8_t* bs, int64_t ldb, int64_t ldsb,
                          int64_t M, int64_t N, int64_t K, void* c, int64_t ldc) {
  GemmArgs g{};
  g.a = a; g.as = as; g.lda = lda; g.ldsa = ldsa;
  g.b = b; g.bs = bs; g.ldb = ldb; g.ldsb = ldsb;
  g.M = M; g.N = N; g.K = K; g.c = c; g.ldc = ldc;
  g.tiles_n = (uint32_t)((N + TN - 1) / TN);
  return g;
}

extern "C" int mx_gemm(const uint8_t* a, const uint8_t* a_scale, int64_t lda, int64_t ldsa,
                       const uint8_t* b, const uint8_t* b_scale, int64_t ldb, int64_t ldsb,
                       int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, int out_dtype,
                       int accum, hipStream_t stream) {
  int st = check_common(M, N, K, ldc, out_dtype, accum);
  if (st) return st;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!c) return MXQ_ERR_NULL;
  if (K % 32 != 0) return MXQ_ERR_SHAPE;
  if (K > 0) {
    if ((st = check_operand(a, a_scale, lda, ldsa, K, true))) return st;
    if ((st = check_operand(b, b_scale, ldb, ldsb, K, true))) return st;
  }
  GemmArgs g = make_args(a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, M, N, K, c, ldc);
  g.rows128 = rows128(M, g.tiles_n);
  const int64_t tiles_m = tiles_of(M, g.rows128 ? TM / 2 : TM);
  return launch_gemm<kDense, false>(g, sat_mul(tiles_m, g.tiles_n), out_dtype, accum,
                                    stream);
}

// c_amax (or null): cleared, then max |C| of the outputs merged into it.
static int per_tensor_gemm(const uint8_t* a, const float* a_scale, int64_t lda,
                           const uint8_t* b, const float* b_scale, int64_t ldb, int64_t M,
                           int64_t N, int64_t K, void* c, int64_t ldc, int out_dtype, int accum,
                           float* c_amax, hipStream_t stream) {
  int st = check_common(M, N, K, ldc, out_dtype, accum);
  if (st) return st;
  if (c_amax && !aligned(c_amax, 4)) return MXQ_ERR_ALIGN;
  if (M > 0 && N > 0) {
    if (!c || !a_scale || !b_scale) return MXQ_ERR_NULL;
    if (K % 32 != 0) return MXQ_ERR_SHAPE;
    if (K > 0) {
      if ((st = check_operand(a, a_scale, lda, 0, K, false))) return st;
      if ((st = check_operand(b, b_scale, ldb, 0, K, false))) return st;
    }
  }
  if (c_amax) {
    // a fill kernel rather than a memset, so that the call can be captured
    // in a HIP graph
    hipLaunchKernelGGL(k_clear_u32, dim3(1), dim3(64), 0, stream,
                       reinterpret_cast<uint32_t*>(c_amax), 1);
    if (hipGetLastError() != hipSuccess) return MXQ_ERR_HIP;
  }
  if (M == 0 || N == 0) return MXQ_OK;
  GemmArgs g = make_args(a, nullptr, lda, 0, b, nullptr, ldb, 0, M, N, K, c, ldc);
  g.pta = a_scale; g.ptb = b_scale;
  g.camax = reinterpret_cast<uint32_t*>(c_amax);
  g.rows128 = rows128(M, g.tiles_n);
  const int64_t tiles_m = tiles_of(M, g.rows128 ? TM / 2 : TM);
  return launch_gemm<kDense, true>(g, sat_mul(tiles_m, g.tiles_n), out_dtype, accum,
                                   stream);
}

extern "C" int fp8_gemm_per_tensor(const uint8_t* a, const float* a_scale, int64_t lda,
                                   const uint8_t* b, const float* b_scale, int64_t ldb,
                                   int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                                   int out_dtype, int accum, hipStream_t stream) {
  return per_tensor_gemm(a, a_scale, lda, b, b_scale, ldb, M, N, K, c, ldc, out_dtype, accum,
                         nullptr, stream);
}

extern "C" int fp8_gemm_per_tensor_amax(const uint8_t* a, const float* a_scale, int64_t lda,
                                        const uint8_t* b, const float* b_scale, int64_t ldb,
                                        int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                                        int out_dtype, int accum, float* c_amax,
                                        hipStream_t stream) {
  if (!c_amax) return MXQ_ERR_NULL;
  return per_tensor_gemm(a, a_scale, lda, b, b_scale, ldb, M, N, K, c, ldc, out_dtype, accum,
                         c_amax, stream);
}

extern "C" int fp8_gemm_blockwise(const uint8_t* a, const float* a_scales, int64_t lda,
                                  int64_t ldsa, const uint8_t* b, const float* b_scales,
                                  int64_t ldb, int64_t ldsb, int64_t M, int64_t N, int64_t K,
                                  void* c, int64_t ldc, int out_dtype, int accum,
                                  hipStream_t stream) {
  int st = check_common(M, N, K, ldc, out_dtype, accum);
  if (st) return st;
  if (K % 128 != 0) return MXQ_ERR_SHAPE;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!c) return MXQ_ERR_NULL;
  if (K > 0) {
    if ((st = check_operand(a, a_scales, lda, 0, K, false))) return st;
    if ((st = check_operand(b, b_scales, ldb, 0, K, false))) return st;
    if (ldsa < K / 128 || ldsb < K / 128) return MXQ_ERR_SHAPE;
    // 32-bit scale offsets: a tile's 256 A rows and two B block rows
    if (sat_add(sat_mul(ldsa, 4 * (TM + 1)), K) >= (1LL << 30) ||
        sat_add(sat_mul(ldsb, 4 * 3), K) >= (1LL << 30))
      return MXQ_ERR_SHAPE;
  }
  if (accum != MXQ_ACC_MFMA_FP8) return MXQ_ERR_ARG;
  GemmArgs g = make_args(a, reinterpret_cast<const uint8_t*>(a_scales), lda, ldsa, b,
                         reinterpret_cast<const uint8_t*>(b_scales), ldb, ldsb, M, N, K, c, ldc);
  const int64_t blocks = sat_mul(tiles_of(M, TM), g.tiles_n);
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  g.nblocks = (uint32_t)blocks;
  if (out_dtype == MXQ_OUT_BF16)
    hipLaunchKernelGGL(k_gemm_blockwise<MXQ_OUT_BF16>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, g);
  else
    hipLaunchKernelGGL(k_gemm_blockwise<MXQ_OUT_FP32>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, g);
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

extern "C" int mx_grouped_gemm(const uint8_t* a, const uint8_t* a_scale, int64_t lda, int64_t ldsa,
                               const uint8_t* b, const uint8_t* b_scale, int64_t ldb, int64_t ldsb,
                               int64_t b_estride, int64_t bs_estride,
                               const int64_t* offsets, int32_t E, int64_t M, int64_t N, int64_t K,
                               void* c, int64_t ldc, int out_dtype, int accum,
                               hipStream_t stream) {
  int st = check_common(M, N, K, ldc, out_dtype, accum);
  if (st) return st;
  if (E < 1 || E > kMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets) return MXQ_ERR_NULL;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!c) return MXQ_ERR_NULL;
  if (K % 32 != 0) return MXQ_ERR_SHAPE;
  if (K > 0) {
    if ((st = check_operand(a, a_scale, lda, ldsa, K, true))) return st;
    if ((st = check_operand(b, b_scale, ldb, ldsb, K, true))) return st;
  }
  if (b_estride < 0 || bs_estride < 0) return MXQ_ERR_SHAPE;
  if (b_estride % 16 != 0) return MXQ_ERR_ALIGN;
  GemmArgs g = make_args(a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, M, N, K, c, ldc);
  g.b_estride = b_estride; g.bs_estride = bs_estride;
  g.offsets = offsets; g.E = E;
  const int64_t mtiles = tiles_of(M, TM) + E;        // upper bound over all group splits
  return launch_gemm<kVarM, false>(g, sat_mul(mtiles, g.tiles_n), out_dtype, accum, stream);
}

extern "C" int mx_grouped_gemm_swiglu(const uint8_t* a, const uint8_t* a_scale, int64_t lda,
                                      int64_t ldsa, const uint8_t* b, const uint8_t* b_scale,
                                      int64_t ldb, int64_t ldsb, int64_t b_estride,
                                      int64_t bs_estride, const int64_t* offsets, int32_t E,
                                      int64_t M, int64_t F, int64_t K, void* gu, int64_t ldgu,
                                      uint8_t* hq, int64_t ldhq, uint8_t* hs, int64_t ldhs,
                                      uint8_t* hqT, int64_t ldhqT, uint8_t* hsT, int64_t ldhsT,
                                      int64_t M_cap, int64_t* offsets_padded,
                                      hipStream_t stream) {
  if (M < 0 || F < 0 || K < 0 || M_cap < 0) return MXQ_ERR_SHAPE;
  if (M > kMaxDim || F > kMaxDim || K > kMaxDim || M_cap > kMaxDim) return MXQ_ERR_SHAPE;
  if (E < 1 || E > kMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets) return MXQ_ERR_NULL;
  if (F % 32 != 0 || K % 32 != 0 || M_cap % 32 != 0) return MXQ_ERR_SHAPE;
  // h's column copy must hold every row after each group is padded to 32
  if (M > 0 && M_cap < M + 31LL * E) return MXQ_ERR_SHAPE;
  if (F == 0) return MXQ_OK;
  if (M > 0 && (!hq || !hs || (M_cap > 0 && (!hqT || !hsT)))) return MXQ_ERR_NULL;
  if (ldhq < F || ldhs < F / 32 || ldhqT < M_cap || ldhsT < M_cap / 32) return MXQ_ERR_SHAPE;
  if (gu && ldgu < 2 * F) return MXQ_ERR_SHAPE;
  int st;
  if (K > 0) {
    // with M == 0 no operand row is read (only the padded offsets are written)
    if (M > 0 && (st = check_operand(a, a_scale, lda, ldsa, K, true))) return st;
    if ((st = check_operand(b, b_scale, ldb, ldsb, K, true))) return st;
  }
  if (b_estride < 0 || bs_estride < 0) return MXQ_ERR_SHAPE;
  // One descriptor spans an expert's 2F weight rows.
  if (sat_add(sat_mul(2 * F, ldb), K) >= (1LL << 30) ||
      sat_add(sat_mul(2 * F, ldsb), K / 32 + 16) >= (1LL << 30))
    return MXQ_ERR_SHAPE;
  if (b_estride % 16 != 0 || ldhq % 16 != 0 || ldhqT % 16 != 0 || !aligned(hq, 16) ||
      !aligned(hqT, 16))
    return MXQ_ERR_ALIGN;
  if (gu && (ldgu % 8 != 0 || !aligned(gu, 16))) return MXQ_ERR_ALIGN;
  GemmArgs g = make_args(a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, M, 2 * F, K, gu, ldgu);
  g.b_estride = b_estride; g.bs_estride = bs_estride;
  g.offsets = offsets; g.E = E;
  g.F = F;
  g.hq = hq; g.hs = hs; g.ldhq = ldhq; g.ldhs = ldhs;
  g.hqT = hqT; g.hsT = hsT; g.ldhqT = ldhqT; g.ldhsT = ldhsT;
  g.hcap = M_cap;
  g.poff = offsets_padded;
  // Every workgroup past the group tiles exits at once; with M == 0 the first
  // one still writes the padded offsets.
  const int64_t blocks = sat_mul(tiles_of(M, TM) + E, g.tiles_n);
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  g.nblocks = (uint32_t)blocks;
  if (ldsa % 16 == 0 && ldsb % 16 == 0)
    hipLaunchKernelGGL((k_gemm_swiglu<true>), dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                       g);
  else
    hipLaunchKernelGGL((k_gemm_swiglu<false>), dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, g);
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

extern "C" int fp8_grouped_gemm_per_group_swiglu(const uint8_t* a, const float* a_scales,
                                                 int64_t lda, const uint8_t* b,
                                                 const float* b_scales, int64_t ldb,
                                                 int64_t b_estride, const int64_t* offsets,
                                                 int32_t E, int64_t M, int64_t F, int64_t K,
                                                 void* gu, int64_t ldgu, uint16_t* h,
                                                 int64_t ldh, float* h_amax,
                                                 hipStream_t stream) {
  if (M < 0 || F < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (M > kMaxDim || F > kMaxDim || K > kMaxDim) return MXQ_ERR_SHAPE;
  if (E < 1 || E > kMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets || !a_scales || !b_scales || !h_amax) return MXQ_ERR_NULL;
  if (F % 32 != 0 || K % 32 != 0) return MXQ_ERR_SHAPE;
  if (M > 0 && F > 0 && !h) return MXQ_ERR_NULL;
  if (F > 0 && (ldh < F || (gu && ldgu < 2 * F))) return MXQ_ERR_SHAPE;
  int st;
  if (K > 0 && M > 0 && F > 0) {
    if ((st = check_operand(a, a_scales, lda, 0, K, false))) return st;
    if ((st = check_operand(b, b_scales, ldb, 0, K, false))) return st;
  }
  if (b_estride < 0) return MXQ_ERR_SHAPE;
  if (sat_add(sat_mul(2 * F, ldb), K) >= (1LL << 30)) return MXQ_ERR_SHAPE;
  if (b_estride % 16 != 0 || ldh % 8 != 0 || !aligned(h, 16)) return MXQ_ERR_ALIGN;
  if (gu && (ldgu % 8 != 0 || !aligned(gu, 16))) return MXQ_ERR_ALIGN;
  // every group's amax starts at zero (also for groups without rows)
  hipLaunchKernelGGL(k_clear_u32, dim3((uint32_t)((E + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(h_amax), E);
  if (hipGetLastError() != hipSuccess) return MXQ_ERR_HIP;
  if (M == 0 || F == 0) return MXQ_OK;
  GemmArgs g = make_args(a, nullptr, lda, 0, b, nullptr, ldb, 0, M, 2 * F, K, gu, ldgu);
  g.b_estride = b_estride;
  g.pta = a_scales; g.ptb = b_scales;
  g.offsets = offsets; g.E = E;
  g.F = F;
  g.h = h; g.ldh = ldh;
  g.hamax = reinterpret_cast<uint32_t*>(h_amax);
  const int64_t blocks = sat_mul(tiles_of(M, TM) + E, g.tiles_n);
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  g.nblocks = (uint32_t)blocks;
  hipLaunchKernelGGL(k_gemm_swiglu_pg, dim3((uint32_t)blocks), dim3(kThreads), 0, stream, g);
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

extern "C" int fp8_grouped_gemm_per_group(const uint8_t* a, const float* a_scales, int64_t lda,
                                          const uint8_t* b, const float* b_scales, int64_t ldb,
                                          int64_t b_estride, const int64_t* offsets, int32_t E,
                                          int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                                          int out_dtype, int accum, hipStream_t stream) {
  int st = check_common(M, N, K, ldc, out_dtype, accum);
  if (st) return st;
  if (E < 1 || E > kMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets || !a_scales || !b_scales) return MXQ_ERR_NULL;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!c) return MXQ_ERR_NULL;
  if (K % 32 != 0) return MXQ_ERR_SHAPE;
  if (K > 0) {
    if ((st = check_operand(a, a_scales, lda, 0, K, false))) return st;
    if ((st = check_operand(b, b_scales, ldb, 0, K, false))) return st;
  }
  if (b_estride < 0) return MXQ_ERR_SHAPE;
  if (b_estride % 16 != 0) return MXQ_ERR_ALIGN;
  GemmArgs g = make_args(a, nullptr, lda, 0, b, nullptr, ldb, 0, M, N, K, c, ldc);
  g.b_estride = b_estride;
  g.pta = a_scales; g.ptb = b_scales;
  g.offsets = offsets; g.E = E;
  const int64_t mtiles = tiles_of(M, TM) + E;        // upper bound over all group splits
  return launch_gemm<kVarM, true>(g, sat_mul(mtiles, g.tiles_n), out_dtype, accum, stream);
}

extern "C" int fp8_grouped_gemm_wgrad_per_group(const uint8_t* at, const float* a_scales,
                                                int64_t lda_t, const uint8_t* bt,
                                                const float* b_scales, int64_t ldb_t,
                                                const int64_t* offsets_padded, int32_t E,
                                                int64_t N, int64_t K, void* c, int64_t ldc,
                                                int out_dtype, int accum, hipStream_t stream) {
  int st = check_common(N, K, 0, ldc, out_dtype, accum);
  if (st) return st;
  if (E < 1 || E > kMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets_padded || !a_scales || !b_scales) return MXQ_ERR_NULL;
  if (N == 0 || K == 0) return MXQ_OK;
  if (!c || !at || !bt) return MXQ_ERR_NULL;
  if (lda_t % 16 != 0 || ldb_t % 16 != 0 || !aligned(at, 16) || !aligned(bt, 16))
    return MXQ_ERR_ALIGN;
  const int64_t cap = lda_t < ldb_t ? lda_t : ldb_t;    // token capacity of both operands
  if (!fits32(lda_t, cap) || !fits32(ldb_t, cap)) return MXQ_ERR_SHAPE;
  GemmArgs g = make_args(at, nullptr, lda_t, 0, bt, nullptr, ldb_t, 0, N, K, cap, c, ldc);
  g.pta = a_scales; g.ptb = b_scales;
  g.offsets = offsets_padded; g.E = E;
  const int64_t blocks = sat_mul(sat_mul(E, tiles_of(N, TM)), g.tiles_n);
  return launch_gemm<kVarK, true>(g, blocks, out_dtype, accum, stream);
}

extern "C" int mx_grouped_gemm_wgrad(const uint8_t* at, const uint8_t* at_scale, int64_t lda_t,
                                     int64_t ldsa_t, const uint8_t* bt, const uint8_t* bt_scale,
                                     int64_t ldb_t, int64_t ldsb_t, const int64_t* offsets_padded,
                                     int32_t E, int64_t N, int64_t K, void* c, int64_t ldc,
                                     int out_dtype, int accum, hipStream_t stream) {
  int st = check_common(N, K, 0, ldc, out_dtype, accum);
  if (st) return st;
  if (E < 1 || E > kMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets_padded) return MXQ_ERR_NULL;
  if (N == 0 || K == 0) return MXQ_OK;
  if (!c || !at || !at_scale || !bt || !bt_scale) return MXQ_ERR_NULL;
  if (lda_t % 16 != 0 || ldb_t % 16 != 0 || !aligned(at, 16) || !aligned(bt, 16))
    return MXQ_ERR_ALIGN;
  // Token capacity: columns readable in both operands.
  int64_t cap = lda_t < ldb_t ? lda_t : ldb_t;
  const int64_t scap = (ldsa_t < ldsb_t ? ldsa_t : ldsb_t) * 32;
  if (scap < cap) cap = scap;
  if (!fits32(lda_t, cap) || !fits32(ldb_t, cap) || !fits32(ldsa_t, cap / 32) ||
      !fits32(ldsb_t, cap / 32))
    return MXQ_ERR_SHAPE;
  // For this kind: M = rows of dW (N), N = columns of dW (K), K = token capacity.
  GemmArgs g = make_args(at, at_scale, lda_t, ldsa_t, bt, bt_scale, ldb_t, ldsb_t, N, K, cap, c,
                         ldc);
  g.offsets = offsets_padded; g.E = E;
  const int64_t blocks = sat_mul(sat_mul(E, tiles_of(N, TM)), g.tiles_n);
  return launch_gemm<kVarK, false>(g, blocks, out_dtype, accum, stream);
}
