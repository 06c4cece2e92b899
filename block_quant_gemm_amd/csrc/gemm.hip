// MX-FP8 GEMM kernels for gfx950 (dense, grouped variable-M, grouped
// variable-K) on the block-scaled FP8 MFMA, with their C-ABI launchers.
//
// Method: "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" §8 (forward, dgrad and
// wgrad are one quantized matmul each on the copy blocked along the
// contraction dim), §5.2 and §13.4 (grouped matmul over per-expert token
// groups); "Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度" §五
// (FP32 accumulation, one rounding to BF16 at the end).
//
// Tiling.  A workgroup of 256 lanes (4 wavefronts, 2 x 2) computes a 256 x 256
// output tile; each wavefront owns 128 x 128 = 4 x 4 MFMA tiles of 32 x 32
// (256 FP32 accumulators per lane).  The K loop steps 64 codes (two
// 32-blocks, one MFMA deep) at a time.  Operand tiles go from HBM straight
// into LDS with buffer_load_dwordx4 ... lds (no register staging) through a
// 4-slot ring, so three steps are in flight while one is multiplied; one
// barrier per step.  Rows and K positions outside the operand read as zero
// through the buffer descriptor's range check.
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

namespace mxq {

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int kThreads = 256;
constexpr int kStages = 4;                        // LDS ring: 3 steps in flight
constexpr int kStage = TM * TK;                   // bytes per operand per stage (16 KB)
constexpr int kGroupM = 4;                        // M tiles per rasterization group
constexpr int kMaxGroups = 256;

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
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m), "v"(off), "s"(r) : "memory");
}
__device__ __forceinline__ void dma_b8(i32x4 r, uint32_t m0, uint32_t off) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ubyte %1, %2, 0 offen lds"
               :: "s"(m), "v"(off), "s"(r) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// LDS offset of 16-byte chunk c (0..3) of tile row r: rows are 64 B; chunks
// are XOR-swizzled with bits 1-2 of the row so 8 consecutive rows read at one
// chunk index cover all 8 16-byte slots of a 128-byte bank line.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * TK + ((c ^ swz(r)) << 4); }

struct GemmArgs {
  const uint8_t* a; const uint8_t* as; int64_t lda, ldsa;
  const uint8_t* b; const uint8_t* bs; int64_t ldb, ldsb;
  int64_t b_estride, bs_estride;                    // per-group B strides (variable M)
  const float* pta; const float* ptb;               // per-tensor scales
  const int64_t* offsets; int32_t E;
  int64_t M, N, K;
  void* c; int64_t ldc;
  uint32_t tiles_n;                                 // output tiles along N
  uint32_t nblocks;                                 // grid size (for the XCD remap)
};

// One operand of a workgroup: codes and scales as buffer resources whose
// offset 0 is the tile's first row at the start of the contraction range.
struct OpTile {
  i32x4 q, s;
  uint32_t ld, lds;
  uint32_t smis;                                    // scale base misalignment (0..3)
  int rows;                                         // valid rows in this tile (<= 256)
};

__device__ __forceinline__ OpTile op_tile(const uint8_t* q, const uint8_t* s, int64_t ld,
                                          int64_t lds, int64_t row0, int64_t k0, int64_t rows,
                                          int64_t kdim, bool scales) {
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
    t.smis = (uint32_t)(a & 3);
    const uint8_t* sb4 = reinterpret_cast<const uint8_t*>(a & ~(uintptr_t)3);
    const uint32_t sbytes = r > 0 ? (uint32_t)((r - 1) * lds + t.smis + ((kdim + 31) >> 5)) : 0;
    t.s = make_rsrc(sb4, sbytes);
  } else {
    t.smis = 0;
    t.s = t.q;
  }
  return t;
}

// Per-lane load offsets of one operand, computed once per workgroup.
// Tile codes: wavefront w fills row groups g = 4w .. 4w+3 of the LDS slot
// (16 rows, 1 KB each); lane i lands at byte 16 i of the group, i.e. row i/4
// and slot i%4, which must hold chunk (i%4) ^ swz(row) under the swizzle.
// Scales: entry e = 128 w + 64 k + i (k = 0, 1) of the slot's 512 scale
// entries is block e%2 of the step for tile row e/2.
struct LaneOffsets {
  uint32_t q[4];            // row * ld + chunk * 16 (0x80000000 for rows past the tile)
  uint32_t kchunk;          // chunk * 16 (the same for the lane's four rows)
  uint32_t s[2];            // smis + row * lds + blk of scale entries k = 0, 1
};

__device__ __forceinline__ LaneOffsets lane_offsets(const OpTile& t) {
  LaneOffsets o;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane >> 2, slot = lane & 3;
  const int chunk = slot ^ swz(rsub);             // swz(16 g + rsub) == swz(rsub)
  o.kchunk = (uint32_t)(chunk * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (w * 4 + j) * 16 + rsub;
    o.q[j] = row < t.rows ? (uint32_t)(row * t.ld) + o.kchunk : 0x80000000u;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = w * 128 + k * 64 + lane;
    o.s[k] = t.smis + (uint32_t)((e >> 1) * t.lds) + (uint32_t)(e & 1);
  }
  return o;
}

// Issue the loads of one k-step of one operand: its 256 x 64 codes into an
// LDS tile slot and, for MX, its 256 x 2 scale bytes into an LDS scale slot.
// `q`, `sr` are the operand's descriptors or zero-range ones for steps past
// the end.  Always 4 (+2) load instructions per wavefront.
template <bool SCALES>
__device__ __forceinline__ void issue_op(const LaneOffsets& o, i32x4 q, i32x4 sr,
                                         uint8_t* tile_slot, uint32_t* scale_slot, int64_t step,
                                         int64_t kdim) {
  const int w = threadIdx.x >> 6;
  const uint32_t kbyte = (uint32_t)(step * TK);
  const bool tail = (int64_t)kbyte + TK > kdim;                  // uniform
  const bool chunk_in = (int64_t)(kbyte + o.kchunk) < kdim;
  const uint32_t tbase = lds_addr(tile_slot) + w * 4 * 1024;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t off = o.q[j] + kbyte;
    if (tail && !chunk_in) off = 0x80000000u;
    dma_b128(q, tbase + j * 1024, off);
  }
  if (SCALES) {
    const uint32_t sbase = lds_addr(scale_slot) + w * 128 * 4;
    const uint32_t kb2 = (uint32_t)(2 * step);
#pragma unroll
    for (int k = 0; k < 2; ++k) dma_b8(sr, sbase + k * 256, o.s[k] + kb2);
  }
}

// Blocks past the end of the contraction range hold zero codes; they get a
// finite scale (2^0) so that 0 * scale cannot become NaN.
__device__ __forceinline__ uint32_t scale_at(uint32_t raw, int64_t step, int half, int64_t kdim) {
  return ((2 * step + half) << 5) < kdim ? raw : 127u;
}

__device__ __forceinline__ i32x8 read_frag(const uint8_t* l, int r, int half) {
  const uint4 x = *reinterpret_cast<const uint4*>(l + lds_off(r, half));
  const uint4 y = *reinterpret_cast<const uint4*>(l + lds_off(r, half + 2));
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
    const __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
    if (n + 3 < N && ((reinterpret_cast<uintptr_t>(p) & 7) == 0)) {
      uint2 u;
      u.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
            ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      u.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
            ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      *reinterpret_cast<uint2*>(p) = u;
    } else {
      if (n < N) p[0] = b0;
      if (n + 1 < N) p[1] = b1;
      if (n + 2 < N) p[2] = b2;
      if (n + 3 < N) p[3] = b3;
    }
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous run of tile indices so tiles sharing operand panels share an L2.
// Only for kinds whose tiles carry equal work.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
  const uint32_t X = 8, per = n / X, rem = n % X;
  const uint32_t x = bid % X, i = bid / X;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

// Tile index -> (tm, tn): groups of kGroupM M-tiles walk N together, so the
// tiles in flight on one XCD read a few A panels and a few B panels.
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

// Vector-memory instructions a wavefront issues per k-step: 4 + 4 tile
// loads, plus 2 + 2 scale-byte loads for MX.
template <bool PT>
constexpr int vmem_per_step() { return PT ? 8 : 12; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N (split field bits 3:0 and 15:14), expcnt and
  // lgkmcnt left at their "don't wait" maxima.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int KIND, bool PT, int OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * 2 * kStage];  // [slot][A, B]
  __shared__ uint32_t ssc[PT ? 1 : kStages * 2 * 2 * TM];           // [slot][A, B][row][blk]
  __shared__ int64_t s_off[KIND == kVarM ? kMaxGroups + 1 : 1];
  __shared__ int32_t s_start[KIND == kVarM ? kMaxGroups + 1 : 1];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, half = lane >> 5;

  // ---- map the workgroup to (group, m0, n0) ----
  int64_t m0 = 0, n0 = 0, kdim = g.K, c_rows = 0;
  void* cbase = g.c;
  OpTile A, B;
  if (KIND == kDense) {
    const uint32_t tiles_m = (uint32_t)((g.M + TM - 1) / TM);
    uint32_t tm, tn;
    raster(xcd_remap(blockIdx.x, g.nblocks), tiles_m, g.tiles_n, tm, tn);
    m0 = (int64_t)tm * TM;
    n0 = (int64_t)tn * TN;
    c_rows = g.M - m0;
    A = op_tile(g.a, g.as, g.lda, g.ldsa, m0, 0, c_rows, kdim, !PT);
    B = op_tile(g.b, g.bs, g.ldb, g.ldsb, n0, 0, g.N - n0, kdim, !PT);
  } else if (KIND == kVarM) {
    group_table(g.offsets, g.E, g.M, s_off, s_start);
    const uint32_t tiles_m = (uint32_t)s_start[g.E];  // data-dependent M-tile count
    const uint32_t tile = xcd_remap(blockIdx.x, g.nblocks);
    if (tile >= tiles_m * g.tiles_n) return;          // surplus workgroup
    uint32_t tm, tn;
    raster(tile, tiles_m, g.tiles_n, tm, tn);
    int lo = 0, hi = g.E - 1;                         // group e: s_start[e] <= tm < s_start[e+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= (int32_t)tm) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    m0 = s_off[e] + (int64_t)(tm - s_start[e]) * TM;
    n0 = (int64_t)tn * TN;
    c_rows = s_off[e + 1] - m0;
    A = op_tile(g.a, g.as, g.lda, g.ldsa, m0, 0, c_rows, kdim, true);
    B = op_tile(g.b + (int64_t)e * g.b_estride, g.bs + (int64_t)e * g.bs_estride, g.ldb, g.ldsb,
                n0, 0, g.N - n0, kdim, true);
  } else {
    // variable K: tile = (e, tm over rows of A = dW rows, tn over rows of B =
    // dW cols).  Work per tile is proportional to the group's tokens, so the
    // plain dispatch order (round-robin over XCDs) is kept for balance.
    const uint32_t tile = blockIdx.x;
    const uint32_t tn = tile % g.tiles_n, tmg = tile / g.tiles_n;
    const uint32_t tiles_m = (uint32_t)((g.M + TM - 1) / TM);
    const int e = (int)(tmg / tiles_m);
    m0 = (int64_t)(tmg % tiles_m) * TM;
    n0 = (int64_t)tn * TN;
    // Padded offsets are multiples of 32; rounding down keeps every access
    // inside [0, capacity) even for malformed offsets.
    int64_t lo_t = g.offsets[e] & ~31LL, hi_t = g.offsets[e + 1] & ~31LL;
    if (lo_t < 0) lo_t = 0;
    if (hi_t > (g.K & ~31LL)) hi_t = g.K & ~31LL;     // g.K holds the token capacity
    kdim = hi_t > lo_t ? hi_t - lo_t : 0;
    c_rows = g.M - m0;
    A = op_tile(g.a, g.as, g.lda, g.ldsa, m0, lo_t, c_rows, kdim, true);
    B = op_tile(g.b, g.bs, g.ldb, g.ldsb, n0, lo_t, g.N - n0, kdim, true);
    cbase = static_cast<uint8_t*>(g.c) + (int64_t)e * g.M * g.ldc * (OUT == MXQ_OUT_FP32 ? 4 : 2);
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t nsteps = (kdim + TK - 1) / TK;
  const LaneOffsets oA = lane_offsets(A);
  const LaneOffsets oB = lane_offsets(B);
  const i32x4 none = make_rsrc(g.c, 0);              // zero range: loads read 0

  // Issue the loads of k-step `step` into ring slot SLOT.  Steps past the end
  // are issued too, through the zero-range descriptor, so each step always
  // issues vmem_per_step<PT>() instructions per wavefront and the wait
  // thresholds below are constants.
  auto issue = [&](int64_t step, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    uint8_t* base = smem + SLOT * 2 * kStage;
    uint32_t* sbase = ssc + (PT ? 0 : SLOT * 2 * 2 * TM);
    const bool live = step < nsteps;
    issue_op<!PT>(oA, uniform(live ? A.q : none), uniform(live ? A.s : none), base, sbase, step,
                  kdim);
    issue_op<!PT>(oB, uniform(live ? B.q : none), uniform(live ? B.s : none), base + kStage,
                  sbase + 2 * TM, step, kdim);
  };
  auto compute = [&](int64_t step, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    const uint8_t* lA = smem + SLOT * 2 * kStage;
    const uint8_t* lB = lA + kStage;
    i32x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = read_frag(lA, wm * 128 + i * 32 + r32, half);
      fb[i] = read_frag(lB, wn * 128 + i * 32 + r32, half);
    }
    uint32_t csa[4], csb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (PT) {
        csa[i] = csb[i] = 127u;
      } else {
        const uint32_t* sA = ssc + SLOT * 2 * 2 * TM;
        const uint32_t* sB = sA + 2 * TM;
        csa[i] = scale_at(sA[(wm * 128 + i * 32 + r32) * 2 + half], step, half, kdim);
        csb[i] = scale_at(sB[(wn * 128 + i * 32 + r32) * 2 + half], step, half, kdim);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[j], fa[i], acc[i][j], 0, 0, 0, (int)csb[j], 0, (int)csa[i]);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  static_assert(kStages == 4, "the unrolled ring below assumes 4 slots");

  // Prologue: steps 0, 1, 2 in flight.
  issue(0, S0{});
  issue(1, S1{});
  issue(2, S2{});
  // Each step: wait until only the 2 later steps are outstanding (this step
  // landed), barrier (visible to all; the slot of the previous step is free),
  // issue step + 3 into that slot, multiply this step.  The loop runs whole
  // groups of kStages steps (one exit keeps the 256 accumulators in place);
  // steps past the end multiply zero tiles.
  constexpr int kWait = (kStages - 2) * vmem_per_step<PT>();
  const int64_t nsteps_pad = (nsteps + kStages - 1) / kStages * kStages;
  for (int64_t s0 = 0; s0 < nsteps_pad; s0 += kStages) {
    wait_vmcnt<kWait>();
    __syncthreads();
    issue(s0 + 3, S3{});
    compute(s0, S0{});
    wait_vmcnt<kWait>();
    __syncthreads();
    issue(s0 + 4, S0{});
    compute(s0 + 1, S1{});
    wait_vmcnt<kWait>();
    __syncthreads();
    issue(s0 + 5, S1{});
    compute(s0 + 2, S2{});
    wait_vmcnt<kWait>();
    __syncthreads();
    issue(s0 + 6, S2{});
    compute(s0 + 3, S3{});
  }
  // Drain the trailing (zero-range) loads before the LDS goes away.
  wait_vmcnt<0>();

  // ---- epilogue: acc[i][j] holds C[m = wm*128 + i*32 + lane%32]
  //                [n = wn*128 + j*32 + 8*(v/4) + 4*(lane/32) + v%4]
  float mul = 1.0f;
  if (PT) mul = (*g.pta) * (*g.ptb);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ml = wm * 128 + i * 32 + r32;
    if (ml >= c_rows) continue;
    const int64_t m = m0 + ml;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 128 + j * 32 + q * 8 + half * 4;
        store4<OUT>(cbase, g.ldc, m, n, g.N, acc[i][j][4 * q] * mul,
                    acc[i][j][4 * q + 1] * mul, acc[i][j][4 * q + 2] * mul,
                    acc[i][j][4 * q + 3] * mul);
      }
    }
  }
}

}  // namespace mxq

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

using namespace mxq;

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <int KIND, bool PT>
static int launch_gemm(GemmArgs& g, int64_t blocks, int out, hipStream_t stream) {
  if (blocks == 0) return MXQ_OK;
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  g.nblocks = (uint32_t)blocks;
  if (out == MXQ_OUT_BF16)
    hipLaunchKernelGGL((k_gemm<KIND, PT, MXQ_OUT_BF16>), dim3((uint32_t)blocks), dim3(kThreads),
                       0, stream, g);
  else
    hipLaunchKernelGGL((k_gemm<KIND, PT, MXQ_OUT_FP32>), dim3((uint32_t)blocks), dim3(kThreads),
                       0, stream, g);
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

static int check_common(int64_t M, int64_t N, int64_t K, int64_t ldc, int out, int accum) {
  if (M < 0 || N < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (out != MXQ_OUT_BF16 && out != MXQ_OUT_FP32) return MXQ_ERR_ARG;
  if (accum != MXQ_ACC_MFMA_FP8 && accum != MXQ_ACC_FP32) return MXQ_ERR_ARG;
  if (ldc < N) return MXQ_ERR_SHAPE;
  return MXQ_OK;
}

// Buffer offsets are 32-bit: one tile of rows must fit.
static bool fits32(int64_t ld, int64_t K) { return ld * (TM + 1) + K < 0x7FFFFFFFLL; }

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
  if (accum != MXQ_ACC_MFMA_FP8) return MXQ_ERR_ARG;   // exact-product mode: not built yet
  GemmArgs g = make_args(a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, M, N, K, c, ldc);
  return launch_gemm<kDense, false>(g, ((M + TM - 1) / TM) * (int64_t)g.tiles_n, out_dtype,
                                    stream);
}

extern "C" int fp8_gemm_per_tensor(const uint8_t* a, const float* a_scale, int64_t lda,
                                   const uint8_t* b, const float* b_scale, int64_t ldb,
                                   int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                                   int out_dtype, int accum, hipStream_t stream) {
  int st = check_common(M, N, K, ldc, out_dtype, accum);
  if (st) return st;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!c || !a_scale || !b_scale) return MXQ_ERR_NULL;
  if (K % 32 != 0) return MXQ_ERR_SHAPE;
  if (K > 0) {
    if ((st = check_operand(a, a_scale, lda, 0, K, false))) return st;
    if ((st = check_operand(b, b_scale, ldb, 0, K, false))) return st;
  }
  if (accum != MXQ_ACC_MFMA_FP8) return MXQ_ERR_ARG;
  GemmArgs g = make_args(a, nullptr, lda, 0, b, nullptr, ldb, 0, M, N, K, c, ldc);
  g.pta = a_scale; g.ptb = b_scale;
  return launch_gemm<kDense, true>(g, ((M + TM - 1) / TM) * (int64_t)g.tiles_n, out_dtype,
                                   stream);
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
  if (accum != MXQ_ACC_MFMA_FP8) return MXQ_ERR_ARG;
  GemmArgs g = make_args(a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, M, N, K, c, ldc);
  g.b_estride = b_estride; g.bs_estride = bs_estride;
  g.offsets = offsets; g.E = E;
  const int64_t mtiles = (M + TM - 1) / TM + E;      // upper bound over all group splits
  return launch_gemm<kVarM, false>(g, mtiles * (int64_t)g.tiles_n, out_dtype, stream);
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
  if (accum != MXQ_ACC_MFMA_FP8) return MXQ_ERR_ARG;
  // For this kind: M = rows of dW (N), N = columns of dW (K), K = token capacity.
  GemmArgs g = make_args(at, at_scale, lda_t, ldsa_t, bt, bt_scale, ldb_t, ldsb_t, N, K, cap, c,
                         ldc);
  g.offsets = offsets_padded; g.E = E;
  const int64_t blocks = (int64_t)E * ((N + TM - 1) / TM) * g.tiles_n;
  return launch_gemm<kVarK, false>(g, blocks, out_dtype, stream);
}
