// MX-FP8 GEMM kernels for gfx950 (dense, grouped variable-M, grouped
// variable-K) on the block-scaled FP8 MFMA, with their C-ABI launchers.
//
// Method: "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" §8 (forward, dgrad and
// wgrad are one quantized matmul each on the copy blocked along the
// contraction dim), §5.2 and §13.4 (grouped matmul over per-expert token
// groups); "Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度" §五
// (FP32 accumulation, one rounding to BF16 at the end).
//
// Tiling: a workgroup of 256 lanes (4 wavefronts, 2 x 2) computes a 128 x 128
// output tile; each wavefront owns 64 x 64 = 2 x 2 MFMA tiles of 32 x 32.  The
// K loop steps 128 codes (four 32-blocks) at a time through LDS.  One
// v_mfma_scale_f32_32x32x64_f8f6f4 consumes, per lane l, 32 codes of row l%32
// (two 16-code halves, one from each 32-block of the 64-wide step) plus one
// E8M0 scale byte, so block scales are applied inside the matrix unit.
// The MFMA is issued with the B tile as its first operand, which makes each
// lane's accumulators hold 4 consecutive output columns of one output row.

#include "common.h"

namespace mxq {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;               // 16 KB per operand tile

enum GemmKind { kDense = 0, kVarM = 1, kVarK = 2 };

// LDS address of 16-byte chunk c of tile row r: rows are 128 B, chunks are
// XOR-swizzled with the row so 8 consecutive rows read at one chunk index
// touch 8 different chunk slots (all banks).
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

struct Operand {
  const uint8_t* q;      // codes; row r, col k at q[r*ld + k]
  const uint8_t* s;      // scales; row r, block j at s[r*lds + j]
  int64_t ld, lds;
  int64_t rows;          // valid rows from q
};

// Stage one 128 x 128 code tile plus its 128 x 4 scales into registers.
struct Stage {
  uint4 a[4], b[4];
  uint32_t sa, sb;       // 4 scale bytes of one row (thread t < 128: A row t, else B row t-128)
};

template <bool PT>
__device__ __forceinline__ void load_stage(Stage& st, const Operand& A, const Operand& B,
                                           int64_t kbase, int64_t kend) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = p * 32 + (t >> 3);
    const int64_t k = kbase + c * 16;
    st.a[p] = (r < A.rows && k < kend) ? *reinterpret_cast<const uint4*>(A.q + r * A.ld + k)
                                       : make_uint4(0, 0, 0, 0);
    st.b[p] = (r < B.rows && k < kend) ? *reinterpret_cast<const uint4*>(B.q + r * B.ld + k)
                                       : make_uint4(0, 0, 0, 0);
  }
  if (!PT) {
    const bool isA = t < 128;
    const int r = isA ? t : t - 128;
    const Operand& O = isA ? A : B;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kb = (kbase >> 5) + j;
      uint32_t v = 127u;                               // 2^0 for padding blocks
      if (r < O.rows && (kb << 5) < kend) v = O.s[r * O.lds + kb];
      w |= v << (8 * j);
    }
    if (isA) st.sa = w; else st.sb = w;
  }
}

template <bool PT>
__device__ __forceinline__ void store_stage(const Stage& st, uint8_t* lA, uint8_t* lB,
                                            uint32_t* lsA, uint32_t* lsB) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = p * 32 + (t >> 3);
    *reinterpret_cast<uint4*>(lA + lds_off(r, c)) = st.a[p];
    *reinterpret_cast<uint4*>(lB + lds_off(r, c)) = st.b[p];
  }
  if (!PT) {
    if (t < 128) lsA[t] = st.sa; else lsB[t - 128] = st.sb;
  }
}

// Operand fragment of one 32x32x64 scaled MFMA for lane (row r, half h):
// bytes 0-15 hold k = 64kk + 16h .. +15 and bytes 16-31 hold
// k = 64kk + 32 + 16h .. +15, i.e. 16-byte chunks 4kk+h and 4kk+2+h.  The
// instruction takes the scale of 32-block 2kk (k 0..31 of the step) from the
// lane with h = 0 and of block 2kk+1 from the lane with h = 1.
__device__ __forceinline__ i32x8 read_frag(const uint8_t* l, int r, int kk, int half) {
  const int c0 = kk * 4 + half;
  uint4 x = *reinterpret_cast<const uint4*>(l + lds_off(r, c0));
  uint4 y = *reinterpret_cast<const uint4*>(l + lds_off(r, c0 + 2));
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
    __bf16 b0 = (__bf16)v0, b1 = (__bf16)v1, b2 = (__bf16)v2, b3 = (__bf16)v3;
    if (n + 3 < N && ((reinterpret_cast<uintptr_t>(p) & 7) == 0)) {
      uint2 u;
      u.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      u.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      *reinterpret_cast<uint2*>(p) = u;
    } else {
      if (n < N) p[0] = b0;
      if (n + 1 < N) p[1] = b1;
      if (n + 2 < N) p[2] = b2;
      if (n + 3 < N) p[3] = b3;
    }
  }
}

struct GemmArgs {
  const uint8_t* a; const uint8_t* as; int64_t lda, ldsa;
  const uint8_t* b; const uint8_t* bs; int64_t ldb, ldsb;
  int64_t b_estride, bs_estride;                    // per-group B strides (variable M)
  const float* pta; const float* ptb;               // per-tensor scales
  const int64_t* offsets; int32_t E;
  int64_t M, N, K;
  void* c; int64_t ldc;
  uint32_t tiles_n;                                 // output tiles along N
};

constexpr int kMaxGroups = 256;

// Per-group tile prefix for the grouped kinds, computed by wavefront 0 into
// LDS: s_start[g] = first tile index of group g (in units of M tiles for
// variable-M), s_off[g] = clamped offsets.
__device__ void group_table(const int64_t* offsets, int E, int64_t M, int64_t* s_off,
                            int32_t* s_start) {
  const int t = threadIdx.x;
  for (int g = t; g <= E; g += blockDim.x) {
    int64_t o = offsets[g];
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
        int64_t d = s_off[g + 1] - s_off[g];
        cnt = d > 0 ? (int32_t)((d + BM - 1) / BM) : 0;
      }
      int32_t v = cnt;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        int32_t u = __shfl_up(v, sh, 64);
        if (t >= sh) v += u;
      }
      if (g < E) s_start[g + 1] = carry + v;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
}

template <int KIND, bool PT, int OUT>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lB[kTileBytes];
  __shared__ uint32_t lsA[BM], lsB[BN];
  __shared__ int64_t s_off[KIND == kDense ? 1 : kMaxGroups + 1];
  __shared__ int32_t s_start[KIND == kVarM ? kMaxGroups + 1 : 1];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;          // wave tile origin (64 x 64)

  // ---- map the workgroup to (group, m0, n0) and set up the operands ----
  const uint32_t tile = blockIdx.x;
  const uint32_t tn = tile % g.tiles_n, tm = tile / g.tiles_n;
  Operand A, B;
  int64_t m0 = 0, n0 = (int64_t)tn * BN, kdim = g.K, c_row0 = 0, c_rows = 0;
  void* cbase = g.c;
  if (KIND == kDense) {
    m0 = (int64_t)tm * BM;
    A = {g.a + m0 * g.lda, g.as + m0 * g.ldsa, g.lda, g.ldsa, g.M - m0};
    B = {g.b + n0 * g.ldb, g.bs + n0 * g.ldsb, g.ldb, g.ldsb, g.N - n0};
    c_row0 = m0; c_rows = g.M - m0;
  } else if (KIND == kVarM) {
    group_table(g.offsets, g.E, g.M, s_off, s_start);
    if ((int32_t)tm >= s_start[g.E]) return;         // beyond the data-dependent tile count
    int lo = 0, hi = g.E - 1;                        // group with s_start[e] <= tm < s_start[e+1]
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_start[mid] <= (int32_t)tm) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    m0 = s_off[e] + (int64_t)(tm - s_start[e]) * BM;
    const int64_t rows = s_off[e + 1] - m0;
    A = {g.a + m0 * g.lda, g.as + m0 * g.ldsa, g.lda, g.ldsa, rows};
    const uint8_t* be = g.b + (int64_t)e * g.b_estride;
    const uint8_t* bse = g.bs + (int64_t)e * g.bs_estride;
    B = {be + n0 * g.ldb, bse + n0 * g.ldsb, g.ldb, g.ldsb, g.N - n0};
    c_row0 = m0; c_rows = rows;
  } else {
    // variable K: tile = (e, tm over N-dim rows of A, tn over K-dim rows of B)
    const uint32_t tiles_m = (uint32_t)((g.M + BM - 1) / BM);   // g.M holds N of dW
    const int e = (int)(tm / tiles_m);
    const uint32_t tme = tm % tiles_m;
    m0 = (int64_t)tme * BM;
    // Padded offsets are multiples of 32; rounding down keeps every access
    // 16-byte aligned and inside [0, capacity) even for malformed offsets.
    int64_t lo_t = g.offsets[e] & ~31LL, hi_t = g.offsets[e + 1] & ~31LL;
    if (lo_t < 0) lo_t = 0;
    if (hi_t > g.K) hi_t = g.K & ~31LL;              // g.K holds the padded token capacity
    kdim = hi_t > lo_t ? hi_t - lo_t : 0;
    A = {g.a + m0 * g.lda + lo_t, g.as + m0 * g.ldsa + (lo_t >> 5), g.lda, g.ldsa, g.M - m0};
    B = {g.b + n0 * g.ldb + lo_t, g.bs + n0 * g.ldsb + (lo_t >> 5), g.ldb, g.ldsb, g.N - n0};
    cbase = static_cast<uint8_t*>(g.c) + (int64_t)e * g.M * g.ldc * (OUT == MXQ_OUT_FP32 ? 4 : 2);
    c_row0 = m0; c_rows = g.M - m0;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t nsteps = (kdim + BK - 1) / BK;
  Stage st;
  if (nsteps > 0) {
    load_stage<PT>(st, A, B, 0, kdim);
    store_stage<PT>(st, lA, lB, lsA, lsB);
  }
  __syncthreads();
  const int r32 = lane & 31, half = lane >> 5;
  for (int64_t s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) load_stage<PT>(st, A, B, (s + 1) * BK, kdim);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x8 fa[2], fb[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm * 64 + i * 32 + r32;
        const int rb = wn * 64 + i * 32 + r32;
        fa[i] = read_frag(lA, ra, kk, half);
        fb[i] = read_frag(lB, rb, kk, half);
        if (PT) {
          sa[i] = 127; sb[i] = 127;
        } else {
          sa[i] = (int)((lsA[ra] >> (8 * (kk * 2 + half))) & 0xFFu);
          sb[i] = (int)((lsB[rb] >> (8 * (kk * 2 + half))) & 0xFFu);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[j], fa[i], acc[i][j], 0, 0, 0, sb[j], 0, sa[i]);
    }
    __syncthreads();
    if (more) {
      store_stage<PT>(st, lA, lB, lsA, lsB);
      __syncthreads();
    }
  }

  // ---- epilogue: acc[i][j] holds C[m = wm*64+i*32 + lane%32][n = wn*64+j*32 + 8*(v/4) + 4*(lane/32) + v%4]
  float mul = 1.0f;
  if (PT) mul = (*g.pta) * (*g.ptb);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t ml = wm * 64 + i * 32 + r32;
    if (ml >= c_rows) continue;
    const int64_t m = c_row0 + ml;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 64 + j * 32 + q * 8 + half * 4;
        store4<OUT>(cbase, g.ldc, m, n, g.N, acc[i][j][4 * q] * mul, acc[i][j][4 * q + 1] * mul,
                    acc[i][j][4 * q + 2] * mul, acc[i][j][4 * q + 3] * mul);
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
static int launch_gemm(const GemmArgs& g, uint32_t blocks, int out, hipStream_t stream) {
  if (blocks == 0) return MXQ_OK;
  if (out == MXQ_OUT_BF16)
    hipLaunchKernelGGL((k_gemm<KIND, PT, MXQ_OUT_BF16>), dim3(blocks), dim3(kThreads), 0, stream, g);
  else
    hipLaunchKernelGGL((k_gemm<KIND, PT, MXQ_OUT_FP32>), dim3(blocks), dim3(kThreads), 0, stream, g);
  return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

static int check_common(int64_t M, int64_t N, int64_t K, int64_t ldc, int out, int accum) {
  if (M < 0 || N < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (out != MXQ_OUT_BF16 && out != MXQ_OUT_FP32) return MXQ_ERR_ARG;
  if (accum != MXQ_ACC_MFMA_FP8 && accum != MXQ_ACC_FP32) return MXQ_ERR_ARG;
  if (ldc < N) return MXQ_ERR_SHAPE;
  return MXQ_OK;
}

static int check_operand(const uint8_t* q, const void* s, int64_t ld, int64_t lds, int64_t K,
                         bool mx) {
  if (!q || !s) return MXQ_ERR_NULL;
  if (ld < K || (mx && lds < K / 32)) return MXQ_ERR_SHAPE;
  if (ld % 16 != 0 || !aligned(q, 16)) return MXQ_ERR_ALIGN;
  if (!mx && !aligned(s, 4)) return MXQ_ERR_ALIGN;
  return MXQ_OK;
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
  GemmArgs g{a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, 0, 0, nullptr, nullptr, nullptr, 0,
             M, N, K, c, ldc, (uint32_t)((N + BN - 1) / BN)};
  const int64_t blocks = ((M + BM - 1) / BM) * (int64_t)g.tiles_n;
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  return launch_gemm<kDense, false>(g, (uint32_t)blocks, out_dtype, stream);
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
  GemmArgs g{a, nullptr, lda, 0, b, nullptr, ldb, 0, 0, 0, a_scale, b_scale, nullptr, 0,
             M, N, K, c, ldc, (uint32_t)((N + BN - 1) / BN)};
  const int64_t blocks = ((M + BM - 1) / BM) * (int64_t)g.tiles_n;
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  return launch_gemm<kDense, true>(g, (uint32_t)blocks, out_dtype, stream);
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
  GemmArgs g{a, a_scale, lda, ldsa, b, b_scale, ldb, ldsb, b_estride, bs_estride, nullptr,
             nullptr, offsets, E, M, N, K, c, ldc, (uint32_t)((N + BN - 1) / BN)};
  const int64_t mtiles = (M + BM - 1) / BM + E;      // upper bound over all group splits
  const int64_t blocks = mtiles * (int64_t)g.tiles_n;
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  return launch_gemm<kVarM, false>(g, (uint32_t)blocks, out_dtype, stream);
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
  int64_t scap = (ldsa_t < ldsb_t ? ldsa_t : ldsb_t) * 32;
  if (scap < cap) cap = scap;
  if (accum != MXQ_ACC_MFMA_FP8) return MXQ_ERR_ARG;
  GemmArgs g{at, at_scale, lda_t, ldsa_t, bt, bt_scale, ldb_t, ldsb_t, 0, 0, nullptr, nullptr,
             offsets_padded, E, N, K, cap, c, ldc, (uint32_t)((K + BN - 1) / BN)};
  // GemmArgs fields for this kind: M = N (rows of dW), N = K (cols of dW), K = token capacity.
  g.M = N; g.N = K; g.K = cap;
  const int64_t blocks = (int64_t)E * ((N + BM - 1) / BM) * g.tiles_n;
  if (blocks > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  return launch_gemm<kVarK, false>(g, (uint32_t)blocks, out_dtype, stream);
}
