// MX (E4M3 + E8M0 per 32 values) and per-tensor FP8 quantization kernels
// for gfx950, with their C-ABI launchers.
//
// Method: "DeepSeek-V3 16B FSDP2 MXFP8/HiF8 训练设计" §3 table (1x32 and 32x1
// blocks, E8M0 scale from the current block) and §3.2 (current scaling: an
// FP32 scale of amax / 448 for a finite non-zero amax, otherwise 1); "低精度训练特性
// （MXFP8 / HiFloat8）" (block size 32; grouped quant for the expert wgrad);
// E4M3 layout from "Transformer 与 LLM（06）：浮点格式、数值稳定性与混合精度" §二.2.
//
// All three kernels are HBM-bound streams: 2 bytes read and 1 + 1/32 bytes
// written per element (MX), or 2 + 2 read and 1 written (per-tensor, two
// passes).  Loads and stores are 16 B (8 B for codes in the row kernel) per
// lane and contiguous across the wavefront.

#include "common.h"

#include <algorithm>
#include <mutex>

namespace mxq {

// ---------------------------------------------------------------------------
// Row-wise MX quantization.
//
// A wavefront owns a segment of 512 consecutive elements of one row; lane l
// holds elements [8l, 8l+8), so the 4 lanes of a DPP quad hold one 32-element
// block.  The block amax is a packed-u16 max over the lane's 8 magnitudes and
// two quad DPP exchanges.  A contiguous matrix is passed as a single row so
// segments run across row ends.
// ---------------------------------------------------------------------------

constexpr int kRowUnroll = 4;

// Code stores are non-temporal: the big output streams then do not
// allocate in the caches on their way to HBM (measured 5-15 % faster than
// plain stores on the expert layer's large operands; non-temporal loads gave
// no gain).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  u32x4 w;
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_stream(void* p, uint2 v) {
  u32x2 w;
  w[0] = v.x; w[1] = v.y;
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ void quant8(uint4 v, uint32_t& lo, uint32_t& hi, uint32_t& code) {
  u16x2 m = __builtin_elementwise_max(absmax2(v.x, v.y), absmax2(v.z, v.w));
  uint32_t am = m.x > m.y ? m.x : m.y;
  uint32_t o = dpp_u32(am, kQuadXor1);
  am = am > o ? am : o;
  o = dpp_u32(am, kQuadXor2);
  am = am > o ? am : o;
  code = mx_scale_code(am);
  if (code == 0xFFu) {                 // NaN or Inf in the block
    lo = hi = 0x7F7F7F7Fu;
    return;
  }
  float inv = mx_inv_scale(code);      // x * 2^-e is exact in FP32
  lo = cvt2_e4m3_sat<false>(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, 0u);
  lo = cvt2_e4m3_sat<true>(bf16_lo(v.y) * inv, bf16_hi(v.y) * inv, lo);
  hi = cvt2_e4m3_sat<false>(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, 0u);
  hi = cvt2_e4m3_sat<true>(bf16_lo(v.w) * inv, bf16_hi(v.w) * inv, hi);
}

// Up to kRowBatch matrices in one launch: item i owns the global segment
// groups [first, first + ceil(total / kRowUnroll) * kRowUnroll), so a group of
// kRowUnroll consecutive segments never straddles two items.
constexpr int kRowBatch = MXQ_ROWWISE_BATCH_MAX;
struct RowItem {
  const uint16_t* x;
  uint8_t* q;
  uint8_t* sc;
  int64_t ldx, ldq, lds;
  uint32_t K, segs_per_row, total, first;
};
struct RowBatch {
  RowItem it[kRowBatch];
  uint32_t n, total;
};

__global__ __launch_bounds__(256) void k_mx_rowwise(RowBatch b) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const uint32_t nwave = gridDim.x * (blockDim.x >> 6);
  for (uint32_t s0 = wave * kRowUnroll; s0 < b.total; s0 += nwave * kRowUnroll) {
    // the item of this group (wave-uniform; items in order of first)
    int i = 0;
#pragma unroll
    for (int k = 1; k < kRowBatch; ++k)
      if ((uint32_t)k < b.n && s0 >= b.it[k].first) i = k;
    const RowItem t = i == 0 ? b.it[0] : i == 1 ? b.it[1] : i == 2 ? b.it[2] : b.it[3];
    static_assert(kRowBatch == 4, "item selection above");
    uint4 v[kRowUnroll];
    uint32_t row[kRowUnroll], col[kRowUnroll];
    bool ok[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      uint32_t s = s0 - t.first + u;
      row[u] = s / t.segs_per_row;                  // wave-uniform
      col[u] = (s - row[u] * t.segs_per_row) * 512u + lane * 8u;
      ok[u] = (s < t.total) && (col[u] < t.K);
      v[u] = ok[u] ? *reinterpret_cast<const uint4*>(t.x + (int64_t)row[u] * t.ldx + col[u])
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      uint32_t lo, hi, code;
      quant8(v[u], lo, hi, code);
      if (ok[u]) {
        store_stream(t.q + (int64_t)row[u] * t.ldq + col[u], make_uint2(lo, hi));
        if ((lane & 3u) == 0u) t.sc[(int64_t)row[u] * t.lds + (col[u] >> 5)] = (uint8_t)code;
      }
    }
  }
}

// Correctly rounded FP32 quotient x / s (s > 0) for the current-scaling
// encoders: q0 = RN(x * r) with r = RN(1/s) and one FMA correction
// RN(q0 + RN'(x - s*q0) * r) (Markstein); a subnormal s divides directly.
__device__ __forceinline__ float pt_div(float xv, float s, float r, bool direct) {
  if (direct) return __fdiv_rn(xv, s);
  float q0 = xv * r;
  float rem = __builtin_fmaf(-q0, s, xv);
  // s > 0, so the quotient has the sign of x; the correction step alone
  // would turn -0 into +0.
  return __builtin_copysignf(__builtin_fmaf(rem, r, q0), xv);
}

// Codes of two BF16 values packed in w, for a tensor whose amax is NaN/Inf
// (s == 1): NaN -> 0x7F|sign, +-Inf -> saturate.
template <bool HI>
__device__ __forceinline__ uint32_t pt_nonfinite_pair(uint32_t w, uint32_t old) {
  uint32_t out = cvt2_e4m3_sat<HI>(bf16_lo(w), bf16_hi(w), old);
  uint32_t sh = HI ? 16u : 0u;
  uint32_t b0 = w & 0x7FFFu, b1 = (w >> 16) & 0x7FFFu;
  if (b0 > 0x7F80u) out = (out & ~(0xFFu << sh)) | ((0x7Fu | ((w >> 8) & 0x80u)) << sh);
  if (b1 > 0x7F80u) out = (out & ~(0xFFu << (sh + 8))) | ((0x7Fu | ((w >> 24) & 0x80u)) << (sh + 8));
  return out;
}

// 8 BF16 values (one 16-byte load) -> 8 codes with scale s (r = RN(1/s)).
__device__ __forceinline__ uint2 pt_encode8(uint4 v, float s, float r, bool direct,
                                            bool nonfinite) {
  uint32_t lo, hi;
  if (nonfinite) {
    lo = pt_nonfinite_pair<false>(v.x, 0u);
    lo = pt_nonfinite_pair<true>(v.y, lo);
    hi = pt_nonfinite_pair<false>(v.z, 0u);
    hi = pt_nonfinite_pair<true>(v.w, hi);
  } else {
    lo = cvt2_e4m3_sat<false>(pt_div(bf16_lo(v.x), s, r, direct), pt_div(bf16_hi(v.x), s, r, direct), 0u);
    lo = cvt2_e4m3_sat<true>(pt_div(bf16_lo(v.y), s, r, direct), pt_div(bf16_hi(v.y), s, r, direct), lo);
    hi = cvt2_e4m3_sat<false>(pt_div(bf16_lo(v.z), s, r, direct), pt_div(bf16_hi(v.z), s, r, direct), 0u);
    hi = cvt2_e4m3_sat<true>(pt_div(bf16_lo(v.w), s, r, direct), pt_div(bf16_hi(v.w), s, r, direct), hi);
  }
  return make_uint2(lo, hi);
}

// ---------------------------------------------------------------------------
// Column-wise (grouped, zero-padded) MX quantization, transposed output.
//
// A workgroup (256 lanes) owns 128 consecutive padded output columns (four
// 32-blocks along M) and walks kColPasses x 64 input columns (K).  The group
// table and the source rows of its four blocks are set up once.  Per pass it
// has the 128 source rows (16 B per lane, whole 128-byte lines along K) in
// registers, prefetched two passes ahead, writes them to LDS, and
// each wave quantizes one 32-block: lane pair (2p, 2p+1) holds input columns
// 2p and 2p+1 for the upper and lower 16 rows of the block, takes a
// packed-u16 max down its 16 rows and one DPP exchange with its partner, and
// puts 16 codes for each of its two columns into an LDS staging tile.  The
// staged 64 x 128 codes then go out as whole 128-byte rows of the transposed
// output, and the 64 x 4 scales as one dword (or four bytes) per row.  The
// grid is one-dimensional with the K chunks of a column tile consecutive, so
// the workgroups in flight read whole source rows rather than 512-byte
// pieces of many rows.
// ---------------------------------------------------------------------------

constexpr int kColTileM = 128;   // padded output columns per workgroup
constexpr int kColTileK = 64;    // input columns per pass
constexpr int kColPasses = 4;    // passes per workgroup
constexpr int kColLdsW = 34;     // LDS row stride of the input tile in dwords (32 + 2 pad)
constexpr int kColOutW = 144;    // LDS row stride of the staged codes in bytes (128 + 16 pad)
constexpr int kColMaxGroupsLds = 256;
constexpr int kColDualGroup = 4;  // column tiles per dispatch block (dual-axis)
// Dual-axis: the row copy's codes and scales of kRowStage passes are staged in
// LDS and leave as whole 128-byte row segments (and one scale dword per row)
// rather than a 64-byte piece and two scale bytes per row and pass.
constexpr int kRowStage = 2;
constexpr int kRowStageW = kRowStage * kColTileK + 16;  // LDS row stride (bytes)

// ROW (dual-axis quantization): the same pass also emits the row-wise (1x32)
// codes and scales of every source row it holds.  Lane tid has 8 consecutive
// columns of a row, and the 4 lanes of a DPP quad one 32-block of it (K is a
// multiple of 32), so the row quantizer's block step applies unchanged.
// PG (per-group current scaling, transposed copy): no block scales; every
// 32-row block takes its group's FP32 scale (gscale, with gmax the group's
// |x| maximum pattern) and encodes as the per-tensor pass does.
// bid / nblk: this workgroup's index among its matrix's nblk workgroups.
template <bool ROW, bool PG>
__device__ __forceinline__ void colwise_body(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const int64_t* __restrict__ offsets, int32_t E,
    uint8_t* __restrict__ qT, int64_t ldqT, int64_t M_cap,
    uint8_t* __restrict__ scT, int64_t ldsT, int64_t* __restrict__ offsets_padded,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ sc, int64_t lds,
    const uint32_t* __restrict__ gmax, const float* __restrict__ gscale, uint32_t bid,
    uint32_t nblk) {
  __shared__ uint32_t tile[kColTileM * kColLdsW];
  __shared__ __attribute__((aligned(16))) uint8_t outq[kColTileK * kColOutW];
  __shared__ __attribute__((aligned(16))) uint8_t outs[kColTileK * 4];
  constexpr bool RSTAGE = ROW && !PG;
  __shared__ __attribute__((aligned(16))) uint8_t rowq[RSTAGE ? kColTileM * kRowStageW : 16];
  __shared__ __attribute__((aligned(16))) uint8_t rowsc[RSTAGE ? kColTileM * 2 * kRowStage : 16];
  __shared__ int64_t s_off[kColMaxGroupsLds + 1];
  __shared__ int64_t s_poff[kColMaxGroupsLds + 1];
  __shared__ int64_t s_src0[4];
  __shared__ int32_t s_nvalid[4];
  __shared__ int32_t s_grp[4];

  const int tid = threadIdx.x;
  // Workgroups along K are consecutive in dispatch order, so the ones in
  // flight read whole source rows together.  With ROW, blocks of kColDualGroup
  // column tiles take the K chunks together (4 adjacent tiles per K chunk), so
  // the transposed stores in flight also form 512-byte runs of each output row.
  const uint32_t nky = (uint32_t)((K + kColTileK * kColPasses - 1) / (kColTileK * kColPasses));
  uint32_t bx, by;
  if (ROW) {
    const uint32_t ngx = nblk / nky, G = kColDualGroup;
    const uint32_t per = G * nky, grp = bid / per, in = bid % per;
    const uint32_t gw = ngx - grp * G < G ? ngx - grp * G : G;
    bx = grp * G + in % gw;
    by = in / gw;
  } else {
    bx = bid / nky;
    by = bid % nky;
  }
  const int64_t p0 = (int64_t)bx * kColTileM;             // first padded column
  const int64_t kw0 = (int64_t)by * kColTileK * kColPasses;  // first input column

  // Group table: s_off = clamped offsets, s_poff = padded prefix sums.
  const int G = offsets ? E : 1;
  for (int g = tid; g <= G; g += blockDim.x) {
    int64_t o = offsets ? offsets[g] : (g == 0 ? 0 : M);
    s_off[g] = o < 0 ? 0 : (o > M ? M : o);
  }
  __syncthreads();
  if (tid < 64) {
    // Wave-wide inclusive scan of padded group sizes, 64 groups per step.
    int64_t carry = 0;
    if (tid == 0) s_poff[0] = 0;
    for (int base = 0; base < G; base += 64) {
      int g = base + tid;
      int64_t cnt = 0;
      if (g < G) {
        int64_t d = s_off[g + 1] - s_off[g];
        cnt = d > 0 ? (d + 31) / 32 * 32 : 0;
      }
      int64_t v = cnt;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        int64_t t = __shfl_up(v, sh, 64);
        if (tid >= sh) v += t;
      }
      if (g < G) s_poff[g + 1] = carry + v;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
  if (offsets_padded && bid == 0)
    for (int g = tid; g <= G; g += blockDim.x) offsets_padded[g] = s_poff[g];
  if (tid < 4) {
    // Source rows of 32-block tid of this tile: find g with
    // poff[g] <= col < poff[g+1] (binary search over the non-decreasing poff).
    int64_t col = p0 + 32 * tid;
    int64_t src0 = 0;
    int32_t nvalid = 0, grp = -1;
    if (col < s_poff[G] && col < M_cap) {
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_poff[mid] <= col) lo = mid; else hi = mid - 1;
      }
      int64_t r0 = s_off[lo] + (col - s_poff[lo]);
      int64_t r1 = s_off[lo + 1];
      src0 = r0;
      int64_t n = r1 - r0;
      nvalid = n <= 0 ? 0 : (n >= 32 ? 32 : (int32_t)n);
      grp = lo;
    }
    s_src0[tid] = src0;
    s_nvalid[tid] = nvalid;
    s_grp[tid] = grp;
  }
  __syncthreads();

  // This lane's loads: tile rows i = 32 u + tid/8 (u = 0..3), 16-byte chunk tid%8.
  const int chunk = tid & 7;
  const uint16_t* src[4];
  int64_t srow[4];
  bool rok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = u * 32 + (tid >> 3), b = i >> 5, r = i & 31;
    rok[u] = r < s_nvalid[b];
    srow[u] = rok[u] ? s_src0[b] + r : 0;
    src[u] = x + srow[u] * ldx + chunk * 8;
  }
  auto load = [&](int64_t kb, uint4* v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = make_uint4(0, 0, 0, 0);
      if (rok[u] && kb + chunk * 8 < K) v[u] = *reinterpret_cast<const uint4*>(src[u] + kb);
    }
  };

  const int w = tid >> 6, lane = tid & 63;
  const int p = lane >> 1, h = lane & 1;
  const int rbase = w * 32 + h * 16;
  const bool scale_dword = ((reinterpret_cast<uintptr_t>(scT + (p0 >> 5)) & 3) == 0) &&
                           (ldsT & 3) == 0 && p0 + kColTileM <= M_cap;
  uint4 cur[4], nxt[4], nx2[4];                     // passes p, p+1 and p+2 in flight
  load(kw0, cur);
  if (kColPasses > 1) load(kw0 + kColTileK, nxt);
  for (int pass = 0; pass < kColPasses; ++pass) {
    const int64_t kb = kw0 + pass * kColTileK;
    if (kb >= K) break;                             // uniform
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(&tile[(u * 32 + (tid >> 3)) * kColLdsW + chunk * 4]) = cur[u];
    if (pass + 2 < kColPasses) load(kb + 2 * kColTileK, nx2);
    if (ROW && PG) {
      // Row-major copy with the group's FP32 scale (rows of block u belong to
      // group s_grp[u]); the scales are the caller's group scales.
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = s_grp[u];
        const float gs = e >= 0 ? gscale[e] : 1.0f;
        const uint2 c = pt_encode8(cur[u], gs, __frcp_rn(gs), gs < 1.17549435e-38f,
                                   e >= 0 && gmax[e] >= 0x7F80u);
        const int64_t k = kb + chunk * 8;
        if (rok[u] && k < K) store_stream(q + srow[u] * ldq + k, c);
      }
    } else if (ROW) {
      // Row-wise codes of the rows held in registers (every lane takes part
      // in the quad exchanges), staged for the flush below.
      const int sp = pass % kRowStage;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t lo, hi, code;
        quant8(cur[u], lo, hi, code);
        const int i = u * 32 + (tid >> 3);
        *reinterpret_cast<uint2*>(&rowq[i * kRowStageW + sp * kColTileK + chunk * 8]) =
            make_uint2(lo, hi);
        if ((chunk & 3) == 0) rowsc[i * 2 * kRowStage + sp * 2 + (chunk >> 2)] = (uint8_t)code;
      }
    }
    __syncthreads();

    // Quantize: wave w -> block w; lane = 2p + h: column pair p, row half h.
    uint32_t vals[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) vals[j] = tile[(rbase + j) * kColLdsW + p];
    uint32_t c0[4], c1[4];
    uint32_t code0 = 0, code1 = 0;
    if (PG) {
      // Padding rows were loaded as zeros and encode to +0.  A group whose
      // amax is NaN/Inf has s = 1: Inf saturates, NaN becomes 0x7F | sign.
      const int e = s_grp[w];
      const float gs = e >= 0 ? gscale[e] : 1.0f;
      const bool nonfinite = e >= 0 && gmax[e] >= 0x7F80u;
      const bool direct = gs < 1.17549435e-38f;    // subnormal scale: divide directly
      const float rc = __frcp_rn(gs);
      // x / 1 is x; dividing would turn +-Inf into NaN through the correction step
      auto enc = [&](float v) { return nonfinite ? v : pt_div(v, gs, rc, direct); };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t a = vals[4 * j], b2 = vals[4 * j + 1], c = vals[4 * j + 2], d = vals[4 * j + 3];
        uint32_t t0 = cvt2_e4m3_sat<false>(enc(bf16_lo(a)), enc(bf16_lo(b2)), 0u);
        c0[j] = cvt2_e4m3_sat<true>(enc(bf16_lo(c)), enc(bf16_lo(d)), t0);
        uint32_t t1 = cvt2_e4m3_sat<false>(enc(bf16_hi(a)), enc(bf16_hi(b2)), 0u);
        c1[j] = cvt2_e4m3_sat<true>(enc(bf16_hi(c)), enc(bf16_hi(d)), t1);
        if (nonfinite) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t v = vals[4 * j + r];
            if ((v & 0x7FFFu) > 0x7F80u)
              c0[j] = (c0[j] & ~(0xFFu << (8 * r))) | ((0x7Fu | ((v >> 8) & 0x80u)) << (8 * r));
            if (((v >> 16) & 0x7FFFu) > 0x7F80u)
              c1[j] = (c1[j] & ~(0xFFu << (8 * r))) | ((0x7Fu | ((v >> 24) & 0x80u)) << (8 * r));
          }
        }
      }
    } else {
      u16x2 m = __builtin_bit_cast(u16x2, 0u);
#pragma unroll
      for (int j = 0; j < 16; j += 2) m = __builtin_elementwise_max(m, absmax2(vals[j], vals[j + 1]));
      uint32_t mw = __builtin_bit_cast(uint32_t, m);
      uint32_t ow = dpp_u32(mw, kQuadXor1);         // partner lane^1: other half
      u16x2 mm = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, ow));
      code0 = mx_scale_code(mm.x);                  // column 2p
      code1 = mx_scale_code(mm.y);                  // column 2p+1
      float inv0 = mx_inv_scale(code0 == 0xFFu ? 127u : code0);
      float inv1 = mx_inv_scale(code1 == 0xFFu ? 127u : code1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t a = vals[4 * j], b2 = vals[4 * j + 1], c = vals[4 * j + 2], d = vals[4 * j + 3];
        uint32_t t0 = cvt2_e4m3_sat<false>(bf16_lo(a) * inv0, bf16_lo(b2) * inv0, 0u);
        c0[j] = cvt2_e4m3_sat<true>(bf16_lo(c) * inv0, bf16_lo(d) * inv0, t0);
        uint32_t t1 = cvt2_e4m3_sat<false>(bf16_hi(a) * inv1, bf16_hi(b2) * inv1, 0u);
        c1[j] = cvt2_e4m3_sat<true>(bf16_hi(c) * inv1, bf16_hi(d) * inv1, t1);
      }
      if (code0 == 0xFFu) c0[0] = c0[1] = c0[2] = c0[3] = 0x7F7F7F7Fu;
      if (code1 == 0xFFu) c1[0] = c1[1] = c1[2] = c1[3] = 0x7F7F7F7Fu;
    }
    *reinterpret_cast<uint4*>(&outq[(2 * p) * kColOutW + w * 32 + h * 16]) =
        make_uint4(c0[0], c0[1], c0[2], c0[3]);
    *reinterpret_cast<uint4*>(&outq[(2 * p + 1) * kColOutW + w * 32 + h * 16]) =
        make_uint4(c1[0], c1[1], c1[2], c1[3]);
    if (!PG && h == 0) {
      outs[(2 * p) * 4 + w] = (uint8_t)code0;
      outs[(2 * p + 1) * 4 + w] = (uint8_t)code1;
    }
    __syncthreads();

    // Stores: 64 rows x 128 codes, 8 lanes x 16 B per row; then 64 x 4 scales.
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row = it * 32 + (tid >> 3), c16 = tid & 7;
      const int64_t k = kb + row, col = p0 + c16 * 16;
      if (k < K && col < M_cap)
        store_stream(qT + k * ldqT + col,
                     *reinterpret_cast<const uint4*>(&outq[row * kColOutW + c16 * 16]));
    }
    if (!PG && tid < kColTileK && kb + tid < K) {
      uint8_t* d = scT + (kb + tid) * ldsT + (p0 >> 5);
      const uint32_t sv = *reinterpret_cast<const uint32_t*>(&outs[tid * 4]);
      if (scale_dword) {
        *reinterpret_cast<uint32_t*>(d) = sv;
      } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
          if (p0 + 32 * bb < M_cap) d[bb] = (uint8_t)(sv >> (8 * bb));
      }
    }
    if (RSTAGE && (pass % kRowStage == kRowStage - 1 || pass + 1 == kColPasses ||
                   kb + kColTileK >= K)) {
      // Flush the staged passes: row segments of kRowStage * 64 bytes, 8 lanes
      // x 16 B per row (valid rows and columns only), then the scales.
      const int64_t k0 = kw0 + (int64_t)(pass - pass % kRowStage) * kColTileK;
      constexpr int kLanesPerRow = kRowStage * kColTileK / 16;
      constexpr int kRowsPerIt = 256 / kLanesPerRow;
#pragma unroll
      for (int it = 0; it < kColTileM / kRowsPerIt; ++it) {
        const int row = it * kRowsPerIt + tid / kLanesPerRow, c16 = tid % kLanesPerRow;
        const int b = row >> 5, r = row & 31;
        const int64_t k = k0 + c16 * 16;
        if (r < s_nvalid[b] && k < K)
          store_stream(q + (s_src0[b] + r) * ldq + k,
                       *reinterpret_cast<const uint4*>(&rowq[row * kRowStageW + c16 * 16]));
      }
      if (tid < kColTileM) {
        const int b = tid >> 5, r = tid & 31;
        if (r < s_nvalid[b]) {
          uint8_t* d = sc + (s_src0[b] + r) * lds + (k0 >> 5);
          const uint32_t sv = *reinterpret_cast<const uint32_t*>(&rowsc[tid * 2 * kRowStage]);
          if (k0 + 32 * 2 * kRowStage <= K && (reinterpret_cast<uintptr_t>(d) & 3) == 0) {
            *reinterpret_cast<uint32_t*>(d) = sv;
          } else {
#pragma unroll
            for (int j = 0; j < 2 * kRowStage; ++j)
              if (k0 + 32 * j < K) d[j] = (uint8_t)(sv >> (8 * j));
          }
        }
      }
      __syncthreads();                              // the next pass refills rowq
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      cur[u] = nxt[u];
      nxt[u] = nx2[u];
    }
  }
}

// Up to kColBatch matrices in one launch (each with its own groups and
// outputs): item i owns workgroups [first, first + nblk) of the grid.
constexpr int kColBatch = MXQ_DUAL_BATCH_MAX;
struct ColItem {
  const uint16_t* x;
  int64_t M, K, ldx;
  const int64_t* offsets;
  uint8_t* qT;
  int64_t ldqT, M_cap;
  uint8_t* scT;
  int64_t ldsT;
  int64_t* offsets_padded;
  uint8_t* q;
  int64_t ldq;
  uint8_t* sc;
  int64_t lds;
  const uint32_t* gmax;
  const float* gscale;
  int32_t E;
  uint32_t first, nblk;
};
struct ColBatch {
  ColItem it[kColBatch];
  uint32_t n;
};

template <bool ROW, bool PG = false>
__global__ __launch_bounds__(256) void k_mx_colwise(ColBatch b) {
  // the item of this workgroup (items in order of first)
  int i = 0;
#pragma unroll
  for (int k = 1; k < kColBatch; ++k)
    if ((uint32_t)k < b.n && blockIdx.x >= b.it[k].first) i = k;
  const ColItem t = i == 0 ? b.it[0] : i == 1 ? b.it[1] : i == 2 ? b.it[2] : b.it[3];
  static_assert(kColBatch == 4, "item selection above");
  colwise_body<ROW, PG>(t.x, t.M, t.K, t.ldx, t.offsets, t.E, t.qT, t.ldqT, t.M_cap, t.scT, t.ldsT,
                        t.offsets_padded, t.q, t.ldq, t.sc, t.lds, t.gmax, t.gscale,
                        blockIdx.x - t.first, t.nblk);
}

// ---------------------------------------------------------------------------
// Per-tensor current scaling: pass 1 reduces |x| to one packed max per
// workgroup; pass 2 re-reduces the partials (every workgroup, same order, so
// the result is deterministic), forms s = fp32(amax) / 448 or 1.0, and
// encodes q = RNE_E4M3(RN(x / s)).  The quotient is the correctly rounded
// FP32 division, formed as q0 = RN(x * r) with r = RN(1/s) and one FMA
// correction RN(q0 + RN'(x - s*q0) * r) (Markstein); when s is subnormal the
// kernel divides directly.
// ---------------------------------------------------------------------------

constexpr int kPtBlocks = 1024;
constexpr int kPtThreads = 256;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  for (int sh = 32; sh >= 1; sh >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, sh, 64);
    v = v > o ? v : o;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = r > red[i] ? r : red[i];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPtThreads) void k_pt_amax(const uint16_t* __restrict__ x, int64_t n,
                                                        uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kPtThreads / 64];
  const int64_t nchunks = n >> 3;
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    uint4 v = reinterpret_cast<const uint4*>(x)[c];
    u16x2 mm = __builtin_elementwise_max(absmax2(v.x, v.y), absmax2(v.z, v.w));
    uint32_t t = mm.x > mm.y ? mm.x : mm.y;
    m = m > t ? m : t;
  }
  // tail (n % 8 elements)
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    uint32_t t = x[(nchunks << 3) + threadIdx.x] & 0x7FFFu;
    m = m > t ? m : t;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// amax_in: the tensor's amax given by the caller (then partial is unused);
// the rule is the same: s = amax / 448 when amax is finite and > 0, else 1.
__global__ __launch_bounds__(kPtThreads) void k_pt_quant(const uint16_t* __restrict__ x, int64_t n,
                                                         const uint32_t* __restrict__ partial, int nparts,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale_out,
                                                         const float* __restrict__ amax_in) {
  __shared__ uint32_t red[kPtThreads / 64];
  bool nonfinite;
  float s = 1.0f;
  if (amax_in) {
    const float a = *amax_in;
    const uint32_t ab = __builtin_bit_cast(uint32_t, a) & 0x7FFFFFFFu;
    nonfinite = ab >= 0x7F800000u;                  // NaN or Inf
    if (!nonfinite && a > 0.0f) s = __fdiv_rn(a, 448.0f);
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = m > partial[i] ? m : partial[i];
    m = block_max_u32(m, red);
    nonfinite = m >= 0x7F80u;
    if (!nonfinite && m != 0u) s = __fdiv_rn(__builtin_bit_cast(float, m << 16), 448.0f);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  const bool direct = s < 1.17549435e-38f;        // subnormal scale: divide directly
  const float r = __frcp_rn(s);

  const int64_t nchunks = n >> 3;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    uint4 v = reinterpret_cast<const uint4*>(x)[c];
    uint32_t lo, hi;
    if (nonfinite) {
      lo = pt_nonfinite_pair<false>(v.x, 0u);
      lo = pt_nonfinite_pair<true>(v.y, lo);
      hi = pt_nonfinite_pair<false>(v.z, 0u);
      hi = pt_nonfinite_pair<true>(v.w, hi);
    } else {
      lo = cvt2_e4m3_sat<false>(pt_div(bf16_lo(v.x), s, r, direct), pt_div(bf16_hi(v.x), s, r, direct), 0u);
      lo = cvt2_e4m3_sat<true>(pt_div(bf16_lo(v.y), s, r, direct), pt_div(bf16_hi(v.y), s, r, direct), lo);
      hi = cvt2_e4m3_sat<false>(pt_div(bf16_lo(v.z), s, r, direct), pt_div(bf16_hi(v.z), s, r, direct), 0u);
      hi = cvt2_e4m3_sat<true>(pt_div(bf16_lo(v.w), s, r, direct), pt_div(bf16_hi(v.w), s, r, direct), hi);
    }
    reinterpret_cast<uint2*>(q)[c] = make_uint2(lo, hi);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    int64_t i = (nchunks << 3) + threadIdx.x;
    uint32_t w = x[i];
    uint32_t out = nonfinite ? pt_nonfinite_pair<false>(w, 0u)
                             : cvt2_e4m3_sat<false>(pt_div(bf16_lo(w), s, r, direct), 0.0f, 0u);
    q[i] = (uint8_t)(out & 0xFFu);
  }
}

// ---------------------------------------------------------------------------
// Blockwise FP8, the comparison recipe ("Transformer 与 LLM（06）：浮点格式、数值
// 稳定性与混合精度" §七.3, DeepSeek-V3's blocks): one FP32 scale per 1x128
// activation block or 128x128 weight block, each block quantized by the
// current-scaling rule (scale = amax / 448, or 1 for a zero or non-finite
// amax; codes RNE_E4M3(x / scale) with an exact FP32 quotient).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float pt_block_scale(uint32_t m) {
  return (m < 0x7F80u && m != 0u) ? __fdiv_rn(__builtin_bit_cast(float, m << 16), 448.0f) : 1.0f;
}

constexpr int kDppRowMirror = 0x140;       // lane i <- lane 15 - i within a row of 16
constexpr int kDppRowHalfMirror = 0x141;   // lane i <- lane 7 - i within each half row

// 1x128 blocks: a wavefront owns 512 consecutive elements of a row (8 per
// lane), so the 16 lanes of a DPP row hold one block; the block amax is the
// packed-u16 magnitude max reduced over the row by four DPP exchanges.
__global__ __launch_bounds__(256) void k_bw_act(const uint16_t* __restrict__ x, int64_t ldx,
                                                uint8_t* __restrict__ q, int64_t ldq,
                                                float* __restrict__ sc, int64_t lds, uint32_t K,
                                                uint32_t segs_per_row, uint32_t total_segs) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const uint32_t nwave = gridDim.x * (blockDim.x >> 6);
  for (uint32_t sg = wave; sg < total_segs; sg += nwave) {
    const uint32_t row = sg / segs_per_row;             // wave-uniform
    const uint32_t col = (sg - row * segs_per_row) * 512u + lane * 8u;
    const bool ok = col < K;
    const uint4 v = ok ? *reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + col)
                       : make_uint4(0, 0, 0, 0);
    const u16x2 mm = __builtin_elementwise_max(absmax2(v.x, v.y), absmax2(v.z, v.w));
    uint32_t am = mm.x > mm.y ? mm.x : mm.y;
    uint32_t o = dpp_u32(am, kQuadXor1);
    am = am > o ? am : o;
    o = dpp_u32(am, kQuadXor2);
    am = am > o ? am : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)am, kDppRowHalfMirror, 0xF, 0xF, false);
    am = am > o ? am : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)am, kDppRowMirror, 0xF, 0xF, false);
    am = am > o ? am : o;
    const bool nonfinite = am >= 0x7F80u;
    const float s = pt_block_scale(am);
    const bool direct = s < 1.17549435e-38f;
    const uint2 c = pt_encode8(v, s, __frcp_rn(s), direct, nonfinite);
    if (ok) {
      store_stream(q + (int64_t)row * ldq + col, c);
      if ((lane & 15u) == 0u) sc[(int64_t)row * lds + (col >> 7)] = s;
    }
  }
}

// 128x128 blocks: one workgroup per block, held in registers across its amax
// reduction.  Each load instruction of a wavefront reads 4 whole 256-byte
// block rows (16 lanes per row); a lane's 8 loads are rows 32w + 4u + t/16,
// u = 0..7, of wavefront w, all at columns 8 (t%16) .. +7.
__global__ __launch_bounds__(256) void k_bw_weight(const uint16_t* __restrict__ w, int64_t N,
                                                   int64_t ldw, uint8_t* __restrict__ q,
                                                   int64_t ldq, float* __restrict__ sc,
                                                   int64_t lds, uint32_t kblocks) {
  __shared__ uint32_t red[4];
  const uint32_t rb = blockIdx.x / kblocks, kb = blockIdx.x - rb * kblocks;
  const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)rb * 128 + wv * 32 + (lane >> 4);
  const int64_t col = (int64_t)kb * 128 + (lane & 15u) * 8;
  uint4 v[8];
  uint32_t am = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t row = row0 + 4 * u;
    v[u] = row < N ? *reinterpret_cast<const uint4*>(w + row * ldw + col)
                   : make_uint4(0, 0, 0, 0);
    const u16x2 mm = __builtin_elementwise_max(absmax2(v[u].x, v[u].y), absmax2(v[u].z, v[u].w));
    const uint32_t t = mm.x > mm.y ? mm.x : mm.y;
    am = am > t ? am : t;
  }
  am = block_max_u32(am, red);
  const bool nonfinite = am >= 0x7F80u;
  const float s = pt_block_scale(am);
  const bool direct = s < 1.17549435e-38f;
  const float r = __frcp_rn(s);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t row = row0 + 4 * u;
    if (row < N) store_stream(q + row * ldq + col, pt_encode8(v[u], s, r, direct, nonfinite));
  }
  if (threadIdx.x == 0) sc[(int64_t)rb * lds + kb] = s;
}

__global__ void k_fill_f32(float* p, float v) {
  if (threadIdx.x == 0) *p = v;
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Per-group (per-expert) current scaling: rows [offsets[e], offsets[e+1])
// share one FP32 scale.  Pass 1 takes each row's packed |x| maximum (one
// wavefront per row, 16-byte loads, four in flight per lane), pass 2 reduces
// each group's rows to its amax and scale (one workgroup per group, so an
// empty group gets 1.0), pass 3 encodes every row with its group's scale
// exactly as the per-tensor pass does.
// ---------------------------------------------------------------------------

constexpr int kPgThreads = 256;
constexpr int kPgMaxGroups = 256;

__global__ __launch_bounds__(kPgThreads) void k_pg_rowmax(const uint16_t* __restrict__ x,
                                                          int64_t M, int64_t K, int64_t ldx,
                                                          uint32_t* __restrict__ rowmax) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kPgThreads / 64);
  for (int64_t r = (int64_t)blockIdx.x * (kPgThreads / 64) + (threadIdx.x >> 6); r < M;
       r += nw) {
    const uint16_t* row = x + r * ldx;
    uint32_t m = 0;
    for (int64_t c0 = lane * 8; c0 < K; c0 += 4 * 512) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = c0 + u * 512 < K ? *reinterpret_cast<const uint4*>(row + c0 + u * 512)
                                : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u16x2 mm = __builtin_elementwise_max(absmax2(v[u].x, v[u].y), absmax2(v[u].z, v[u].w));
        const uint32_t t = mm.x > mm.y ? mm.x : mm.y;
        m = m > t ? m : t;
      }
    }
    for (int sh = 32; sh >= 1; sh >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, sh, 64);
      m = m > o ? m : o;
    }
    if (lane == 0) rowmax[r] = m;
  }
}

__global__ __launch_bounds__(kPgThreads) void k_pg_scale(const uint32_t* __restrict__ rowmax,
                                                         const int64_t* __restrict__ offsets,
                                                         int64_t M, uint32_t* __restrict__ gmax,
                                                         float* __restrict__ scales) {
  __shared__ uint32_t red[kPgThreads / 64];
  const int e = blockIdx.x;
  int64_t lo = offsets[e], hi = offsets[e + 1];
  lo = lo < 0 ? 0 : (lo > M ? M : lo);
  hi = hi < lo ? lo : (hi > M ? M : hi);
  uint32_t m = 0;
  for (int64_t r = lo + threadIdx.x; r < hi; r += blockDim.x) m = m > rowmax[r] ? m : rowmax[r];
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) {
    float sc = 1.0f;
    if (m < 0x7F80u && m != 0u) sc = __fdiv_rn(__builtin_bit_cast(float, m << 16), 448.0f);
    scales[e] = sc;
    gmax[e] = m;
  }
}

// Group scales from given group amaxes (FP32, e.g. from the producing
// matmul's epilogue): the same rule as k_pg_scale; gmax receives the BF16
// magnitude pattern k_pg_quant tests for NaN/Inf.
__global__ void k_pg_scale_amax(const float* __restrict__ amax, int32_t E,
                                uint32_t* __restrict__ gmax, float* __restrict__ scales) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const uint32_t bits = __builtin_bit_cast(uint32_t, amax[e]) & 0x7FFFFFFFu;
  float sc = 1.0f;
  if (bits < 0x7F800000u && bits != 0u) sc = __fdiv_rn(__builtin_bit_cast(float, bits), 448.0f);
  scales[e] = sc;
  gmax[e] = bits >> 16;
}

__global__ __launch_bounds__(kPgThreads) void k_pg_quant(const uint16_t* __restrict__ x,
                                                         int64_t M, int64_t K, int64_t ldx,
                                                         const int64_t* __restrict__ offsets,
                                                         int32_t E, const uint32_t* __restrict__ gmax,
                                                         const float* __restrict__ scales,
                                                         uint8_t* __restrict__ q, int64_t ldq) {
  __shared__ int64_t s_off[kPgMaxGroups + 1];
  for (int i = threadIdx.x; i <= E; i += blockDim.x) s_off[i] = offsets[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * (kPgThreads / 64);
  for (int64_t r = (int64_t)blockIdx.x * (kPgThreads / 64) + (threadIdx.x >> 6); r < M;
       r += nw) {
    // group of row r: the last e with offsets[e] <= r (empty groups skipped)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const bool nonfinite = gmax[lo] >= 0x7F80u;
    const float sc = scales[lo];
    const bool direct = sc < 1.17549435e-38f;     // subnormal scale: divide directly
    const float rc = __frcp_rn(sc);
    const uint16_t* row = x + r * ldx;
    uint8_t* qrow = q + r * ldq;
    for (int64_t c = lane * 8; c < K; c += 512) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + c);
      uint32_t lo32, hi32;
      if (nonfinite) {
        lo32 = pt_nonfinite_pair<false>(v.x, 0u);
        lo32 = pt_nonfinite_pair<true>(v.y, lo32);
        hi32 = pt_nonfinite_pair<false>(v.z, 0u);
        hi32 = pt_nonfinite_pair<true>(v.w, hi32);
      } else {
        lo32 = cvt2_e4m3_sat<false>(pt_div(bf16_lo(v.x), sc, rc, direct),
                                    pt_div(bf16_hi(v.x), sc, rc, direct), 0u);
        lo32 = cvt2_e4m3_sat<true>(pt_div(bf16_lo(v.y), sc, rc, direct),
                                   pt_div(bf16_hi(v.y), sc, rc, direct), lo32);
        hi32 = cvt2_e4m3_sat<false>(pt_div(bf16_lo(v.z), sc, rc, direct),
                                    pt_div(bf16_hi(v.z), sc, rc, direct), 0u);
        hi32 = cvt2_e4m3_sat<true>(pt_div(bf16_lo(v.w), sc, rc, direct),
                                   pt_div(bf16_hi(v.w), sc, rc, direct), hi32);
      }
      *reinterpret_cast<uint2*>(qrow + c) = make_uint2(lo32, hi32);
    }
  }
}

}  // namespace mxq

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

using namespace mxq;

static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

static int num_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
  }
  return cus;
}

// Checks one row-wise item and fills its segment range (first and total are
// set by the caller).  Returns MXQ_OK with it->total == 0 for an empty item.
static int rowwise_item(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                        int64_t ldq, uint8_t* scale, int64_t lds, RowItem* it) {
  *it = RowItem{};
  if (M < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (M == 0 || K == 0) return MXQ_OK;
  if (!x || !q || !scale) return MXQ_ERR_NULL;
  if (K % 32 != 0 || ldx < K || ldq < K || lds < K / 32) return MXQ_ERR_SHAPE;
  if (ldx % 8 != 0 || ldq % 16 != 0 || !aligned(x, 16) || !aligned(q, 16)) return MXQ_ERR_ALIGN;
  // A contiguous matrix is one long row: segments then cross row ends.
  int64_t rows = M, cols = K;
  if (ldx == K && ldq == K && lds == K / 32 && sat_mul(M, K) <= 0xFFFFFFFFLL) {
    rows = 1;
    cols = M * K;
  }
  if (cols > 0xFFFFFFFFLL) return MXQ_ERR_SHAPE;
  const int64_t segs_per_row = (cols + 511) / 512;
  const int64_t total = sat_mul(rows, segs_per_row);
  if (total > 0x7FFFFFFFLL - 2 * kRowUnroll) return MXQ_ERR_SHAPE;
  it->x = x;
  it->q = q;
  it->sc = scale;
  it->ldx = rows == 1 ? cols : ldx;
  it->ldq = rows == 1 ? cols : ldq;
  it->lds = rows == 1 ? cols / 32 : lds;
  it->K = (uint32_t)cols;
  it->segs_per_row = (uint32_t)segs_per_row;
  it->total = (uint32_t)total;
  return MXQ_OK;
}

static int launch_rowwise(RowBatch& b, hipStream_t stream) {
  // pack the non-empty items, each starting on a group boundary
  uint32_t n = 0;
  int64_t first = 0;
  for (uint32_t i = 0; i < b.n; ++i) {
    if (b.it[i].total == 0) continue;
    b.it[n] = b.it[i];
    b.it[n].first = (uint32_t)first;
    first += ((int64_t)b.it[i].total + kRowUnroll - 1) / kRowUnroll * kRowUnroll;
    if (first > 0x7FFFFFFFLL) return MXQ_ERR_SHAPE;
    ++n;
  }
  if (n == 0) return MXQ_OK;
  b.n = n;
  b.total = (uint32_t)first;
  const int64_t waves = first / kRowUnroll;
  int64_t blocks = (waves + 3) / 4;
  const int64_t cap = (int64_t)num_cus() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_mx_rowwise, dim3((uint32_t)blocks), dim3(256), 0, stream, b);
  return launch_status();
}

extern "C" int mx_quantize_rowwise(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* q, int64_t ldq, uint8_t* scale, int64_t lds,
                                   hipStream_t stream) {
  RowBatch b{};
  const int st = rowwise_item(x, M, K, ldx, q, ldq, scale, lds, &b.it[0]);
  if (st != MXQ_OK) return st;
  b.n = 1;
  return launch_rowwise(b, stream);
}

extern "C" int mx_quantize_rowwise_batch(const mxq_rowwise_item* items, int32_t n,
                                         hipStream_t stream) {
  if (n < 1 || n > kRowBatch) return MXQ_ERR_SHAPE;
  if (!items) return MXQ_ERR_NULL;
  RowBatch b{};
  for (int32_t i = 0; i < n; ++i) {
    const mxq_rowwise_item& it = items[i];
    const int st = rowwise_item(it.x, it.M, it.K, it.ldx, it.q, it.ldq, it.scale, it.lds,
                                &b.it[i]);
    if (st != MXQ_OK) return st;
  }
  b.n = (uint32_t)n;
  return launch_rowwise(b, stream);
}

// Columns a grouped column copy may need: every group padded to a multiple
// of 32 adds at most 31 (the offsets are on the device, so the bound is
// checked, not the padded total).  No groups: M rounded up to 32.  An empty
// input needs nothing.
static int64_t padded_capacity(int64_t M, int32_t E) {
  if (M <= 0) return 0;
  return E > 0 ? sat_add(M, 31LL * E) : sat_add(M, 31) / 32 * 32;
}

// Workgroups of one column-tile item: M_cap in 128-column tiles times K in
// chunks of kColPasses passes.
static int col_blocks(int64_t M_cap, int64_t K, uint32_t* nblk) {
  const int64_t gx = sat_add(M_cap, kColTileM - 1) / kColTileM;
  const int64_t gy = sat_add(K, kColTileK * kColPasses - 1) / (kColTileK * kColPasses);
  const int64_t n = sat_mul(gx, gy);
  if (n > 0x7FFFFFFFLL) return MXQ_ERR_SHAPE;
  *nblk = (uint32_t)n;
  return MXQ_OK;
}

template <bool ROW, bool PG>
static int launch_colwise(ColBatch& b, hipStream_t stream) {
  // pack the non-empty items, each owning a contiguous run of workgroups
  uint32_t n = 0;
  int64_t first = 0;
  for (uint32_t i = 0; i < b.n; ++i) {
    if (b.it[i].nblk == 0) continue;
    b.it[n] = b.it[i];
    b.it[n].first = (uint32_t)first;
    first += b.it[i].nblk;
    if (first > 0x7FFFFFFFLL) return MXQ_ERR_SHAPE;
    ++n;
  }
  if (n == 0) return MXQ_OK;
  b.n = n;
  hipLaunchKernelGGL((k_mx_colwise<ROW, PG>), dim3((uint32_t)first), dim3(256), 0, stream, b);
  return launch_status();
}

extern "C" int mx_quantize_colwise(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   const int64_t* offsets, int32_t E, uint8_t* qT, int64_t ldqT,
                                   int64_t M_cap, uint8_t* scaleT, int64_t ldsT,
                                   int64_t* offsets_padded, hipStream_t stream) {
  if (M < 0 || K < 0 || M_cap < 0) return MXQ_ERR_SHAPE;
  if (offsets && (E < 1 || E > kColMaxGroupsLds)) return MXQ_ERR_SHAPE;
  if (M_cap < padded_capacity(M, offsets ? E : 0)) return MXQ_ERR_SHAPE;
  if (K == 0 || M_cap == 0) return MXQ_OK;
  if (!qT || !scaleT || (M > 0 && !x)) return MXQ_ERR_NULL;
  if (K % 8 != 0 || M_cap % 32 != 0 || ldqT < M_cap || ldsT < M_cap / 32 || ldx < K)
    return MXQ_ERR_SHAPE;
  if (ldqT % 16 != 0 || ldx % 8 != 0 || !aligned(qT, 16) || (x && !aligned(x, 16)))
    return MXQ_ERR_ALIGN;
  ColBatch b{};
  ColItem& t = b.it[0];
  if (col_blocks(M_cap, K, &t.nblk) != MXQ_OK) return MXQ_ERR_SHAPE;
  t.x = x; t.M = M; t.K = K; t.ldx = ldx; t.offsets = offsets; t.E = E;
  t.qT = qT; t.ldqT = ldqT; t.M_cap = M_cap; t.scT = scaleT; t.ldsT = ldsT;
  t.offsets_padded = offsets_padded;
  b.n = 1;
  return launch_colwise<false, false>(b, stream);
}

// Checks one dual-axis item and fills it (nblk == 0 for an item that writes
// nothing).
static int dual_item(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     const int64_t* offsets, int32_t E, uint8_t* q, int64_t ldq, uint8_t* scale,
                     int64_t lds, uint8_t* qT, int64_t ldqT, int64_t M_cap, uint8_t* scaleT,
                     int64_t ldsT, int64_t* offsets_padded, ColItem* t) {
  *t = ColItem{};
  if (M < 0 || K < 0 || M_cap < 0) return MXQ_ERR_SHAPE;
  if (offsets && (E < 1 || E > kColMaxGroupsLds)) return MXQ_ERR_SHAPE;
  // every row must land in the column copy: the row copy is written from the
  // same column tiles
  if (M_cap < padded_capacity(M, offsets ? E : 0)) return MXQ_ERR_SHAPE;
  if (K == 0 || M_cap == 0) return MXQ_OK;
  if (!qT || !scaleT || (M > 0 && (!x || !q || !scale))) return MXQ_ERR_NULL;
  if (K % 32 != 0 || M_cap % 32 != 0 || ldqT < M_cap || ldsT < M_cap / 32 || ldx < K ||
      ldq < K || lds < K / 32)
    return MXQ_ERR_SHAPE;
  if (ldqT % 16 != 0 || ldx % 8 != 0 || ldq % 16 != 0 || !aligned(qT, 16) ||
      (x && !aligned(x, 16)) || (q && !aligned(q, 16)))
    return MXQ_ERR_ALIGN;
  uint32_t nblk = 0;
  if (col_blocks(M_cap, K, &nblk) != MXQ_OK) return MXQ_ERR_SHAPE;
  t->x = x; t->M = M; t->K = K; t->ldx = ldx; t->offsets = offsets; t->E = E;
  t->qT = qT; t->ldqT = ldqT; t->M_cap = M_cap; t->scT = scaleT; t->ldsT = ldsT;
  t->offsets_padded = offsets_padded;
  t->q = q; t->ldq = ldq; t->sc = scale; t->lds = lds;
  t->nblk = nblk;
  return MXQ_OK;
}

extern "C" int mx_quantize_dual(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                const int64_t* offsets, int32_t E, uint8_t* q, int64_t ldq,
                                uint8_t* scale, int64_t lds, uint8_t* qT, int64_t ldqT,
                                int64_t M_cap, uint8_t* scaleT, int64_t ldsT,
                                int64_t* offsets_padded, hipStream_t stream) {
  ColBatch b{};
  const int st = dual_item(x, M, K, ldx, offsets, E, q, ldq, scale, lds, qT, ldqT, M_cap, scaleT,
                           ldsT, offsets_padded, &b.it[0]);
  if (st != MXQ_OK) return st;
  b.n = 1;
  return launch_colwise<true, false>(b, stream);
}

extern "C" int mx_quantize_dual_batch(const mxq_dual_item* items, int32_t n,
                                      hipStream_t stream) {
  if (n < 1 || n > kColBatch) return MXQ_ERR_SHAPE;
  if (!items) return MXQ_ERR_NULL;
  ColBatch b{};
  for (int32_t i = 0; i < n; ++i) {
    const mxq_dual_item& d = items[i];
    const int st = dual_item(d.x, d.M, d.K, d.ldx, d.offsets, d.E, d.q, d.ldq, d.scale, d.lds,
                             d.qT, d.ldqT, d.M_cap, d.scaleT, d.ldsT, d.offsets_padded, &b.it[i]);
    if (st != MXQ_OK) return st;
  }
  b.n = (uint32_t)n;
  return launch_colwise<true, false>(b, stream);
}

extern "C" size_t mxq_workspace_size(int op, int64_t n, int64_t a1, int64_t, int64_t) {
  if (op == MXQ_WS_PER_TENSOR) return n > 0 ? kPtBlocks * sizeof(uint32_t) : 0;
  if (op == MXQ_WS_PER_GROUP && n >= 0 && a1 > 0) {   // n = rows, a1 = groups
    const int64_t words = sat_add(n, a1);
    return words > INT64_MAX / (int64_t)sizeof(uint32_t) ? SIZE_MAX
                                                          : (size_t)words * sizeof(uint32_t);
  }
  return 0;
}

// Group scales into scales[E] and the NaN/Inf patterns into gmax: from the
// given amaxes, or from a row-maxima pass over x (rowmax: M entries).
static int pg_scales(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     const int64_t* offsets, int32_t E, const float* amax, uint32_t* rowmax,
                     uint32_t* gmax, float* scales, uint32_t blocks, hipStream_t stream) {
  if (amax) {
    hipLaunchKernelGGL(k_pg_scale_amax, dim3((uint32_t)((E + 255) / 256)), dim3(256), 0, stream,
                       amax, E, gmax, scales);
    return launch_status();
  }
  if (M > 0 && K > 0) {
    hipLaunchKernelGGL(k_pg_rowmax, dim3(blocks), dim3(kPgThreads), 0, stream, x, M, K, ldx,
                       rowmax);
  } else if (M > 0) {
    hipLaunchKernelGGL(k_fill_u32, dim3((uint32_t)((M + 255) / 256)), dim3(256), 0, stream,
                       rowmax, M, 0u);
  }
  int st = launch_status();
  if (st != MXQ_OK) return st;
  hipLaunchKernelGGL(k_pg_scale, dim3((uint32_t)E), dim3(kPgThreads), 0, stream, rowmax, offsets,
                     M, gmax, scales);
  return launch_status();
}

// Arguments of the row-major per-group quantization (workspace aside).
static int per_group_args(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                          const int64_t* offsets, int32_t E, const uint8_t* q, int64_t ldq,
                          const float* scales) {
  if (M < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (E < 1 || E > kPgMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets || !scales) return MXQ_ERR_NULL;
  if (M > 0 && K > 0 && (!x || !q)) return MXQ_ERR_NULL;
  if (K % 8 != 0) return MXQ_ERR_SHAPE;
  if (M > 0 && K > 0) {                              // strides of empty inputs are not used
    if (ldx < K || ldq < K) return MXQ_ERR_SHAPE;
    if (ldx % 8 != 0 || ldq % 8 != 0 || !aligned(x, 16) || !aligned(q, 8)) return MXQ_ERR_ALIGN;
  }
  return MXQ_OK;
}

static int quantize_per_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const int64_t* offsets, int32_t E, const float* amax, uint8_t* q,
                              int64_t ldq, float* scales, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const int a = per_group_args(x, M, K, ldx, offsets, E, q, ldq, scales);
  if (a != MXQ_OK) return a;
  if (!workspace) return MXQ_ERR_NULL;
  if (!aligned(workspace, 4)) return MXQ_ERR_ALIGN;
  const int64_t ws_rows = amax ? 0 : M;              // row maxima only without amaxes
  if (workspace_bytes < mxq_workspace_size(MXQ_WS_PER_GROUP, ws_rows, E, 0, 0))
    return MXQ_ERR_WORKSPACE;
  uint32_t* rowmax = static_cast<uint32_t*>(workspace);
  uint32_t* gmax = rowmax + ws_rows;
  const int64_t waves = (int64_t)num_cus() * 64;    // rows in flight: 16 wavefronts per CU
  const int64_t rows_blocks = sat_add(M, 3) / 4;
  const uint32_t blocks = (uint32_t)(rows_blocks < waves / 4 ? (rows_blocks > 0 ? rows_blocks : 1)
                                                             : waves / 4);
  int st = pg_scales(x, M, K, ldx, offsets, E, amax, rowmax, gmax, scales, blocks, stream);
  if (st != MXQ_OK || M == 0 || K == 0) return st;
  hipLaunchKernelGGL(k_pg_quant, dim3(blocks), dim3(kPgThreads), 0, stream, x, M, K, ldx,
                     offsets, E, gmax, scales, q, ldq);
  return launch_status();
}

extern "C" int fp8_quantize_per_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      const int64_t* offsets, int32_t E, uint8_t* q,
                                      int64_t ldq, float* scales, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return quantize_per_group(x, M, K, ldx, offsets, E, nullptr, q, ldq, scales, workspace,
                            workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free per-group quantization.  The row maxima and group maxima
// that fp8_quantize_per_group keeps in the caller's workspace live in this
// file-scope device array instead: one copy per GPU, held until the process
// ends, shared by every call on that GPU (calls that overlap on one GPU race).
// In host code `scratch` names a host-side stand-in, never the device memory:
// its device address is looked up once per device and only that is used.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchWords = 1 << 18;          // 1 MiB: M + E <= 262144
static __device__ __align__(256) uint32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static uint32_t* g_scratch_ptr[kMaxDevices];        // device address of `scratch` per device

// Device address of the current device's `scratch`, looked up on its first
// use on that device (with it current) and kept.
static int current_scratch(uint32_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MXQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MXQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXQ_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MXQ_OK;
}

extern "C" int fp8_quantize_per_group_noalloc(const uint16_t* x, int64_t M, int64_t K,
                                              int64_t ldx, const int64_t* offsets, int32_t E,
                                              uint8_t* q, int64_t ldq, float* scales,
                                              hipStream_t stream) {
  const int a = per_group_args(x, M, K, ldx, offsets, E, q, ldq, scales);
  if (a != MXQ_OK) return a;
  // row maxima [M] then group maxima [E]; every word read is written earlier
  // in the same call, so nothing needs clearing between calls
  if (sat_add(M, E) > kScratchWords) return MXQ_ERR_SHAPE;
  uint32_t* ws = nullptr;
  const int st = current_scratch(&ws);
  if (st != MXQ_OK) return st;
  return quantize_per_group(x, M, K, ldx, offsets, E, nullptr, q, ldq, scales, ws,
                            (size_t)kScratchWords * sizeof(uint32_t), stream);
}

extern "C" int fp8_quantize_per_group_amax(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                           const int64_t* offsets, int32_t E,
                                           const float* amax, uint8_t* q, int64_t ldq,
                                           float* scales, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (!amax) return MXQ_ERR_NULL;
  return quantize_per_group(x, M, K, ldx, offsets, E, amax, q, ldq, scales, workspace,
                            workspace_bytes, stream);
}

static int quantize_per_group_colwise(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                     const int64_t* offsets, int32_t E, const float* amax,
                                     uint8_t* qT, int64_t ldqT, int64_t M_cap, float* scales,
                                     int64_t* offsets_padded, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || K < 0 || M_cap < 0) return MXQ_ERR_SHAPE;
  if (E < 1 || E > kPgMaxGroups) return MXQ_ERR_SHAPE;
  if (!offsets || !scales || !workspace) return MXQ_ERR_NULL;
  if (K % 8 != 0 || M_cap % 32 != 0 || M_cap < padded_capacity(M, E)) return MXQ_ERR_SHAPE;
  if (K > 0 && M_cap > 0) {
    if (!qT || (M > 0 && !x)) return MXQ_ERR_NULL;
    if (ldqT < M_cap || (M > 0 && ldx < K)) return MXQ_ERR_SHAPE;
    if (ldqT % 16 != 0 || !aligned(qT, 16) || (M > 0 && (ldx % 8 != 0 || !aligned(x, 16))))
      return MXQ_ERR_ALIGN;
  }
  if (!aligned(workspace, 4)) return MXQ_ERR_ALIGN;
  const int64_t ws_rows = amax ? 0 : M;
  if (workspace_bytes < mxq_workspace_size(MXQ_WS_PER_GROUP, ws_rows, E, 0, 0))
    return MXQ_ERR_WORKSPACE;
  uint32_t* rowmax = static_cast<uint32_t*>(workspace);
  uint32_t* gmax = rowmax + ws_rows;
  const int64_t waves = (int64_t)num_cus() * 64;
  const int64_t rows_blocks = sat_add(M, 3) / 4;
  const uint32_t blocks = (uint32_t)(rows_blocks < waves / 4 ? (rows_blocks > 0 ? rows_blocks : 1)
                                                             : waves / 4);
  int st = pg_scales(x, M, K, ldx, offsets, E, amax, rowmax, gmax, scales, blocks, stream);
  if (st != MXQ_OK || K == 0 || M_cap == 0) return st;
  ColBatch b{};
  ColItem& t = b.it[0];
  if (col_blocks(M_cap, K, &t.nblk) != MXQ_OK) return MXQ_ERR_SHAPE;
  t.x = x; t.M = M; t.K = K; t.ldx = ldx; t.offsets = offsets; t.E = E;
  t.qT = qT; t.ldqT = ldqT; t.M_cap = M_cap; t.offsets_padded = offsets_padded;
  t.gmax = gmax; t.gscale = scales;
  b.n = 1;
  return launch_colwise<false, true>(b, stream);
}

extern "C" int fp8_quantize_per_group_colwise(const uint16_t* x, int64_t M, int64_t K,
                                              int64_t ldx, const int64_t* offsets, int32_t E,
                                              uint8_t* qT, int64_t ldqT, int64_t M_cap,
                                              float* scales, int64_t* offsets_padded,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  return quantize_per_group_colwise(x, M, K, ldx, offsets, E, nullptr, qT, ldqT, M_cap, scales,
                                    offsets_padded, workspace, workspace_bytes, stream);
}

extern "C" int fp8_quantize_per_group_colwise_amax(const uint16_t* x, int64_t M, int64_t K,
                                                   int64_t ldx, const int64_t* offsets,
                                                   int32_t E, const float* amax, uint8_t* qT,
                                                   int64_t ldqT, int64_t M_cap, float* scales,
                                                   int64_t* offsets_padded, void* workspace,
                                                   size_t workspace_bytes, hipStream_t stream) {
  if (!amax) return MXQ_ERR_NULL;
  return quantize_per_group_colwise(x, M, K, ldx, offsets, E, amax, qT, ldqT, M_cap, scales,
                                    offsets_padded, workspace, workspace_bytes, stream);
}

extern "C" int fp8_quantize_per_group_dual(const uint16_t* x, int64_t M, int64_t K,
                                           int64_t ldx, const int64_t* offsets, int32_t E,
                                           const float* amax,
                                           uint8_t* q, int64_t ldq, uint8_t* qT, int64_t ldqT,
                                           int64_t M_cap, float* scales,
                                           int64_t* offsets_padded, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || K < 0 || M_cap < 0) return MXQ_ERR_SHAPE;
  if (E < 1 || E > kPgMaxGroups || E > kColMaxGroupsLds) return MXQ_ERR_SHAPE;
  if (!offsets || !scales || !workspace) return MXQ_ERR_NULL;
  if (K % 8 != 0 || M_cap % 32 != 0 || M_cap < padded_capacity(M, E)) return MXQ_ERR_SHAPE;
  if (K > 0 && M_cap > 0) {
    if (!qT || (M > 0 && (!x || !q))) return MXQ_ERR_NULL;
    if (ldqT < M_cap || (M > 0 && (ldx < K || ldq < K))) return MXQ_ERR_SHAPE;
    if (ldqT % 16 != 0 || !aligned(qT, 16) ||
        (M > 0 && (ldx % 8 != 0 || !aligned(x, 16) || ldq % 8 != 0 || !aligned(q, 8))))
      return MXQ_ERR_ALIGN;
  }
  if (!aligned(workspace, 4)) return MXQ_ERR_ALIGN;
  const int64_t ws_rows = amax ? 0 : M;              // row maxima only without amaxes
  if (workspace_bytes < mxq_workspace_size(MXQ_WS_PER_GROUP, ws_rows, E, 0, 0))
    return MXQ_ERR_WORKSPACE;
  uint32_t* rowmax = static_cast<uint32_t*>(workspace);
  uint32_t* gmax = rowmax + ws_rows;
  const int64_t waves = (int64_t)num_cus() * 64;
  const int64_t rows_blocks = sat_add(M, 3) / 4;
  const uint32_t blocks = (uint32_t)(rows_blocks < waves / 4 ? (rows_blocks > 0 ? rows_blocks : 1)
                                                             : waves / 4);
  int st = pg_scales(x, M, K, ldx, offsets, E, amax, rowmax, gmax, scales, blocks, stream);
  if (st != MXQ_OK || K == 0 || M_cap == 0) return st;
  ColBatch b{};
  ColItem& t = b.it[0];
  if (col_blocks(M_cap, K, &t.nblk) != MXQ_OK) return MXQ_ERR_SHAPE;
  t.x = x; t.M = M; t.K = K; t.ldx = ldx; t.offsets = offsets; t.E = E;
  t.qT = qT; t.ldqT = ldqT; t.M_cap = M_cap; t.offsets_padded = offsets_padded;
  t.q = q; t.ldq = ldq; t.gmax = gmax; t.gscale = scales;
  b.n = 1;
  return launch_colwise<true, true>(b, stream);
}

extern "C" int fp8_quantize_per_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* scale,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (n < 0) return MXQ_ERR_SHAPE;
  if (!scale) return MXQ_ERR_NULL;
  if (n == 0) {
    // Empty tensor: no amax to take, the scale is 1.0.
    hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(64), 0, stream, scale, 1.0f);
    return launch_status();
  }
  if (!x || !q || !workspace) return MXQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(workspace, 4)) return MXQ_ERR_ALIGN;
  if (workspace_bytes < mxq_workspace_size(MXQ_WS_PER_TENSOR, n, 0, 0, 0)) return MXQ_ERR_WORKSPACE;
  int64_t chunks = n / 8;
  int64_t blocks = (chunks + kPtThreads - 1) / kPtThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > kPtBlocks) blocks = kPtBlocks;
  uint32_t* partial = static_cast<uint32_t*>(workspace);
  hipLaunchKernelGGL(k_pt_amax, dim3((uint32_t)blocks), dim3(kPtThreads), 0, stream, x, n, partial);
  int st = launch_status();
  if (st != MXQ_OK) return st;
  hipLaunchKernelGGL(k_pt_quant, dim3((uint32_t)blocks), dim3(kPtThreads), 0, stream, x, n,
                     partial, (int)blocks, q, scale, nullptr);
  return launch_status();
}

extern "C" int fp8_quantize_per_tensor_amax(const uint16_t* x, int64_t n, const float* amax,
                                            uint8_t* q, float* scale, hipStream_t stream) {
  if (n < 0) return MXQ_ERR_SHAPE;
  if (!scale || !amax) return MXQ_ERR_NULL;
  if (n > 0 && (!x || !q)) return MXQ_ERR_NULL;
  if (n > 0 && (!aligned(x, 16) || !aligned(q, 16))) return MXQ_ERR_ALIGN;
  int64_t blocks = (n / 8 + kPtThreads - 1) / kPtThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > kPtBlocks) blocks = kPtBlocks;
  hipLaunchKernelGGL(k_pt_quant, dim3((uint32_t)blocks), dim3(kPtThreads), 0, stream, x, n,
                     nullptr, 0, q, scale, amax);
  return launch_status();
}

extern "C" int fp8_quantize_blockwise_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                          uint8_t* q, int64_t ldq, float* scales, int64_t lds,
                                          hipStream_t stream) {
  if (M < 0 || K < 0 || K % 128 != 0) return MXQ_ERR_SHAPE;
  if (M == 0 || K == 0) return MXQ_OK;
  if (!x || !q || !scales) return MXQ_ERR_NULL;
  if (ldx < K || ldq < K || lds < K / 128) return MXQ_ERR_SHAPE;
  if (ldx % 8 != 0 || ldq % 8 != 0 || !aligned(x, 16) || !aligned(q, 8) || !aligned(scales, 4))
    return MXQ_ERR_ALIGN;
  // A contiguous matrix is one long row (blocks never cross row ends: K % 128 == 0).
  int64_t rows = M, cols = K;
  if (ldx == K && ldq == K && lds == K / 128 && sat_mul(M, K) <= 0xFFFFFFFFLL) {
    rows = 1;
    cols = M * K;
  }
  if (cols > 0xFFFFFFFFLL) return MXQ_ERR_SHAPE;
  const int64_t segs_per_row = (cols + 511) / 512;
  const int64_t total = sat_mul(rows, segs_per_row);
  if (cols > 0xFFFFFFFFLL || total > 0x7FFFFFFFLL) return MXQ_ERR_SHAPE;
  int64_t blocks = (total + 3) / 4;
  const int64_t cap = (int64_t)num_cus() * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_bw_act, dim3((uint32_t)blocks), dim3(256), 0, stream, x,
                     rows == 1 ? cols : ldx, q, rows == 1 ? cols : ldq, scales,
                     rows == 1 ? cols / 128 : lds, (uint32_t)cols, (uint32_t)segs_per_row,
                     (uint32_t)total);
  return launch_status();
}

extern "C" int fp8_quantize_blockwise_weight(const uint16_t* w, int64_t N, int64_t K,
                                             int64_t ldw, uint8_t* q, int64_t ldq,
                                             float* scales, int64_t lds, hipStream_t stream) {
  if (N < 0 || K < 0 || K % 128 != 0) return MXQ_ERR_SHAPE;
  if (N == 0 || K == 0) return MXQ_OK;
  if (!w || !q || !scales) return MXQ_ERR_NULL;
  if (ldw < K || ldq < K || lds < K / 128) return MXQ_ERR_SHAPE;
  if (ldw % 8 != 0 || ldq % 8 != 0 || !aligned(w, 16) || !aligned(q, 8) || !aligned(scales, 4))
    return MXQ_ERR_ALIGN;
  const int64_t nblocks = sat_mul(sat_add(N, 127) / 128, K / 128);
  if (nblocks > 0x7FFFFFFFLL) return MXQ_ERR_SHAPE;
  hipLaunchKernelGGL(k_bw_weight, dim3((uint32_t)nblocks), dim3(256), 0, stream, w, N, ldw, q,
                     ldq, scales, lds, (uint32_t)(K / 128));
  return launch_status();
}
