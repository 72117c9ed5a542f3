// Two-stage drafter LM head (jialefu.github.io, "EAGLE-4: Notes on the Efficient LM Head").
//
// Stage one screens the whole vocabulary with a low-rank head, u = B h, then A u, and keeps
// candidates with a local top-k fused into each tile of (shuffled) vocabulary rows, so the
// approximate scores never leave the chip.  Stage two gathers the candidates' rows of the full
// head W and recomputes their logits exactly.  The drafter's children are the K best candidates,
// with confidences from a softmax over the candidates.
//
// The arithmetic is float32 in a fixed order of the kernels' choosing (the page defines the
// stages, not a summation order; results are valid wherever two values lie within float32
// rounding of each other, and each term passes through a bounded number of roundings):
//   * lm_dot (u = B h, logits = W[token] h; d a multiple of 512): lane j of a wavefront runs a
//     chain of fused multiply-adds from 0 over elements 512 p + 8 j + e (p = 0, 1, ... outer,
//     e = 0 .. 7 inner), so every 16-byte load of the wavefront covers 1 KB contiguously; the
//     64 chain sums are then combined by a butterfly, j with j^32, then j^16, ..., j^1, which
//     leaves the same value in every lane (d/64 + 6 roundings per term);
//   * screening (A u), ranks up to 256: on v_mfma_f32_32x32x16_bf16 (v_mfma_f32_16x16x32_bf16
//     for at most 16 hidden states) with u split exactly into three bfloat16 parts
//     (u = hi + mid + lo), so every product with A is exact in float32 and a term passes through
//     at most k + 3 ceil(r / k) roundings (k = 16 or 32 products inside its MFMA, one per later
//     MFMA of the chain); larger ranks: one chain of fused multiply-adds over the rank index, in
//     order, from 0 (r roundings per term).
// Ranking uses an unsigned key of the float (-0 as +0); equal values go to the smaller row
// (screening) or the smaller token (children).
//
// Kernels:
//   lm_project_kernel  one wavefront per (i, m), u[m, i] = B[i] . h[m]          (2 MB of B)
//   lm_screen_mfma_kernel  one workgroup per tile of rows (ranks up to 256): each wavefront
//                      loads 64 rows of A straight into MFMA operands, u's three bfloat16 parts
//                      sit in LDS one block of 32 (or 16) hidden states at a time, each lane
//                      picks the k best of the 32 (or 16) rows its accumulators hold for one
//                      hidden state (a sorting network on float64 stand-ins of the keys for
//                      k <= 4), and the 8 (or 16) lists of a hidden state merge
//   lm_screen_kernel   (larger ranks) one workgroup per tile of rows: the tile's A rows stream
//                      through LDS in 64-element slices (each row's 128 B XOR-swizzled by
//                      16-byte piece so a thread reading its row is free of bank conflicts), a
//                      thread runs half of the M chains for two rows (one LDS read of u serves
//                      both), then each wavefront picks its k best rows per hidden state by
//                      wavefront maxima and the two wavefronts' picks of each hidden state are
//                      merged
//   lm_rescore_kernel  one wavefront per (m, c): W[cand] . h[m]                  (8 KB per row)
//   lm_topk_kernel     one workgroup per hidden state: each wavefront takes K rounds of
//                      wavefront maxima over its share of the candidates, the 4K picks are
//                      merged by rank, and the softmax denominator covers all valid candidates
#include <hip/hip_runtime.h>

#include "tree_device.h"

namespace tv {
namespace {

constexpr int kLmMaxM = 64;       // hidden states per call
constexpr int kLmMaxTile = 256;   // rows per screening tile (one thread each)
constexpr int kLmMaxKTile = 16;   // candidates kept per tile and hidden state
constexpr int kLmMaxK = 64;       // children per hidden state
constexpr int kLmSlice = 64;      // rank elements per LDS slice (128 B per row)

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unsigned key in the float's order, -0 taken as +0.
__device__ inline uint32_t fkey(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  // negative: all bits flipped; otherwise the sign bit set
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ inline float fkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// A 64-bit value moved by one DPP control, both halves alike; lanes without a source (or in
// rows outside kRowMask) keep their own value.
template <int kCtrl, int kRowMask>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const int lo2 = __builtin_amdgcn_update_dpp(lo, lo, kCtrl, kRowMask, 0xf, false);
  const int hi2 = __builtin_amdgcn_update_dpp(hi, hi, kCtrl, kRowMask, 0xf, false);
  return ((uint64_t)(uint32_t)hi2 << 32) | (uint32_t)lo2;
}

// A 32-bit value moved by one DPP control (lanes without a source keep their own value).
template <int kCtrl, int kRowMask>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, kRowMask, 0xf, false);
}

// Maximum of a 32-bit value over the wavefront, in every lane (the scan of wave_max_u64 below).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xf>(v));  // row_shr:1
  v = max(v, dpp_u32<0x112, 0xf>(v));  // row_shr:2
  v = max(v, dpp_u32<0x114, 0xf>(v));  // row_shr:4
  v = max(v, dpp_u32<0x118, 0xf>(v));  // row_shr:8
  v = max(v, dpp_u32<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
  v = max(v, dpp_u32<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Maximum of a float over the wavefront, in every lane (by the order-preserving key).
__device__ inline float wave_max_f32(float v) { return fkey_value(wave_max_u32(fkey(v))); }

// Sum of a float over the wavefront, in every lane: the scan of wave_max_u32 with addition,
// lanes without a source adding 0.
template <int kCtrl, int kRowMask>
__device__ inline float dpp_f32_or0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf,
                                                    false));
}
__device__ inline float wave_sum_f32(float v) {
  v += dpp_f32_or0<0x111, 0xf>(v);  // row_shr:1
  v += dpp_f32_or0<0x112, 0xf>(v);  // row_shr:2
  v += dpp_f32_or0<0x114, 0xf>(v);  // row_shr:4
  v += dpp_f32_or0<0x118, 0xf>(v);  // row_shr:8
  v += dpp_f32_or0<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f32_or0<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Maximum over the wavefront, returned to every lane.  An inclusive max scan runs within each
// row of 16 lanes (row shifts by 1, 2, 4, 8), then across rows (lane 15 of a row broadcast to
// the next row, then lane 31 to rows 2 and 3), so lane 63 ends with the maximum, which is read
// out as a uniform value.  All steps stay in the vector ALU; no LDS round trips.
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<0x111, 0xf>(v));  // row_shr:1
  v = mx(v, dpp_u64<0x112, 0xf>(v));  // row_shr:2
  v = mx(v, dpp_u64<0x114, 0xf>(v));  // row_shr:4
  v = mx(v, dpp_u64<0x118, 0xf>(v));  // row_shr:8
  v = mx(v, dpp_u64<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
  v = mx(v, dpp_u64<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// The fixed-order dot product of two bfloat16 rows of length d (d % 512 == 0), by the calling
// wavefront: lane j's pieces are the 16 bytes at element 512 p + 8 j.
__device__ inline float lm_dot(const uint16_t* __restrict__ x, const uint16_t* __restrict__ y,
                               int d) {
  const int lane = threadIdx.x & 63;
  const uint4* xs = reinterpret_cast<const uint4*>(x) + lane;  // 64 pieces per 512 elements
  const uint4* ys = reinterpret_cast<const uint4*>(y) + lane;
  float acc = 0.f;
  auto chain = [&](const uint4& a, const uint4& b) {
    acc = __builtin_fmaf(bf16_lo(a.x), bf16_lo(b.x), acc);
    acc = __builtin_fmaf(bf16_hi(a.x), bf16_hi(b.x), acc);
    acc = __builtin_fmaf(bf16_lo(a.y), bf16_lo(b.y), acc);
    acc = __builtin_fmaf(bf16_hi(a.y), bf16_hi(b.y), acc);
    acc = __builtin_fmaf(bf16_lo(a.z), bf16_lo(b.z), acc);
    acc = __builtin_fmaf(bf16_hi(a.z), bf16_hi(b.z), acc);
    acc = __builtin_fmaf(bf16_lo(a.w), bf16_lo(b.w), acc);
    acc = __builtin_fmaf(bf16_hi(a.w), bf16_hi(b.w), acc);
  };
  // eight pieces of each vector in flight at a time (4096 elements: one memory round trip),
  // then the chain over them in order
  const int np = d >> 9;
  int p = 0;
  for (; p + 8 <= np; p += 8) {
    uint4 a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = xs[64 * (p + k)];
      b[k] = ys[64 * (p + k)];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) chain(a[k], b[k]);
  }
  for (; p < np; ++p) chain(xs[64 * p], ys[64 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
  return acc;
}

__global__ __launch_bounds__(256) void lm_project_kernel(const uint16_t* __restrict__ h,
                                                         const uint16_t* __restrict__ Bm, int M,
                                                         int r, int d, float* __restrict__ u) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);  // p = i * M + m: waves of a block share B[i]
  if (p >= M * r) return;
  const int i = p / M, m = p - i * M;
  const float v = lm_dot(Bm + (size_t)i * d, h + (size_t)m * d, d);
  if ((threadIdx.x & 63) == 0) u[(size_t)m * r + i] = v;
}

// The tile's k_tile best rows per hidden state from its scores (thread (half, p) of the 256
// holds rows p and p + 128 for hidden states half * kM/2 + i), written as candidates best first.
// s_pick is LDS for M * 2 * k_tile 64-bit picks that no thread still reads.
template <int kM>
__device__ inline void screen_picks(const float (&acc)[2][kM / 2], uint64_t* s_pick,
                                    const int32_t* __restrict__ row_token, int M, int n, int tile,
                                    int k_tile, int32_t* __restrict__ cand,
                                    float* __restrict__ cand_score) {
  constexpr int kH = kM / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = tid >> 7, p = tid & 127;
  const int t = blockIdx.x;
  const int r0 = t * tile;
  const int rows = min(tile, n - r0);
  // Each wavefront's k best rows per hidden state, then the merge of the two wavefronts of the
  // half.  A wavefront holds rows q0 = 64 (wave & 1) + lane and q0 + 128, so among its rows
  // with the best score the smallest row is the lowest lane holding it in its first row, else
  // in its second: a 32-bit maximum and ballots replace a 64-bit (score, row) maximum.  The
  // hidden states' reductions of one round are independent, so they interleave.
  const int wh = wave & 1;
  const bool real0 = p < rows, real1 = p + 128 < rows;
  uint64_t taken0 = 0, taken1 = 0;  // bit i: the row was picked for hidden state half*kH + i
  for (int j = 0; j < k_tile; ++j) {
#pragma unroll
    for (int i = 0; i < kH; ++i) {
      const int m = half * kH + i;
      if (m < M) {
        const bool open0 = real0 && !((taken0 >> i) & 1);
        const bool open1 = real1 && !((taken1 >> i) & 1);
        const uint32_t k0 = open0 ? fkey(acc[0][i]) : 0u, k1 = open1 ? fkey(acc[1][i]) : 0u;
        const uint32_t best = wave_max_u32(max(k0, k1));
        const uint64_t h0 = __ballot(open0 && k0 == best);
        const uint64_t h1 = __ballot(open1 && k1 == best);
        uint64_t pick = 0;  // none left: fewer real rows than picks
        if (h0 | h1) {
          const int w = __builtin_ctzll(h0 ? h0 : h1);
          const int q = (h0 ? 0 : 128) + wh * 64 + w;
          if (lane == w) {
            if (h0) taken0 |= 1ull << i;
            else taken1 |= 1ull << i;
          }
          pick = ((uint64_t)best << 32) | (0xffffffffu - (uint32_t)(r0 + q));
        }
        if (lane == 0) s_pick[(m * 2 + wh) * k_tile + j] = pick;
      }
    }
  }
  __syncthreads();
  const int C = ceil_div(n, tile) * k_tile;
  const int per_m = 2 * k_tile;
  for (int x = tid; x < M * per_m; x += 256) {
    const int m = x / per_m, e = x - m * per_m;
    const uint64_t* pm = s_pick + m * per_m;
    const uint64_t me = pm[e];
    int rank = 0;  // picks are distinct except padding (0), which ranks by entry
    for (int o = 0; o < per_m; ++o) rank += pm[o] > me || (pm[o] == me && o < e);
    if (rank >= k_tile) continue;
    const size_t out = (size_t)m * C + (size_t)t * k_tile + rank;
    if (me == 0) {  // the tile has fewer real rows than k_tile: padding picks rank last
      cand[out] = -1;
      cand_score[out] = -INFINITY;
    } else {
      const int row = (int)(0xffffffffu - (uint32_t)me);
      cand[out] = row_token[row];
      cand_score[out] = fkey_value((uint32_t)(me >> 32));
    }
  }
}

// Screening of tile blockIdx.x by float32 chains on the vector ALU (ranks beyond the MFMA
// kernel's reach): rows r0 .. r0 + rows - 1 of A [n, r]; u [M, r] fp32 staged in LDS (dynamic
// shared memory, kM * r floats, rows m >= M zero) and read with 16-byte reads that every lane
// of a wavefront takes from the same address; k_tile candidates per hidden state.  kM >= M
// (even) is the number of chains a row runs, half of them in each half of the workgroup (a
// compile-time count so the accumulators stay in registers; the chains of m >= M are
// discarded).
template <int kM>
__global__ __launch_bounds__(256) void lm_screen_kernel(
    const uint16_t* __restrict__ A, const float* __restrict__ u, const int32_t* __restrict__ row_token,
    int M, int r, int n, int tile, int k_tile, int32_t* __restrict__ cand,
    float* __restrict__ cand_score) {
  // two slices of the tile's rows: [row][128 B], piece v of row q at ((v ^ (q & 7)) * 16)
  __shared__ __attribute__((aligned(16))) char s_a[2][kLmMaxTile * 128];
  extern __shared__ __attribute__((aligned(16))) float s_u[];  // [kM][r]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int r0 = t * tile;
  const int rows = min(tile, n - r0);
  const int n_slices = ceil_div(r, kLmSlice);

  // slice loads: piece L = k * 256 + tid of the slice is (row L / 8, 16-byte piece L % 8);
  // pieces past the row's rank or past the tile read as zero and are never used
  uint4 pre[kLmMaxTile * 8 / 256];
  auto fetch = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kLmMaxTile * 8 / 256; ++k) {
      const int L = k * 256 + tid, row = L >> 3, pc = L & 7;
      const int i0 = sl * kLmSlice + pc * 8;
      pre[k] = make_uint4(0, 0, 0, 0);
      if (row < rows && i0 < r) pre[k] = *reinterpret_cast<const uint4*>(A + (size_t)(r0 + row) * r + i0);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kLmMaxTile * 8 / 256; ++k) {
      const int L = k * 256 + tid, row = L >> 3, pc = L & 7;
      *reinterpret_cast<uint4*>(&s_a[buf][row * 128 + ((pc ^ (row & 7)) << 4)]) = pre[k];
    }
  };

  // Thread (half, p) runs the chains of hidden states half * kH .. half * kH + kH - 1 for rows p
  // and p + 128 of the tile: each u value read from LDS serves two rows.
  constexpr int kH = kM / 2;
  const int half = tid >> 7, p = tid & 127;
  float acc[2][kH];
#pragma unroll
  for (int i = 0; i < kH; ++i) acc[0][i] = acc[1][i] = 0.f;

  fetch(0);
  // u into LDS while the first slice is in flight: float4 pieces (r % 8 == 0), every load of a
  // pass issued before its stores
  {
    constexpr int kPass = 4;
    const int n4 = kM * r / 4, m4 = M * r / 4;
    for (int base = 0; base < n4; base += kPass * 256) {
      float4 v[kPass];
#pragma unroll
      for (int i = 0; i < kPass; ++i) {
        const int x = base + i * 256 + tid;
        v[i] = x < m4 ? reinterpret_cast<const float4*>(u)[x] : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < kPass; ++i) {
        const int x = base + i * 256 + tid;
        if (x < n4) reinterpret_cast<float4*>(s_u)[x] = v[i];
      }
    }
  }
  store(0);
  for (int sl = 0; sl < n_slices; ++sl) {
    if (sl + 1 < n_slices) fetch(sl + 1);
    __syncthreads();  // slice sl (and, the first time, u) is in LDS
    const int i_end = min(kLmSlice, r - sl * kLmSlice);
    const float* us = s_u + (size_t)half * kH * r + sl * kLmSlice;
    const char* sa = &s_a[sl & 1][0];
#pragma unroll 2
    for (int v = 0; v < (i_end >> 3); ++v) {
      // rows p and p + 128 (same swizzle: (p + 128) & 7 == p & 7)
      const int off = p * 128 + ((v ^ (p & 7)) << 4);
      const uint4 a0 = *reinterpret_cast<const uint4*>(sa + off);
      const uint4 a1 = *reinterpret_cast<const uint4*>(sa + off + 128 * 128);
      const float x0[8] = {bf16_lo(a0.x), bf16_hi(a0.x), bf16_lo(a0.y), bf16_hi(a0.y),
                           bf16_lo(a0.z), bf16_hi(a0.z), bf16_lo(a0.w), bf16_hi(a0.w)};
      const float x1[8] = {bf16_lo(a1.x), bf16_hi(a1.x), bf16_lo(a1.y), bf16_hi(a1.y),
                           bf16_lo(a1.z), bf16_hi(a1.z), bf16_lo(a1.w), bf16_hi(a1.w)};
#pragma unroll
      for (int i = 0; i < kH; ++i) {
        // u[m][8v .. 8v+7], the same for every lane
        const float* um = us + i * r + v * 8;
        const float4 u0 = *reinterpret_cast<const float4*>(um);
        const float4 u1 = *reinterpret_cast<const float4*>(um + 4);
        const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float c0 = acc[0][i], c1 = acc[1][i];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          c0 = __builtin_fmaf(x0[e], uv[e], c0);
          c1 = __builtin_fmaf(x1[e], uv[e], c1);
        }
        acc[0][i] = c0;
        acc[1][i] = c1;
      }
    }
    if (sl + 1 < n_slices) store((sl + 1) & 1);
  }
  __syncthreads();  // every thread is done with the slices: their LDS holds the picks now
  screen_picks<kM>(acc, reinterpret_cast<uint64_t*>(&s_a[0][0]), row_token, M, n, tile, k_tile,
                   cand, cand_score);
}

// u = hi + mid + lo with three bfloat16 parts: hi = bf16(x), mid = bf16(x - hi), lo = the rest.
// Each subtraction is exact (the operands are within a factor of two), and the rest has at most
// eight significant bits, so the parts sum to x exactly (for |x| well above 2^-110).
__device__ inline void split3(float x, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = (__bf16)x;
  const float r1 = x - (float)hi;
  mid = (__bf16)r1;
  lo = (__bf16)(r1 - (float)mid);
}

constexpr int kMfmaMaxR = 256;  // ranks the MFMA screening kernel holds in registers

// a >= b afterwards (neither is NaN)
__device__ inline void cmp_swap_desc(double& a, double& b) {
  const double hi = __builtin_fmax(a, b), lo = __builtin_fmin(a, b);
  a = hi;
  b = lo;
}

// The k_tile best of kL sorted lists of picks (64-bit keys, best first, 0 for no row) of one
// hidden state, written as candidates out[0 .. k_tile) of cand / cand_score from index `at`:
// the lists' heads sit in registers, and k_tile rounds take the best head and refill that list's
// head from LDS.  Keys of real rows are distinct; padding keys (0) come last.
template <int kL>
__device__ inline void merge_pick_lists(const uint64_t* pm, int k_tile, size_t at,
                                        const int32_t* __restrict__ row_token,
                                        int32_t* __restrict__ cand,
                                        float* __restrict__ cand_score) {
  uint64_t head[kL];
  int pos[kL];
#pragma unroll
  for (int L = 0; L < kL; ++L) {
    head[L] = pm[L * k_tile];
    pos[L] = 0;
  }
  for (int j = 0; j < k_tile; ++j) {
    uint64_t best = head[0];
    int bl = 0;
#pragma unroll
    for (int L = 1; L < kL; ++L)
      if (head[L] > best) {
        best = head[L];
        bl = L;
      }
    if (best == 0) {  // the tile has fewer real rows than k_tile
      cand[at + j] = -1;
      cand_score[at + j] = -INFINITY;
    } else {
      const int row = (int)(0xffffffffu - (uint32_t)best);
      cand[at + j] = row_token[row];
      cand_score[at + j] = fkey_value((uint32_t)(best >> 32));
    }
    int np = 0;
#pragma unroll
    for (int L = 0; L < kL; ++L) np = L == bl ? pos[L] + 1 : np;
    const uint64_t nh = np < k_tile ? pm[bl * k_tile + np] : 0ull;
#pragma unroll
    for (int L = 0; L < kL; ++L)
      if (L == bl) {
        pos[L] = np;
        head[L] = nh;
      }
  }
}

// Screening of tile blockIdx.x on the matrix cores: scores S = A_tile u^T with u split into
// three bfloat16 parts, so every product A_i * part is exact in float32.  The hidden states go
// in blocks of kN: v_mfma_f32_32x32x16_bf16 for kN = 32, and v_mfma_f32_16x16x32_bf16 for
// kN = 16 (kM <= 16), which pads fewer hidden states and leaves each lane half as many rows to
// pick from.  A term passes through at most kK + 3 ceil(r / kK) roundings (kK = 512 / kN
// products inside its MFMA, then one per later MFMA of the chain).
//  * Wavefront w owns rows 64 w .. 64 w + 63 as 64 / kN blocks of kN rows; lane (q, h) =
//    (lane % kN, lane / kN) holds, for every kK-element k-step s, elements kK s + 8 h .. + 7 of
//    row q of each block: the MFMA's A operand, loaded straight from memory (16 bytes per lane;
//    pieces past r zeroed, rows past the tile computed from its last row and dropped at the
//    picks).
//  * The three parts of u sit in LDS (rows padded by 16 bytes so the rows of a B-operand read
//    fall in different banks); a block of kN hidden states reads its B operand there (lane
//    (q, h): hidden state q, the same elements), and every B operand serves all row blocks.
//  * Element e of a row block's accumulator is row 4 kLG (e / 4) + 4 h + e % 4 of the block for
//    hidden state q (kLG = 64 / kN lane groups), so each lane picks from 64 / kLG rows of one
//    hidden state; the 4 kLG sorted lists of a hidden state then merge.
template <int kM>
__global__ __launch_bounds__(256) void lm_screen_mfma_kernel(
    const uint16_t* __restrict__ A, const float* __restrict__ u,
    const int32_t* __restrict__ row_token, int M, int r, int n, int tile, int k_tile,
    int32_t* __restrict__ cand, float* __restrict__ cand_score) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int kN = kM <= 16 ? 16 : 32;  // hidden states per MFMA block
  constexpr int kLG = 64 / kN;             // lane groups along k (4 or 2)
  constexpr int kK = 8 * kLG;              // products per MFMA output (32 or 16)
  constexpr int kRB = 64 / kN;             // row blocks per wavefront (4 or 2)
  constexpr int kE = kN * kN / 64;         // accumulator elements per lane (4 or 16)
  constexpr int kKeys = kRB * kE;          // rows a lane picks from (16 or 32)
  constexpr int kLists = 4 * kLG;          // sorted pick lists per hidden state (16 or 8)
  constexpr int kNMB = (kM + kN - 1) / kN;  // hidden-state blocks
  constexpr int kMpad = kNMB * kN;
  constexpr int kKS = kMfmaMaxR / kK;      // k-steps
  typedef float accv __attribute__((ext_vector_type(kE)));
  // u's parts for one block of kN hidden states (r <= kMfmaMaxR), then the picks
  // (M * kLists * k_tile 64-bit words); two workgroups fit a compute unit
  constexpr int kPartsLds = 3 * kN * (2 * kMfmaMaxR + 16);
  constexpr int kPickLds = kMpad * kLists * kLmMaxKTile * 8;
  constexpr int kLds = kPartsLds > kPickLds ? kPartsLds : kPickLds;
  __shared__ __attribute__((aligned(16))) char s_dyn[kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane % kN, h = lane / kN;
  const int t = blockIdx.x;
  const int r0 = t * tile;
  const int rows = min(tile, n - r0);
  // every row of a part holds kMfmaMaxR elements (zero from r on) and 16 bytes of padding, so
  // the k-step loop below runs all kKS steps without a branch: a step past r adds exact zeros
  constexpr int u_row = 2 * kMfmaMaxR + 16;  // bytes per row of a part
  constexpr int u_part = kN * u_row;

  constexpr int per_row = kMfmaMaxR / 8;
  constexpr int kUIt = kN * per_row / 256;  // 8-element pieces of a u block per thread
  // u's raw values of hidden states kN mb .. kN mb + kN - 1: thread piece k covers hidden state
  // j = x / per_row, elements i0 .. i0 + 7, x = tid + 256 k (zero for hidden states >= M or
  // i >= r)
  auto load_u = [&](int mb, float (&v)[kUIt][8]) {
#pragma unroll
    for (int k = 0; k < kUIt; ++k) {
      const int x = tid + 256 * k;
      const int j = x / per_row, i0 = (x - j * per_row) * 8, m = kN * mb + j;
      // clamped, not branched, so that every load is issued and the waits count exactly
      const float* src = u + (size_t)min(m, M - 1) * r + min(i0, r - 8);
      const float4 v0 = *reinterpret_cast<const float4*>(src);
      const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
      const bool in = m < M && i0 < r;
      v[k][0] = in ? v0.x : 0.f; v[k][1] = in ? v0.y : 0.f;
      v[k][2] = in ? v0.z : 0.f; v[k][3] = in ? v0.w : 0.f;
      v[k][4] = in ? v1.x : 0.f; v[k][5] = in ? v1.y : 0.f;
      v[k][6] = in ? v1.z : 0.f; v[k][7] = in ? v1.w : 0.f;
    }
  };
  // their three parts into LDS: part p, hidden state j, element i at p*u_part + j*u_row + 2 i
  auto stage_u = [&](const float (&v)[kUIt][8]) {
#pragma unroll
    for (int k = 0; k < kUIt; ++k) {
      const int x = tid + 256 * k;
      const int j = x / per_row, i0 = (x - j * per_row) * 8;
      uint32_t w[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 h0, m0, l0, h1, m1, l1;
        split3(v[k][2 * e], h0, m0, l0);
        split3(v[k][2 * e + 1], h1, m1, l1);
        w[0][e] = __builtin_bit_cast(uint32_t, bf16x2{h0, h1});
        w[1][e] = __builtin_bit_cast(uint32_t, bf16x2{m0, m1});
        w[2][e] = __builtin_bit_cast(uint32_t, bf16x2{l0, l1});
      }
#pragma unroll
      for (int pt = 0; pt < 3; ++pt)
        *reinterpret_cast<uint4*>(s_dyn + pt * u_part + j * u_row + 2 * i0) =
            make_uint4(w[pt][0], w[pt][1], w[pt][2], w[pt][3]);
    }
  };

  // The first block of u is read before the tile, and the tile's A operands are issued k-step
  // by k-step, so the MFMA chain below starts on the first steps while the later ones are
  // still in flight (loads complete in issue order).
  float uv[kUIt][8];
  load_u(0, uv);
  bf16x8 a[kRB][kKS];
#pragma unroll
  for (int s = 0; s < kKS; ++s)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      // Clamped, not branched, so that every load is issued and the MFMAs wait for exactly
      // the steps they use: rows past the tile repeat its last row (their keys are 0 below),
      // and pieces past r (r % 8 == 0: a piece is all in or all out) repeat the row's last
      // piece until zeroed below.
      const int row = 64 * wave + kN * rb + q, i0 = kK * s + 8 * h;
      a[rb][s] = *reinterpret_cast<const bf16x8*>(A + (size_t)(r0 + min(row, rows - 1)) * r +
                                                  min(i0, r - 8));
    }
  if (r < kMfmaMaxR) {
    // The k-step loop runs all kKS steps without a branch, so a step past r must add exact
    // zeros: u's parts are zero there, and the repeated pieces, which may hold an infinity,
    // are zeroed (uniform branch: at the full rank no wait is spent here).
#pragma unroll
    for (int s = 0; s < kKS; ++s)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        if (kK * s + 8 * h >= r) a[rb][s] = bf16x8{};
  }

  accv acc[kRB][kNMB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) acc[rb][mb] = accv{};
#pragma unroll
  for (int mb = 0; mb < kNMB; ++mb) {
    if (mb > 0) {
      load_u(mb, uv);
      __syncthreads();  // the previous block's parts are no longer read
    }
    stage_u(uv);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kKS; ++s)
#pragma unroll
      for (int pt = 0; pt < 3; ++pt) {
        const bf16x8 bq = *reinterpret_cast<const bf16x8*>(s_dyn + pt * u_part + q * u_row +
                                                           2 * (kK * s + 8 * h));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          if constexpr (kN == 32)
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb][s], bq, acc[rb][mb], 0, 0, 0);
          else
            acc[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb][s], bq, acc[rb][mb], 0, 0, 0);
        }
      }
  }
  __syncthreads();  // every wavefront is done with u's parts: their LDS takes the picks

  // Picks straight from the accumulators: each lane holds kKeys rows of hidden state
  // kN mb + q.  A row's key is (fkey(score) << 32) | ~row: the larger key is the better row,
  // ties going to the smaller row; rows past the tile have key 0.  Each lane takes its k_tile
  // best keys, best first (keys of real rows are distinct: a sorting network for k_tile <= 4,
  // else rounds of a maximum and its removal), into s_pick[m][kLG w + h][j]; then the kLists
  // sorted lists of each hidden state merge: by counting ranks when the picks are few
  // (M * kLists * k_tile <= 512), by one thread per hidden state otherwise (at M = 64 the ranks
  // took 44.8 us against 38.3 us, at M = 10 24.0 us against 25.8 us).
  uint64_t* s_pick = reinterpret_cast<uint64_t*>(s_dyn);  // [M][kLists][k_tile]
  // the row in the tile of this lane's element x = kE rb + e (increasing with x)
  auto tile_row = [&](int x) {
    const int rb = x / kE, e = x % kE;
    return 64 * wave + kN * rb + 4 * kLG * (e >> 2) + 4 * h + (e & 3);
  };
#pragma unroll
  for (int mb = 0; mb < kNMB; ++mb) {
    const int m = kN * mb + q;
    if (m < M) {
      uint64_t* out = s_pick + ((size_t)m * kLists + kLG * wave + h) * k_tile;
      if (k_tile <= 4) {
        // Sorting network: sorted groups of four, then bitonic merges that keep the best four
        // of two groups (with 32 keys 68 compare-exchanges and 28 maxima, where four rounds
        // take 124 maxima and 128 compares for the removals).  It runs on float64 stand-ins
        // of the keys: the bits (fkey << 31) | (2^31 - 1 - row in the tile) are a non-negative
        // double, and below the NaN patterns once fkey is capped under them (which only moves
        // NaN scores, all to one place above +inf, ties by row), so the doubles order as the
        // keys do and a compare-exchange is one v_max_f64 and one v_min_f64.  Rows past the
        // tile are +0.0, below every real row.
        constexpr int kG = kKeys / 4;  // groups
        double g[kG][4];
#pragma unroll
        for (int x = 0; x < kKeys; ++x) {
          const uint32_t fk = min(fkey(acc[x / kE][mb][x % kE]), 0xffdfffffu);
          const uint32_t lo = (fk << 31) | (0x7fffffffu - (uint32_t)tile_row(x)), hi = fk >> 1;
          g[x >> 2][x & 3] = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
        }
        if (__builtin_expect(rows < 256, 0)) {  // uniform: only the vocabulary's last tile
#pragma unroll
          for (int x = 0; x < kKeys; ++x)
            if (tile_row(x) >= rows) g[x >> 2][x & 3] = 0.0;
        }
#pragma unroll
        for (int x = 0; x < kG; ++x) {
          cmp_swap_desc(g[x][0], g[x][1]);
          cmp_swap_desc(g[x][2], g[x][3]);
          cmp_swap_desc(g[x][0], g[x][2]);
          cmp_swap_desc(g[x][1], g[x][3]);
          cmp_swap_desc(g[x][1], g[x][2]);
        }
#pragma unroll
        for (int w = kG / 2; w >= 1; w >>= 1)
#pragma unroll
          for (int x = 0; x < w; ++x) {
            // g[x] descending, g[x + w] descending: the larger of g[x][e] and g[x + w][3 - e]
            // are the best four, in bitonic order; two half-cleaners sort them
            double c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] = __builtin_fmax(g[x][e], g[x + w][3 - e]);
            cmp_swap_desc(c[0], c[2]);
            cmp_swap_desc(c[1], c[3]);
            cmp_swap_desc(c[0], c[1]);
            cmp_swap_desc(c[2], c[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) g[x][e] = c[e];
          }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < k_tile) {  // back to the key (0: no real row left)
            const uint64_t d = (uint64_t)__double_as_longlong(g[0][j]);
            const uint32_t row = 0x7fffffffu - (uint32_t)(d & 0x7fffffffu);
            out[j] = d ? ((d >> 31) << 32) | (0xffffffffu - (uint32_t)r0 - row) : 0ull;
          }
      } else {
        // rounds of a maximum and its removal
        uint64_t key[kKeys];
#pragma unroll
        for (int x = 0; x < kKeys; ++x)
          key[x] = tile_row(x) < rows ? ((uint64_t)fkey(acc[x / kE][mb][x % kE]) << 32) |
                                            (0xffffffffu - (uint32_t)(r0 + tile_row(x)))
                                      : 0ull;
        for (int j = 0; j < k_tile; ++j) {
          uint64_t best = key[0];
#pragma unroll
          for (int x = 1; x < kKeys; ++x) best = key[x] > best ? key[x] : best;
#pragma unroll
          for (int x = 0; x < kKeys; ++x) key[x] = key[x] == best ? 0ull : key[x];
          out[j] = best;  // 0: no real row left
        }
      }
    }
  }
  __syncthreads();
  const int C = ceil_div(n, tile) * k_tile;
  const int per_m = kLists * k_tile;
  if (M * per_m <= 512) {
    // few picks: every (hidden state, pick) pair counts the picks ahead of it, two pairs per
    // thread at most
    for (int x = tid; x < M * per_m; x += 256) {
      const int m = x / per_m, e = x - m * per_m;
      const uint64_t* pm = s_pick + (size_t)m * per_m;
      const uint64_t me = pm[e];
      int rank = 0;  // picks are distinct except padding (0), which ranks by entry
      for (int o = 0; o < per_m; ++o) rank += pm[o] > me || (pm[o] == me && o < e);
      if (rank >= k_tile) continue;
      const size_t o_at = (size_t)m * C + (size_t)t * k_tile + rank;
      if (me == 0) {  // the tile has fewer real rows than k_tile: padding picks rank last
        cand[o_at] = -1;
        cand_score[o_at] = -INFINITY;
      } else {
        const int row = (int)(0xffffffffu - (uint32_t)me);
        cand[o_at] = row_token[row];
        cand_score[o_at] = fkey_value((uint32_t)(me >> 32));
      }
    }
  } else if (tid < M) {  // many: one thread per hidden state merges its sorted lists
    merge_pick_lists<kLists>(s_pick + (size_t)tid * per_m, k_tile,
                             (size_t)tid * C + (size_t)t * k_tile, row_token, cand, cand_score);
  }
}

__global__ __launch_bounds__(256) void lm_rescore_kernel(const uint16_t* __restrict__ W,
                                                         const uint16_t* __restrict__ h,
                                                         const int32_t* __restrict__ cand, int M,
                                                         int C, int d, int V,
                                                         float* __restrict__ logits,
                                                         int32_t* __restrict__ status) {
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);  // p = m * C + c
  if (p >= M * C) return;
  const int m = p / C;
  const int tok = cand[p];
  const bool ok = tok >= 0 && tok < V;
  float v = -INFINITY;
  if (ok) v = lm_dot(W + (size_t)tok * d, h + (size_t)m * d, d);
  if ((threadIdx.x & 63) == 0) {
    logits[p] = v;
    if (!ok && tok != -1 && status) atomicOr(status + m, TV_BAD_TOKEN);
  }
}

// Children of hidden state blockIdx.x.  The 64-bit key (logit key << 32 | ~token) of every
// valid candidate; each wavefront takes K rounds of wavefront maxima over its candidates, the
// 4K picks (0 = none) are merged by rank; confidences exp(l - max) / sum over valid ones.
template <int kPer>  // candidates per thread: C <= 256 * kPer
__global__ __launch_bounds__(256) void lm_topk_kernel(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ cand, int C,
                                                      int K, int V, int32_t* __restrict__ out_tok,
                                                      float* __restrict__ out_conf) {
  __shared__ uint64_t s_pick[4 * kLmMaxK];
  __shared__ float s_f[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* l = logits + (size_t)m * C;
  const int32_t* cm = cand + (size_t)m * C;
  uint64_t key[kPer];
  float mx = -INFINITY;
  // every slot's token and logit are loaded before any is used: clamped to the last candidate
  // rather than branched, so the 2 kPer loads are in flight together
  int tok[kPer];
  float lv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = min(k * 256 + tid, C - 1);
    tok[k] = cm[c];
    lv[k] = l[c];
  }
  // the values are taken here, so all the loads above are issued before the first wait
  // rather than sunk into the conditional uses below
#pragma unroll
  for (int k = 0; k < kPer; ++k) __asm__ volatile("" ::"v"(tok[k]), "v"(lv[k]));
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const bool ok = k * 256 + tid < C && tok[k] >= 0 && tok[k] < V;
    key[k] = ok ? ((uint64_t)fkey(lv[k]) << 32) | (0xffffffffu - (uint32_t)tok[k]) : 0ull;
    mx = ok ? fmaxf(mx, lv[k]) : mx;
  }
  // max and sum of exponentials over the valid candidates
  mx = wave_max_f32(mx);
  if (lane == 0) s_f[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_f[0], s_f[1]), fmaxf(s_f[2], s_f[3]));
  __syncthreads();
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (key[k]) z += expf(fkey_value((uint32_t)(key[k] >> 32)) - mx);
  z = wave_sum_f32(z);
  if (lane == 0) s_f[wave] = z;

  // this wavefront's K best: the best score by a 32-bit maximum; the token decides only
  // between lanes holding equal scores (a 64-bit maximum over those lanes, rarely needed).
  // Each round removes one copy of the best key (candidates may repeat a token): the first
  // slot holding it in the lowest lane holding it.
  // With eight slots a lane's keys are sorted once (a 19-exchange network), so its best is its
  // first key and a removal shifts the rest up.
  if constexpr (kPer == 8) {
    auto cx = [&](int i, int k) {
      const uint64_t hi = key[i] > key[k] ? key[i] : key[k], lo = key[i] > key[k] ? key[k] : key[i];
      key[i] = hi;
      key[k] = lo;
    };
    cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
    cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
    cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
    cx(2, 4); cx(3, 5);
    cx(1, 4); cx(3, 6);
    cx(1, 2); cx(3, 4); cx(5, 6);
  }
  for (int j = 0; j < K; ++j) {
    uint64_t mine = key[0];  // this lane's best key (0: none)
    if constexpr (kPer != 8) {
#pragma unroll
      for (int k = 1; k < kPer; ++k) mine = key[k] > mine ? key[k] : mine;
    }
    const uint32_t top = wave_max_u32((uint32_t)(mine >> 32));
    const uint64_t holders = __ballot(mine != 0 && (uint32_t)(mine >> 32) == top);
    uint64_t best = 0;
    if (holders) {
      if ((holders & (holders - 1)) == 0) {
        const int w = __builtin_ctzll(holders);
        best = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), w) << 32) |
               (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, w);
      } else {
        best = wave_max_u64((uint32_t)(mine >> 32) == top ? mine : 0);
      }
      const int owner = __builtin_ctzll(__ballot(mine == best));
      if (lane == owner) {
        if constexpr (kPer == 8) {  // the best is the first key: the rest move up
#pragma unroll
          for (int k = 0; k < kPer - 1; ++k) key[k] = key[k + 1];
          key[kPer - 1] = 0;
        } else {
          bool done = false;
#pragma unroll
          for (int k = 0; k < kPer; ++k)
            if (!done && key[k] == best) {
              key[k] = 0;
              done = true;
            }
        }
      }
    }
    if (lane == 0) s_pick[wave * K + j] = best;
  }
  __syncthreads();
  z = (s_f[0] + s_f[1]) + (s_f[2] + s_f[3]);
  for (int e = tid; e < 4 * K; e += 256) {
    const uint64_t me = s_pick[e];
    int rank = 0;  // equal picks (a repeated token's copies, or 0 for none) rank by entry
    // eight LDS reads in flight per step (4 K is a multiple of 4; entries past it read 0)
    for (int o0 = 0; o0 < 4 * K; o0 += 8) {
      uint64_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = o0 + i < 4 * K ? s_pick[o0 + i] : 0ull;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rank += o0 + i < 4 * K && (v[i] > me || (v[i] == me && o0 + i < e));
    }
    if (rank >= K) continue;
    const size_t o = (size_t)m * K + rank;
    if (me == 0) {
      out_tok[o] = -1;
      out_conf[o] = 0.f;
    } else {
      out_tok[o] = (int)(0xffffffffu - (uint32_t)me);
      out_conf[o] = expf(fkey_value((uint32_t)(me >> 32)) - mx) / z;
    }
  }
}

}  // namespace
}  // namespace tv

using namespace tv;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

extern "C" int lm_head_project(const void* h, const void* B, int M, int r, int d, float* u,
                               void* stream) {
  if (!h || !B || !u || !aligned16(h) || !aligned16(B) || M < 1 || M > kLmMaxM || r < 1 ||
      d < 512 || d % 512 != 0 || (long long)M * r > (1 << 24))
    return TV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(lm_project_kernel, dim3(ceil_div(M * r, 4)), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)h, (const uint16_t*)B, M, r, d, u);
  return launch_status();
}

namespace tv {
namespace {
// Chains per thread for M hidden states: the smallest instantiated count >= M.
constexpr int kScreenM[] = {2, 4, 6, 8, 10, 12, 16, 24, 32, 48, 64};

template <int kM>
void launch_screen(const void* A, const float* u, const int32_t* row_token, int M, int r, int n,
                   int tile, int k_tile, int32_t* cand, float* cand_score, hipStream_t stream) {
  if (r <= kMfmaMaxR) {  // matrix cores
    hipLaunchKernelGGL(lm_screen_mfma_kernel<kM>, dim3(ceil_div(n, tile)), dim3(256), 0, stream,
                       (const uint16_t*)A, u, row_token, M, r, n, tile, k_tile, cand, cand_score);
  } else  // larger ranks run the float32 chains
    hipLaunchKernelGGL(lm_screen_kernel<kM>, dim3(ceil_div(n, tile)), dim3(256),
                       (size_t)kM * r * sizeof(float), stream, (const uint16_t*)A, u, row_token, M,
                       r, n, tile, k_tile, cand, cand_score);
}
}  // namespace
}  // namespace tv

extern "C" int lm_head_screen(const void* A, const float* u, const int32_t* row_token, int M,
                              int r, int n, int tile, int k_tile, int32_t* cand, float* cand_score,
                              void* stream) {
  if (!A || !u || !row_token || !cand || !cand_score || !aligned16(A) || !aligned16(u) || M < 1 ||
      M > kLmMaxM || r < 8 || r % 8 != 0 || n < 1 || tile < 1 || tile > kLmMaxTile ||
      k_tile < 1 || k_tile > kLmMaxKTile || (long long)ceil_div(n, tile) * k_tile * M >= (1LL << 31))
    return TV_ERR_INVALID_ARG;
  int kM = kLmMaxM;
  for (int c : kScreenM)
    if (c >= M) {
      kM = c;
      break;
    }
  if ((size_t)kM * r * sizeof(float) > 65536) return TV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  switch (kM) {
    case 2: launch_screen<2>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 4: launch_screen<4>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 6: launch_screen<6>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 8: launch_screen<8>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 10: launch_screen<10>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 12: launch_screen<12>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 16: launch_screen<16>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 24: launch_screen<24>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 32: launch_screen<32>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    case 48: launch_screen<48>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
    default: launch_screen<64>(A, u, row_token, M, r, n, tile, k_tile, cand, cand_score, st); break;
  }
  return launch_status();
}

extern "C" int lm_head_rescore(const void* W, const void* h, const int32_t* cand, int M, int C,
                               int d, int V, float* logits, int32_t* status, void* stream) {
  if (!W || !h || !cand || !logits || !aligned16(W) || !aligned16(h) || M < 1 || M > kLmMaxM ||
      C < 1 || V < 1 || d < 512 || d % 512 != 0 || (long long)M * C >= (1LL << 31))
    return TV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(lm_rescore_kernel, dim3(ceil_div(M * C, 4)), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)W, (const uint16_t*)h, cand, M, C, d, V,
                     logits, status);
  return launch_status();
}

extern "C" int lm_head_topk(const float* logits, const int32_t* cand, int M, int C, int K, int V,
                            int32_t* out_tok, float* out_conf, void* stream) {
  if (!logits || !cand || !out_tok || !out_conf || M < 1 || C < 1 || C > 256 * 32 || K < 1 ||
      K > kLmMaxK || V < 1)
    return TV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (C <= 256 * 8)
    hipLaunchKernelGGL(lm_topk_kernel<8>, dim3(M), dim3(256), 0, st, logits, cand, C, K, V, out_tok,
                       out_conf);
  else if (C <= 256 * 16)
    hipLaunchKernelGGL(lm_topk_kernel<16>, dim3(M), dim3(256), 0, st, logits, cand, C, K, V,
                       out_tok, out_conf);
  else
    hipLaunchKernelGGL(lm_topk_kernel<32>, dim3(M), dim3(256), 0, st, logits, cand, C, K, V,
                       out_tok, out_conf);
  return launch_status();
}
