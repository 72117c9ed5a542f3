// Two-stage drafter LM head (jialefu.github.io, "EAGLE-4: Notes on the Efficient LM Head").
//
// Stage one screens the whole vocabulary with a low-rank head, u = B h, then A u, and keeps
// candidates with a local top-k fused into each tile of (shuffled) vocabulary rows, so the
// approximate scores never leave the chip.  Stage two gathers the candidates' rows of the full
// head W and recomputes their logits exactly.  The drafter's children are the K best candidates,
// with confidences from a softmax over the candidates.
//
// The candidates and children are chosen by float32 values, so every dot product has a stated
// order, part of the definition of the result:
//   * lm_dot (u = B h, logits = W[token] h; d a multiple of 512): lane j of a wavefront runs a
//     chain of fused multiply-adds from 0 over elements 512 p + 8 j + e (p = 0, 1, ... outer,
//     e = 0 .. 7 inner), so every 16-byte load of the wavefront covers 1 KB contiguously; the
//     64 chain sums are then combined by a butterfly, j with j^32, then j^16, ..., j^1, which
//     leaves the same value in every lane;
//   * screening (A u): one chain of fused multiply-adds over the rank index, in order, from 0.
// Ranking uses an unsigned key of the float (-0 as +0); equal values go to the smaller row
// (screening) or the smaller token (children).
//
// Kernels:
//   lm_project_kernel  one wavefront per (i, m), u[m, i] = B[i] . h[m]          (2 MB of B)
//   lm_screen_kernel   one workgroup per tile of rows: the tile's A rows stream through LDS in
//                      64-element slices (each row's 128 B XOR-swizzled by 16-byte piece so a
//                      thread reading its row is free of bank conflicts), one thread per row
//                      runs the M chains, then each wavefront picks its k best rows per hidden
//                      state by wavefront maxima and the four wavefronts' picks are merged
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
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float fkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = shfl64(v, (int)(threadIdx.x & 63) ^ off);
    v = o > v ? o : v;
  }
  return v;
}

// The fixed-order dot product of two bfloat16 rows of length d (d % 512 == 0), by the calling
// wavefront: lane j's pieces are the 16 bytes at element 512 p + 8 j.
__device__ inline float lm_dot(const uint16_t* __restrict__ x, const uint16_t* __restrict__ y,
                               int d) {
  const int lane = threadIdx.x & 63;
  const uint4* xs = reinterpret_cast<const uint4*>(x) + lane;  // 64 pieces per 512 elements
  const uint4* ys = reinterpret_cast<const uint4*>(y) + lane;
  float acc = 0.f;
  for (int p = 0; p < (d >> 9); ++p) {
    const uint4 a = xs[64 * p], b = ys[64 * p];
    acc = __builtin_fmaf(bf16_lo(a.x), bf16_lo(b.x), acc);
    acc = __builtin_fmaf(bf16_hi(a.x), bf16_hi(b.x), acc);
    acc = __builtin_fmaf(bf16_lo(a.y), bf16_lo(b.y), acc);
    acc = __builtin_fmaf(bf16_hi(a.y), bf16_hi(b.y), acc);
    acc = __builtin_fmaf(bf16_lo(a.z), bf16_lo(b.z), acc);
    acc = __builtin_fmaf(bf16_hi(a.z), bf16_hi(b.z), acc);
    acc = __builtin_fmaf(bf16_lo(a.w), bf16_lo(b.w), acc);
    acc = __builtin_fmaf(bf16_hi(a.w), bf16_hi(b.w), acc);
  }
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

// Screening of tile blockIdx.x: rows r0 .. r0 + rows - 1 of A [n, r]; u [M, r] fp32 staged in
// LDS (dynamic shared memory, kM * r floats, rows m >= M zero) and read with 16-byte reads
// that every lane of a wavefront takes from the same address; k_tile candidates per hidden
// state.  kM >= M is the number of chains each thread runs (a compile-time count so the
// accumulators stay in registers; the chains of m >= M are discarded).
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

  for (int x = tid; x < kM * r; x += 256) s_u[x] = x < M * r ? u[x] : 0.f;

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

  float acc[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) acc[m] = 0.f;

  fetch(0);
  store(0);
  for (int sl = 0; sl < n_slices; ++sl) {
    if (sl + 1 < n_slices) fetch(sl + 1);
    __syncthreads();  // slice sl (and, the first time, u) is in LDS
    const int q = tid;
    const int i_end = min(kLmSlice, r - sl * kLmSlice);
    const float* us = s_u + sl * kLmSlice;
#pragma unroll 2
    for (int v = 0; v < (i_end >> 3); ++v) {
      const uint4 a = *reinterpret_cast<const uint4*>(&s_a[sl & 1][q * 128 + ((v ^ (q & 7)) << 4)]);
      const float av[8] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y),
                           bf16_lo(a.z), bf16_hi(a.z), bf16_lo(a.w), bf16_hi(a.w)};
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        // u[m][8v .. 8v+7], the same for every lane
        const float* um = us + m * r + v * 8;
        const float4 u0 = *reinterpret_cast<const float4*>(um);
        const float4 u1 = *reinterpret_cast<const float4*>(um + 4);
        float a_m = acc[m];
        a_m = __builtin_fmaf(av[0], u0.x, a_m);
        a_m = __builtin_fmaf(av[1], u0.y, a_m);
        a_m = __builtin_fmaf(av[2], u0.z, a_m);
        a_m = __builtin_fmaf(av[3], u0.w, a_m);
        a_m = __builtin_fmaf(av[4], u1.x, a_m);
        a_m = __builtin_fmaf(av[5], u1.y, a_m);
        a_m = __builtin_fmaf(av[6], u1.z, a_m);
        a_m = __builtin_fmaf(av[7], u1.w, a_m);
        acc[m] = a_m;
      }
    }
    if (sl + 1 < n_slices) store((sl + 1) & 1);
  }
  __syncthreads();  // every thread is done with the slices: their LDS holds the picks now

  // each wavefront's k best rows per hidden state, then the merge of the four wavefronts
  uint64_t* s_pick = reinterpret_cast<uint64_t*>(&s_a[0][0]);  // [M][4][k_tile]
  const bool real = tid < rows;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m < M) {
      uint64_t key =
          real ? ((uint64_t)fkey(acc[m]) << 32) | (0xffffffffu - (uint32_t)(r0 + tid)) : 0;
      for (int j = 0; j < k_tile; ++j) {
        const uint64_t best = wave_max_u64(key);
        if (key == best) key = 0;  // keys of real rows are distinct
        if (lane == 0) s_pick[(m * 4 + wave) * k_tile + j] = best;
      }
    }
  }
  __syncthreads();
  const int C = ceil_div(n, tile) * k_tile;
  const int per_m = 4 * k_tile;
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
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = k * 256 + tid;
    key[k] = 0;
    if (c < C) {
      const int tok = cm[c];
      if (tok >= 0 && tok < V) {
        key[k] = ((uint64_t)fkey(l[c]) << 32) | (0xffffffffu - (uint32_t)tok);
        mx = fmaxf(mx, l[c]);
      }
    }
  }
  // max and sum of exponentials over the valid candidates
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) s_f[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_f[0], s_f[1]), fmaxf(s_f[2], s_f[3]));
  __syncthreads();
  float z = 0.f;
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (key[k]) z += expf(fkey_value((uint32_t)(key[k] >> 32)) - mx);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (lane == 0) s_f[wave] = z;

  // this wavefront's K best
  for (int j = 0; j < K; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) best = key[k] > best ? key[k] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int k = 0; k < kPer; ++k) key[k] = key[k] == best ? 0 : key[k];
    if (lane == 0) s_pick[wave * K + j] = best;
  }
  __syncthreads();
  z = (s_f[0] + s_f[1]) + (s_f[2] + s_f[3]);
  for (int e = tid; e < 4 * K; e += 256) {
    const uint64_t me = s_pick[e];
    int rank = 0;  // picks are distinct except 0 (none), which ranks by entry
    for (int o = 0; o < 4 * K; ++o) rank += s_pick[o] > me || (s_pick[o] == me && o < e);
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

extern "C" int lm_head_project(const void* h, const void* B, int M, int r, int d, float* u,
                               void* stream) {
  if (!h || !B || !u || M < 1 || M > kLmMaxM || r < 1 || d < 512 || d % 512 != 0 ||
      (long long)M * r > (1 << 24))
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
  hipLaunchKernelGGL(lm_screen_kernel<kM>, dim3(ceil_div(n, tile)), dim3(256),
                     (size_t)kM * r * sizeof(float), stream, (const uint16_t*)A, u, row_token, M, r,
                     n, tile, k_tile, cand, cand_score);
}
}  // namespace
}  // namespace tv

extern "C" int lm_head_screen(const void* A, const float* u, const int32_t* row_token, int M,
                              int r, int n, int tile, int k_tile, int32_t* cand, float* cand_score,
                              void* stream) {
  if (!A || !u || !row_token || !cand || !cand_score || M < 1 || M > kLmMaxM || r < 8 ||
      r % 8 != 0 || n < 1 || tile < 1 || tile > kLmMaxTile || k_tile < 1 ||
      k_tile > kLmMaxKTile || (long long)ceil_div(n, tile) * k_tile * M >= (1LL << 31))
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
  if (!W || !h || !cand || !logits || M < 1 || M > kLmMaxM || C < 1 || V < 1 || d < 512 ||
      d % 512 != 0 || (long long)M * C >= (1LL << 31))
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
