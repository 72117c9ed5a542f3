// Stochastic acceptance of a draft tree: rejection sampling tried child by child
// (lesty.tech "EAGLE-2 vs. Medusa", section 4).
//
// Reformulation used by the kernel (exact up to rounding).  Let the children of the current
// node u be tried in order with tokens x_1, x_2, ...  The page's residual after a rejection is
// p_{j+1} = max(0, p_j - q_j) / Z_j.  Writing p_j = U_j / S_j with U_1 = p and S_1 = 1, and
// using max(0, max(0, a) - b) = max(0, a - b) for b >= 0, every residual is
//
//     U_j(y) = max(0, p(y) - C_{j-1} q(y)),   S_j = sum_y U_j(y),
//     C_j = C_{j-1} + S_j / N_j,              C_0 = 0,
//
// where q_j = q / N_j is the draft distribution child j is tested against: N_j = 1 when siblings
// are independent draws from q, and N_j = 1 - (q mass of the distinct tokens rejected so far)
// when they are drawn without replacement (the rejected token's residual is already zero, so
// removing it from q changes nothing else).  A child is kept iff u * q_j(x) * S_j < U_j(x).
// So the walk carries three scalars per node, and each rejection costs one sweep of the
// vocabulary that sums max(0, p - C q) in fp64.  The bonus token is an inverse-CDF draw from
// U (smallest y whose running sum exceeds u * total).
//
// One workgroup of 512 threads per sequence.  Every wavefront runs the same walk on the same
// data (child tokens and their p, q values live in its lanes), so decisions need no broadcast;
// only the sweep totals go through LDS.
#include "tree_device.h"

namespace tv {
namespace {

constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / 64;
constexpr int kChunk = 256;       // vocabulary elements per wavefront step: 64 lanes x 4
constexpr int kMaxChunks = 4096;  // chunk sums kept in LDS for the draw
constexpr int kUnroll = 8;        // chunks in flight per wavefront

struct StochArgs {
  const uint64_t* anc;
  const int32_t* draft;
  const float* p;
  const float* q;
  const double* u_acc;
  const double* u_res;
  int32_t* path;
  int32_t* alen;
  int32_t* bonus;
  int32_t* status;
  int T, W, V, mode;
};

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;  // identical in every lane: each butterfly step adds the same pair
}

// Inclusive prefix sum over the lanes of a wavefront.
__device__ inline double wave_scan_f64(double v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Highest ancestor bit below c in a mask row: c's parent, or -1.
__device__ inline int parent_from_row(int c, uint64_t lo, uint64_t hi) {
  if (c >= 64) {
    const uint64_t h = hi & (bit64(c - 64) - 1);
    if (h) return 64 + 63 - __clzll(h);
    return lo ? 63 - __clzll(lo) : -1;
  }
  const uint64_t l = lo & (bit64(c) - 1);
  return l ? 63 - __clzll(l) : -1;
}

// Four consecutive elements of a row starting at i (zeros past V).
template <bool kVec>
__device__ inline void load4(const float* __restrict__ row, int i, int V, float (&v)[4]) {
  if constexpr (kVec) {
    if (i < V) {
      const float4 t = *reinterpret_cast<const float4*>(row + i);
      v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
    } else {
      v[0] = v[1] = v[2] = v[3] = 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = i + e < V ? row[i + e] : 0.f;
  }
}

__device__ inline double resid(float p, float q, double C) {
  const double d = fma(-C, (double)q, (double)p);
  return d > 0.0 ? d : 0.0;
}

// Sum over the vocabulary of U(y) = max(0, p(y) - C q(y)), chunk k = 256 consecutive elements
// handled by wavefront k % 16.  With kDraw the chunk sums go to s_chunk and last_nz tracks the
// largest y with U(y) > 0.  Returns this thread's share of the sum.
template <bool kVec, bool kDraw>
__device__ double sweep(const float* __restrict__ pu, const float* __restrict__ qu, double C,
                        int V, int wave, int lane, double* s_chunk, int& last_nz) {
  const int nchunks = ceil_div(V, kChunk);
  const bool use_q = C != 0.0;
  double acc = 0.0;
  for (int k0 = wave; k0 < nchunks; k0 += kSWaves * kUnroll) {
    float pv[kUnroll][4], qv[kUnroll][4];
#pragma unroll
    for (int s = 0; s < kUnroll; ++s) {
      const int k = k0 + s * kSWaves;
      const int i = k < nchunks ? k * kChunk + lane * 4 : V;
      load4<kVec>(pu, i, V, pv[s]);
      if (use_q) {
        load4<kVec>(qu, i, V, qv[s]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[s][e] = 0.f;
      }
    }
#pragma unroll
    for (int s = 0; s < kUnroll; ++s) {
      const int k = k0 + s * kSWaves;
      double cs = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d = resid(pv[s][e], qv[s][e], C);
        cs += d;
        if (kDraw && d > 0.0) last_nz = k * kChunk + lane * 4 + e;
      }
      if constexpr (kDraw) {
        const double t = wave_sum_f64(cs);
        if (lane == 0 && k < nchunks) s_chunk[k] = t;
      }
      acc += cs;
    }
  }
  return acc;
}

template <bool kVec>
__global__ __launch_bounds__(kSThreads) void accept_stochastic_kernel(StochArgs a) {
  __shared__ double s_red[2][kSWaves];
  __shared__ int s_ired[kSWaves];
  __shared__ double s_chunk[kMaxChunks];
  __shared__ int s_path[kMaxT];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V;

  // the lane's two nodes: parent, token, acceptance uniform
  int par[2], tok[2];
  double ua[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    par[k] = -2;
    tok[k] = -1;
    ua[k] = 0.0;
    if (c < T) {
      const uint64_t* row = a.anc + ((size_t)b * T + c) * a.W;
      par[k] = parent_from_row(c, row[0], a.W > 1 ? row[1] : 0ull);
      tok[k] = a.draft[(size_t)b * T + c];
      ua[k] = a.u_acc[(size_t)b * T + c];
    }
  }

  int u = 0, n = 1, buf = 0, bad = 0, bonus = -1;
  if (tid == 0) s_path[0] = 0;
  for (;;) {
    const float* pu = a.p + ((size_t)b * T + u) * V;
    const float* qu = a.q + ((size_t)b * T + u) * V;
    // children of u with an in-vocabulary token, and their p, q values
    bool ch[2], ok[2];
    float px[2], qx[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ch[k] = par[k] == u;
      ok[k] = ch[k] && tok[k] >= 0 && tok[k] < V;
      px[k] = ok[k] ? pu[tok[k]] : 0.f;
      qx[k] = ok[k] ? qu[tok[k]] : 0.f;
    }
    uint64_t m0 = __ballot(ok[0]), m1 = __ballot(ok[1]);
    const uint64_t bad0 = __ballot(ch[0] && !ok[0]), bad1 = __ballot(ch[1] && !ok[1]);
    uint64_t rj0 = 0, rj1 = 0;  // lanes of rejected children
    double C = 0.0, S = 1.0, N = 1.0;
    int next = -1;
    while (m0 | m1) {
      const int k = m0 ? 0 : 1;
      const int l = __builtin_ctzll(k ? m1 : m0);
      if (k) m1 &= m1 - 1; else m0 &= m0 - 1;
      const int c = l + 64 * k;
      const int x = __shfl(k ? tok[1] : tok[0], l, 64);
      const double pxd = (double)__shfl(k ? px[1] : px[0], l, 64);
      const double qxd = (double)__shfl(k ? qx[1] : qx[0], l, 64);
      const double uac = __shfl(k ? ua[1] : ua[0], l, 64);
      bool excl = false;
      if (a.mode) {
        const bool same = ((rj0 >> lane) & 1 && tok[0] == x) || ((rj1 >> lane) & 1 && tok[1] == x);
        excl = __ballot(same) != 0;
      }
      const double Ux = fmax(fma(-C, qxd, pxd), 0.0);  // U_j(x) = p_j(x) * S_j
      const double qj = (excl || !(N > 0.0)) ? 0.0 : qxd / N;
      if (uac * qj * S < Ux) {
        next = c;
        break;
      }
      // rejected: the residual for the next sibling
      const double Cn = C + (N > 0.0 ? S / N : 0.0);
      int dummy = 0;
      const double part = wave_sum_f64(sweep<kVec, false>(pu, qu, Cn, V, wave, lane, nullptr, dummy));
      if (lane == 0) s_red[buf][wave] = part;
      __syncthreads();
      double Sn = 0.0;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) Sn += s_red[buf][w];
      buf ^= 1;
      if (!(Sn > 0.0)) break;  // no mass left: draw from the distribution child j faced
      C = Cn;
      S = Sn;
      if (a.mode && !excl) N -= qxd;
      if (k) rj1 |= bit64(l); else rj0 |= bit64(l);
    }
    // children passed over with an out-of-vocabulary token (those before the kept one)
    {
      uint64_t lo, hi;
      low_bits(next < 0 ? T : next, lo, hi);
      if ((bad0 & lo) | (bad1 & hi)) bad = 1;
    }
    if (next >= 0) {
      if (tid == 0) s_path[n] = next;
      ++n;
      u = next;
      continue;
    }
    // bonus draw at u from U = max(0, p - C q)
    int last_nz = -1;
    sweep<kVec, true>(pu, qu, C, V, wave, lane, s_chunk, last_nz);
    last_nz = wave_max(last_nz);
    if (lane == 0) s_ired[wave] = last_nz;
    __syncthreads();
    for (int w = 0; w < kSWaves; ++w) last_nz = max(last_nz, s_ired[w]);
    const int nchunks = ceil_div(V, kChunk);
    const int per = ceil_div(nchunks, 64);
    double local = 0.0;
    for (int j = 0; j < per; ++j) {
      const int kk = lane * per + j;
      if (kk < nchunks) local += s_chunk[kk];
    }
    // running sum before lane l's chunks, and the lane where it first exceeds u * total
    const double incl = wave_scan_f64(local, lane);
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    const double total = __shfl(incl, 63, 64);
    const double thr = a.u_res[(size_t)b * T + u] * total;
    const uint64_t over = __ballot(excl + local > thr);
    bonus = last_nz;  // no running sum exceeds the threshold (u >= 1, rounding): last token with mass
    if (over) {
      const int L = __builtin_ctzll(over);
      const double excl_L = __shfl(excl, L, 64);
      // chunk of lane L where the running sum first exceeds thr (walked by every lane alike)
      int kc = -1;
      double before = excl_L, run = 0.0;
      for (int j = 0; j < per; ++j) {
        const int kk = L * per + j;
        if (kk >= nchunks) break;
        const double ck = s_chunk[kk];
        if (excl_L + (run + ck) > thr && ck > 0.0) {
          kc = kk;
          before = excl_L + run;
          break;
        }
        run += ck;
      }
      if (kc >= 0) {
        float pv[4], qv[4] = {0.f, 0.f, 0.f, 0.f};
        const int i = kc * kChunk + lane * 4;
        load4<kVec>(pu, i, V, pv);
        if (C != 0.0) load4<kVec>(qu, i, V, qv);
        double uv[4], ls = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uv[e] = resid(pv[e], qv[e], C);
          ls += uv[e];
        }
        const double inc2 = wave_scan_f64(ls, lane);
        double r = before + (inc2 - ls);
        int hit = -1, lastpos = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r += uv[e];
          if (uv[e] > 0.0) {
            lastpos = i + e;
            if (hit < 0 && r > thr) hit = i + e;
          }
        }
        const uint64_t hits = __ballot(hit >= 0);
        if (hits) {
          bonus = __shfl(hit, __builtin_ctzll(hits), 64);
        } else {
          bonus = wave_max(lastpos);  // rounding tie at the chunk's end: its last token with mass
        }
      }
    }
    break;
  }
  __syncthreads();
  for (int t = tid; t < T; t += kSThreads) a.path[(size_t)b * T + t] = t < n ? s_path[t] : -1;
  if (tid == 0) {
    a.alen[b] = n;
    a.bonus[b] = bonus;
    if (bad && a.status) atomicOr(a.status + b, TV_BAD_TOKEN);
  }
}

}  // namespace
}  // namespace tv

using namespace tv;

extern "C" int tree_accept_stochastic(const uint64_t* anc_mask, const int32_t* draft_tok,
                                      const float* p, const float* q, const double* u_acc,
                                      const double* u_res, int B, int T, int V,
                                      int without_replacement, int32_t* accept_path,
                                      int32_t* accept_len, int32_t* bonus_tok, int32_t* status,
                                      void* stream) {
  if (!anc_mask || !draft_tok || !p || !q || !u_acc || !u_res || !accept_path || !accept_len ||
      !bonus_tok || B < 1 || T < 1 || T > kMaxT || V < 1 || V > kChunk * kMaxChunks ||
      (without_replacement != 0 && without_replacement != 1))
    return TV_ERR_INVALID_ARG;
  StochArgs a{anc_mask, draft_tok, p, q, u_acc, u_res, accept_path, accept_len, bonus_tok, status,
              T, ceil_div(T, 64), V, without_replacement};
  const bool vec = V % 4 == 0 && ((uintptr_t)p % 16) == 0 && ((uintptr_t)q % 16) == 0;
  if (vec)
    hipLaunchKernelGGL(accept_stochastic_kernel<true>, dim3(B), dim3(kSThreads), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(accept_stochastic_kernel<false>, dim3(B), dim3(kSThreads), 0,
                       (hipStream_t)stream, a);
  return launch_status();
}
