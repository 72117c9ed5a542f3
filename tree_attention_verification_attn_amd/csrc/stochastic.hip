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
// Work split.  G workgroups of 512 threads serve one sequence, each sweeping its own slice of the
// vocabulary.  Every workgroup, and every wavefront in it, runs the same walk on the same data
// (child tokens and their p, q values live in its lanes), so decisions need no broadcast: only
// per-slice sums are exchanged.  With G > 1 the partial sums of a sweep meet in a workspace: each
// workgroup stores its value with a device-coherent atomic, in a form that is never zero, and
// waits (bounded) until every value of that sweep is there; all workgroups then add the G values
// in the same order, so they take the same decisions.  Each workgroup counts itself out after its
// last exchange, and the last one to do so clears the slots the
// call used, so the workspace is all zeros between calls.  The host keeps B * G within the
// compute units, so all workgroups of a sequence are resident together.
#include <hip/hip_ext.h>

#include <algorithm>

#include "tree_device.h"

namespace tv {
namespace {

constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / 64;
constexpr int kChunk = 256;       // vocabulary elements per wavefront step: 64 lanes x 4
constexpr int kMaxChunks = 4096;  // chunk sums kept in LDS for the draw
constexpr int kUnroll = 8;        // chunks in flight per wavefront
constexpr int kMaxG = 64;         // workgroups per sequence (one polling lane each)
constexpr uint32_t kSpinLimit = 1u << 16;  // polls before a wait gives up (tens of ms)

// One workgroup's contribution to one sweep: its partial sum and its largest token with mass
// (draws only), each stored once as a 64-bit word XOR kMagic, so that a word is nonzero exactly
// when it has been written: the word is its own ready flag, and no fence is needed between a
// value and a flag.  kMagic is a NaN bit pattern that no sum produces.
constexpr uint64_t kMagic = 0xFFF4A5C3E1D2B987ull;
struct XSlot {
  uint64_t val;
  uint64_t nz;
};

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
  XSlot* xch;       // [B][T][G]: sweep r of sequence b, workgroup g (G > 1 only)
  uint32_t* exitc;  // [B]: workgroups of the sequence that have finished
  int T, W, V, mode, G;
};

// DPP move of a double (both halves alike); a lane without a source takes 0.
template <int kCtrl, int kRowMask = 0xf>
__device__ inline double dpp_f64_or0(double v) {
  const long long x = __double_as_longlong(v);
  const int lo = dpp_mov<kCtrl, kRowMask>((int)(uint32_t)x, 0);
  const int hi = dpp_mov<kCtrl, kRowMask>((int)(x >> 32), 0);
  return __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
}

__device__ inline double readlane_f64(double v, int l) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
}

// Inclusive prefix sum over the lanes of a wavefront (row shifts, then row broadcasts).
__device__ inline double wave_scan_f64(double v) {
  v += dpp_f64_or0<0x111>(v);
  v += dpp_f64_or0<0x112>(v);
  v += dpp_f64_or0<0x114>(v);
  v += dpp_f64_or0<0x118>(v);
  v += dpp_f64_or0<0x142, 0xa>(v);
  v += dpp_f64_or0<0x143, 0xc>(v);
  return v;
}

// Sum over the wavefront, the same in every lane (lane 63's prefix, read out as uniform).
__device__ inline double wave_sum_f64(double v) { return readlane_f64(wave_scan_f64(v), 63); }

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

// Four consecutive elements of a row starting at i (zeros past V).  Branch-free: the load
// reads a group clamped into the row and the select zeroes what lies past V, so the loads of
// several groups can all be in flight at once.
template <bool kVec>
__device__ inline void load4(const float* __restrict__ row, int i, int V, float (&v)[4]) {
  if constexpr (kVec) {  // V % 4 == 0, so V >= 4 and a group is all in or all out
    const float4 t = *reinterpret_cast<const float4*>(row + min(i, V - 4));
    const bool in = i < V;
    v[0] = in ? t.x : 0.f;
    v[1] = in ? t.y : 0.f;
    v[2] = in ? t.z : 0.f;
    v[3] = in ? t.w : 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = row[min(i + e, V - 1)];
      v[e] = i + e < V ? x : 0.f;
    }
  }
}

__device__ inline double resid(float p, float q, double C) {
  const double d = fma(-C, (double)q, (double)p);
  return d > 0.0 ? d : 0.0;
}

// Sum of U(y) = max(0, p(y) - C q(y)) over chunks [k_lo, k_hi) of the vocabulary (chunk k =
// 256 consecutive elements, handled by wavefront (k - k_lo) % 8).  With kDraw the chunk sums go
// to s_chunk[k - k_lo] and last_nz tracks the largest y with U(y) > 0.  kQ = false when C == 0
// (U = p; q is not read).  All loads of an unrolled step are issued before any is used.
// Returns this thread's share of the sum.
template <bool kVec, bool kDraw, bool kQ>
__device__ double sweep_impl(const float* __restrict__ pu, const float* __restrict__ qu, double C,
                             int V, int k_lo, int k_hi, int wave, int lane, double* s_chunk,
                             int& last_nz) {
  double acc = 0.0;
  for (int k0 = k_lo + wave; k0 < k_hi; k0 += kSWaves * kUnroll) {
    float pv[kUnroll][4], qv[kUnroll][4];
#pragma unroll
    for (int s = 0; s < kUnroll; ++s) {
      const int k = k0 + s * kSWaves;
      const int i = k < k_hi ? k * kChunk + lane * 4 : V;
      load4<kVec>(pu, i, V, pv[s]);
      if constexpr (kQ) {
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
        if (lane == 0 && k < k_hi) s_chunk[k - k_lo] = t;
      }
      acc += cs;
    }
  }
  return acc;
}

template <bool kVec, bool kDraw>
__device__ double sweep(const float* __restrict__ pu, const float* __restrict__ qu, double C,
                        int V, int k_lo, int k_hi, int wave, int lane, double* s_chunk,
                        int& last_nz) {
  return C != 0.0
             ? sweep_impl<kVec, kDraw, true>(pu, qu, C, V, k_lo, k_hi, wave, lane, s_chunk, last_nz)
             : sweep_impl<kVec, kDraw, false>(pu, qu, C, V, k_lo, k_hi, wave, lane, s_chunk,
                                              last_nz);
}

// Sweep r of sequence b: publishes this workgroup's (val, nz) and fills s_xval / s_xnz with every
// workgroup's values, in workgroup order.  Called by all threads; ends with a barrier.  The
// words go through device-coherent atomics (relaxed: each word is written once and read until it
// is nonzero).
__device__ void exchange(const StochArgs& a, int b, int g, int r, double val, int nz, int tid,
                         double* s_xval, int* s_xnz, int* s_timeout) {
  XSlot* row = a.xch + ((size_t)b * a.T + r) * a.G;
  if (tid == 0) {
    __hip_atomic_store(&row[g].val, (uint64_t)__double_as_longlong(val) ^ kMagic,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&row[g].nz, (uint64_t)(uint32_t)(nz + 1) ^ kMagic, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < 64) {  // wavefront 0 polls, one lane per workgroup
    const int lane = tid;
    uint64_t v = 1, z = 1;
    uint32_t spins = 0;
    bool ok = true;
    for (;;) {
      if (lane < a.G) {
        v = __hip_atomic_load(&row[lane].val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        z = __hip_atomic_load(&row[lane].nz, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (__all(v != 0 && z != 0)) break;
      if (++spins > kSpinLimit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane < a.G) {
      s_xval[lane] = __longlong_as_double((long long)(v ^ kMagic));
      s_xnz[lane] = (int)(uint32_t)(z ^ kMagic) - 1;
    }
    if (lane == 0 && !ok) *s_timeout = 1;
  }
  __syncthreads();
}

template <bool kVec>
__global__ __launch_bounds__(kSThreads) void accept_stochastic_kernel(StochArgs a) {
  __shared__ double s_red[2][kSWaves];
  __shared__ int s_ired[kSWaves];
  __shared__ double s_chunk[kMaxChunks];
  __shared__ int s_path[kMaxT];
  __shared__ double s_xval[kMaxG];
  __shared__ int s_xnz[kMaxG];
  __shared__ int s_timeout, s_last;

  const int G = a.G;
  const int b = blockIdx.x / G, g = blockIdx.x - b * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, V = a.V;
  // this workgroup's slice of the vocabulary, in chunks
  const int nchunks = ceil_div(V, kChunk);
  const int per_wg = ceil_div(nchunks, G);
  const int k_lo = min(nchunks, g * per_wg), k_hi = min(nchunks, k_lo + per_wg);

  // the lane's two nodes: parent, token, acceptance and residual uniforms (the residual one is
  // read only by the bonus draw, but fetched here so its load is long done by then)
  int par[2], tok[2];
  double ua[2], ur[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    par[k] = -2;
    tok[k] = -1;
    ua[k] = 0.0;
    ur[k] = 0.0;
    if (c < T) {
      const uint64_t* row = a.anc + ((size_t)b * T + c) * a.W;
      par[k] = parent_from_row(c, row[0], a.W > 1 ? row[1] : 0ull);
      tok[k] = a.draft[(size_t)b * T + c];
      ua[k] = a.u_acc[(size_t)b * T + c];
      ur[k] = a.u_res[(size_t)b * T + c];
    }
  }

  // p and q of every node's token under its parent's distributions, all gathered up front (the
  // tests at a node read its children's raw p, q values whatever the walk did before)
  float pg[2], qg[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bool g_ok = par[k] >= 0 && tok[k] >= 0 && tok[k] < V;
    const size_t at = ((size_t)b * T + max(par[k], 0)) * V + (g_ok ? tok[k] : 0);
    pg[k] = g_ok ? a.p[at] : 0.f;
    qg[k] = g_ok ? a.q[at] : 0.f;
  }

  int u = 0, n = 1, buf = 0, bad = 0, rounds = 0;
  uint32_t exit_prev = 0;  // the sequence's exit count before this workgroup's (thread 0)
  int bonus = -1;
  bool writer = false;  // this workgroup writes bonus_tok[b]
  if (tid == 0) {
    s_path[0] = 0;
    s_timeout = 0;
  }
  __syncthreads();
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
      px[k] = pg[k];
      qx[k] = qg[k];
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
      // the child's token, probabilities and uniform from its lane (l is uniform)
      const int x = __builtin_amdgcn_readlane(k ? tok[1] : tok[0], l);
      const double pxd = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(k ? px[1] : px[0]), l));
      const double qxd = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(k ? qx[1] : qx[0]), l));
      const double uac = readlane_f64(k ? ua[1] : ua[0], l);
      bool excl = false;
      if (a.mode) {
        const bool same = ((rj0 >> lane) & 1 && tok[0] == x) || ((rj1 >> lane) & 1 && tok[1] == x);
        excl = __ballot(same) != 0;
      }
      const double Ux = fmax(fma(-C, qxd, pxd), 0.0);  // U_j(x) = p_j(x) * S_j
      // (x / 1 is x exactly: independent siblings skip the divisions)
      const double qj = (excl || !(N > 0.0)) ? 0.0 : (N == 1.0 ? qxd : qxd / N);
      if (uac * qj * S < Ux) {
        next = c;
        break;
      }
      // rejected: the residual for the next sibling
      const double Cn = C + (N > 0.0 ? (N == 1.0 ? S : S / N) : 0.0);
      int unused = -1;
      const double part =
          wave_sum_f64(sweep<kVec, false>(pu, qu, Cn, V, k_lo, k_hi, wave, lane, nullptr, unused));
      if (lane == 0) s_red[buf][wave] = part;
      __syncthreads();
      double Sn = 0.0;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) Sn += s_red[buf][w];
      buf ^= 1;
      if (G > 1) {
        exchange(a, b, g, rounds, Sn, -1, tid, s_xval, s_xnz, &s_timeout);
        Sn = 0.0;
        for (int h = 0; h < G; ++h) Sn += s_xval[h];
      }
      ++rounds;
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

    // ---- bonus draw at u from U = max(0, p - C q) ----
    const double u_draw = readlane_f64(u < 64 ? ur[0] : ur[1], u & 63);
    // chunk sums of this workgroup's slice into LDS, and its last token with mass
    int last_nz = -1;
    sweep<kVec, true>(pu, qu, C, V, k_lo, k_hi, wave, lane, s_chunk, last_nz);
    last_nz = wave_max(last_nz);
    if (lane == 0) s_ired[wave] = last_nz;
    __syncthreads();
    for (int w = 0; w < kSWaves; ++w) last_nz = max(last_nz, s_ired[w]);
    // per lane: the running sum of the slice before its chunks (excl) and over them (local)
    const int nloc = k_hi - k_lo;
    const int per = ceil_div(nloc, 64);
    double local = 0.0;
    for (int j = 0; j < per; ++j) {
      const int kk = lane * per + j;
      if (kk < nloc) local += s_chunk[kk];
    }
    const double incl = wave_scan_f64(local);
    const double excl = dpp_f64_or0<0x138>(incl);  // wave_shr:1: the previous lane's (0 in lane 0)
    // the slice where the running sum first exceeds u * total (owner), the running sum before
    // it (base), and the last token with mass over the whole vocabulary (gnz)
    double total = readlane_f64(incl, 63), base = 0.0;
    int owner = 0, gnz = last_nz;
    if (G > 1) {
      exchange(a, b, g, rounds, total, last_nz, tid, s_xval, s_xnz, &s_timeout);
      // every walk ends with this exchange, its last use of the slots: count this workgroup
      // out now, so the atomic's round trip overlaps the rest of the draw
      if (tid == 0)
        exit_prev = __hip_atomic_fetch_add(a.exitc + b, 1u, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
      total = 0.0;
      for (int h = 0; h < G; ++h) total += s_xval[h];
      const double thr_all = u_draw * total;
      double pre = 0.0;
      owner = -1;
      gnz = -1;
      for (int h = 0; h < G; ++h) {
        gnz = max(gnz, s_xnz[h]);
        if (owner < 0 && pre + s_xval[h] > thr_all) {
          owner = h;
          base = pre;
        }
        pre += s_xval[h];
      }
    }
    ++rounds;
    const double thr = u_draw * total;
    if (owner < 0) {  // no running sum exceeds the threshold (u >= 1, rounding)
      writer = g == 0;
      bonus = gnz;
      break;
    }
    if (owner != g) break;
    writer = true;
    // this slice: without a crossing found below (rounding), its last token with mass
    bonus = G > 1 ? last_nz : gnz;
    const uint64_t over = __ballot(base + (excl + local) > thr);
    if (over) {
      const int L = __builtin_ctzll(over);
      const double excl_L = base + readlane_f64(excl, L);
      // chunk of lane L where the running sum first exceeds thr (walked by every lane alike)
      int kc = -1;
      double before = excl_L, run = 0.0;
      for (int j = 0; j < per; ++j) {
        const int kk = L * per + j;
        if (kk >= nloc) break;
        const double ck = s_chunk[kk];
        if (excl_L + (run + ck) > thr && ck > 0.0) {
          kc = k_lo + kk;
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
        const double inc2 = wave_scan_f64(ls);
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
        bonus = hits ? __builtin_amdgcn_readlane(hit, __builtin_ctzll(hits))
                     : wave_max(lastpos);  // rounding tie at the chunk's end
      }
    }
    break;
  }
  __syncthreads();
  if (tid == 0) {
    if (g == 0) a.alen[b] = n;
    if (writer) a.bonus[b] = bonus;
    const int bits = (g == 0 && bad ? TV_BAD_TOKEN : 0) | (s_timeout ? TV_SYNC_TIMEOUT : 0);
    if (bits && a.status) atomicOr(a.status + b, bits);
  }
  if (g == 0)
    for (int t = tid; t < T; t += kSThreads) a.path[(size_t)b * T + t] = t < n ? s_path[t] : -1;
  if (G > 1) {
    // the last workgroup of the sequence to count out clears the slots this call used
    if (tid == 0) s_last = exit_prev == (uint32_t)(G - 1);
    __syncthreads();
    if (s_last) {
      XSlot* rows = a.xch + (size_t)b * T * G;
      for (int i = tid; i < rounds * G; i += kSThreads) rows[i] = XSlot{0ull, 0ull};
      if (tid == 0) a.exitc[b] = 0u;
    }
  }
}

// Profiling events recorded around the kernel (tv_profile_accept_stochastic).
hipEvent_t g_st_before = nullptr, g_st_after = nullptr;

template <bool kVec>
void launch_stochastic(const StochArgs& a, int B, hipStream_t stream) {
  const dim3 grid(B * a.G), block(kSThreads);
  if (g_st_before)  // the events take the kernel's own start and end timestamps
    hipExtLaunchKernelGGL(accept_stochastic_kernel<kVec>, grid, block, 0, stream, g_st_before,
                          g_st_after, 0, a);
  else
    hipLaunchKernelGGL(accept_stochastic_kernel<kVec>, grid, block, 0, stream, a);
}

// Workgroups per sequence: as many as keep B * G within the compute units, at most 8, and at
// least 32 chunks (8192 tokens) of the vocabulary per workgroup.  (Past 8 the exchange costs
// more than the smaller slices save: 128256 tokens at batch 1 take 24 us with 8, 25 with 16
// and 29 with 32.)
int auto_groups(int B, int V) {
  const int nchunks = ceil_div(V, kChunk);
  int G = device_cu_count() / B;
  G = std::min(G, 8);
  G = std::min(G, nchunks / 32);
  return std::max(G, 1);
}

size_t workspace_bytes_for(int B, int T, int G) {
  if (G <= 1) return 0;
  return (size_t)B * T * G * sizeof(XSlot) + (size_t)B * sizeof(uint32_t);
}

}  // namespace
}  // namespace tv

using namespace tv;

extern "C" int tv_profile_accept_stochastic(void* ev_before, void* ev_after) {
  if ((ev_before == nullptr) != (ev_after == nullptr)) return TV_ERR_INVALID_ARG;
  g_st_before = (hipEvent_t)ev_before;
  g_st_after = (hipEvent_t)ev_after;
  return TV_OK;
}

extern "C" size_t tree_accept_stochastic_workspace_size(int B, int T, int V,
                                                        int workgroups_per_seq) {
  if (B < 1 || T < 1 || T > kMaxT || V < 1 || V > kChunk * kMaxChunks || workgroups_per_seq < 0 ||
      workgroups_per_seq > kMaxG)
    return 0;
  const int G = workgroups_per_seq ? workgroups_per_seq : auto_groups(B, V);
  return workspace_bytes_for(B, T, G);
}

extern "C" int tree_accept_stochastic(const uint64_t* anc_mask, const int32_t* draft_tok,
                                      const float* p, const float* q, const double* u_acc,
                                      const double* u_res, int B, int T, int V,
                                      int without_replacement, int workgroups_per_seq,
                                      void* workspace, size_t workspace_bytes,
                                      int32_t* accept_path, int32_t* accept_len,
                                      int32_t* bonus_tok, int32_t* status, void* stream) {
  if (!anc_mask || !draft_tok || !p || !q || !u_acc || !u_res || !accept_path || !accept_len ||
      !bonus_tok || B < 1 || T < 1 || T > kMaxT || V < 1 || V > kChunk * kMaxChunks ||
      (without_replacement != 0 && without_replacement != 1) || workgroups_per_seq < 0 ||
      workgroups_per_seq > kMaxG)
    return TV_ERR_INVALID_ARG;
  const int G = workgroups_per_seq ? workgroups_per_seq : auto_groups(B, V);
  // every workgroup of a sequence must be resident at once (one per compute unit)
  if (G > 1 && (long long)B * G > device_cu_count()) return TV_ERR_INVALID_ARG;
  const size_t need = workspace_bytes_for(B, T, G);
  if (need && (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16) != 0))
    return TV_ERR_WORKSPACE;
  XSlot* xch = need ? static_cast<XSlot*>(workspace) : nullptr;
  uint32_t* exitc = need ? reinterpret_cast<uint32_t*>(xch + (size_t)B * T * G) : nullptr;
  StochArgs a{anc_mask, draft_tok, p, q, u_acc, u_res, accept_path, accept_len, bonus_tok, status,
              xch, exitc, T, ceil_div(T, 64), V, without_replacement, G};
  const bool vec = V % 4 == 0 && ((uintptr_t)p % 16) == 0 && ((uintptr_t)q % 16) == 0;
  if (vec)
    launch_stochastic<true>(a, B, (hipStream_t)stream);
  else
    launch_stochastic<false>(a, B, (hipStream_t)stream);
  return launch_status();
}
