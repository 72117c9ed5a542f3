// EAGLE-2 dynamic draft tree built on the device (rainlin.net "EAGLE 系列", section 7).
//
//   * Expansion (section 7.1), one launch per level, between the drafter's forward passes:
//     every frontier node of the previous level receives the `branch` candidate children the
//     drafter proposed for it.  A child's global acceptance value is its parent's value times
//     its confidence (the product of the confidences on its root path, in float32), and the
//     frontier of the new level is its k best children, best first.  One workgroup per
//     sequence; a child's rank is the number of this level's children that outrank it (larger
//     value, or equal value and smaller node id), counted over LDS by up to four threads, each
//     over a quarter of the values.
//   * Reranking and flattening (section 7.2), one launch after the last level: the T best nodes
//     of the whole table are kept, and the kept tree is flattened in level order (depth, then
//     the parent's flattened index, then node id), ready for tree_build_mask.  One workgroup
//     of 1024 threads per sequence: a radix select over the 48-bit keys
//     (value bits << 16 | 0xFFFF - id), six 8-bit passes with an LDS histogram and a wavefront
//     suffix scan, finds the T-th best key; then wavefront 0 alone sorts the kept nodes by id,
//     finds their depths by pointer jumping over the kept list and flattens the levels one
//     after another, without workgroup barriers.
//
// Node ids: the root is node 0; child c of frontier slot r of level l is node
// n_l + r * branch + c, with n_l the nodes of the levels before l, so ids grow with depth and
// equal values resolve towards the shallower node.
#include <hip/hip_runtime.h>

#include "tree_device.h"

namespace tv {
namespace {

constexpr int kExpandMax = 1024;        // children of one level (k * branch)
constexpr int kRerankThreads = 1024;
constexpr int kRerankMaxNodes = 16384;  // node values staged in LDS (64 KB); ids fit 16 bits

// A drafter confidence used as a probability: NaN and negatives count as 0, values above 1 as 1.
__device__ inline float as_prob(float c) { return c > 0.f ? (c < 1.f ? c : 1.f) : 0.f; }
// A node value as it is ranked: NaN and negatives count as 0 (so its bits order as an integer).
__device__ inline float rank_value(float v) { return v > 0.f ? v : 0.f; }

// One expansion level of sequence blockIdx.x.  F parents: the root at level 1, otherwise
// frontier[b, 0..F) (ids of the previous level, [prev_lo, base)).  Children go to ids
// base .. base + F*branch - 1; the new frontier (min(k, F*branch) ids, best first, padded with
// -1 to k) overwrites frontier[b] after every parent entry has been read.
__global__ __launch_bounds__(kExpandMax) void expand_kernel(
    int level, const int32_t* __restrict__ root_tok, const int32_t* __restrict__ child_tok,
    const float* __restrict__ child_conf, int k, int branch, int F, int prev_lo, int base,
    int n_max, int32_t* __restrict__ node_tok, int32_t* __restrict__ node_parent,
    float* __restrict__ node_value, int32_t* __restrict__ frontier, int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(16))) float s_val[kExpandMax];
  __shared__ int s_part[kExpandMax];  // partial ranks, [group][child]
  const int b = blockIdx.x, tid = threadIdx.x;
  const int n = F * branch;
  const int n_front = min(k, n);
  // npad threads per group (one per child); G groups split each child's rank count
  const int npad = (max(n, k) + 63) & ~63;
  const int G = blockDim.x / npad;
  const int g = tid / npad, c = tid - g * npad;
  const size_t row = (size_t)b * n_max;
  int bits = 0;
  float v = 0.f;
  if (g == 0 && c < n) {
    const int r = c / branch, cc = c - r * branch;
    // the child's own token and confidence first: they go out with the frontier read, not
    // behind the parent's value, which waits for it
    const size_t src = ((size_t)b * k + r) * branch + cc;
    const float conf = child_conf[src];
    const int32_t ctok = child_tok[src];
    int pid = 0;
    float pv = 1.f;
    bool ok = true;
    if (level > 1) {
      pid = frontier[(size_t)b * k + r];
      ok = pid >= prev_lo && pid < base;
      pv = ok ? node_value[row + pid] : 0.f;
      if (!ok) bits |= TV_BAD_TREE;
    }
    if (!(conf >= 0.f && conf <= 1.f)) bits |= TV_BAD_CONF;
    v = rank_value(pv * as_prob(conf));
    node_tok[row + base + c] = ctok;
    node_parent[row + base + c] = ok ? pid : -1;
    node_value[row + base + c] = v;
    s_val[c] = v;
  }
  if (g == 0 && c >= n && c < ((n + 3) & ~3)) s_val[c] = -1.f;  // padding: below every value
  if (level == 1 && tid == 0) {
    node_tok[row] = root_tok[b];
    node_parent[row] = -1;
    node_value[row] = 1.f;
  }
  __syncthreads();  // every parent entry of the frontier has been read
  // group g counts, for child c, the outranking children among words [q0, q1) of the values
  int rank = 0;
  if (c < n) {
    if (g > 0) v = s_val[c];
    const int Q = (n + 3) >> 2, Qg = (Q + G - 1) / G;
    const int q0 = g * Qg, q1 = min(Q, q0 + Qg);
    // four values per LDS read (every lane reads the same address), several reads in flight
    const float4* sv = reinterpret_cast<const float4*>(s_val);
#pragma unroll 4
    for (int q = q0; q < q1; ++q) {
      const float4 w = sv[q];
      const int j = 4 * q;
      rank += (w.x > v) || (w.x == v && j < c);
      rank += (w.y > v) || (w.y == v && j + 1 < c);
      rank += (w.z > v) || (w.z == v && j + 2 < c);
      rank += (w.w > v) || (w.w == v && j + 3 < c);
    }
  }
  if (G > 1) {
    s_part[tid] = rank;
    __syncthreads();
    if (g == 0 && c < n)
      for (int q = 1; q < G; ++q) rank += s_part[q * npad + c];
  }
  if (g == 0) {
    if (c < n && rank < n_front) frontier[(size_t)b * k + rank] = base + c;
    if (c >= n_front && c < k) frontier[(size_t)b * k + c] = -1;
    if (bits) atomicOr(status + b, bits);
  }
}

// Inclusive prefix sum over the wavefront (DPP row shifts, then row broadcasts; lanes without a
// source add 0), in every lane.
template <int kCtrl, int kRowMask>
__device__ inline int dpp_i32_or0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, false);
}
__device__ inline int wave_prefix_sum(int v) {
  v += dpp_i32_or0<0x111, 0xf>(v);  // row_shr:1
  v += dpp_i32_or0<0x112, 0xf>(v);  // row_shr:2
  v += dpp_i32_or0<0x114, 0xf>(v);  // row_shr:4
  v += dpp_i32_or0<0x118, 0xf>(v);  // row_shr:8
  v += dpp_i32_or0<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i32_or0<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Reranking and flattening of sequence blockIdx.x's table of n nodes (row stride n_max).  All
// 1024 threads stage the table and run the radix select; the kept nodes (at most 128) are then
// sorted, linked and flattened by wavefront 0 alone, two nodes per lane, with no workgroup
// barrier.
__global__ __launch_bounds__(kRerankThreads) void rerank_kernel(
    const int32_t* __restrict__ node_tok, const int32_t* __restrict__ node_parent,
    const float* __restrict__ node_value, int n, int n_max, int T, int32_t* __restrict__ parent_out,
    int32_t* __restrict__ tok_out, int32_t* __restrict__ depth_out, int32_t* __restrict__ node_out,
    int32_t* __restrict__ status) {
  __shared__ uint32_t s_key[kRerankMaxNodes];  // rank_value bits of every node
  __shared__ int32_t s_par[kRerankMaxNodes];   // every node's parent
  __shared__ int s_hist[2][256];               // one pass counts while the other is cleared
  __shared__ int s_sel[2];  // digit of the pass, count still to take at or below it
  __shared__ int s_cnt;
  __shared__ __attribute__((aligned(16))) int s_kept[kMaxT];
  __shared__ __attribute__((aligned(16))) int s_dep[kMaxT];
  __shared__ __attribute__((aligned(16))) int s_lp[kMaxT];
  __shared__ int s_id[kMaxT], s_ptr[kMaxT], s_flat[kMaxT];
  __shared__ int s_cc[kMaxT];                         // children of list position t
  __shared__ __attribute__((aligned(8))) int s_A[kMaxT], s_E[kMaxT];  // by level-order index
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = (size_t)b * n_max;
  const size_t orow = (size_t)b * T;
  const int T4 = (T + 3) & ~3;  // lists padded to whole 16-byte reads

  // four nodes per thread in flight at a time: loads clamped to the last node rather than
  // branched, so a batch costs one memory round trip (n >= 1)
  for (int base = 0; base < n; base += 4 * kRerankThreads) {
    float v[4];
    int pp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = min(base + k * kRerankThreads + tid, n - 1);
      v[k] = node_value[row + i];
      pp[k] = node_parent[row + i];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = base + k * kRerankThreads + tid;
      if (i < n) {
        s_key[i] = __float_as_uint(rank_value(v[k]));
        s_par[i] = pp[k];
      }
    }
  }
  if (tid < 512) (&s_hist[0][0])[tid] = 0;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  // a tree whose values never grow from parent to child: then a parent outranks its children
  // and the kept set is closed under parents
  int bad = 0;
  for (int i = tid; i < n; i += kRerankThreads) {
    const int p = s_par[i];
    bad |= i == 0 ? p != -1 : (p < 0 || p >= i || s_key[i] > s_key[p]);
  }
  if (__syncthreads_or(bad)) {
    for (int f = tid; f < T; f += kRerankThreads) {
      parent_out[orow + f] = -1;
      tok_out[orow + f] = -1;
      depth_out[orow + f] = 0;
      node_out[orow + f] = -1;
    }
    if (tid == 0) atomicOr(status + b, TV_BAD_TREE);
    return;
  }

  // ---- radix select of the T-th best key, 8 bits per pass from the top -------------------
  auto key48 = [&](int i) -> uint64_t {
    return ((uint64_t)s_key[i] << 16) | (uint32_t)(0xFFFF - i);
  };
  uint64_t prefix = 0;
  int need = T;
  for (int pass = 0; pass < 6; ++pass) {
    const int shift = 40 - 8 * pass;
    int* hist = s_hist[pass & 1];
    for (int i = tid; i < n; i += kRerankThreads) {
      const uint64_t key = key48(i);
      if ((key >> (shift + 8)) == (prefix >> (shift + 8)))
        atomicAdd(&hist[(int)(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 4l .. 4l+3; S = keys in bins of lanes >= l (a suffix sum)
      int h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = hist[4 * lane + j];
      const int mine = h[0] + h[1] + h[2] + h[3];
      const int P = wave_prefix_sum(mine);
      const int S = __builtin_amdgcn_readlane(P, 63) - P + mine;
      const int above = S - mine;
      if (above < need && need <= S) {  // exactly one lane
        int acc = above, d = 4 * lane;
        for (int j = 3; j >= 0; --j) {
          if (acc + h[j] >= need) {
            d = 4 * lane + j;
            break;
          }
          acc += h[j];
        }
        s_sel[0] = d;
        s_sel[1] = need - acc;
      }
    } else if (wave >= 4 && wave < 8) {
      s_hist[(pass + 1) & 1][tid - 256] = 0;  // the next pass's histogram (read last pass)
    }
    __syncthreads();
    prefix |= (uint64_t)s_sel[0] << shift;
    need = s_sel[1];
  }
  // keys are distinct, so exactly T nodes have a key at or above the T-th best

  for (int i = tid; i < n; i += kRerankThreads)
    if (key48(i) >= prefix) {
      const int slot = atomicAdd(&s_cnt, 1);
      if (slot < kMaxT) s_kept[slot] = i;
    }
  __syncthreads();
  if (wave != 0) return;

  // ---- wavefront 0: kept nodes in id order, parents, depths, level order --------------------
  // lane l handles list positions l and l + 64
  if (lane < T4 - T) {
    s_kept[T + lane] = 0x7fffffff;  // padding: after every id
    s_lp[T + lane] = -2;            // padding: nobody's sibling
  }
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = lane + 64 * h;
    if (t < T) {
      const int u = s_kept[t];
      const int4* sk = reinterpret_cast<const int4*>(s_kept);
      int r = 0;
#pragma unroll 4
      for (int q = 0; q < T4 >> 2; ++q) {
        const int4 w = sk[q];
        r += (w.x < u) + (w.y < u) + (w.z < u) + (w.w < u);
      }
      s_id[r] = u;
    }
  }
  wave_lds_sync();
  int tok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = lane + 64 * h;
    tok[h] = 0;
    if (t < T) {
      const int u = s_id[t];
      tok[h] = node_tok[row + u];  // used at the end; the load runs under the work below
      // position of the parent in the id-ordered list (node 0, the best node, is at position 0)
      int pos = -1;
      if (t > 0) {
        const int pu = s_par[u];
        int lo = 0, hi = t - 1;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_id[mid] < pu) lo = mid + 1;
          else hi = mid;
        }
        pos = lo;
      }
      s_lp[t] = pos;
      s_ptr[t] = pos;
      s_dep[t] = pos < 0 ? 0 : 1;
      s_cc[t] = 0;
    }
  }
  // pointer jumping: s_dep is the distance to s_ptr, which doubles every round
  for (int span = 1; span < T; span <<= 1) {
    wave_lds_sync();
    int nd[2] = {0, 0}, np[2] = {-1, -1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lane + 64 * h;
      if (t < T) {
        const int p = s_ptr[t];
        nd[h] = s_dep[t] + (p >= 0 ? s_dep[p] : 0);
        np[h] = p >= 0 ? s_ptr[p] : -1;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lane + 64 * h;
      if (t < T) {
        s_dep[t] = nd[h];
        s_ptr[t] = np[h];
      }
    }
  }
  wave_lds_sync();
  // depths, children counts, and each node's rank among its siblings in id order
  int dep[2] = {0, 0}, lp[2] = {-1, -1}, sib[2] = {0, 0};
  int dmax = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = lane + 64 * h;
    if (t < T) {
      dep[h] = s_dep[t];
      dmax = max(dmax, dep[h]);
      lp[h] = s_lp[t];
      if (lp[h] >= 0) atomicAdd(&s_cc[lp[h]], 1);
      const int4* sl = reinterpret_cast<const int4*>(s_lp);
#pragma unroll 4
      for (int q = 0; q < T4 >> 2; ++q) {
        const int4 w = sl[q];
        sib[h] += (w.x == lp[h] && 4 * q < t) + (w.y == lp[h] && 4 * q + 1 < t) +
                  (w.z == lp[h] && 4 * q + 2 < t) + (w.w == lp[h] && 4 * q + 3 < t);
      }
    }
  }
  dmax = __reduce_max_sync(~0ull, dmax);

  // ---- level order (depth, then the parent's index in it, then id) ---------------------------
  // In that order a node's children follow every child of the nodes placed before it, so a
  // child at depth d takes index 1 + (children of the nodes before its parent) + (its rank
  // among its siblings).  Level by level: s_A holds each placed node's children count at its
  // index, s_E the exclusive prefix sums of s_A (a wavefront scan over index pairs).
  wave_lds_sync();
  *reinterpret_cast<int2*>(&s_A[2 * lane]) = int2{0, 0};
  wave_lds_sync();
  if (lane == 0) {
    s_flat[0] = 0;  // the root
    s_A[0] = s_cc[0];
  }
  for (int d = 1; d <= dmax; ++d) {
    wave_lds_sync();
    const int2 a = *reinterpret_cast<const int2*>(&s_A[2 * lane]);
    const int e0 = wave_prefix_sum(a.x + a.y) - (a.x + a.y);
    *reinterpret_cast<int2*>(&s_E[2 * lane]) = int2{e0, e0 + a.x};
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = lane + 64 * h;
      if (t < T && dep[h] == d) {
        const int f = 1 + s_E[s_flat[lp[h]]] + sib[h];
        s_flat[t] = f;
        s_A[f] = s_cc[t];
      }
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = lane + 64 * h;
    if (t < T) {
      const int f = s_flat[t];
      parent_out[orow + f] = lp[h] < 0 ? -1 : s_flat[lp[h]];
      tok_out[orow + f] = tok[h];
      depth_out[orow + f] = dep[h];
      node_out[orow + f] = s_id[t];
    }
  }
}

// Nodes after `levels` expansion levels and the frontier size after the last one (host).
long long node_count(int levels, int k, int branch, int* front) {
  long long n = 1, F = 1;
  for (int l = 0; l < levels; ++l) {
    n += F * branch;
    F = F * branch < k ? F * branch : k;
    if (n > (1LL << 30)) return -1;
  }
  if (front) *front = (int)F;
  return n;
}

}  // namespace
}  // namespace tv

using namespace tv;

extern "C" int eagle2_node_count(int depth, int k, int branch) {
  if (depth < 0 || k < 1 || branch < 1) return -1;
  return (int)node_count(depth, k, branch, nullptr);
}

extern "C" int eagle2_expand(const int32_t* root_tok, const int32_t* child_tok,
                             const float* child_conf, int B, int level, int k, int branch,
                             int32_t* node_tok, int32_t* node_parent, float* node_value,
                             int n_max, int32_t* frontier, int32_t* status, void* stream) {
  if (!child_tok || !child_conf || !node_tok || !node_parent || !node_value || !frontier ||
      !status || B < 1 || level < 1 || k < 1 || branch < 1 || (long long)k * branch > kExpandMax)
    return TV_ERR_INVALID_ARG;
  if (level == 1 && !root_tok) return TV_ERR_INVALID_ARG;
  int F = 1;  // parents of this level: the frontier after level - 1
  const long long base = node_count(level - 1, k, branch, &F);
  const long long prev_lo = level == 1 ? 0 : node_count(level - 2, k, branch, nullptr);
  if (base < 0 || base + (long long)F * branch > n_max) return TV_ERR_INVALID_ARG;
  // one thread per child, in up to four groups that split the rank counts
  const int npad = ceil_div(max(F * branch, k), 64) * 64;
  const int threads = npad * (npad <= kExpandMax / 4 ? 4 : npad <= kExpandMax / 2 ? 2 : 1);
  hipLaunchKernelGGL(expand_kernel, dim3(B), dim3(threads), 0, (hipStream_t)stream, level,
                     root_tok, child_tok, child_conf, k, branch, F, (int)prev_lo, (int)base, n_max,
                     node_tok, node_parent, node_value, frontier, status);
  return launch_status();
}

extern "C" int eagle2_rerank(const int32_t* node_tok, const int32_t* node_parent,
                             const float* node_value, int n_nodes, int n_max, int B, int T,
                             int32_t* parent_out, int32_t* tok_out, int32_t* depth_out,
                             int32_t* node_out, int32_t* status, void* stream) {
  if (!node_tok || !node_parent || !node_value || !parent_out || !tok_out || !depth_out ||
      !node_out || !status || B < 1 || T < 1 || T > kMaxT || n_nodes < T ||
      n_nodes > kRerankMaxNodes || n_max < n_nodes)
    return TV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(rerank_kernel, dim3(B), dim3(kRerankThreads), 0, (hipStream_t)stream,
                     node_tok, node_parent, node_value, n_nodes, n_max, T, parent_out, tok_out,
                     depth_out, node_out, status);
  return launch_status();
}
