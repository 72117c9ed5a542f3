// Integer kernels of the verification step: ancestor masks, the acceptance walk and the
// compaction of the accepted K/V rows.  One wavefront (64 lanes) owns one sequence for the
// mask and acceptance kernels; T <= 128 nodes means two nodes per lane.
#include <hip/hip_runtime.h>

#include "tree_device.h"

namespace tv {
namespace {

// ------------------------------------------------------------------------------------------
// tree_build_mask: anc[i] = anc[parent(i)] | bit(i), computed by pointer jumping.
// Each node keeps the set of its ancestors closer than 2^r and a pointer to the ancestor at
// distance 2^r; one round merges the pointed-to node's set and doubles the pointer.  After
// ceil(log2 T) rounds every pointer has left the tree and the sets are complete.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void build_mask_kernel(const int32_t* __restrict__ parent,
                                                        int T, int W,
                                                        uint64_t* __restrict__ anc,
                                                        int32_t* __restrict__ status) {
  __shared__ uint64_t s_lo[kMaxT], s_hi[kMaxT];
  __shared__ int s_ptr[kMaxT];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int32_t* pb = parent + (size_t)b * T;

  uint64_t lo[2], hi[2];
  int ptr[2];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    lo[k] = hi[k] = 0;
    ptr[k] = -1;
    if (i < T) {
      const int p = pb[i];
      const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
      bad |= !ok;
      ptr[k] = (i > 0 && ok) ? p : -1;
      lo[k] = k == 0 ? bit64(i) : 0;
      hi[k] = k == 1 ? bit64(i) : 0;
      s_lo[i] = lo[k];
      s_hi[i] = hi[k];
      s_ptr[i] = ptr[k];
    }
  }
  bad = __ballot(bad) != 0;
  __syncthreads();
  for (int span = 1; span < T; span <<= 1) {
    int nptr[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      nptr[k] = ptr[k];
      if (ptr[k] >= 0) {
        lo[k] |= s_lo[ptr[k]];
        hi[k] |= s_hi[ptr[k]];
        nptr[k] = s_ptr[ptr[k]];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = lane + 64 * k;
      ptr[k] = nptr[k];
      if (i < T) {
        s_lo[i] = lo[k];
        s_hi[i] = hi[k];
        s_ptr[i] = ptr[k];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    if (i < T) {
      if (bad) {
        lo[k] = k == 0 ? bit64(i) : 0;
        hi[k] = k == 1 ? bit64(i) : 0;
      }
      uint64_t* row = anc + ((size_t)b * T + i) * W;
      row[0] = lo[k];
      if (W == 2) row[1] = hi[k];
    }
  }
  if (lane == 0) status[b] = bad ? TV_BAD_TREE : 0;
}

// ------------------------------------------------------------------------------------------
// tree_accept: one wavefront per sequence runs the acceptance walk (accept_walk).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void accept_kernel(const uint64_t* __restrict__ anc,
                                                    const int32_t* __restrict__ draft,
                                                    const int32_t* __restrict__ target, int T,
                                                    int W, int32_t* __restrict__ accept_path,
                                                    int32_t* __restrict__ accept_len,
                                                    int32_t* __restrict__ bonus_tok) {
  accept_walk(blockIdx.x, T, W, anc, draft, target, accept_path, accept_len, bonus_tok, nullptr);
}

// ------------------------------------------------------------------------------------------
// kv_compact_accepted: one workgroup per (sequence, group of KV heads).  Every accepted row of
// the group's heads is staged in LDS before any cache row is written, so tree rows that live in
// the cache's own tail are safe.  Rows move as 16-byte chunks.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void compact_kernel(
    char* kc, char* vc, const int32_t* cache_len,
    int32_t* cache_len_out, const char* kt, const char* vt, const int32_t* __restrict__ path,
    const int32_t* __restrict__ alen, int T, int Hkv, int Lmax, int row_bytes,
    int heads_per_wg, int stage_rows, int32_t* status) {
  extern __shared__ uint4 stage[];
  __shared__ int s_bits;
  __shared__ int s_path[kMaxT];
  const int b = blockIdx.x, hg = blockIdx.y, tid = threadIdx.x;
  // the whole path row is read with the lengths (one round trip), then checked from LDS
  const int L = cache_len[b];
  const int n = alen[b];
  if (tid < T) s_path[tid] = path[(size_t)b * T + tid];
  if (tid == 0) s_bits = 0;
  __syncthreads();
  int bits = 0;
  if (L < 0 || L > Lmax) bits |= TV_BAD_LEN;
  if (n < 0 || n > T) {
    bits |= TV_BAD_PATH;
  } else if (tid < n) {
    const int j = s_path[tid];
    if (j < 0 || j >= T) atomicOr(&s_bits, TV_BAD_PATH);
  }
  __syncthreads();
  bits |= s_bits;
  if (!bits && (long long)L + n > Lmax) bits |= TV_OVERFLOW;
  if (bits) {
    if (hg == 0 && tid == 0) {
      if (status) atomicOr(status + b, bits);
      cache_len_out[b] = L;
    }
    return;
  }
  const int cpr = row_bytes / 16;
  const int h0 = hg * heads_per_wg, h1 = min(Hkv, h0 + heads_per_wg);
  const int heads_per_phase = n > 0 ? max(1, stage_rows / (2 * n)) : 1;
  for (int h = h0; h < h1 && n > 0; h += heads_per_phase) {
    const int hh = min(h1, h + heads_per_phase);
    const int total = (hh - h) * 2 * n * cpr;
    for (int q = tid; q < total; q += 256) {
      const int chunk = q % cpr;
      int r = q / cpr;
      const int i = r % n;
      r /= n;
      const int kv = r & 1, head = h + (r >> 1);
      const int j = s_path[i];
      const char* src = (kv ? vt : kt) + (((size_t)b * T + j) * Hkv + head) * row_bytes;
      stage[q] = reinterpret_cast<const uint4*>(src)[chunk];
    }
    __syncthreads();
    for (int q = tid; q < total; q += 256) {
      const int chunk = q % cpr;
      int r = q / cpr;
      const int i = r % n;
      r /= n;
      const int kv = r & 1, head = h + (r >> 1);
      char* dst = (kv ? vc : kc) + (((size_t)b * Hkv + head) * Lmax + L + i) * row_bytes;
      reinterpret_cast<uint4*>(dst)[chunk] = stage[q];
    }
    __syncthreads();
  }
  if (hg == 0 && tid == 0) cache_len_out[b] = L + n;
}

// ------------------------------------------------------------------------------------------
// kv_commit_paged: one wavefront per sequence runs commit_paged_wave on the path in memory.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void commit_paged_kernel(
    int32_t* __restrict__ table, int max_pages, const int32_t* cache_len, int32_t* cache_len_out,
    const int32_t* __restrict__ tree_slot, const int32_t* __restrict__ path,
    const int32_t* __restrict__ alen, int T, int num_slots, int32_t* __restrict__ free_slots,
    int32_t* __restrict__ free_top, int32_t* status) {
  __shared__ int s_on[kMaxT];  // times each node appears on the path
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = cache_len[b];  // read before cache_len_out[b] is written (they may alias)
  const int n = alen[b];
  int pe[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    pe[k] = c < T ? path[(size_t)b * T + c] : -1;
  }
  commit_paged_wave(b, L, n, pe, table, max_pages, tree_slot, T, num_slots, free_slots, free_top,
                    status, cache_len_out, s_on);
}

}  // namespace
}  // namespace tv

using namespace tv;

extern "C" const char* tv_status_string(int code) {
  switch (code) {
    case TV_OK: return "TV_OK";
    case TV_ERR_INVALID_ARG: return "TV_ERR_INVALID_ARG: null pointer, bad shape or limit";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED: dtype or head_dim not supported";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE: workspace missing or too small";
    case TV_ERR_HIP: return "TV_ERR_HIP: HIP runtime or launch failure";
    case TV_BAD_TREE: return "TV_BAD_TREE: parent array is not a level-ordered single-root tree";
    case TV_OVERFLOW: return "TV_OVERFLOW: cache_len + accept_len exceeds Lmax";
    case TV_BAD_LEN: return "TV_BAD_LEN: cache_len outside [0, Lmax]";
    case TV_BAD_PATH: return "TV_BAD_PATH: accept_len or an accepted index out of range";
    case TV_BAD_PAGE: return "TV_BAD_PAGE: a block-table entry or tree slot outside the pool";
    case TV_BAD_TOKEN: return "TV_BAD_TOKEN: a tried child's token is outside the vocabulary";
    case TV_SYNC_TIMEOUT:
      return "TV_SYNC_TIMEOUT: the workgroups of a sequence did not all meet; re-zero the workspace";
    case TV_BAD_CONF: return "TV_BAD_CONF: a drafter confidence outside [0, 1] (used clamped)";
    case TV_FREE_FULL: return "TV_FREE_FULL: the free list had no room for some rejected slots";
    default: return "unknown tree_verify status";
  }
}

extern "C" int tree_build_mask(const int32_t* parent, int B, int T, uint64_t* anc_mask,
                               int32_t* status, void* stream) {
  if (!parent || !anc_mask || !status || B < 1 || T < 1 || T > kMaxT) return TV_ERR_INVALID_ARG;
  const int W = ceil_div(T, 64);
  hipLaunchKernelGGL(build_mask_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, parent, T, W,
                     anc_mask, status);
  return launch_status();
}

extern "C" int tree_accept(const uint64_t* anc_mask, const int32_t* draft_tok,
                           const int32_t* target_tok, int B, int T, int32_t* accept_path,
                           int32_t* accept_len, int32_t* bonus_tok, void* stream) {
  if (!anc_mask || !draft_tok || !target_tok || !accept_path || !accept_len || !bonus_tok ||
      B < 1 || T < 1 || T > kMaxT)
    return TV_ERR_INVALID_ARG;
  const int W = ceil_div(T, 64);
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, anc_mask,
                     draft_tok, target_tok, T, W, accept_path, accept_len, bonus_tok);
  return launch_status();
}

extern "C" int kv_compact_accepted(void* k_cache, void* v_cache, const int32_t* cache_len,
                                   int32_t* cache_len_out, const void* k_tree,
                                   const void* v_tree, const int32_t* accept_path,
                                   const int32_t* accept_len, int B, int T, int Hkv, int D,
                                   int Lmax, int dtype, int32_t* status, void* stream) {
  if (!k_cache || !v_cache || !cache_len || !cache_len_out || !k_tree || !v_tree ||
      !accept_path || !accept_len || B < 1 || T < 1 || T > kMaxT || Hkv < 1 || Lmax < 0)
    return TV_ERR_INVALID_ARG;
  if ((dtype != TV_F32 && dtype != TV_BF16) || (D != 64 && D != 128)) return TV_ERR_UNSUPPORTED;
  const int row_bytes = D * (dtype == TV_F32 ? 4 : 2);
  // When the output length array is the input one, a single workgroup per sequence reads
  // cache_len[b] before it writes cache_len_out[b]; otherwise one workgroup per KV head.
  const bool same_len = cache_len_out == cache_len;
  const int heads_per_wg = same_len ? Hkv : 1;
  const int stage_rows = 2 * T;  // one head's K and V rows at the largest accepted length
  const size_t lds = (size_t)stage_rows * row_bytes;
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&compact_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return TV_ERR_HIP;
  hipLaunchKernelGGL(compact_kernel, dim3(B, same_len ? 1 : Hkv), dim3(256), lds,
                     (hipStream_t)stream, (char*)k_cache, (char*)v_cache, cache_len,
                     cache_len_out, (const char*)k_tree, (const char*)v_tree, accept_path,
                     accept_len, T, Hkv, Lmax, row_bytes, heads_per_wg, stage_rows, status);
  return launch_status();
}

extern "C" int kv_commit_paged(int32_t* block_table, int max_pages, int page_size,
                               const int32_t* cache_len, int32_t* cache_len_out,
                               const int32_t* tree_slot, const int32_t* accept_path,
                               const int32_t* accept_len, int32_t* free_slots, int32_t* free_top,
                               int num_slots, int B, int T, int32_t* status, void* stream) {
  if (!block_table || !cache_len || !cache_len_out || !tree_slot || !accept_path ||
      !accept_len || !free_slots || !free_top || B < 1 || T < 1 || T > kMaxT || max_pages < 1 ||
      num_slots < 1)
    return TV_ERR_INVALID_ARG;
  if (page_size != 1) return TV_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(commit_paged_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, block_table,
                     max_pages, cache_len, cache_len_out, tree_slot, accept_path, accept_len, T,
                     num_slots, free_slots, free_top, status);
  return launch_status();
}
