// Device code shared by the acceptance kernel and the fused verification-step tail: the
// greedy acceptance walk over one sequence's tree, run by one wavefront.  Not part of the ABI.
#pragma once

#include "tv_internal.h"

namespace tv {

__device__ inline uint64_t bit64(int j) { return (uint64_t)1 << (j & 63); }

// Bits [0, n) of a two-word mask (n in [0, 128]).
__device__ inline void low_bits(int n, uint64_t& lo, uint64_t& hi) {
  lo = n >= 64 ? ~0ull : (n <= 0 ? 0ull : bit64(n) - 1);
  hi = n >= 128 ? ~0ull : (n <= 64 ? 0ull : bit64(n - 64) - 1);
}

// One DPP move of a 32-bit value across the lanes of a wavefront (controls: row_shr:n is
// 0x110 + n, wave_shr:1 is 0x138, row_bcast:15 is 0x142, row_bcast:31 is 0x143); a lane
// without a source, or in a row outside kRowMask, takes `fill`.
template <int kCtrl, int kRowMask = 0xf>
__device__ inline int dpp_mov(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, kCtrl, kRowMask, 0xf, false);
}

// Maximum over the wavefront, the same in every lane: an inclusive max scan (row shifts by 1,
// 2, 4, 8, then lane 15 of a row into the next row and lane 31 into rows 2 and 3) leaves it in
// lane 63, read out as a uniform value.  All in the vector ALU, no LDS round trips.
__device__ inline int wave_max(int v) {
  v = max(v, dpp_mov<0x111>(v, v));
  v = max(v, dpp_mov<0x112>(v, v));
  v = max(v, dpp_mov<0x114>(v, v));
  v = max(v, dpp_mov<0x118>(v, v));
  v = max(v, dpp_mov<0x142, 0xa>(v, v));
  v = max(v, dpp_mov<0x143, 0xc>(v, v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ inline uint64_t shfl64(uint64_t v, int src) {
  const int lo = __shfl((int)(uint32_t)v, src, 64);
  const int hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Orders the LDS accesses of one wavefront around it: a wavefront's LDS operations complete in
// issue order, so after this its lanes see each other's earlier writes.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Lane src's value of v in every lane; src must be the same in all lanes.
__device__ inline uint64_t readlane64(uint64_t v, int src) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Acceptance walk of sequence b by the calling wavefront (all 64 lanes, lane = threadIdx % 64):
// ok[c] = (c is the root) or draft[c] == target[parent(c)], with parent(c) the highest set bit
// of anc[c] below c.  A node is accepted iff its whole mask lies inside the ok ballot.  The
// deepest accepted node wins (popcount of its mask), ties to the smaller index.  Writes
// accept_path / accept_len / bonus_tok of b; if s_path is not null the path (root first) also
// goes there.  Returns accept_len.
//
// All global loads (mask rows, draft and target tokens of the lane's two nodes) are issued
// together; the parent's target token then comes from another lane by a shuffle and the winner's
// mask row by lane reads, so the walk makes one round trip to memory before its writes.
__device__ inline int accept_walk(int b, int T, int W, const uint64_t* __restrict__ anc,
                                  const int32_t* __restrict__ draft,
                                  const int32_t* __restrict__ target,
                                  int32_t* __restrict__ accept_path,
                                  int32_t* __restrict__ accept_len,
                                  int32_t* __restrict__ bonus_tok, int* s_path) {
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)b * T;
  uint64_t in_lo, in_hi;  // bits of real nodes: garbage above T is ignored
  low_bits(T, in_lo, in_hi);

  uint64_t a0[2], a1[2];
  int dr[2], tg[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    a0[k] = a1[k] = 0;
    dr[k] = tg[k] = 0;
    if (c < T) {
      const uint64_t* row = anc + (base + c) * W;
      a0[k] = row[0] & in_lo;
      a1[k] = (W == 2 ? row[1] : 0) & in_hi;
      dr[k] = draft[base + c];
      tg[k] = target[base + c];
    }
  }
  bool ok[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    uint64_t blo, bhi;  // strictly below c
    low_bits(c, blo, bhi);
    const uint64_t m0 = a0[k] & blo, m1 = a1[k] & bhi;
    const int p = m1 ? 64 + 63 - __clzll(m1) : (m0 ? 63 - __clzll(m0) : -1);
    // target token of node p, held by lane p % 64 in slot p / 64 (every lane takes part)
    const int pp = max(p, 0);
    const int t0 = __shfl(tg[0], pp & 63, 64), t1 = __shfl(tg[1], pp & 63, 64);
    const int tp = pp >= 64 ? t1 : t0;
    ok[k] = c < T && ((c == 0) || (p >= 0 && dr[k] == tp));
  }
  const uint64_t ok_lo = __ballot(ok[0]);
  const uint64_t ok_hi = __ballot(ok[1]);

  int key = -1;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < T && (a0[k] & ~ok_lo) == 0 && (a1[k] & ~ok_hi) == 0) {
      const int depth = __popcll(a0[k]) + __popcll(a1[k]);
      key = max(key, (depth << 8) | (255 - c));
    }
  }
  key = wave_max(key);
  const int best = key >= 0 ? 255 - (key & 255) : 0;

  // the winner's mask row and target token, from lane best % 64, slot best / 64
  const int src = best & 63;
  const bool hi_slot = best >= 64;
  const uint64_t b0 = readlane64(hi_slot ? a0[1] : a0[0], src);
  const uint64_t b1 = readlane64(hi_slot ? a1[1] : a1[0], src);
  const int bonus = __builtin_amdgcn_readlane(hi_slot ? tg[1] : tg[0], src);
  const int n = __popcll(b0) + __popcll(b1);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < T) {
      const bool on_path = k == 0 ? ((b0 >> c) & 1) : ((b1 >> (c - 64)) & 1);
      if (on_path) {
        uint64_t blo, bhi;
        low_bits(c, blo, bhi);
        const int pos = __popcll(b0 & blo) + __popcll(b1 & bhi);
        accept_path[base + pos] = c;
        if (s_path) s_path[pos] = c;
      }
      if (c >= n) accept_path[base + c] = -1;
    }
  }
  if (lane == 0) {
    accept_len[b] = n;
    bonus_tok[b] = bonus;
  }
  return n;
}

// Pointer-swap commit of sequence b ("EAGLE-2 vs. Medusa" section 8, pages of one token) by the
// calling wavefront (all 64 lanes): block_table[b][L + i] = tree_slot[b][path[i]] for i < n, and
// the slots of the nodes not on the path go back to the free list, reserved with one atomic add
// on free_top and written in node order.  Nothing is copied.  pe[k] is path entry lane + 64k
// (only entries below n are used), L the sequence's length before the step.  A bad length, path
// or tree slot, or a table too short for L + n, commits and frees nothing, keeps the length and
// OR-s the reason into status[b] (if status is not null).  Rejected slots that find no room in
// the free list (past num_slots) are not written, and TV_FREE_FULL is OR-ed in.  s_on is LDS
// scratch of kMaxT ints used by this wavefront alone.
__device__ inline void commit_paged_wave(int b, int L, int n, const int pe[2],
                                         int32_t* __restrict__ table, int max_pages,
                                         const int32_t* __restrict__ tree_slot, int T,
                                         int num_slots, int32_t* __restrict__ free_slots,
                                         int32_t* __restrict__ free_top, int32_t* status,
                                         int32_t* cache_len_out, int* s_on) {
  const int lane = threadIdx.x & 63;
  int ts[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    ts[k] = c < T ? tree_slot[(size_t)b * T + c] : 0;
    if (c < kMaxT) s_on[c] = 0;
  }
  wave_lds_sync();
  int bits = 0;
  if (L < 0 || L > max_pages) bits |= TV_BAD_LEN;
  bool bad = n < 0 || n > T;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < T && (ts[k] < 0 || ts[k] >= num_slots)) bad = true;
    if (!(n < 0 || n > T) && c < n) {
      if (pe[k] < 0 || pe[k] >= T) bad = true;
      else atomicAdd(&s_on[pe[k]], 1);
    }
  }
  wave_lds_sync();
  bool rej[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    const int cnt = c < T ? s_on[c] : 0;
    if (cnt > 1) bad = true;  // a node twice on the path
    rej[k] = c < T && cnt == 0;
  }
  if (__ballot(bad)) bits |= TV_BAD_PATH;
  if (!bits && (long long)L + n > max_pages) bits |= TV_OVERFLOW;
  if (bits) {
    if (lane == 0) {
      if (status) atomicOr(status + b, bits);
      cache_len_out[b] = L;
    }
    return;
  }
  // the table takes the accepted nodes' slots, in path order (slot of node p from its lane)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = lane + 64 * k;
    const int p = max(pe[k], 0);
    const int t0 = __shfl(ts[0], p & 63, 64), t1 = __shfl(ts[1], p & 63, 64);
    if (i < n) table[(size_t)b * max_pages + L + i] = p >= 64 ? t1 : t0;
  }
  // the rejected nodes' slots return to the free list
  const uint64_t m0 = __ballot(rej[0]), m1 = __ballot(rej[1]);
  const int cnt = __popcll(m0) + __popcll(m1);
  int at = 0;
  if (lane == 0 && cnt) at = atomicAdd(free_top, cnt);
  at = __builtin_amdgcn_readfirstlane(at);
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (!rej[k]) continue;
    const int r = k == 0 ? __popcll(m0 & below) : __popcll(m0) + __popcll(m1 & below);
    if (at + r < num_slots) free_slots[at + r] = ts[k];
  }
  // slots that found no room in the free list are lost to it: report that
  if (lane == 0 && status && cnt && (long long)at + cnt > num_slots)
    atomicOr(status + b, TV_FREE_FULL);
  // release: a workgroup that reads the new length (cache_len_out may be cache_len) with an
  // acquire also sees the table entries written above
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (lane == 0) __hip_atomic_store(cache_len_out + b, L + n, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace tv
