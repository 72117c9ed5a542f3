// tree_verify_attn: tree attention of a flattened draft tree over its sequence's KV prefix.
//
// Work decomposition (one KV head at a time, GQA-grouped):
//   * The G*T query rows of one (sequence b, KV head) are ordered r = t*G + g (node t, query
//     head kvh*G + g).  A workgroup owns 256 of them: 8 wavefronts x 32 rows, two wavefronts per
//     SIMD, so one wavefront's softmax overlaps the other's matrix instructions.  Every prefix
//     key is visible to every row, so a K/V tile staged in LDS serves all 256 rows.
//   * K/V tiles of 64 keys move HBM -> LDS by direct-to-LDS loads (global_load_lds_dwordx4)
//     through a ring of four LDS stages; no registers hold staged data.  Each wavefront waits
//     only for its own loads of the tile it needs, then one barrier per tile publishes the tile
//     and frees a stage for the next load.
//   * A sequence's keys form 64-key tiles: its tree tiles (masked per row by the ancestor
//     bitmask), then its prefix tiles.  They are cut into equal chunks of `chunk_tiles` tiles
//     (split-K), each processed by its own workgroup.  Partial results (unnormalised O, running
//     max m, sum l) are merged by attn_combine; a sequence with a single chunk is written
//     directly.
//   * A tile is two 32-key blocks.  Per block: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from
//     LDS as the A operand, Q held in registers as the B operand), masking, online softmax in
//     the log2 domain, then O^T += V^T P^T (V^T fragments from LDS with the gfx950 transpose
//     read, P taken straight from the S^T accumulators).  In this transposed form a lane holds
//     one query row in both the score and the output accumulators, so the softmax statistics
//     never leave the lane pair (l, l^32).
//   * The blocks run as a two-deep software pipeline: while the softmax of block j runs on the
//     vector ALU, the matrix core computes S of block j+1 and O of block j-1, within one
//     wavefront and across the two wavefronts of each SIMD.  The pipeline runs across tile
//     barriers, so the tile of block j-1 is still read after the barrier of the next tile.
//   * LDS rows are unpadded; 16-byte chunks are XOR-swizzled by row so the K reads (16 keys x
//     one chunk), the transposed V reads (4 keys x 4 chunks per 16 lanes) and the 1 KB
//     direct-load writes are all free of bank conflicts.
//   * Online softmax with lazy rescaling: p = 2^(S c - m) against the running max m, accepted
//     as long as no lane's block sum exceeds 1024; only then is the block max taken, m raised
//     and O rescaled.
//   * fp32 inputs use v_mfma_f32_32x32x2_f32 and run the blocks one after the other.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "tree_device.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup
constexpr int kKT = 64;             // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSumLimit = 1024.f;  // a lane's block sum above this forces a rescale

struct AttnArgs {
  const char* q;
  const char* kc;
  const char* vc;
  const int32_t* cache_len;
  const char* kt;
  const char* vt;
  const uint64_t* anc;      // ancestor masks, or (masks built in the kernel) their output
  const int32_t* parent;    // parent array when the kernel builds the masks itself
  char* out;
  float* lse;
  int32_t* status;
  char* part_o;    // [slot][kRows*D] elements of the input type, in register order
  float* part_ml;  // [slot][kRows][2]: running max m and sum l per row
  int32_t* nsplit; // [B] non-empty chunks of each sequence, for the merge
  // paged K/V: kc / vc are pools [num_slots, Hkv, D]; position p of sequence b lives in slot
  // table[b][p >> log2P] * P + (p & (P-1)), tree node j in slot tree_slot[b][j]
  const int32_t* table;
  const int32_t* tree_slot;
  int max_pages, log2P, num_slots;
  int B, T, Hq, Hkv, G, Lmax, W, GT, RB, S, chunk_tiles;
  int lpt;         // dispatch the (sequence, chunk) pairs longest first (see lpt_item)
  float c;         // scale * log2(e)
};

template <typename E, int D>
struct Layout {
  static constexpr bool kBF16 = std::is_same<E, __bf16>::value;
  static constexpr int kElem = sizeof(E);
  static constexpr int kRowBytes = D * kElem;          // 128, 256 or 512
  static constexpr int kCPR = kRowBytes / 16;          // 16-byte chunks per row
  static constexpr int kTile = kKT * kRowBytes;        // bytes of one K (or V) tile
  static constexpr int kStage = 2 * kTile;             // one K tile and one V tile
  static constexpr int kStages = kStage <= 32768 ? 4 : 2;
  // K stage s at s * kTile, V stage s at kVBase + s * kTile: every K stage lies within the first
  // 64 KB and every V stage within 64 KB of kVBase, so (bf16) a fragment read takes its stage as
  // an immediate offset from one fixed per-lane address
  static constexpr int kVBase = kStages * kTile;
  // bf16 pipelines blocks across tile barriers: four stages hold the tile read for S, the tile
  // read for O and two in flight.  fp32 (the small exact path) runs its blocks one after the
  // other, with every stage but the current one in flight.
  static constexpr bool kCrossTile = kBF16;
  static constexpr int kAhead = kCrossTile ? kStages - 2 : kStages - 1;
  static constexpr int kRowsPerDma = 1024 / kRowBytes; // rows one wavefront-wide load fills
  static constexpr int kDmaPerWave = kTile / 1024 / kWaves;  // per K (or V) tile
  static constexpr int kDB = D / 32;                   // 32-wide d blocks
  static constexpr int kKS = kBF16 ? D / 16 : D / 2;   // MFMA k-steps over D

  // XOR applied to the chunk index of tile row `row` (depends on row mod 16 only).
  __device__ static inline int swz(int row) {
    return kCPR == 8 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3))
                     : (((row & 3) << 2) | ((row >> 2) & 3));
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane l ^ 32 (hi: the calling lane is one of lanes 32..63).
__device__ inline float partner(float x, int hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(hi ? r[0] : r[1]);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Streaming stores for the split-K partials.  They are read once, by the merge in the next
// launch; written through instead of left dirty in the XCD's L2, they reach memory during the
// epilogue rather than in the write-back at the kernel's end (1 us of the 15 us main kernel at
// batch 1, where 11 MB of partials are written in the last microsecond).
__device__ inline void store_stream(uint2* p, uint2 v) {
  __builtin_nontemporal_store((unsigned long long)v.x | ((unsigned long long)v.y << 32),
                              reinterpret_cast<unsigned long long*>(p));
}
__device__ inline void store_stream(float2* p, float2 v) {
  store_stream(reinterpret_cast<uint2*>(p), uint2{__float_as_uint(v.x), __float_as_uint(v.y)});
}
__device__ inline void store_stream(float4* p, float4 v) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4v*>(p));
}

// One wavefront-wide direct-to-LDS load: lane l's 16 bytes at sbase + voff land at LDS address
// lds + 16*l.  Issued from inline assembly so that the compiler does not order LDS reads behind
// every in-flight tile; the kernel waits for these loads itself (vm_wait) before its barriers.
// M0 carries the LDS address and is restored afterwards.
__device__ inline void lds_dma16(uint32_t lds, const void* sbase, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(sbase)
      : "memory");
}

// The same load from a 64-bit address in a VGPR pair (paged K/V: rows anywhere in a pool).
__device__ inline void lds_dma16_addr(uint32_t lds, const void* addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(addr)
      : "memory");
}

// One wavefront-wide 4-byte direct-to-LDS load: lane l's dword at `addr` lands at lds + 4*l.
__device__ inline void lds_dma4_addr(uint32_t lds, const void* addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(addr)
      : "memory");
}

// s_waitcnt vmcnt(n) (n <= 63), other counters untouched.
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Logical work item -> hardware workgroup id.  Workgroups are dealt to the 8 XCDs round-robin;
// this gives every XCD a contiguous range of logical items, so items that read the same K/V
// chunk (consecutive row blocks) or the same Q rows (consecutive splits) share an L2.
__device__ inline int xcd_remap(int bid, int n) {
  const int per = n / 8, rem = n % 8;
  const int xcd = bid % 8, slot = bid / 8;
  return xcd * per + min(xcd, rem) + slot;
}

// Work order for sequences of different lengths, longest processing time first.  Every
// workgroup ranks the B*S (sequence, chunk) pairs by their tile count, largest first (ties by
// index), from cache_len, in LDS scratch (P <= kLptMaxPairs).  Unit U = rank * Hkv + kvh.
// Hardware ids are dealt to the 8 XCDs in turn and dispatched in order, so units go out in
// groups of 8, one per XCD, and the RB row blocks of a unit (which read the same K/V tiles)
// follow each other on the same XCD: every XCD gets a longest-first share of the work.
constexpr int kLptMaxPairs = 256;

__device__ inline void lpt_item(const AttnArgs& a, int* lds, int& b, int& s, int& kvh,
                                int& rb, int& L_raw) {
  const int P = a.B * a.S;
  const int P4 = (P + 3) & ~3;
  const int tid = threadIdx.x;
  const int tree_tiles = ceil_div(a.T, kKT);
  int* sz = lds;        // [P4] tiles of each pair; padding -1 ranks after every pair
  int* ord = lds + P4;  // [P] pair of each rank
  int* len = ord + P;   // [P] cache_len of each pair's sequence, as given
  for (int i = tid; i < P4; i += kThreads) {
    int v = -1;
    if (i < P) {
      const int bi = i / a.S, si = i - bi * a.S;
      const int Lr = a.cache_len[bi];
      const int L = min(max(Lr, 0), a.Lmax);
      v = min(max(tree_tiles + ceil_div(L, kKT) - si * a.chunk_tiles, 0), a.chunk_tiles);
      len[i] = Lr;
    }
    sz[i] = v;
  }
  __syncthreads();
  // The rank of pair i counts the pairs ahead of it.  tpp consecutive lanes (a power of two, at
  // most a wavefront) share a pair: each counts every tpp-th int4 of sz, and the counts meet by
  // butterfly shuffles, so all wavefronts rank and each lane waits on few LDS reads.
  {
    const int lg = P > 1 ? 32 - __clz(P - 1) : 0;  // ceil(log2 P); P <= kLptMaxPairs
    const int lt = min(6, __builtin_ctz(kThreads) - lg);
    const int tpp = 1 << lt;
    const int i = tid >> lt, j = tid & (tpp - 1);
    const int4* s4 = reinterpret_cast<const int4*>(sz);
    int r = 0;
    if (i < P) {
      const int me = sz[i];
#pragma unroll 4
      for (int q = j; q < P4 >> 2; q += tpp) {
        const int4 o = s4[q];
        const int c = 4 * q;
        r += (o.x > me || (o.x == me && c < i)) + (o.y > me || (o.y == me && c + 1 < i)) +
             (o.z > me || (o.z == me && c + 2 < i)) + (o.w > me || (o.w == me && c + 3 < i));
      }
    }
    for (int off = tpp >> 1; off > 0; off >>= 1) r += __shfl_xor(r, off, 64);
    if (i < P && j == 0) ord[r] = i;
  }
  __syncthreads();
  const int n_units = P * a.Hkv;
  const int per = 8 * a.RB;
  const int h = blockIdx.x, g = h / per, w = h - g * per;
  const int m = min(8, n_units - g * 8);  // units in this group (fewer in the last one)
  const int U = g * 8 + w % m;
  rb = w / m;
  kvh = U % a.Hkv;
  const int pair = ord[U / a.Hkv];
  b = pair / a.S;
  s = pair - b * a.S;
  L_raw = len[pair];  // (no second global read of cache_len[b])
  __syncthreads();  // this LDS is the K/V ring, which the first tile loads overwrite
}

// Score block j = 32 keys: tile j/2, half j%2.  P of a block: bf16 operands or fp32 values.
template <bool kBF16>
struct PBlock;
template <>
struct PBlock<true> {
  bf16x8 v[2];  // 16-key steps st = 0, 1
};
template <>
struct PBlock<false> {
  float v[16];  // element e of the S^T accumulator
};

// Ancestor masks of sequence b built by wavefront 0 from the parent array, by pointer jumping
// through LDS: node c = lane + 64*k lives in lane c % 64, slot k.  Each node keeps the set of
// its ancestors closer than 2^r and a pointer to the ancestor at distance 2^r; one round reads
// the pointed-to node's set and pointer, then merges the set and takes over the pointer.  A
// round's reads all come before its writes (the wavefront's LDS instructions execute in order;
// compiler barriers keep them in place), and its writes have completed (lgkmcnt) before the next
// round reads.  Rounds stop once no pointer is left (after ceil(log2(depth + 1)) rounds).  A
// tree that is not level-ordered with one root gets only each node's own bit (as
// tree_build_mask).  par[k] is parent[b, lane + 64*k].  Writes the masks to s_anc (and to
// anc_out when not null); s_ptr is LDS for T pointers.  Returns whether the tree was bad.
__device__ inline bool build_masks_wave(const int (&par)[2], int b, int T,
                                        uint64_t (*s_anc)[2], int* s_ptr, uint64_t* anc_out) {
  const int lane = threadIdx.x & 63;
  const int W = T > 64 ? 2 : 1;
  uint64_t lo[2], hi[2];
  int ptr[2];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    lo[k] = hi[k] = 0;
    ptr[k] = -1;
    if (c < T) {
      const int p = par[k];
      const bool ok = c == 0 ? p == -1 : (p >= 0 && p < c);
      bad |= !ok;
      ptr[k] = (c > 0 && ok) ? p : -1;
      lo[k] = k == 0 ? bit64(c) : 0;
      hi[k] = k == 1 ? bit64(c) : 0;
      s_anc[c][0] = lo[k];
      s_anc[c][1] = hi[k];
      s_ptr[c] = ptr[k];
    }
  }
  bad = __ballot(bad) != 0;
  // a pointer's distance doubles every round, so ceil(log2 T) rounds reach past every root
  for (int span = 1; span < T && __ballot(ptr[0] >= 0 || ptr[1] >= 0); span <<= 1) {
    uint64_t plo[2], phi[2];
    int pp[2];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the previous round's writes are done
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int src = max(ptr[k], 0);  // lanes without a pointer read node 0 and drop it
      plo[k] = s_anc[src][0];
      phi[k] = s_anc[src][1];
      pp[k] = s_ptr[src];
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = lane + 64 * k;
      if (ptr[k] >= 0) {  // (only nodes c < T have one)
        lo[k] |= plo[k];
        hi[k] |= phi[k];
        ptr[k] = pp[k];
        s_anc[c][0] = lo[k];
        s_anc[c][1] = hi[k];
        s_ptr[c] = ptr[k];
      }
    }
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < T) {
      if (bad) {
        lo[k] = k == 0 ? bit64(c) : 0;
        hi[k] = k == 1 ? bit64(c) : 0;
        s_anc[c][0] = lo[k];
        s_anc[c][1] = hi[k];
      }
      if (anc_out) {
        uint64_t* row = anc_out + ((size_t)b * T + c) * W;
        row[0] = lo[k];
        if (W == 2) row[1] = hi[k];
      }
    }
  }
  return bad;
}

// kPaged: 0 dense caches; 1 paged, rows addressed by 64-bit pointers; 2 paged, by 32-bit offsets
// from the pool's base (pools under 4 GB: no 64-bit address arithmetic per load)
template <typename E, int D, bool kSplit, bool kMasks, int kPaged>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void attn_main(AttnArgs a) {
  using Lay = Layout<E, D>;
  constexpr bool kBF16 = Lay::kBF16;
  constexpr int kDB = Lay::kDB;
  constexpr int kKS = Lay::kKS;
  constexpr int kRB = Lay::kRowBytes;
  constexpr int kNS = Lay::kStages;
  constexpr int kDPW = Lay::kDmaPerWave;
  __shared__ __attribute__((aligned(1024))) char smem[kNS * Lay::kStage];

  int rb, s, kvh, b, L_lpt = 0;
  if (a.lpt) {
    lpt_item(a, reinterpret_cast<int*>(smem), b, s, kvh, rb, L_lpt);
  } else {
    const int n_items = a.B * a.Hkv * a.S * a.RB;
    const int item = xcd_remap(blockIdx.x, n_items);
    rb = item % a.RB;
    s = (item / a.RB) % a.S;
    kvh = (item / (a.RB * a.S)) % a.Hkv;
    b = item / (a.RB * a.S * a.Hkv);
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  const int L_raw = a.lpt ? L_lpt : a.cache_len[b];
  const int L = min(max(L_raw, 0), a.Lmax);
  // one workgroup per sequence reports its status (and, building masks, writes them)
  const bool writer = kvh == 0 && s == 0 && rb == 0;
  if (!kMasks && a.status && (L_raw < 0 || L_raw > a.Lmax) && writer && tid == 0)
    atomicOr(a.status + b, TV_BAD_LEN);
  // Chunks are cut from the sequence's tiles in the order tree tiles, then prefix tiles, so
  // the chunk that carries the tree does no more work than the others.
  const int tree_tiles = ceil_div(a.T, kKT);
  const int all_tiles = tree_tiles + ceil_div(L, kKT);
  const int n_split = ceil_div(all_tiles, a.chunk_tiles);
  if (kSplit && kvh == 0 && s == 0 && rb == 0 && tid == 0) a.nsplit[b] = n_split;
  if (s >= n_split) return;  // empty chunk: nothing to merge
  const bool direct = !kSplit || n_split == 1;

  const int v0 = s * a.chunk_tiles, v1 = min(v0 + a.chunk_tiles, all_tiles);
  const int n_tree_tiles = max(0, min(v1, tree_tiles) - v0);
  const int k0 = max(v0 - tree_tiles, 0) * kKT;
  const int k1 = min(max(v1 - tree_tiles, 0) * kKT, L);
  const int n_prefix_tiles = k1 > k0 ? ceil_div(k1 - k0, kKT) : 0;
  const int n_tiles = n_tree_tiles + n_prefix_tiles;  // >= 1 for every non-empty chunk
  const int mask_from = n_prefix_tiles > 0 && (k1 - k0) % kKT != 0 ? n_tiles - 1 : n_tiles;

  // ---- the lane's query row: r = rb*256 + wave*32 + n -------------------------------------
  const int r = rb * kRows + wave * 32 + n;
  const bool row_ok = r < a.GT;
  const int row_t = row_ok ? r / a.G : 0;  // padding rows load a real row; never written
  const int row_head = kvh * a.G + (row_ok ? r % a.G : 0);

  // ---- direct-to-LDS tile loads ------------------------------------------------------------
  // Wavefront w fills K rows [w*kDPW*kRowsPerDma, ...) of a tile, and the same V rows; lane l
  // writes chunk slot l % kCPR of row l / kCPR, which holds logical chunk slot ^ swz(row).
  const char* kc_head = a.kc + (((size_t)b * a.Hkv + kvh) * a.Lmax) * kRB;
  const char* vc_head = a.vc + (((size_t)b * a.Hkv + kvh) * a.Lmax) * kRB;
  const char* kt_head = a.kt + ((size_t)b * a.T * a.Hkv + kvh) * kRB;
  const char* vt_head = a.vt + ((size_t)b * a.T * a.Hkv + kvh) * kRB;
  const uint32_t tree_stride = (uint32_t)a.Hkv * kRB;
  int dma_row[kDPW];
  uint32_t dma_chunk[kDPW];
#pragma unroll
  for (int i = 0; i < kDPW; ++i) {
    dma_row[i] = (wave * kDPW + i) * Lay::kRowsPerDma + lane / Lay::kCPR;
    dma_chunk[i] = (uint32_t)(((lane % Lay::kCPR) ^ Lay::swz(dma_row[i])) << 4);
  }
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  // Paged K/V: the rows of one direct-load instruction are kRowsPerDma consecutive keys, one
  // per group of kCPR lanes.  Each lane's table entry (the page of its prefix key, or the slot
  // of its tree node) is itself brought in by a 4-byte direct-to-LDS load into a small per-
  // wavefront area, ahead of the tile: the entry loads join the tile loads in the one in-order
  // vmcnt stream, so the waits below stay exact and no scalar load shares lgkmcnt with the LDS
  // fragment reads.  At issue each lane reads its entry back and forms the slot.  Entries
  // outside the pool are clamped into it and reported.
  __shared__ __attribute__((aligned(256))) int32_t s_ent[kPaged ? 2 * kWaves * kDPW * 64 : 1];
  bool bad_slot = false;
  // key position (prefix tiles) or node (tree tiles) of this lane's row in instruction i
  auto row_key = [&](int tile, int i) __attribute__((always_inline)) -> int {
    const int r = (wave * kDPW + i) * Lay::kRowsPerDma + lane / Lay::kCPR;
    return tile < n_tree_tiles ? min((v0 + tile) * kKT + r, a.T - 1)
                               : min(k0 + (tile - n_tree_tiles) * kKT + r, k1 - 1);
  };
  auto ent_lds = [&](int tile, int i) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(uintptr_t)s_ent + ((((tile & 1) * kWaves + wave) * kDPW + i) * 64) * 4;
  };
  auto load_entries = [&](int tile) __attribute__((always_inline)) {  // kDPW loads
    if constexpr (kPaged) {
#pragma unroll
      for (int i = 0; i < kDPW; ++i) {
        const int key = row_key(tile, i);
        const int32_t* src = tile < n_tree_tiles
                                 ? a.tree_slot + (size_t)b * a.T + key
                                 : a.table + (size_t)b * a.max_pages + (key >> a.log2P);
        lds_dma4_addr(ent_lds(tile, i), src);
      }
    }
  };
  // the tile's entries have landed (the caller waited for them)
  auto issue_tile_paged = [&](int tile, uint32_t kl, uint32_t vl) __attribute__((always_inline)) {
    const size_t hstride = (size_t)a.Hkv * kRB;  // bytes per pool slot
    const char* kpool = a.kc + (size_t)kvh * kRB;
    const char* vpool = a.vc + (size_t)kvh * kRB;
    const int pmask = (1 << a.log2P) - 1;
#pragma unroll
    for (int i = 0; i < kDPW; ++i) {
      const int e = *(const int32_t*)((const char*)s_ent + (ent_lds(tile, i) -
                                                            (uint32_t)(uintptr_t)s_ent) + 4 * lane);
      const long long slot =
          tile < n_tree_tiles
              ? (long long)e
              : (e < 0 ? -1LL : ((long long)e << a.log2P) + (row_key(tile, i) & pmask));
      const bool out = slot < 0 || slot >= a.num_slots;
      bad_slot = bad_slot || out;
      const int mine = out ? (slot < 0 ? 0 : a.num_slots - 1) : (int)slot;
      if constexpr (kPaged == 2) {
        const uint32_t off = (uint32_t)mine * (uint32_t)hstride + dma_chunk[i];
        lds_dma16(kl + i * 1024, kpool, off);
        lds_dma16(vl + i * 1024, vpool, off);
      } else {
        const size_t off = (size_t)mine * hstride + dma_chunk[i];
        lds_dma16_addr(kl + i * 1024, kpool + off);
        lds_dma16_addr(vl + i * 1024, vpool + off);
      }
    }
  };

  // `part`: 1 the K rows, 2 the V rows, 3 both.  The dense bf16 pipeline issues a tile's K rows
  // at one tile barrier and its V rows half a tile later, so each wavefront's tile loads leave
  // in two groups.
  constexpr bool kSplitIssue = !kPaged && Lay::kCrossTile;
  auto issue_tile = [&](int tile, int stage, int part) __attribute__((always_inline)) {
    const uint32_t kl = smem_base + stage * Lay::kTile + wave * kDPW * 1024;
    const uint32_t vl = kl + Lay::kVBase;
    if constexpr (kPaged) {
      if constexpr (!Lay::kCrossTile) {
        // fp32 (the small exact path): entries fetched at issue, waiting for everything
        load_entries(tile);
        vm_wait<0>();
      }
      issue_tile_paged(tile, kl, vl);
      return;
    }
    if (tile < n_tree_tiles) {
      const int base = (v0 + tile) * kKT;
#pragma unroll
      for (int i = 0; i < kDPW; ++i) {
        // keys past the tree load the last node's row: masked to -inf, they add exactly 0
        const uint32_t off = (uint32_t)min(base + dma_row[i], a.T - 1) * tree_stride + dma_chunk[i];
        if (part & 1) lds_dma16(kl + i * 1024, kt_head, off);
        if (part & 2) lds_dma16(vl + i * 1024, vt_head, off);
      }
    } else {
      const int base = k0 + (tile - n_tree_tiles) * kKT;
#pragma unroll
      for (int i = 0; i < kDPW; ++i) {
        // keys past the chunk load its last row (never a row at or past cache_len)
        const uint32_t off = (uint32_t)min(base + dma_row[i], k1 - 1) * kRB + dma_chunk[i];
        if (part & 1) lds_dma16(kl + i * 1024, kc_head, off);
        if (part & 2) lds_dma16(vl + i * 1024, vc_head, off);
      }
    }
  };

  // The first tiles go out before the Q loads so the two latencies overlap; they are complete
  // before the block pipeline starts (vm_wait<0> below), so no compiler-tracked load is pending
  // inside it and its own waits count tile loads only.
  if constexpr (kPaged && Lay::kCrossTile) {
    // entries of tiles 0 and 1, then their data; the entries of tile 2 follow (the pipeline
    // below keeps the entries of tile t+2 ahead of the data of tile t+1)
    load_entries(0);
    if (n_tiles > 1) load_entries(1);
    vm_wait<0>();
  }
#pragma unroll
  for (int t = 0; t < Lay::kAhead; ++t)
    if (t < n_tiles) issue_tile(t, t, 3);
  if constexpr (kPaged && Lay::kCrossTile) {
    if (n_tiles > 2) load_entries(2);
  }

  // ---- Q fragments (B operand): row n, d = 16*ks + 8*h .. +7 (bf16) or 2*ks + h (fp32) -----
  using QFrag = typename std::conditional<kBF16, bf16x8, float>::type;
  QFrag qf[kKS];
  {
    const E* qrow = reinterpret_cast<const E*>(a.q) +
                    (((size_t)b * a.T + row_t) * a.Hq + row_head) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if constexpr (kBF16) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + 8 * h);
      } else {
        qf[ks] = qrow[ks * 2 + h];
      }
    }
  }
  // ancestor mask words of the lane's row (padding rows see only the root)
  uint64_t mk0 = 1, mk1 = 0;
  if (!kMasks && row_ok && n_tree_tiles) {
    const uint64_t* mrow = a.anc + ((size_t)b * a.T + row_t) * a.W;
    mk0 = mrow[0];
    mk1 = a.W > 1 ? mrow[1] : 0;
  }
  // Masks built here: wavefront 0 of every workgroup that reads tree keys, and of the
  // sequence's writer, runs the pointer jumping once its tile loads have landed; the other
  // wavefronts read their rows' masks after the first tile barrier.
  __shared__ __attribute__((aligned(16))) uint64_t s_anc[kMasks ? kMaxT : 1][2];
  __shared__ int s_ptr[kMasks ? kMaxT : 1];
  const bool need_masks = kMasks && (n_tree_tiles > 0 || writer);
  int par[2] = {-1, -1};
  if (need_masks && wave == 0) {
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (lane + 64 * k < a.T) par[k] = a.parent[(size_t)b * a.T + lane + 64 * k];
  }

  // ---- per-lane LDS fragment offsets (bytes within a K or V tile) --------------------------
  uint32_t koff[kBF16 ? kKS : 1];
  uint32_t voff[kBF16 ? 2 * kDB : 1];
  if constexpr (kBF16) {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      koff[ks] = n * kRB + ((((2 * ks + h) ^ Lay::swz(n))) << 4);
    const int tr_key = 4 * h + ((lane & 15) >> 2);             // key within an 8-key half
    const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // d within a 32-wide block
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int row = 8 * sec + tr_key;
        // V tiles sit at kVBase and above: the base is held here, so the stage and block
        // offsets (under 64 KB) fit the reads' immediate field
        voff[sec * kDB + db] = Lay::kVBase + row * kRB +
                               (((4 * db + (tr_d >> 3)) ^ Lay::swz(row)) << 4) + (tr_d & 7) * 2;
        asm volatile("" : "+v"(voff[sec * kDB + db]));
      }
  }

  vm_wait<0>();
  if constexpr (kMasks) {
    if (need_masks && wave == 0) {
      const bool bad = build_masks_wave(par, b, a.T, s_anc, s_ptr,
                                        writer ? const_cast<uint64_t*>(a.anc) : nullptr);
      if (writer && lane == 0 && a.status)
        a.status[b] = (bad ? TV_BAD_TREE : 0) | ((L_raw < 0 || L_raw > a.Lmax) ? TV_BAD_LEN : 0);
    }
  }

  // ---- accumulators and running statistics -------------------------------------------------
  f32x16 oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max of S*c (log2 domain) over the row
  float l_run = 0.f;        // the lane's part of the row sum of 2^(S*c - m_run)
  float alpha = 1.f;        // O rescale factor decided by the latest softmax
  bool rescale_o = false;

  // Barrier of tile t: every wavefront's loads of tile t have landed, and every wavefront is
  // done with the tile whose stage tile t + kAhead takes (across tiles, tile t-2, whose last
  // reader is the O^T step of block 2t-3; one block after another, tile t-1), so that tile is
  // loaded now.
  auto barrier_tile = [&](int t, int next_stage) __attribute__((always_inline)) {
    if constexpr (kPaged && Lay::kCrossTile) {
      // Issue order per barrier t: entries of tile t+3, then data of tile t+2.  Loads newer
      // than tile t's data: entries of t+2 and data of t+1 (issued at barrier t-1).
      constexpr int En = kDPW, Dd = 2 * kDPW;
      if (t + 2 < n_tiles) vm_wait<En + Dd>();
      else if (t + 1 < n_tiles) vm_wait<Dd>();
      else vm_wait<0>();
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 3 < n_tiles) load_entries(t + 3);
      if (t + 2 < n_tiles) {
        // entries of t+2 have landed once only data of t+1 and entries of t+3 may remain
        if (t + 3 < n_tiles) vm_wait<Dd + En>();
        else vm_wait<Dd>();
        asm volatile("" ::: "memory");
        issue_tile(t + 2, next_stage, 3);
      }
      return;
    }
    // newer tiles may stay in flight
    if (Lay::kAhead >= 3 && t + 2 < n_tiles) vm_wait<(Lay::kAhead >= 3 ? 4 * kDPW : 0)>();
    else if (Lay::kAhead >= 2 && t + 1 < n_tiles) vm_wait<(Lay::kAhead >= 2 ? 2 * kDPW : 0)>();
    else vm_wait<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): earlier LDS reads are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + Lay::kAhead < n_tiles) issue_tile(t + Lay::kAhead, next_stage, kSplitIssue ? 1 : 3);
  };

  // LDS byte offset of the K (V) tile of ring stage st.  In the bf16 pipeline the stage is a
  // compile-time constant, so the fragment reads below take it as an immediate offset from the
  // fixed per-lane koff / voff.
  auto kbase = [&](int st) __attribute__((always_inline)) -> uint32_t { return st * Lay::kTile; };
  auto vbase = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return Lay::kVBase + st * Lay::kTile;
  };
  // bf16 V reads: voff already holds kVBase
  auto vbase_rel = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return st * Lay::kTile;
  };

  // S^T = K Q^T for block j, its K tile at LDS offset kb0
  auto qk = [&](int j, f32x16& S, uint32_t kb0) __attribute__((always_inline)) {
    const int kb = j & 1;
    S = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if constexpr (kBF16) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(smem + koff[ks] + (kb0 + kb * 32 * kRB));
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S, 0, 0, 0);
      } else {
        const int key = kb * 32 + n;
        const int d = 2 * ks + h;
        const float kf = *reinterpret_cast<const float*>(
            smem + kb0 + key * kRB + ((((d >> 2) ^ Lay::swz(key))) << 4) + (d & 3) * 4);
        S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[ks], S, 0, 0, 0);
      }
    }
  };

  // O^T += V^T P^T for block j, its V tile at LDS offset vb0 (bf16: relative to kVBase, which
  // voff holds; fp32: absolute)
  auto pv = [&](int j, const PBlock<kBF16>& P, uint32_t vb0) __attribute__((always_inline)) {
    const int kb = j & 1;
    if constexpr (kBF16) {
      // 16-key step st: keys kb*32 + 16st + {4h..4h+3} (elements 0-3) and kb*32 + 16st + 8 +
      // {4h..4h+3} (elements 4-7); a transpose read gives lane i of each 16-lane group four
      // consecutive keys at d = D0 + i.
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint32_t vo = vb0 + (kb * 32 + 16 * st) * kRB;  // stage offset of V, relative
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const i16x4 x0 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + voff[db] + vo));
          const i16x4 x1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + voff[kDB + db] + vo));
          const i16x8 v = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v),
                                                            P.v[st], oacc[db], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int d = db * 32 + n;
          const float vf = *reinterpret_cast<const float*>(
              smem + vb0 + key * kRB + ((((d >> 2) ^ Lay::swz(key))) << 4) + (d & 3) * 4);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, P.v[e], oacc[db], 0, 0, 0);
        }
      }
    }
  };

  // Mask block j's scores where needed: tree keys by the row's ancestor bits, keys at or past
  // the end of the tree or of the chunk.  Element e is key kb*32 + 8*(e/4) + 4*h + e%4 of the
  // tile; a tree tile covers nodes 64*tile .. 64*tile+63, so one mask word per row.
  auto mask_block = [&](int j, f32x16& S) __attribute__((always_inline)) {
    const int tile = j >> 1, kb = j & 1;
    if (tile >= n_tree_tiles && tile < mask_from) return;
    const bool is_tree = tile < n_tree_tiles;
    const int base = is_tree ? (v0 + tile) * kKT : k0 + (tile - n_tree_tiles) * kKT;
    const int lim = (is_tree ? a.T : k1) - base - kb * 32;  // keys of this block that exist
    if (!is_tree && lim >= 32) return;
    const uint32_t lenbits = lim >= 32 ? 0xffffffffu : (lim <= 0 ? 0u : (1u << lim) - 1u);
    const uint64_t mw = !is_tree ? ~0ull : (base == 0 ? mk0 : mk1);
    const uint32_t bits = (((uint32_t)(mw >> (32 * kb))) & lenbits) >> (4 * h);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int keep = -(int)((bits >> (8 * (e >> 2) + (e & 3))) & 1u);  // all ones or zero
      S[e] = __int_as_float((__float_as_int(S[e]) & keep) | (__float_as_int(-INFINITY) & ~keep));
    }
  };

  // p = 2^(S*c - m_run), packed as the P operand; returns the lane's sum of the p it packed.
  auto exp_pack = [&](const f32x16& S, float mb, PBlock<kBF16>& P) __attribute__((always_inline)) -> float {
    float sum = 0.f;
    if constexpr (kBF16) {
      // the row sum adds the fp32 values; only the O^T operand is rounded to bf16
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = fast_exp2(__builtin_fmaf(S[e], a.c, -mb));
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[8 * st + 2 * e], p[8 * st + 2 * e + 1]);
        P.v[st] = __builtin_bit_cast(bf16x8, w);
      }
      sum = p[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) sum += p[e];
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        P.v[e] = fast_exp2(__builtin_fmaf(S[e], a.c, -mb));
        sum += P.v[e];
      }
    }
    return sum;
  };

  // Online softmax of one block with lazy rescaling.  The fast path keeps m_run: a lane whose
  // block sum is at most kSumLimit has every p in range (p <= sum), and the block is taken as
  // is.  Otherwise (a score outgrew m_run, or m_run is unset) the wavefront takes the
  // slow path: exact row max over the block, new m_run, alpha = 2^(m_old - m_new), p again.
  // In a pipeline region (sched) the region's instructions are ordered for the scheduler: the
  // eight K-fragment reads first, four S^T MFMAs each followed by two vector instructions, the
  // sixteen V-fragment reads, then the other twelve MFMAs each followed by three (1 % faster on
  // the MFMA-bound workloads than the compiler's own order, which waits on each K read just
  // before its MFMA).
  auto softmax = [&](const f32x16& S, PBlock<kBF16>& P, bool sched = false)
                     __attribute__((always_inline)) {
    float bsum = exp_pack(S, m_run, P);
    if (kBF16 && sched) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads: K fragments
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads: V fragments
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    }
    rescale_o = __ballot(!(bsum <= kSumLimit)) != 0;  // also catches inf and NaN
    if (rescale_o) {
      float mx = S[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[e]);
      mx = fmaxf(mx, partner(mx, h));
      const float m_new = fmaxf(m_run, mx * a.c);
      alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);  // 0 while m_run is unset
      m_run = m_new;
      bsum = exp_pack(S, m_new == -INFINITY ? 0.f : m_new, P);
      l_run = __builtin_fmaf(l_run, alpha, bsum);
    } else {
      l_run += bsum;
    }
  };

  auto rescale = [&]() __attribute__((always_inline)) {
    if (rescale_o) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) oacc[db] *= alpha;
    }
  };

  // Keeps the softmax of a region inside it: without a use here the compiler sinks the
  // exponentials and sums to their next uses, out of reach of the region's matrix work.
  auto end_region = [&](const PBlock<kBF16>& P) __attribute__((always_inline)) {
    if constexpr (kBF16) {
#pragma unroll
      for (int st = 0; st < 2; ++st) asm volatile("" ::"v"(P.v[st]));
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) asm volatile("" ::"v"(P.v[e]));
    }
    asm volatile("" ::"v"(l_run));
  };

  // ---- block pipeline ----------------------------------------------------------------------
  // Region R(j) issues the S^T product of block j+1, the O^T product of block j-1 and the
  // softmax of block j, in one basic block, so that the matrix work of one block and the vector
  // work of another interleave in the wavefront's instruction stream.  Between regions: the
  // mask of block j+1 and the O rescale decided by block j.  Even blocks' S and P live in
  // Se / Pe, odd blocks' in So / Po.
  f32x16 Se, So;
  PBlock<kBF16> Pe, Po;
  auto masks_from_lds = [&]() __attribute__((always_inline)) {
    if constexpr (kMasks) {
      if (row_ok && n_tree_tiles) {
        mk0 = s_anc[row_t][0];
        mk1 = s_anc[row_t][1];
      }
    }
  };
  if constexpr (Lay::kCrossTile) {
    static_assert(kNS == 4, "the bf16 pipeline unrolls its tile loop over four ring stages");
    barrier_tile(0, Lay::kAhead % kNS);
    masks_from_lds();
    qk(0, Se, kbase(0));
    mask_block(0, Se);
    // R(0)
    qk(1, So, kbase(0));
    softmax(Se, Pe);
    end_region(Pe);
    mask_block(1, So);
    rescale();
    if (kSplitIssue && Lay::kAhead < n_tiles)
      issue_tile(Lay::kAhead, Lay::kAhead % kNS, 2);  // V rows of tile 2
    // Tile t (stage t % 4) reads K of tile t and V of tile t - 1.  The stage is a template
    // constant of each unrolled copy, so every fragment address is fixed per lane.
    auto tile_step = [&](int t, auto stage) __attribute__((always_inline)) {
      constexpr int SK = decltype(stage)::value, SV = (SK + kNS - 1) % kNS;
      barrier_tile(t, (SK + Lay::kAhead) % kNS);
      // R(2t-1): S of block 2t, O of block 2t-2, softmax of block 2t-1
      qk(2 * t, Se, kbase(SK));
      pv(2 * t - 2, Pe, vbase_rel(SV));
      softmax(So, Po, true);
      end_region(Po);
      mask_block(2 * t, Se);
      rescale();
      if (kSplitIssue && t + Lay::kAhead < n_tiles)
        issue_tile(t + Lay::kAhead, (SK + Lay::kAhead) % kNS, 2);  // V rows of tile t + 2
      // R(2t): S of block 2t+1, O of block 2t-1, softmax of block 2t
      qk(2 * t + 1, So, kbase(SK));
      pv(2 * t - 1, Po, vbase_rel(SV));
      softmax(Se, Pe, true);
      end_region(Pe);
      mask_block(2 * t + 1, So);
      rescale();
    };
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    using S0 = std::integral_constant<int, 0>;
    for (int t = 1; t < n_tiles; t += 4) {  // t % 4 == 1 at the top of every pass
      tile_step(t, S1{});
      if (t + 1 >= n_tiles) break;
      tile_step(t + 1, S2{});
      if (t + 2 >= n_tiles) break;
      tile_step(t + 2, S3{});
      if (t + 3 >= n_tiles) break;
      tile_step(t + 3, S0{});
    }
    // R(2n-1): O of block 2n-2, softmax of block 2n-1; then O of block 2n-1
    const uint32_t vlast = vbase_rel((n_tiles - 1) % kNS);
    pv(2 * n_tiles - 2, Pe, vlast);
    softmax(So, Po);
    end_region(Po);
    rescale();
    pv(2 * n_tiles - 1, Po, vlast);
  } else {
    for (int t = 0; t < n_tiles; ++t) {
      barrier_tile(t, (t + Lay::kAhead) % kNS);
      if (t == 0) masks_from_lds();
      const uint32_t kb0 = kbase(t % kNS), vb0 = vbase(t % kNS);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        qk(2 * t + kb, Se, kb0);
        mask_block(2 * t + kb, Se);
        softmax(Se, Pe);
        rescale();
        pv(2 * t + kb, Pe, vb0);
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------------------
  // (when the kernel builds the masks, its mask writer stores status[b] with a plain write, so
  // the fused step's second kernel reports bad pages instead)
  if (kPaged && !kMasks && __ballot(bad_slot) && lane == 0 && a.status)
    atomicOr(a.status + b, TV_BAD_PAGE);
  l_run += partner(l_run, h);

  if (direct) {
    if (row_ok) {
      const float inv = 1.f / l_run;
      const size_t orow = ((size_t)b * a.T + row_t) * a.Hq + row_head;
      E* o = reinterpret_cast<E*>(a.out) + orow * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + 8 * j + 4 * h;
          const f32x16& acc = oacc[db];
          if constexpr (kBF16) {
            uint2 w;
            w.x = pack_bf16x2(acc[4 * j] * inv, acc[4 * j + 1] * inv);
            w.y = pack_bf16x2(acc[4 * j + 2] * inv, acc[4 * j + 3] * inv);
            *reinterpret_cast<uint2*>(o + d) = w;
          } else {
            *reinterpret_cast<float4*>(o + d) =
                float4{acc[4 * j] * inv, acc[4 * j + 1] * inv, acc[4 * j + 2] * inv,
                       acc[4 * j + 3] * inv};
          }
        }
      if (a.lse && h == 0) a.lse[orow] = (m_run + __log2f(l_run)) * kLn2;
    }
  } else if (row_ok) {  // padding rows are never merged
    // unnormalised O in fp32 whatever the input type (the fp32 accumulation is never rounded
    // before the merge), four consecutive d per lane and group: group index
    // ((wave*kDB + db)*4 + j)*64 + lane, so a wavefront's store is one 1 KB run
    const size_t slot = (((size_t)b * a.Hkv + kvh) * a.RB + rb) * a.S + s;
    float4* po = reinterpret_cast<float4*>(a.part_o + slot * (size_t)kRows * D * sizeof(float));
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& acc = oacc[db];
        store_stream(&po[(((wave * kDB + db) * 4 + j) << 6) + lane],
                     float4{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]});
      }
    if (h == 0) {
      float2* pml = reinterpret_cast<float2*>(a.part_ml + slot * (size_t)kRows * 2);
      store_stream(&pml[wave * 32 + n], float2{m_run, l_run});
    }
  }
}

// Merge the per-chunk partials of sequences with more than one non-empty chunk:
//   M = max_s m_s,  O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  lse = (M + log2 den) ln 2.
// The unit of work is a piece: 16 bytes of a slot's partial in the partials' register order,
// that is one row and four consecutive d in fp32.  Chunks are taken kBatch at a time, exactly as
// many as the sequence has, with all their loads in flight, and M is raised per batch (online,
// as in the main kernel).
//  * Few chunks (S <= 8): every thread owns kP pieces of one (b, kvh, rb) and merges all its
//    chunks in one batch, the loads of all kP pieces in flight together (kP * kBatch = 8
//    loads of 16 bytes).  Sequences that were not split leave their workgroups with nothing
//    to do but one read of the chunk count, so fewer, fuller workgroups keep the merge from
//    being bound by dispatch and that read's latency (batch 32: 2048 workgroups, not 8192).
//  * More chunks: the four wavefronts of a workgroup own the same 64 pieces and take every
//    fourth chunk each, then combine their (M, den, O) through LDS: four times the workgroups
//    and a quarter of the round trips, for the long splits of short batches.
// Workgroups are dealt to XCDs in the same (b, kvh) order as attn_main's, so a merge reads
// partials from the L2 they were written to.

// the merge's compile-time shape for a plan with S chunks per (b, kvh, rb)
struct CombineShape {
  int batch;  // chunks loaded per round by one thread
  int sw;     // wavefronts sharing one piece (1 or 4)
};
inline CombineShape combine_shape(int S) {
  if (S <= 2) return {2, 1};
  if (S <= 4) return {4, 1};
  if (S <= 8) return {8, 1};
  return {8, 4};
}

// pieces per thread: eight 16-byte partial loads in flight per thread
constexpr int combine_pieces(int batch, int sw) { return sw == 1 ? 8 / batch : 1; }

template <int D, int kBatch, int kSW>
constexpr int combine_wgs_per_item() {  // workgroups per (b, kvh, rb)
  return kRows * D / 4 * kSW / combine_pieces(kBatch, kSW) / 256;
}

template <int D>
int combine_grid(int items, int S) {
  const CombineShape c = combine_shape(S);
  const int per = c.sw == 4 ? combine_wgs_per_item<D, 8, 4>()
                  : c.batch == 2 ? combine_wgs_per_item<D, 2, 1>()
                  : c.batch == 4 ? combine_wgs_per_item<D, 4, 1>()
                                 : combine_wgs_per_item<D, 8, 1>();
  return items * per;
}

// Logical merge workgroup c (of B * Hkv * RB * combine_wgs_per_item), 256 threads.  The chunk
// count comes from the workspace (written by attn_main), not from cache_len, which a fused
// compaction may be updating at the same time.
template <typename E, int D, int kBatch, int kSW>
__device__ void combine_group(const AttnArgs& a, int c) {
  constexpr bool kBF16 = std::is_same<E, __bf16>::value;
  constexpr int kDB = D / 32;
  constexpr int kP = combine_pieces(kBatch, kSW);
  constexpr int kWGs = combine_wgs_per_item<D, kBatch, kSW>();
  constexpr int kPer = 256 / kSW;          // pieces per workgroup and per-thread piece index
  constexpr int kStride = kRows * D / 4;   // pieces per slot
  static_assert(kSW == 1 || kP == 1, "shared pieces are merged one per thread");
  const int tid = threadIdx.x;
  const int pl = tid % kPer, sg = tid / kPer;  // piece within the workgroup, chunk group
  int b, item, n_split;
  if constexpr (kSW == 1) {
    // Logical workgroups go to split sequences only, in sequence order: logical workgroup c
    // serves the (c / per_seq)-th sequence with more than one chunk, so all the merge's work
    // sits in the first workgroups (the hardware deals them to the XCDs in turn) and the rest,
    // up to the grid's bound for a plan that splits every sequence, leave at once.  Wavefront
    // 0 ranks the sequences by ballots over their chunk counts.
    // The chunk count of the sequence found goes along with it, so the partials' loads wait
    // for one read of the counts, not two.
    __shared__ int s_b, s_n;
    const int per_seq = a.Hkv * a.RB * kWGs;
    const int rank = c / per_seq;
    if (tid < 64) {
      int found = -1, found_n = 0, before = 0;
      for (int base = 0; base < a.B && found < 0; base += 256) {
        int ns[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int bi = base + 64 * k + tid;
          ns[k] = bi < a.B ? a.nsplit[bi] : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint64_t m = __ballot(ns[k] > 1);
          const int cnt = __popcll(m);
          if (found < 0 && rank < before + cnt) {
            uint64_t mm = m;  // the (rank - before)-th set lane
            for (int i = rank - before; i > 0; --i) mm &= mm - 1;
            const int lane = __builtin_ctzll(mm);
            found = base + 64 * k + lane;
            found_n = __shfl(ns[k], lane, 64);
          }
          before += cnt;
        }
      }
      if (tid == 0) {
        s_b = found;
        s_n = found_n;
      }
    }
    __syncthreads();
    b = s_b;
    if (b < 0) return;  // more logical workgroups than the split sequences need (uniform)
    n_split = s_n;
    item = b * a.Hkv * a.RB + (c % per_seq) / kWGs;
  } else {
    // the chunk count is read here but first needed after the first batch's loads are issued
    item = c / kWGs;
    b = item / (a.RB * a.Hkv);
    n_split = a.nsplit[b];
  }
  const int rb = item % a.RB;
  const int kvh = (item / a.RB) % a.Hkv;
  const size_t slot0 = (((size_t)b * a.Hkv + kvh) * a.RB + rb) * a.S;
  const float4* po = reinterpret_cast<const float4*>(a.part_o) + slot0 * kStride;
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + slot0 * kRows;

  // piece q of this thread: register-order group g = ((wave*kDB + db)*4 + j)*64 + lane, that is
  // row wave*32 + lane%32 and d = db*32 + 8j + 4*(lane/32); consecutive threads own consecutive
  // groups, so each of the thread's loads is part of one 4 KB run per workgroup
  int g[kP], rloc[kP], dq[kP];
  bool live[kP];
#pragma unroll
  for (int q = 0; q < kP; ++q) {
    g[q] = ((c % kWGs) * kP + q) * kPer + pl;
    const int lane = g[q] & 63, j = (g[q] >> 6) & 3, db = (g[q] >> 8) % kDB;
    const int wave = (g[q] >> 8) / kDB;
    rloc[q] = wave * 32 + (lane & 31);
    live[q] = rb * kRows + rloc[q] < a.GT;  // padding rows were never written
    dq[q] = db * 32 + 8 * j + 4 * (lane >> 5);
  }

  float M[kP], den[kP];
  float4 acc[kP];
#pragma unroll
  for (int q = 0; q < kP; ++q) {
    M[q] = -INFINITY;
    den[q] = 0.f;
    acc[q] = float4{0.f, 0.f, 0.f, 0.f};
  }
  // chunk group sg takes chunks sg, sg + kSW, sg + 2 kSW, ...
  float4 v[kP][kBatch];
  float2 ml[kP][kBatch];
  auto load_batch = [&](int k0, int nb) {
#pragma unroll
    for (int q = 0; q < kP; ++q)
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (u < nb && live[q]) {
          const size_t sidx = (size_t)(k0 + u) * kSW + sg;
          v[q][u] = po[sidx * kStride + g[q]];
          ml[q][u] = pml[sidx * kRows + rloc[q]];
        } else {
          v[q][u] = float4{0.f, 0.f, 0.f, 0.f};
          ml[q][u] = float2{-INFINITY, 0.f};
        }
  };
  // The first batch is loaded as far as the plan's chunk count, which bounds the sequence's
  // own and whose slots all exist, so with shared pieces these loads need not wait for the
  // count.  Slots past the sequence's count hold stale values; they only ever pass the u < nb
  // selects below, never the arithmetic.
  const int n_plan = kSW == 1 ? n_split : a.S;
  load_batch(0, min(kBatch, sg < n_plan ? (n_plan - sg + kSW - 1) / kSW : 0));
  const int n_mine = sg < n_split ? (n_split - sg + kSW - 1) / kSW : 0;
  for (int k0 = 0;;) {
    const int nb = min(kBatch, n_mine - k0);  // uniform across the workgroup; 0 if none
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      // A chunk in which a row sees no key (a second tree tile that holds none of the row's
      // ancestors, cut into a chunk of its own) carries m = -inf, l = 0, O = 0.  When every
      // chunk so far is such a chunk, Mb is -inf too; the exponents are then taken against 0,
      // so those chunks weigh 0 instead of 2^(-inf - -inf) = NaN.
      float Mb = M[q];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (u < nb) Mb = fmaxf(Mb, ml[q][u].x);
      const float Me = Mb == -INFINITY ? 0.f : Mb;
      const float sc = fast_exp2(M[q] - Me);  // 0 on the first batch
      den[q] *= sc;
      acc[q].x *= sc;
      acc[q].y *= sc;
      acc[q].z *= sc;
      acc[q].w *= sc;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (u < nb) {
          const float w = fast_exp2(ml[q][u].x - Me);
          const float4 x = v[q][u];
          den[q] += w * ml[q][u].y;
          acc[q].x += w * x.x;
          acc[q].y += w * x.y;
          acc[q].z += w * x.z;
          acc[q].w += w * x.w;
        }
      M[q] = Mb;
    }
    k0 += kBatch;
    if (k0 >= n_mine) break;
    load_batch(k0, min(kBatch, n_mine - k0));
  }
  if (n_split <= 1) return;  // written directly by attn_main (uniform: the whole workgroup)
  if constexpr (kSW > 1) {
    // the chunk groups' partial merges meet in LDS; group 0 combines them in group order
    __shared__ float4 s_acc[kSW][kPer];
    __shared__ float2 s_mden[kSW][kPer];
    s_acc[sg][pl] = acc[0];
    s_mden[sg][pl] = float2{M[0], den[0]};
    __syncthreads();
    if (sg != 0) return;
    float Mt = M[0];
#pragma unroll
    for (int w = 1; w < kSW; ++w) Mt = fmaxf(Mt, s_mden[w][pl].x);
    // group 0 always holds chunk 0, whose first tile holds the root (visible to every row),
    // so Mt is finite for live rows; a group that saw no key has M = -inf, den = 0, O = 0
    // and weight 0
    const float sc = fast_exp2(M[0] - Mt);
    den[0] *= sc;
    acc[0].x *= sc;
    acc[0].y *= sc;
    acc[0].z *= sc;
    acc[0].w *= sc;
#pragma unroll
    for (int w = 1; w < kSW; ++w) {
      const float2 md = s_mden[w][pl];
      const float4 x = s_acc[w][pl];
      const float wt = fast_exp2(md.x - Mt);
      den[0] += wt * md.y;
      acc[0].x += wt * x.x;
      acc[0].y += wt * x.y;
      acc[0].z += wt * x.z;
      acc[0].w += wt * x.w;
    }
    M[0] = Mt;
  }
  // output row of a (live) row index of this item
  auto out_row = [&](int r) -> size_t {
    const int t = r / a.G, head = kvh * a.G + r % a.G;
    return ((size_t)b * a.T + t) * a.Hq + head;
  };
  if constexpr (kSW == 1) {
    // The workgroup's pieces cover a block of whole row segments: kRowsWG rows (32 consecutive
    // per 8 D pieces) by kDSpan consecutive d.  Stored piece by piece, every store instruction
    // would write 16 bytes into each of 32 rows; staged through LDS (rows padded by 16 bytes,
    // so the 32 rows of a staging write fall in different banks), every row segment leaves in
    // contiguous 16-byte stores.
    constexpr int kWGPieces = 256 * kP;
    constexpr int kGroupPieces = 8 * D;  // pieces of 32 whole rows
    constexpr int kRowsWG = kWGPieces >= kGroupPieces ? 32 * (kWGPieces / kGroupPieces) : 32;
    constexpr int kDSpan = kWGPieces >= kGroupPieces ? D : D * kWGPieces / kGroupPieces;
    constexpr int kSegBytes = kDSpan * (int)sizeof(E);
    constexpr int kLdsRow = kSegBytes + 16;
    constexpr int kChunks = kRowsWG * kSegBytes / 16;  // 16-byte stores of the block
    __shared__ __attribute__((aligned(16))) char s_out[kRowsWG * kLdsRow];
    const int gb = (c % kWGs) * kWGPieces >> 8;  // (wave * kDB + db) of the block's first piece
    const int row0 = (gb / kDB) * 32;              // first row of the block within the item
    const int d0 = kDSpan == D ? 0 : (gb % kDB) * 32;
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      if (!live[q]) continue;
      const float inv = 1.f / den[q];
      char* dst = s_out + (rloc[q] - row0) * kLdsRow + (dq[q] - d0) * (int)sizeof(E);
      if constexpr (kBF16) {
        *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(acc[q].x * inv, acc[q].y * inv),
                                               pack_bf16x2(acc[q].z * inv, acc[q].w * inv)};
      } else {
        *reinterpret_cast<float4*>(dst) =
            float4{acc[q].x * inv, acc[q].y * inv, acc[q].z * inv, acc[q].w * inv};
      }
      if (a.lse && dq[q] == 0)
        a.lse[out_row(rb * kRows + rloc[q])] = (M[q] + __log2f(den[q])) * kLn2;
    }
    __syncthreads();
#pragma unroll
    for (int k = tid; k < kChunks; k += 256) {
      const int rr = k / (kSegBytes / 16), off = (k % (kSegBytes / 16)) * 16;
      const int r = rb * kRows + row0 + rr;
      if (r >= a.GT) continue;  // padding rows are never written
      char* o = a.out + (out_row(r) * D + d0) * sizeof(E) + off;
      *reinterpret_cast<uint4*>(o) = *reinterpret_cast<const uint4*>(s_out + rr * kLdsRow + off);
    }
  } else {
    if (!live[0]) return;
    const int r = rb * kRows + rloc[0];
    const float inv = 1.f / den[0];
    const size_t orow = out_row(r);
    E* o = reinterpret_cast<E*>(a.out) + orow * D;
    const int d = dq[0];
    if constexpr (kBF16) {
      *reinterpret_cast<uint2*>(o + d) = uint2{pack_bf16x2(acc[0].x * inv, acc[0].y * inv),
                                               pack_bf16x2(acc[0].z * inv, acc[0].w * inv)};
    } else {
      *reinterpret_cast<float4*>(o + d) =
          float4{acc[0].x * inv, acc[0].y * inv, acc[0].z * inv, acc[0].w * inv};
    }
    if (a.lse && d == 0) a.lse[orow] = (M[0] + __log2f(den[0])) * kLn2;
  }
}

template <typename E, int D, int kBatch, int kSW>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  // (few chunks: split sequences first, in hardware order; many: XCD-aligned with attn_main)
  combine_group<E, D, kBatch, kSW>(
      a, kSW == 1 ? (int)blockIdx.x
                  : xcd_remap(blockIdx.x, a.B * a.Hkv * a.RB *
                                              combine_wgs_per_item<D, kBatch, kSW>()));
}

// ---- fused tail of a verification step -----------------------------------------------------
// Workgroup b < B runs the acceptance walk of sequence b on its first wavefront, then all four
// wavefronts copy the accepted K/V rows of every KV head into the cache; they come first so
// they run under the merge.  Workgroups from n_acc (B rounded up to a multiple of the 8 XCDs,
// so the merge keeps attn_combine's XCD order) merge split-K partials.  Used only when the
// tree K/V does not overlap the cache, so rows are copied directly, without staging.
struct TailArgs {
  const uint64_t* anc;
  const int32_t* draft;
  const int32_t* target;
  int32_t* accept_path;
  int32_t* accept_len;
  int32_t* bonus_tok;
  char* kc;  // writable views of the caches
  char* vc;
  int32_t* cache_len_out;
  int32_t* status;
  int n_comb, n_acc, W, row_bytes;
  // paged step (table not null): pointer-swap commit into the block table and free list, and
  // n_scan workgroups (scan_per_seq per sequence) checking the entries the attention read
  int32_t* table;
  int32_t* free_slots;
  int32_t* free_top;
  int n_scan, scan_per_seq;
};

constexpr int kScanPerThread = 16;                  // table entries per thread of a scan
constexpr int kScanSlice = 256 * kScanPerThread;    // table entries per scan workgroup

// Acceptance workgroup of the paged step (one-token pages): wavefront 0 walks the tree and then
// commits the path by pointer swap.
__device__ inline void tail_commit_paged(const AttnArgs& a, const TailArgs& t, int b, int L,
                                         int* s_path) {
  __shared__ int s_on[kMaxT];
  const int tid = threadIdx.x;
  if (tid >= 64) return;
  const int n = accept_walk(b, a.T, t.W, t.anc, t.draft, t.target, t.accept_path, t.accept_len,
                            t.bonus_tok, s_path);
  wave_lds_sync();
  int pe[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = tid + 64 * k;
    pe[k] = c < n ? s_path[c] : -1;
  }
  commit_paged_wave(b, L, n, pe, t.table, a.max_pages, a.tree_slot, a.T, a.num_slots,
                    t.free_slots, t.free_top, t.status, t.cache_len_out, s_on);
}

// Scan workgroup k of the paged step: checks the block-table entries of positions
// [slice * kScanSlice, +kScanSlice) below the attention's clamped length of its sequence, and
// (slice 0) every tree slot, and ORs TV_BAD_PAGE as tree_verify_attn_paged does.  The mask
// writer of the step's main kernel stores status[b] with a plain write, so that kernel leaves
// bad pages to these workgroups, which run after it.  All loads of a thread are in flight at
// once.
__device__ inline void tail_scan_pages(const AttnArgs& a, const TailArgs& t, int k) {
  const int b = k / t.scan_per_seq, slice = k - b * t.scan_per_seq;
  const int tid = threadIdx.x;
  // With cache_len_out aliasing cache_len, the acceptance workgroup of b may already have
  // committed L + n.  Read with acquire against the commit's release, the new length comes with
  // the n new entries, which are tree slots the commit found inside the pool, so the verdict
  // is the same as over the L entries the attention read.  One thread reads it, so the whole
  // workgroup uses one value.
  __shared__ int s_len;
  if (tid == 0) {
    s_len = __hip_atomic_load(const_cast<int32_t*>(a.cache_len) + b, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  const int Lc = min(max(s_len, 0), a.Lmax);
  const int lo = slice * kScanSlice;
  if (lo >= Lc && slice > 0) return;  // uniform
  const int32_t* row = a.table + (size_t)b * a.max_pages;
  const int last = max(Lc - 1, 0);  // row[0] exists (max_pages >= 1)
  int e[kScanPerThread];
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j) e[j] = row[min(lo + j * 256 + tid, last)];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j)
    bad = bad || (lo + j * 256 + tid < Lc && (e[j] < 0 || e[j] >= a.num_slots));
  if (slice == 0 && tid < a.T) {
    const int ts = a.tree_slot[(size_t)b * a.T + tid];
    bad = bad || ts < 0 || ts >= a.num_slots;
  }
  if (__syncthreads_or(bad) && tid == 0 && t.status) atomicOr(t.status + b, TV_BAD_PAGE);
}

template <typename E, int D, int kBatch, int kSW>
__global__ __launch_bounds__(256) void step_tail(AttnArgs a, TailArgs t) {
  if ((int)blockIdx.x >= t.n_acc) {
    const int c = blockIdx.x - t.n_acc;
    combine_group<E, D, kBatch, kSW>(a, kSW == 1 ? c : xcd_remap(c, t.n_comb));
    return;
  }
  if ((int)blockIdx.x >= a.B) {  // bad-page scans, then XCD alignment padding
    if ((int)blockIdx.x - a.B < t.n_scan) tail_scan_pages(a, t, blockIdx.x - a.B);
    return;
  }
  __shared__ int s_path[kMaxT];
  __shared__ int s_n;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = a.cache_len[b];  // read before this workgroup writes cache_len_out[b]
  if (t.table) {
    tail_commit_paged(a, t, b, L, s_path);
    return;
  }
  if (tid < 64) {
    const int n = accept_walk(b, a.T, t.W, t.anc, t.draft, t.target, t.accept_path, t.accept_len,
                              t.bonus_tok, s_path);
    if (tid == 0) s_n = n;
  }
  __syncthreads();
  const int n = s_n;  // in [1, T]; the path's entries are valid node indices
  int bits = 0;
  if (L < 0 || L > a.Lmax) bits |= TV_BAD_LEN;
  else if ((long long)L + n > a.Lmax) bits |= TV_OVERFLOW;
  if (!bits) {
    const int cpr = t.row_bytes / 16;
    const int total = a.Hkv * 2 * n * cpr;
    for (int q = tid; q < total; q += 256) {
      const int chunk = q % cpr;
      int r = q / cpr;
      const int i = r % n;
      r /= n;
      const int kv = r & 1, head = r >> 1;
      const int j = s_path[i];
      const char* src = (kv ? a.vt : a.kt) + (((size_t)b * a.T + j) * a.Hkv + head) * t.row_bytes;
      char* dst = (kv ? t.vc : t.kc) + (((size_t)b * a.Hkv + head) * a.Lmax + L + i) * t.row_bytes;
      reinterpret_cast<uint4*>(dst)[chunk] = reinterpret_cast<const uint4*>(src)[chunk];
    }
  }
  if (tid == 0) {
    if (bits && t.status) atomicOr(t.status + b, bits);
    t.cache_len_out[b] = bits ? L : L + n;
  }
}

struct Plan {
  int RB, S, chunk_tiles;
  size_t ws_bytes;
};

Plan make_plan(int B, int T, int Hq, int Hkv, int D, int Lmax, int split_keys) {
  Plan p;
  const int G = Hq / Hkv;
  p.RB = ceil_div(G * T, kRows);
  // tiles of the longest sequence: its tree tiles, then its prefix tiles
  const int tiles = ceil_div(T, kKT) + ceil_div(Lmax, kKT);
  int chunk_tiles;
  if (split_keys > 0) {
    chunk_tiles = ceil_div(split_keys, kKT);
  } else {
    // One workgroup per compute unit.  A chunk costs a prologue (Q and the first tiles), a
    // 128 KB fp32 partial (256 rows x D = 128) written and merged, so splitting pays only where
    // CUs would otherwise idle:
    //  * fewer (sequence, KV head, row block) units than CUs: one round of workgroups, with
    //    chunks of at least 4 tiles (3-tile chunks write a larger partial than the 96 KB of K/V
    //    they read: 20.8 against 19.9 us at batch 1, prefix 4096).  Two rounds pay a second
    //    prologue and twice the partials: 543.5 against 533.0 us for the step at batch 8,
    //    prefix 32768;
    //  * at least as many units as CUs, but fewer than twice: only sequences longer than 3/4
    //    of the longest split, into a 3/4 chunk and the rest, which the longest-first dispatch
    //    places in the second round (126 us against 143 us for halves at batch 32, prefixes of
    //    512..4096: most sequences then need no merge at all);
    //  * twice the CUs or more: no split; the longest-first dispatch balances the rounds.
    const long long units = (long long)B * Hkv * p.RB;
    const long long cus = device_cu_count();
    if (units >= 2 * cus) {
      chunk_tiles = tiles;
    } else if (units >= cus) {
      chunk_tiles = std::max(1, ceil_div(3 * tiles, 4));
    } else {
      const int S = (int)std::min<long long>(std::max<long long>(1, ceil_div_ll(cus, units)),
                                             std::max(1, ceil_div(tiles, 4)));
      chunk_tiles = ceil_div(tiles, S);
    }
  }
  p.chunk_tiles = chunk_tiles;
  p.S = ceil_div(tiles, chunk_tiles);
  // per slot: kRows x D partial O in fp32, then kRows x (m, l) in fp32; then the chunk count
  // of every sequence
  p.ws_bytes = p.S > 1 ? (size_t)B * Hkv * p.RB * p.S * kRows * ((size_t)D * 4 + 8) +
                             (size_t)B * sizeof(int32_t)
                       : 0;
  return p;
}

// Profiling events recorded around the main kernel (tv_profile_attn_main).
hipEvent_t g_prof_before = nullptr, g_prof_after = nullptr;

template <typename E, int D, bool kMasks = false, int kPaged = 0>
int launch_main(const AttnArgs& a, hipStream_t stream) {
  const int n_items = a.B * a.Hkv * a.S * a.RB;
  auto kernel = a.S > 1 ? attn_main<E, D, true, kMasks, kPaged>
                        : attn_main<E, D, false, kMasks, kPaged>;
  if (g_prof_before) {
    // the events take the kernel's own start and end timestamps
    hipExtLaunchKernelGGL(kernel, dim3(n_items), dim3(kThreads), 0, stream, g_prof_before,
                          g_prof_after, 0, a);
  } else {
    hipLaunchKernelGGL(kernel, dim3(n_items), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

template <typename E, int D, int kPaged = 0>
int launch_attn(const AttnArgs& a, hipStream_t stream) {
  const int rc = launch_main<E, D, false, kPaged>(a, stream);
  if (rc != TV_OK) return rc;
  if (a.S > 1) {
    const dim3 grid(combine_grid<D>(a.B * a.Hkv * a.RB, a.S)), block(256);
    switch (combine_shape(a.S).batch * combine_shape(a.S).sw) {
      case 2: hipLaunchKernelGGL((attn_combine<E, D, 2, 1>), grid, block, 0, stream, a); break;
      case 4: hipLaunchKernelGGL((attn_combine<E, D, 4, 1>), grid, block, 0, stream, a); break;
      case 8: hipLaunchKernelGGL((attn_combine<E, D, 8, 1>), grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL((attn_combine<E, D, 8, 4>), grid, block, 0, stream, a);
    }
  }
  return launch_status();
}

template <typename E, int D, int kPaged = 0>
int launch_step(const AttnArgs& a, TailArgs t, hipStream_t stream) {
  const int rc = launch_main<E, D, true, kPaged>(a, stream);
  if (rc != TV_OK) return rc;
  t.n_comb = a.S > 1 ? combine_grid<D>(a.B * a.Hkv * a.RB, a.S) : 0;
  t.n_acc = (a.B + t.n_scan + 7) / 8 * 8;
  const dim3 grid(t.n_acc + t.n_comb), block(256);
  switch (combine_shape(a.S).batch * combine_shape(a.S).sw) {
    case 2: hipLaunchKernelGGL((step_tail<E, D, 2, 1>), grid, block, 0, stream, a, t); break;
    case 4: hipLaunchKernelGGL((step_tail<E, D, 4, 1>), grid, block, 0, stream, a, t); break;
    case 8: hipLaunchKernelGGL((step_tail<E, D, 8, 1>), grid, block, 0, stream, a, t); break;
    default: hipLaunchKernelGGL((step_tail<E, D, 8, 4>), grid, block, 0, stream, a, t);
  }
  return launch_status();
}

}  // namespace

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
      cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

}  // namespace tv

using namespace tv;

static bool attn_shapes_ok(int B, int T, int Hq, int Hkv, int Lmax) {
  return B >= 1 && T >= 1 && T <= kMaxT && Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0 && Lmax >= 0 &&
         (long long)B * Hkv * 64 * ceil_div(Hq / Hkv * T, kRows) < (1LL << 31);
}

extern "C" int tv_profile_attn_main(void* ev_before, void* ev_after) {
  if ((ev_before == nullptr) != (ev_after == nullptr)) return TV_ERR_INVALID_ARG;
  g_prof_before = (hipEvent_t)ev_before;
  g_prof_after = (hipEvent_t)ev_after;
  return TV_OK;
}

extern "C" size_t tree_verify_attn_workspace_size(int B, int T, int Hq, int Hkv, int D, int Lmax,
                                                  int dtype, int split_keys) {
  if (!attn_shapes_ok(B, T, Hq, Hkv, Lmax) || (D != 64 && D != 128) ||
      (dtype != TV_F32 && dtype != TV_BF16))
    return 0;
  return make_plan(B, T, Hq, Hkv, D, Lmax, split_keys).ws_bytes;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Checks the attention arguments and fills `a`; returns TV_OK or the error to report.
static int prepare_attn(AttnArgs& a, Plan& p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_len, const void* k_tree,
                        const void* v_tree, const uint64_t* anc_mask, void* out, float* lse,
                        int32_t* status, int B, int T, int Hq, int Hkv, int D, int Lmax,
                        int dtype, float scale, int split_keys, void* workspace,
                        size_t workspace_bytes) {
  if (!q || !k_cache || !v_cache || !cache_len || !k_tree || !v_tree || !anc_mask || !out ||
      !attn_shapes_ok(B, T, Hq, Hkv, Lmax) || split_keys < 0)
    return TV_ERR_INVALID_ARG;
  // q, K and V rows are read 16 bytes at a time (fp32 output rows are written so too)
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_tree) ||
      !aligned16(v_tree) || !aligned16(out))
    return TV_ERR_INVALID_ARG;
  if ((dtype != TV_F32 && dtype != TV_BF16) || (D != 64 && D != 128)) return TV_ERR_UNSUPPORTED;
  p = make_plan(B, T, Hq, Hkv, D, Lmax, split_keys);
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes)) return TV_ERR_WORKSPACE;
  if ((long long)B * Hkv * p.RB * p.S >= (1LL << 31)) return TV_ERR_INVALID_ARG;

  a.q = (const char*)q;
  a.kc = (const char*)k_cache;
  a.vc = (const char*)v_cache;
  a.cache_len = cache_len;
  a.kt = (const char*)k_tree;
  a.vt = (const char*)v_tree;
  a.anc = anc_mask;
  a.parent = nullptr;
  a.table = nullptr;
  a.tree_slot = nullptr;
  a.max_pages = 0;
  a.log2P = 0;
  a.num_slots = 0;
  a.out = (char*)out;
  a.lse = lse;
  a.status = status;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Lmax = Lmax;
  a.W = ceil_div(T, 64);
  a.GT = a.G * T;
  a.RB = p.RB;
  a.S = p.S;
  a.chunk_tiles = p.chunk_tiles;
  // lengths differ between sequences only when there are several
  a.lpt = B > 1 && (long long)B * p.S <= kLptMaxPairs;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  a.c = sc * kLog2e;
  char* ws = (char*)workspace;
  const size_t slots = (size_t)B * Hkv * p.RB * p.S;
  a.part_o = ws;
  a.part_ml = p.ws_bytes ? (float*)(ws + slots * kRows * D * sizeof(float)) : nullptr;
  a.nsplit = p.ws_bytes ? (int32_t*)(ws + slots * kRows * ((size_t)D * sizeof(float) + 8)) : nullptr;
  return TV_OK;
}

// The dense main kernel forms each K/V row's byte offset in 32 bits, within one (b, kvh) cache
// slab and within the sequence's tree rows; larger slabs are refused rather than wrapped.
static bool dense_offsets_ok(int T, int Hkv, int D, int Lmax, int dtype) {
  const long long row = (long long)D * (dtype == TV_BF16 ? 2 : 4);
  return (long long)Lmax * row <= (1LL << 32) && (long long)T * Hkv * row <= (1LL << 32);
}

extern "C" int tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* cache_len, const void* k_tree, const void* v_tree,
                                const uint64_t* anc_mask, void* out, float* lse, int32_t* status,
                                int B, int T, int Hq, int Hkv, int D, int Lmax, int dtype,
                                float scale, int split_keys, void* workspace,
                                size_t workspace_bytes, void* stream) {
  AttnArgs a;
  Plan p;
  const int rc = prepare_attn(a, p, q, k_cache, v_cache, cache_len, k_tree, v_tree, anc_mask,
                              out, lse, status, B, T, Hq, Hkv, D, Lmax, dtype, scale, split_keys,
                              workspace, workspace_bytes);
  if (rc != TV_OK) return rc;
  if (!dense_offsets_ok(T, Hkv, D, Lmax, dtype)) return TV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == TV_BF16)
    return D == 128 ? launch_attn<__bf16, 128>(a, st) : launch_attn<__bf16, 64>(a, st);
  return D == 128 ? launch_attn<float, 128>(a, st) : launch_attn<float, 64>(a, st);
}

extern "C" int tree_verify_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                                      int num_slots, const int32_t* block_table, int max_pages,
                                      int page_size, const int32_t* cache_len,
                                      const int32_t* tree_slot, const uint64_t* anc_mask,
                                      void* out, float* lse, int32_t* status, int B, int T,
                                      int Hq, int Hkv, int D, int dtype, float scale,
                                      int split_keys, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!block_table || !tree_slot || num_slots < 1 || max_pages < 1 || page_size < 1 ||
      (page_size & (page_size - 1)) || (long long)max_pages * page_size >= (1LL << 30))
    return TV_ERR_INVALID_ARG;
  AttnArgs a;
  Plan p;
  const int cap = max_pages * page_size;  // positions the table can name
  // the dense argument checks, with the pools standing in for the caches and the tree K/V
  const int rc = prepare_attn(a, p, q, k_pool, v_pool, cache_len, k_pool, v_pool, anc_mask, out,
                              lse, status, B, T, Hq, Hkv, D, cap, dtype, scale, split_keys,
                              workspace, workspace_bytes);
  if (rc != TV_OK) return rc;
  a.table = block_table;
  a.tree_slot = tree_slot;
  a.max_pages = max_pages;
  a.log2P = 31 - __builtin_clz((unsigned)page_size);
  a.num_slots = num_slots;
  hipStream_t st = (hipStream_t)stream;
  // a pool of at most 4 GB per cache is addressed by 32-bit offsets from its base
  const bool off32 =
      (unsigned long long)num_slots * Hkv * D * (dtype == TV_BF16 ? 2 : 4) <= 0xffffffffull;
  if (dtype == TV_BF16) {
    if (off32)
      return D == 128 ? launch_attn<__bf16, 128, 2>(a, st) : launch_attn<__bf16, 64, 2>(a, st);
    return D == 128 ? launch_attn<__bf16, 128, 1>(a, st) : launch_attn<__bf16, 64, 1>(a, st);
  }
  return D == 128 ? launch_attn<float, 128, 1>(a, st) : launch_attn<float, 64, 1>(a, st);
}

// True when byte ranges [a, a + na) and [b, b + nb) intersect.
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

extern "C" int tree_verify_step(const int32_t* parent, const int32_t* draft_tok,
                                const int32_t* target_tok, const void* q, void* k_cache,
                                void* v_cache, const int32_t* cache_len, int32_t* cache_len_out,
                                const void* k_tree, const void* v_tree, uint64_t* anc_mask,
                                void* out, float* lse, int32_t* accept_path, int32_t* accept_len,
                                int32_t* bonus_tok, int32_t* status, int B, int T, int Hq,
                                int Hkv, int D, int Lmax, int dtype, float scale,
                                int split_keys, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!parent || !draft_tok || !target_tok || !cache_len_out || !accept_path || !accept_len ||
      !bonus_tok || !status)
    return TV_ERR_INVALID_ARG;
  AttnArgs a;
  Plan p;
  int rc = prepare_attn(a, p, q, k_cache, v_cache, cache_len, k_tree, v_tree, anc_mask, out, lse,
                        status, B, T, Hq, Hkv, D, Lmax, dtype, scale, split_keys, workspace,
                        workspace_bytes);
  if (rc != TV_OK) return rc;
  if (!dense_offsets_ok(T, Hkv, D, Lmax, dtype)) return TV_ERR_INVALID_ARG;
  if (cache_len_out != cache_len &&
      overlaps(cache_len_out, (size_t)B * 4, cache_len, (size_t)B * 4))
    return TV_ERR_INVALID_ARG;
  const size_t elem = dtype == TV_BF16 ? 2 : 4;
  const size_t cache_bytes = (size_t)B * Hkv * Lmax * D * elem;
  const size_t tree_bytes = (size_t)B * T * Hkv * D * elem;
  if (overlaps(k_tree, tree_bytes, k_cache, cache_bytes) ||
      overlaps(k_tree, tree_bytes, v_cache, cache_bytes) ||
      overlaps(v_tree, tree_bytes, k_cache, cache_bytes) ||
      overlaps(v_tree, tree_bytes, v_cache, cache_bytes)) {
    // Tree rows inside the cache: the compaction must stage rows (kv_compact_accepted).
    rc = tree_build_mask(parent, B, T, anc_mask, status, stream);
    if (rc != TV_OK) return rc;
    rc = tree_verify_attn(q, k_cache, v_cache, cache_len, k_tree, v_tree, anc_mask, out, lse,
                          status, B, T, Hq, Hkv, D, Lmax, dtype, scale, split_keys, workspace,
                          workspace_bytes, stream);
    if (rc != TV_OK) return rc;
    rc = tree_accept(anc_mask, draft_tok, target_tok, B, T, accept_path, accept_len, bonus_tok,
                     stream);
    if (rc != TV_OK) return rc;
    return kv_compact_accepted(k_cache, v_cache, cache_len, cache_len_out, k_tree, v_tree,
                               accept_path, accept_len, B, T, Hkv, D, Lmax, dtype, status,
                               stream);
  }
  // attention main kernel (building the ancestor masks), then merge + acceptance + compaction
  a.parent = parent;
  TailArgs t;
  t.anc = anc_mask;
  t.draft = draft_tok;
  t.target = target_tok;
  t.accept_path = accept_path;
  t.accept_len = accept_len;
  t.bonus_tok = bonus_tok;
  t.kc = (char*)k_cache;
  t.vc = (char*)v_cache;
  t.cache_len_out = cache_len_out;
  t.status = status;
  t.n_comb = 0;
  t.W = ceil_div(T, 64);
  t.row_bytes = D * (int)elem;
  t.table = t.free_slots = t.free_top = nullptr;
  t.n_scan = t.scan_per_seq = 0;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == TV_BF16)
    return D == 128 ? launch_step<__bf16, 128>(a, t, st) : launch_step<__bf16, 64>(a, t, st);
  return D == 128 ? launch_step<float, 128>(a, t, st) : launch_step<float, 64>(a, t, st);
}

extern "C" int tree_verify_step_paged(
    const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok, const void* q,
    const void* k_pool, const void* v_pool, int num_slots, int32_t* block_table, int max_pages,
    int page_size, const int32_t* cache_len, int32_t* cache_len_out, const int32_t* tree_slot,
    uint64_t* anc_mask, void* out, float* lse, int32_t* accept_path, int32_t* accept_len,
    int32_t* bonus_tok, int32_t* free_slots, int32_t* free_top, int32_t* status, int B, int T,
    int Hq, int Hkv, int D, int dtype, float scale, int split_keys, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (!parent || !draft_tok || !target_tok || !cache_len_out || !accept_path || !accept_len ||
      !bonus_tok || !status || !block_table || !tree_slot || !free_slots || !free_top ||
      num_slots < 1 || max_pages < 1 || page_size < 1 || (page_size & (page_size - 1)) ||
      max_pages >= (1 << 30))
    return TV_ERR_INVALID_ARG;
  if (page_size != 1) return TV_ERR_UNSUPPORTED;  // the pointer-swap commit needs token pages
  if (cache_len_out != cache_len &&
      overlaps(cache_len_out, (size_t)B * 4, cache_len, (size_t)B * 4))
    return TV_ERR_INVALID_ARG;
  AttnArgs a;
  Plan p;
  // the dense argument checks, with the pools standing in for the caches and the tree K/V
  const int rc = prepare_attn(a, p, q, k_pool, v_pool, cache_len, k_pool, v_pool, anc_mask, out,
                              lse, status, B, T, Hq, Hkv, D, max_pages, dtype, scale, split_keys,
                              workspace, workspace_bytes);
  if (rc != TV_OK) return rc;
  a.table = block_table;
  a.tree_slot = tree_slot;
  a.max_pages = max_pages;
  a.log2P = 0;
  a.num_slots = num_slots;
  a.parent = parent;
  TailArgs t;
  t.anc = anc_mask;
  t.draft = draft_tok;
  t.target = target_tok;
  t.accept_path = accept_path;
  t.accept_len = accept_len;
  t.bonus_tok = bonus_tok;
  t.kc = t.vc = nullptr;  // nothing is copied
  t.cache_len_out = cache_len_out;
  t.status = status;
  t.n_comb = 0;
  t.W = ceil_div(T, 64);
  t.row_bytes = 0;
  t.table = block_table;
  t.free_slots = free_slots;
  t.free_top = free_top;
  t.scan_per_seq = ceil_div(max_pages, kScanSlice);
  if ((long long)B * t.scan_per_seq > (1 << 24)) return TV_ERR_INVALID_ARG;
  t.n_scan = B * t.scan_per_seq;
  hipStream_t st = (hipStream_t)stream;
  const bool off32 =
      (unsigned long long)num_slots * Hkv * D * (dtype == TV_BF16 ? 2 : 4) <= 0xffffffffull;
  if (dtype == TV_BF16) {
    if (off32)
      return D == 128 ? launch_step<__bf16, 128, 2>(a, t, st) : launch_step<__bf16, 64, 2>(a, t, st);
    return D == 128 ? launch_step<__bf16, 128, 1>(a, t, st) : launch_step<__bf16, 64, 1>(a, t, st);
  }
  return D == 128 ? launch_step<float, 128, 1>(a, t, st) : launch_step<float, 64, 1>(a, t, st);
}

// ---- tree_verify_step_noalloc: the step with a library-owned workspace ----------------------
// The split-K partials live in this array instead of a caller's workspace.  Every GPU the
// library runs on holds its own copy for the life of the process.  In host code the name is
// only a host-side handle: the device address is looked up once per device (scratch_on_device)
// and only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[TV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on that device (with
// that device current).
int scratch_on_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TV_OK;
}
}  // namespace

extern "C" int tree_verify_step_noalloc(const int32_t* parent, const int32_t* draft_tok,
                                        const int32_t* target_tok, const void* q, void* k_cache,
                                        void* v_cache, const int32_t* cache_len,
                                        int32_t* cache_len_out, const void* k_tree,
                                        const void* v_tree, uint64_t* anc_mask, void* out,
                                        float* lse, int32_t* accept_path, int32_t* accept_len,
                                        int32_t* bonus_tok, int32_t* status, int B, int T,
                                        int Hq, int Hkv, int D, int Lmax, int dtype, float scale,
                                        int split_keys, void* stream) {
  // the size check comes first: a plan beyond the array is refused before any device call
  const size_t need =
      tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, Lmax, dtype, split_keys);
  if (need > (size_t)TV_NOALLOC_SCRATCH_BYTES) return TV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_on_device(&ws);
    if (rc != TV_OK) return rc;
  }
  return tree_verify_step(parent, draft_tok, target_tok, q, k_cache, v_cache, cache_len,
                          cache_len_out, k_tree, v_tree, anc_mask, out, lse, accept_path,
                          accept_len, bonus_tok, status, B, T, Hq, Hkv, D, Lmax, dtype, scale,
                          split_keys, ws, need, stream);
}
