/*
 * tree_verify.h — C ABI of libtreeverify.so: the verification step of tree speculative decoding
 * on an AMD Instinct MI355X (gfx950).
 *
 * One verification step, as described on lesty.tech "EAGLE-2 vs. Medusa" (sections 4, 5, 8) and
 * rainlin.net "大模型投机解码（二）：EAGLE 系列" (sections 3.2, 4, 7):
 *   1. tree_build_mask      per-node ancestor bitmask of the flattened draft tree;
 *   2. tree_verify_attn     every tree node attends to its sequence's KV prefix plus only its
 *                           own root-to-node path;
 *   3. tree_accept          greedy acceptance, keep the single longest accepted path;
 *   4. kv_compact_accepted  append the accepted nodes' K/V to the cache, drop the rest.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers, except where a parameter says otherwise.  The caller
 *     owns every buffer; the library never allocates, frees, copies to the host or
 *     synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     outputs are valid once that stream reaches the end of the call's work.
 *   - Tensors are dense, row-major, in the shapes given in brackets.  One floating dtype per
 *     call (tv_dtype): fp32, or bfloat16 stored as 16-bit words.
 *   - The tree is flattened in level order with a single root at index 0 and parent[i] < i for
 *     i > 0 (the worked tree It/is/has/a/the/to/good/be flattens to
 *     [It, is, has, a, the, to, good, be] with parent = [-1,0,0,1,1,2,3,5]).
 *   - Ancestor masks are W = ceil(T/64) 64-bit words per node; bit (j % 64) of word (j / 64)
 *     refers to node j.
 *   - Limits: 1 <= T <= 128, D in {64, 128}, Hq % Hkv == 0, B >= 1, Lmax >= 0.
 *   - Return value: TV_OK, or a negative tv_status.  Host-checkable problems (null pointers,
 *     shapes, limits, dtype, workspace size) are reported before anything is launched.  A
 *     launch failure is reported as TV_ERR_HIP.  Problems in the data itself are found on the
 *     device and reported as bits in a caller-owned int32 status[B] array; they never cause an
 *     out-of-bounds access.
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_ERR_INVALID_ARG = -1, /* null pointer, bad shape or limit */
  TV_ERR_UNSUPPORTED = -2, /* dtype or head_dim outside what the kernels are built for */
  TV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than tree_verify_attn_workspace_size */
  TV_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Device status bits (per sequence b). */
#define TV_BAD_TREE 0x1 /* parent[0] != -1, or parent[i] < 0 or >= i for some i > 0 */
#define TV_OVERFLOW 0x2 /* cache_len[b] + accept_len[b] > Lmax: nothing committed */
#define TV_BAD_LEN 0x4  /* cache_len[b] < 0 or > Lmax */
#define TV_BAD_PATH 0x8 /* accept_len[b] outside [0, T] or an accepted index outside [0, T) */
#define TV_BAD_PAGE 0x10 /* paged K/V: a block-table entry or tree slot outside the pool */
#define TV_BAD_TOKEN 0x20 /* stochastic acceptance: a tried child's token outside [0, V) */
#define TV_SYNC_TIMEOUT 0x40 /* stochastic acceptance: its workgroups did not all meet (they were
                                not resident together); results invalid, re-zero the workspace */
#define TV_BAD_CONF 0x80 /* draft tree: a drafter confidence outside [0, 1] (used clamped) */
#define TV_FREE_FULL 0x100 /* paged commit: the free list had no room for some rejected slots */

/* Human-readable name of a tv_status return value or of a single status bit. */
const char* tv_status_string(int code);

/*
 * tree_build_mask — ancestor bitmask of every node.
 * Defined by the tree-attention mask of lesty.tech section 5 (mask[i, j] is set iff j is i or
 * an ancestor of i, found by following parent pointers) and the worked example of rainlin.net
 * section 4 ("good" sees exactly [It, is, a, good]).
 *
 *   parent    [B,T]    int32, -1 at the root
 *   anc_mask  [B,T,W]  uint64 out: bit j of row i set iff j is on the root-to-i path
 *   status    [B]      int32 out: WRITTEN (not OR-ed) with TV_BAD_TREE or 0.  For a bad tree
 *                      every row of that sequence is written with only its own bit set.
 */
int tree_build_mask(const int32_t* parent, int B, int T, uint64_t* anc_mask, int32_t* status,
                    void* stream);

/*
 * Bytes of workspace tree_verify_attn needs for these shapes and this split setting (0 when
 * the prefix is not split).  Deterministic for the same arguments on the same device.
 */
size_t tree_verify_attn_workspace_size(int B, int T, int Hq, int Hkv, int D, int Lmax, int dtype,
                                       int split_keys);

/*
 * tree_verify_attn — tree attention over the KV prefix plus each node's ancestors.
 * A tree node attends to every prefix row of its sequence and, among the tree's own rows, only
 * to the nodes on its root-to-node path; siblings are invisible (lesty.tech section 5; the
 * path-by-path equivalence of rainlin.net section 4).  Query head h reads KV head
 * h / (Hq / Hkv).  Scores are scale * q.k; softmax over the visible keys; output = weighted sum
 * of the visible V rows.
 *
 *   q          [B,T,Hq,D]      dtype   queries of the tree tokens
 *   k_cache    [B,Hkv,Lmax,D]  dtype   prefix keys; rows 0..cache_len[b]-1 are read, no others
 *   v_cache    [B,Hkv,Lmax,D]  dtype   prefix values, same rows
 *   cache_len  [B]             int32   prefix length L_b (clamped into [0, Lmax]; an
 *                                      out-of-range value sets TV_BAD_LEN in status)
 *   k_tree     [B,T,Hkv,D]     dtype   keys of the tree tokens
 *   v_tree     [B,T,Hkv,D]     dtype   values of the tree tokens
 *   anc_mask   [B,T,W]         uint64  from tree_build_mask (bit 0 must be set in every row)
 *   out        [B,T,Hq,D]      dtype   out: attention output (bf16 rounded to nearest even)
 *   lse        [B,T,Hq]        fp32    out, optional (NULL): natural-log sum of exp of scores
 *   status     [B]             int32   optional (NULL): TV_BAD_LEN is OR-ed in
 *   scale      <= 0 selects 1/sqrt(D)
 *   split_keys keys per split-K chunk, rounded up to a multiple of 64; a sequence's keys are
 *              counted as its tree tiles (ceil(T/64) tiles of 64) followed by its prefix.
 *              0 = automatic.  Results agree across split settings to rounding.
 *   workspace  device buffer of at least tree_verify_attn_workspace_size(...) bytes (may be
 *              NULL when that size is 0); holds per-split partial results, no state across
 *              calls.
 * Row offsets are 32-bit within one (b, kvh) cache slab and within one sequence's tree rows:
 * Lmax * D * elem and T * Hkv * D * elem may not exceed 4 GiB (TV_ERR_INVALID_ARG otherwise;
 * also for tree_verify_step).
 * q, k_cache, v_cache, k_tree and v_tree are read 16 bytes at a time, and out is written in
 * pieces of up to 16 bytes: each must be 16-byte aligned, as any device allocation is
 * (TV_ERR_INVALID_ARG otherwise; also for tree_verify_step and, with the pools in place of the
 * caches, the paged entry points).
 */
int tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cache_len, const void* k_tree, const void* v_tree,
                     const uint64_t* anc_mask, void* out, float* lse, int32_t* status, int B,
                     int T, int Hq, int Hkv, int D, int Lmax, int dtype, float scale,
                     int split_keys, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tv_profile_attn_main — profiling hook for the attention main kernel.
 * While set, every tree_verify_attn and tree_verify_step call launches its main kernel with
 * hipExtLaunchKernel so that `ev_before` and `ev_after` (hipEvent_t) take that kernel's own
 * start and end timestamps; hipEventElapsedTime then gives the main kernel's duration alone
 * (not the split-K merge, not the launch).  Pass NULL, NULL to turn it off.  Process-wide
 * setting, not synchronised: set it while no other thread calls either function.  Returns
 * TV_ERR_INVALID_ARG if exactly one event is NULL.
 */
int tv_profile_attn_main(void* ev_before, void* ev_after);

/*
 * tree_accept — greedy acceptance and the single longest accepted path.
 * A drafted token is accepted iff it equals the target model's greedy choice at its parent
 * (lesty.tech section 4); a node is accepted iff every node on its root path is; the root (the
 * token the target emitted last step) is always accepted.  The deepest accepted node is kept,
 * ties going to the smallest flattened index (lesty.tech section 8: only the single longest
 * accepted path is retained; rainlin.net section 3.2: the longest valid branch is accepted).
 *
 *   anc_mask     [B,T,W]  uint64  from tree_build_mask
 *   draft_tok    [B,T]    int32   drafted token of each node (entry 0 is not checked)
 *   target_tok   [B,T]    int32   target model's greedy token at each node
 *   accept_path  [B,T]    int32   out: accepted node indices root first, -1 after accept_len
 *   accept_len   [B]      int32   out: nodes kept, counting the root (>= 1)
 *   bonus_tok    [B]      int32   out: target_tok at the last kept node
 */
int tree_accept(const uint64_t* anc_mask, const int32_t* draft_tok, const int32_t* target_tok,
                int B, int T, int32_t* accept_path, int32_t* accept_len, int32_t* bonus_tok,
                void* stream);

/*
 * tree_accept_stochastic — acceptance under sampling (temperature > 0) by rejection sampling,
 * tried child by child (lesty.tech section 4: a drafted token x is kept with probability
 * min(1, p(x)/q(x)); after a rejection the token comes from the residual max(0, p - q),
 * normalised).  p[b,u,:] is the target model's next-token distribution after node u and
 * q[b,u,:] the draft model's, from which u's children were drawn.  From the root (always kept)
 * the walk tries the children of the current node in index order: child c with token x is kept
 * iff u_acc[b,c] * q_j(x) < p_j(x); a rejection replaces p_j by the residual for the next child
 * (and, with without_replacement = 1, removes x from q_j and renormalises it by 1 - q_j(x)).  The
 * first kept child becomes the current node.  When none is kept, the bonus token is the smallest
 * y whose running sum of p_j exceeds u_res[b,u] times its total (the last token with mass if
 * none does; -1 if p_j has none).  If a residual has no mass left (possible only when p or q
 * does not sum to one), no further child is tried and the bonus is drawn from the p_j the
 * rejected child faced.  Results are exact up to fp64 rounding: each rejection sums the
 * vocabulary once in fp64.
 *
 *   anc_mask     [B,T,W]  uint64  from tree_build_mask (a node's parent is its highest
 *                                 ancestor bit below itself)
 *   draft_tok    [B,T]    int32   drafted token of each node (entry 0 is not used)
 *   p, q         [B,T,V]  float32 non-negative distributions; q rows of childless nodes and p
 *                                 rows off the walk are not read
 *   u_acc, u_res [B,T]    float64 uniforms in [0, 1): u_acc[b,c] is used when child c is tried,
 *                                 u_res[b,u] when the bonus is drawn at u
 *   without_replacement   0: siblings are independent draws from q; 1: drawn without
 *                         replacement (q loses each rejected token)
 *   workgroups_per_seq    workgroups that share each vocabulary sweep of a sequence (0 =
 *                         automatic: as many as keep B * G within the compute units, at most
 *                         32, at least 2048 tokens each).  With G > 1 the workgroups of a
 *                         sequence exchange partial sums and must all be resident together:
 *                         B * G may not exceed the device's compute units (TV_ERR_INVALID_ARG).
 *   workspace    device buffer of tree_accept_stochastic_workspace_size(...) bytes (NULL
 *                allowed when that is 0), 16-byte aligned, zero-filled by the caller once
 *                before its first use and not written by the caller afterwards: every call
 *                leaves it all zeros again.  Calls that share a workspace must be ordered on
 *                one stream.
 *   accept_path, accept_len, bonus_tok   out, as for tree_accept
 *   status       [B]      int32   optional (NULL): TV_BAD_TOKEN OR-ed in when a child tried
 *                                 before the kept one (or any child, if none is kept) has a
 *                                 token outside [0, V); that child is skipped.
 *                                 TV_SYNC_TIMEOUT if the workgroups of a sequence did not all
 *                                 meet within about 0.1 s (another kernel held compute units)
 * Limits: 1 <= T <= 128, 1 <= V <= 1048576, 0 <= workgroups_per_seq <= 64.
 */
size_t tree_accept_stochastic_workspace_size(int B, int T, int V, int workgroups_per_seq);
int tree_accept_stochastic(const uint64_t* anc_mask, const int32_t* draft_tok, const float* p,
                           const float* q, const double* u_acc, const double* u_res, int B, int T,
                           int V, int without_replacement, int workgroups_per_seq,
                           void* workspace, size_t workspace_bytes, int32_t* accept_path,
                           int32_t* accept_len, int32_t* bonus_tok, int32_t* status, void* stream);

/*
 * tv_profile_accept_stochastic — profiling hook for tree_accept_stochastic's kernel, as
 * tv_profile_attn_main is for the attention: while set, the kernel is launched with
 * hipExtLaunchKernel so that the two hipEvent_t take its own start and end timestamps.  NULL,
 * NULL turns it off.  Process-wide, not synchronised.  TV_ERR_INVALID_ARG if exactly one event
 * is NULL.
 */
int tv_profile_accept_stochastic(void* ev_before, void* ev_after);

/*
 * kv_compact_accepted — commit the accepted path's K/V to the cache.
 * The tree's K/V rows were written to scratch during the verification pass; the surviving
 * path's rows enter the cache and the rejected ones are dropped (lesty.tech section 8).  For
 * every KV head, cache rows L_b .. L_b + accept_len[b] - 1 receive tree rows accept_path[b, 0..]
 * in path order; no other cache row is written; cache_len_out[b] = L_b + accept_len[b].
 *
 *   k_cache, v_cache  [B,Hkv,Lmax,D]  dtype  in/out
 *   cache_len         [B]             int32  L_b
 *   cache_len_out     [B]             int32  out; may be the same pointer as cache_len (it must
 *                                            then be exactly equal, not partly overlapping)
 *   k_tree, v_tree    [B,T,Hkv,D]     dtype  may live inside the cache: every accepted row of a
 *                                            (sequence, KV head) is read before any is written
 *   accept_path [B,T], accept_len [B]  int32  from tree_accept
 *   status            [B]             int32  optional (NULL): TV_BAD_LEN, TV_BAD_PATH or
 *                                            TV_OVERFLOW OR-ed in; such a sequence commits
 *                                            nothing and gets cache_len_out[b] = cache_len[b]
 */
int kv_compact_accepted(void* k_cache, void* v_cache, const int32_t* cache_len,
                        int32_t* cache_len_out, const void* k_tree, const void* v_tree,
                        const int32_t* accept_path, const int32_t* accept_len, int B, int T,
                        int Hkv, int D, int Lmax, int dtype, int32_t* status, void* stream);

/*
 * tree_verify_attn_paged — tree_verify_attn over a paged KV cache.
 * The K/V rows live in a pool of token slots, as in the PagedAttention scheme of lesty.tech
 * section 8: speculative tree nodes are written into reserved scratch slots of the pool and the
 * sequence's prefix is reached through a block table.  Results equal tree_verify_attn on the
 * dense cache those rows form.
 *
 *   k_pool, v_pool [num_slots,Hkv,D]  dtype   slot s holds one token's rows for every KV head
 *   block_table    [B,max_pages]      int32   page of each group of page_size positions:
 *                                             position p of sequence b is slot
 *                                             block_table[b][p / page_size] * page_size +
 *                                             p % page_size
 *   page_size      power of two >= 1
 *   cache_len      [B]                int32   L_b, clamped into [0, max_pages * page_size]
 *                                             (TV_BAD_LEN otherwise)
 *   tree_slot      [B,T]              int32   slot of each tree node's K/V rows
 *   other arguments as for tree_verify_attn, with Lmax = max_pages * page_size for the
 *   workspace size (tree_verify_attn_workspace_size).  A table entry or tree slot outside the
 *   pool is never read through: it is clamped into the pool and TV_BAD_PAGE is OR-ed into
 *   status[b].
 */
int tree_verify_attn_paged(const void* q, const void* k_pool, const void* v_pool, int num_slots,
                           const int32_t* block_table, int max_pages, int page_size,
                           const int32_t* cache_len, const int32_t* tree_slot,
                           const uint64_t* anc_mask, void* out, float* lse, int32_t* status,
                           int B, int T, int Hq, int Hkv, int D, int dtype, float scale,
                           int split_keys, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_commit_paged — commit the accepted path by pointer swap (lesty.tech section 8): the block
 * table's entries for positions L_b .. L_b + accept_len[b] - 1 take the accepted nodes' slots,
 * in path order, and the slots of the tree's rejected nodes are returned to the free list by
 * one atomic increment of free_top; no K/V row is copied.  Pages hold one token (page_size must
 * be 1: accepted nodes are scattered over the tree's slots, so only token-sized pages can adopt
 * them exactly; kv_compact_accepted is the copying commit).
 *
 *   block_table [B,max_pages]  int32  in/out
 *   cache_len, cache_len_out   as for kv_compact_accepted (may be the same pointer)
 *   tree_slot [B,T], accept_path [B,T], accept_len [B]  int32
 *   free_slots  [num_slots]    int32  out: rejected slots are written at free_top, free_top+1, ..
 *                                     in node order per sequence (the order between sequences
 *                                     follows the atomics); entries at or past num_slots are not
 *                                     written, and a sequence whose rejected slots do not all fit
 *                                     gets TV_FREE_FULL (which sequence that is, when several
 *                                     commit into a full list, follows the atomics)
 *   free_top    [1]            int32  in/out: advanced by the number of rejected nodes
 *   status      [B]            int32  optional (NULL): TV_BAD_LEN (cache_len outside
 *                                     [0, max_pages]), TV_BAD_PATH (bad accept_len, an accepted
 *                                     index outside [0, T) or repeated, a tree slot outside the
 *                                     pool) or TV_OVERFLOW (L_b + accept_len[b] > max_pages)
 *                                     OR-ed in; such a sequence commits nothing, frees nothing
 *                                     and keeps cache_len_out[b] = cache_len[b].  TV_FREE_FULL
 *                                     is OR-ed in as well by a sequence that committed but
 *                                     could not write every rejected slot
 */
int kv_commit_paged(int32_t* block_table, int max_pages, int page_size, const int32_t* cache_len,
                    int32_t* cache_len_out, const int32_t* tree_slot, const int32_t* accept_path,
                    const int32_t* accept_len, int32_t* free_slots, int32_t* free_top,
                    int num_slots, int B, int T, int32_t* status, void* stream);

/*
 * tree_verify_step — one whole verification step: tree_build_mask, tree_verify_attn,
 * tree_accept and kv_compact_accepted, in that order and with the same results and status
 * bits, fused into two kernel launches (the attention main kernel, which also builds the
 * ancestor masks; the split-K merge together with the acceptance walk and the compaction).  The step is the one
 * the pages describe: attention of the flattened tree (lesty.tech section 5), greedy
 * acceptance of the longest path (section 4; rainlin.net section 3.2), commit of its K/V
 * (lesty.tech section 8).
 *
 * Arguments are those of the four calls: parent, draft_tok, target_tok as for tree_build_mask
 * and tree_accept; q, k_cache, v_cache, cache_len, k_tree, v_tree, out, lse, scale,
 * split_keys, workspace as for tree_verify_attn (the same workspace size); anc_mask is an
 * output here; accept_path, accept_len, bonus_tok as for tree_accept; cache_len_out as for
 * kv_compact_accepted (it may be the same pointer as cache_len, not partly overlapping).
 * status [B] is required; it is written by the mask stage and OR-ed by the others.  When
 * k_tree or v_tree overlaps a cache buffer, the step runs the four calls one after the other,
 * so that rows are staged as kv_compact_accepted does.
 */
int tree_verify_step(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok,
                     const void* q, void* k_cache, void* v_cache, const int32_t* cache_len,
                     int32_t* cache_len_out, const void* k_tree, const void* v_tree,
                     uint64_t* anc_mask, void* out, float* lse, int32_t* accept_path,
                     int32_t* accept_len, int32_t* bonus_tok, int32_t* status, int B, int T,
                     int Hq, int Hkv, int D, int Lmax, int dtype, float scale, int split_keys,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * tree_verify_step_noalloc — tree_verify_step for callers that cannot allocate device memory:
 * code under HIP graph capture that may not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation.  It calls no allocating routine.  The split-K partials go to a device array
 * owned by the library, TV_NOALLOC_SCRATCH_BYTES on each GPU the library runs on, held until
 * the process ends; its device address is looked up once per device, on the first call with
 * that device current.
 *
 * Arguments, results and status bits as for tree_verify_step, without workspace and
 * workspace_bytes.  Returns TV_ERR_WORKSPACE, launching nothing, when
 * tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, Lmax, dtype, split_keys) exceeds
 * TV_NOALLOC_SCRATCH_BYTES.  The automatic split (split_keys = 0) always fits on a 256-CU
 * device: a plan splits only while there are fewer than 512 (sequence, KV head, row block)
 * units, so it holds fewer than 1024 partial slots of 256 rows x (D + 2) floats, at most
 * 136.2 MB.  An explicit split_keys may need more; a larger one needs less.
 * Every call on one GPU uses that GPU's one array, and each call rewrites what it reads, so no
 * state carries over between calls; calls that overlap in time on one GPU (on different
 * streams or from different host threads) race on the array and give wrong results.
 */
#define TV_NOALLOC_SCRATCH_BYTES (144u << 20)
int tree_verify_step_noalloc(const int32_t* parent, const int32_t* draft_tok,
                             const int32_t* target_tok, const void* q, void* k_cache,
                             void* v_cache, const int32_t* cache_len, int32_t* cache_len_out,
                             const void* k_tree, const void* v_tree, uint64_t* anc_mask,
                             void* out, float* lse, int32_t* accept_path, int32_t* accept_len,
                             int32_t* bonus_tok, int32_t* status, int B, int T, int Hq, int Hkv,
                             int D, int Lmax, int dtype, float scale, int split_keys,
                             void* stream);

/*
 * tree_verify_step_paged — the verification step over a paged cache: tree_build_mask,
 * tree_verify_attn_paged, tree_accept and kv_commit_paged, in that order and with the same
 * results and status bits, fused into two kernel launches (the paged attention main kernel,
 * which also builds the ancestor masks; the split-K merge together with the acceptance walk and
 * the pointer-swap commit).  The serving layout of lesty.tech section 8: the prefix in the
 * sequence's pages, the tree nodes in scratch slots of the same pool, the accepted nodes'
 * slots adopted by the block table and the rest returned to the free list.
 *
 * Arguments are those of the four calls: parent, draft_tok, target_tok as for tree_build_mask
 * and tree_accept; q, k_pool, v_pool, num_slots, block_table, max_pages, cache_len, tree_slot,
 * out, lse, scale, split_keys, workspace as for tree_verify_attn_paged (the same workspace
 * size); anc_mask is an output here; accept_path, accept_len, bonus_tok as for tree_accept;
 * block_table (in/out), cache_len_out, free_slots, free_top as for kv_commit_paged
 * (cache_len_out may be the same pointer as cache_len, not partly overlapping).  page_size
 * must be 1 (TV_ERR_UNSUPPORTED otherwise), as for kv_commit_paged.  status [B] is required;
 * it is written by the mask stage and OR-ed by the others.  The block table's entries that the
 * attention reads (positions below cache_len) and those the commit writes (from cache_len on)
 * do not meet, and the commit runs after every attention read.
 */
int tree_verify_step_paged(const int32_t* parent, const int32_t* draft_tok,
                           const int32_t* target_tok, const void* q, const void* k_pool,
                           const void* v_pool, int num_slots, int32_t* block_table, int max_pages,
                           int page_size, const int32_t* cache_len, int32_t* cache_len_out,
                           const int32_t* tree_slot, uint64_t* anc_mask, void* out, float* lse,
                           int32_t* accept_path, int32_t* accept_len, int32_t* bonus_tok,
                           int32_t* free_slots, int32_t* free_top, int32_t* status, int B, int T,
                           int Hq, int Hkv, int D, int dtype, float scale, int split_keys,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dynamic draft tree of EAGLE-2 (rainlin.net "EAGLE 系列", section 7), built on the device.
 *
 * Expansion (section 7.1): from the deepest level of the tree, the k nodes with the largest
 * global acceptance value go to the drafter for the next level, a node's value being the
 * product of the drafter's confidences on its root path.  Reranking (section 7.2): after the
 * last level, the T nodes of largest value are kept (a child never outranks its parent, so they
 * form a tree) and flattened into one sequence for verification.
 *
 * Node table of a sequence (caller-owned, row stride n_max): node_tok, node_parent (id of the
 * parent, -1 at the root) and node_value (float32).  The root is node 0 with value 1; child c of
 * frontier slot r of level l is node n_l + r * branch + c, where n_l = eagle2_node_count(l - 1,
 * k, branch) counts the nodes of the levels before.  Node A outranks node B iff A's value is
 * larger, or equal and A's id smaller (created earlier, so never deeper).  Values are float32
 * products parent value * confidence, rounded to nearest even; every decision compares them
 * exactly, so results are bit-exact.
 */

/* Nodes in the table after `depth` levels (the root, then branch children of every frontier
 * node of each level, a frontier holding min(k, children of its level) nodes); -1 for bad
 * arguments.  Host function, no device work. */
int eagle2_node_count(int depth, int k, int branch);

/*
 * eagle2_expand — level `level` (1, 2, ...) of the expansion, for every sequence.
 *
 *   root_tok    [B]              int32  token of the root (the token the target model emitted
 *                                       last); read at level 1 only (may be NULL otherwise)
 *   child_tok   [B,k,branch]     int32  the drafter's candidate tokens for each frontier slot
 *                                       (slot 0 only at level 1, whose parent is the root)
 *   child_conf  [B,k,branch]     fp32   their confidences; one outside [0, 1] (or NaN) is used
 *                                       clamped into it (NaN as 0) and TV_BAD_CONF is OR-ed in
 *   node_tok, node_parent, node_value  [B,n_max]  the node table: level 1 writes the root and
 *                                       its children, level l > 1 appends level l's nodes;
 *                                       n_max >= eagle2_node_count(level, k, branch)
 *   frontier    [B,k]            int32  in (level > 1): the previous level's frontier, as the
 *                                       previous call left it; out: this level's frontier, its
 *                                       min(k, children) best children, best first, then -1
 *   status      [B]              int32  OR-ed: TV_BAD_CONF; TV_BAD_TREE if a frontier entry is
 *                                       not a node of the previous level (that slot's children
 *                                       get parent -1 and value 0, and eagle2_rerank rejects
 *                                       the table)
 * Limits: B >= 1, level >= 1, k >= 1, branch >= 1, k * branch <= 1024.
 */
int eagle2_expand(const int32_t* root_tok, const int32_t* child_tok, const float* child_conf,
                  int B, int level, int k, int branch, int32_t* node_tok, int32_t* node_parent,
                  float* node_value, int n_max, int32_t* frontier, int32_t* status, void* stream);

/*
 * eagle2_rerank — keep the T best nodes of each table and flatten them in level order: by
 * depth, then by the flattened index of the parent, then by node id (siblings in the drafter's
 * order).  The output is a level-ordered tree with its root at 0, ready for tree_build_mask.
 *
 *   node_tok, node_parent, node_value  [B,n_max]  tables of n_nodes nodes (any source: they
 *                                       must form a tree with node 0 the root, parent ids below
 *                                       the node's own, no value above its parent's; NaN and
 *                                       negative values count as 0)
 *   parent_out  [B,T]  int32  out: flattened index of each position's parent (-1 at 0)
 *   tok_out     [B,T]  int32  out: its token (the draft tokens of the verification step)
 *   depth_out   [B,T]  int32  out: its depth (the root is 0; position offsets for the target)
 *   node_out    [B,T]  int32  out: its node id in the table
 *   status      [B]    int32  OR-ed: TV_BAD_TREE for a table that is not such a tree; its
 *                             outputs are parent -1, token -1, depth 0, node -1 everywhere
 * Limits: B >= 1, 1 <= T <= min(128, n_nodes), n_nodes <= min(n_max, 16384).
 */
int eagle2_rerank(const int32_t* node_tok, const int32_t* node_parent, const float* node_value,
                  int n_nodes, int n_max, int B, int T, int32_t* parent_out, int32_t* tok_out,
                  int32_t* depth_out, int32_t* node_out, int32_t* status, void* stream);

/*
 * Two-stage drafter LM head (jialefu.github.io, "EAGLE-4: Notes on the Efficient LM Head").
 *
 * Stage one scores the whole vocabulary with low-rank factors of the head, u = B h then A u,
 * and keeps candidates by a local top-k inside each tile of vocabulary rows (the rows of A were
 * shuffled before tiling; row_token names each row's token), so the approximate scores never
 * go to memory.  Stage two gathers the candidates' rows of the full head W and recomputes their
 * logits exactly.  The drafter's children are the K best candidates (their tokens and
 * confidences feed eagle2_expand).  h, A, B and W are bfloat16 (16-bit words); results are
 * float32.  The sums are float32 in an order of the kernels' own (fixed, so a call repeats
 * bit for bit); each value is therefore the exact dot product of its bfloat16 operands within
 * float32 rounding: d/64 + 6 roundings per term for u = B h and for the exact logits (each of
 * 64 lanes sums d/64 products, then six pairwise combining steps); for a screening score
 * A[row] . u[m], at most max(r, 16 + 3 ceil(r/16), 32 + 3 ceil(r/32)) roundings per term, with
 * u split exactly into three bfloat16 parts whose magnitudes add up to at most (1 + 2^-8) |u|
 * (ranks up to 256 run on the matrix cores, 16 or 32 products per instruction, then one rounding
 * per later instruction; larger ranks one chain over the rank index).  Choices made on such
 * values (which candidates a tile keeps, which children win) are those of the exact values
 * except where two of them lie within that rounding of each other.  Values rank by their float
 * order with -0 as +0 (a NaN score ranks above +inf with its sign bit clear, below -inf with it
 * set); equal values go to the smaller row of A (screening) or the smaller token (children).
 * h, B, A, W and u are read 16 bytes at a time: each must be 16-byte aligned (as any device
 * allocation is), else the call returns TV_ERR_INVALID_ARG.
 */

/* lm_head_project — u [M, r] fp32 = B [r, d] h [M, d] (rows of h are hidden states).
 * Limits: 1 <= M <= 64, r >= 1, d a positive multiple of 512. */
int lm_head_project(const void* h, const void* B, int M, int r, int d, float* u, void* stream);

/* lm_head_screen — local top-k screening.  A [n, r] bfloat16 (rows in shuffled order),
 * u [M, r] fp32 from lm_head_project, row_token [n] int32.  Tile t holds rows t*tile ..
 * t*tile + tile - 1 (the last one may be shorter); its k_tile best rows for hidden state m
 * become cand[m, t*k_tile + j] = row_token[row] (best first) with cand_score = the row's
 * score; a tile with fewer than k_tile rows pads with token -1 and score -inf.
 * C = ceil(n / tile) * k_tile candidates per hidden state.
 * Limits: 1 <= M <= 64, r a positive multiple of 8 with (M rounded up to the next of 2, 4, 6,
 * 8, 10, 12, 16, 24, 32, 48, 64) * r * 4 <= 65536, 1 <= tile <= 256, 1 <= k_tile <= 16. */
int lm_head_screen(const void* A, const float* u, const int32_t* row_token, int M, int r, int n,
                   int tile, int k_tile, int32_t* cand, float* cand_score, void* stream);

/* lm_head_rescore — exact logits of the candidates: logits [M, C] fp32 = W[cand[m, c]] . h[m]
 * with W [V, d] bfloat16 in token order.  A candidate outside [0, V) gets -inf; one other than
 * -1 also ORs TV_BAD_TOKEN into status[m] (status may be NULL).
 * Limits: 1 <= M <= 64, C >= 1, V >= 1, d a positive multiple of 512. */
int lm_head_rescore(const void* W, const void* h, const int32_t* cand, int M, int C, int d,
                    int V, float* logits, int32_t* status, void* stream);

/* lm_head_topk — the drafter's children: the K best valid candidates (tokens in [0, V)) of
 * each hidden state by exact logit, best first, out_tok [M, K] int32, and their confidences
 * out_conf [M, K] fp32, the softmax of the logits over all valid candidates of that hidden
 * state (fp32 sums; confidences agree with an fp64 evaluation to about 1e-6 relative).  With
 * fewer than K valid candidates the rest are token -1, confidence 0.  Every entry of cand is
 * a candidate of its own: a token listed twice (lm_head_screen never does) can be chosen twice
 * and counts twice in the softmax.
 * Limits: M >= 1, 1 <= C <= 8192, 1 <= K <= 64, V >= 1. */
int lm_head_topk(const float* logits, const int32_t* cand, int M, int C, int K, int V,
                 int32_t* out_tok, float* out_conf, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TREE_VERIFY_H */
