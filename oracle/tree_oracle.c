/*
 * CPU oracle for tree-attention verification of a speculative draft tree.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Everything is written as the plain definition, in fp64, with no blocking or fusion:
 *
 *   path(i)        root..i, found by following parent pointers until -1 and reversing
 *                  (lesty.tech "EAGLE-2 vs. Medusa", section 5, tree-attention mask code).
 *   mask row i     bit j set iff j lies on path(i): a node sees itself and its ancestors only,
 *                  never a sibling branch (same section; rainlin.net "EAGLE 系列", section 4,
 *                  where "good" sees exactly [It, is, a, good]).
 *   attention      for query head h of node i: ordinary softmax attention of q[b,i,h] over the
 *                  sequence prefix rows 0..L_b-1 followed by the K/V rows of path(i).  This is
 *                  the causal attention of the last position of prefix ++ path(i); a tree pass
 *                  equals verifying every root-to-node path on its own (rainlin.net section 4),
 *                  so no mask is needed.  Query head h reads KV head h / (Hq / Hkv).
 *   acceptance     greedy: a drafted token is accepted iff it equals the target model's choice
 *                  at its parent (lesty.tech section 4); a node is accepted iff every node on its
 *                  path is; the single longest accepted path is kept (lesty.tech section 8;
 *                  rainlin.net section 3.2).  Ties at equal depth go to the smallest index.
 *   compaction     the accepted path's K/V rows are appended to the cache after the prefix, in
 *                  path order, and nothing else is written (lesty.tech section 8).
 *   paged KV       (lesty.tech section 8, PagedAttention blocks) the K/V rows live in a pool of
 *                  token slots [num_slots, Hkv, D]; logical position p of sequence b is slot
 *                  table[b][p / P] * P + p % P for pages of P tokens, and tree node j is slot
 *                  tree_slot[b][j].  Attention over a paged cache is attention over the rows
 *                  the table names: oracle_paged_gather copies them into the dense layout.
 *                  Committing the accepted path by pointer swap makes the table's entries for
 *                  positions L_b .. L_b+n-1 name the accepted nodes' slots, in path order, and
 *                  returns the rejected nodes' slots to a free list; no row is copied.
 *   stochastic     (lesty.tech section 4, rejection sampling) a drafted token x is accepted with
 *   acceptance     probability min(1, p(x)/q(x)); after a rejection the residual
 *                  max(0, p - q), normalised, is what the next sibling is tested against, and
 *                  what the bonus token is drawn from when no child is accepted.  The random
 *                  numbers are inputs (one uniform per tested child, one per sampling node).
 *   draft tree     (rainlin.net "EAGLE 系列", section 7) EAGLE-2's dynamic tree: each level
 *   construction   expands the top-k nodes of the deepest layer by global acceptance value (the
 *                  product of the drafter's confidences on the root path), then all nodes are
 *                  reranked and the best T kept and flattened in level order.  Which node
 *                  outranks which is decided on float32 products, the precision of the GPU
 *                  kernels, since these decisions choose integers (node ids).
 *   drafter LM     (jialefu.github.io, EAGLE-4 efficient LM head) two stages: a low-rank head
 *   head           scores the vocabulary and a local top-k per tile of shuffled rows keeps
 *                  candidates; the full head's rows recompute their logits exactly; the
 *                  drafter's children are the best of them.  All in fp64 (plain dot
 *                  products); the float32 kernels are checked for validity against these
 *                  exact values within the float32 rounding bound.
 *
 * Floating inputs are either float32 (elem_bits = 32) or raw bfloat16 bit patterns
 * (elem_bits = 16), which are widened exactly.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BAD_TREE 0x1
#define ORC_OVERFLOW 0x2
#define ORC_BAD_LEN 0x4
#define ORC_BAD_PATH 0x8
#define ORC_FREE_FULL 0x100 /* pointer-swap commit: the free list had no room for a rejected slot */

/* ------------------------------------------------------------------------------------------ */
/* tree paths                                                                                  */
/* ------------------------------------------------------------------------------------------ */

/* A tree is valid iff node 0 is the only root and every other node's parent comes before it
 * (the flattened level order of the worked tree). */
static int tree_is_valid(const int32_t* parent, int T) {
  if (T < 1 || parent[0] != -1) return 0;
  for (int i = 1; i < T; ++i)
    if (parent[i] < 0 || parent[i] >= i) return 0;
  return 1;
}

/* Writes path(i) = [root, ..., parent(i), i] to out and returns its length.  For an invalid
 * tree every node's path is just the node itself. */
static int node_path(const int32_t* parent, int T, int valid, int i, int32_t* out) {
  (void)T;
  if (!valid) {
    out[0] = i;
    return 1;
  }
  int n = 0;
  for (int cur = i; cur != -1; cur = parent[cur]) out[n++] = cur;
  for (int a = 0, z = n - 1; a < z; ++a, --z) {
    int32_t t = out[a];
    out[a] = out[z];
    out[z] = t;
  }
  return n;
}

/* paths[i*T + k] = k-th node of path(i) (-1 past its length), plen[i] = its length.
 * Returns the status bits of the tree. */
int oracle_tree_paths(const int32_t* parent, int T, int32_t* paths, int32_t* plen) {
  int valid = tree_is_valid(parent, T);
  for (int i = 0; i < T; ++i) {
    for (int k = 0; k < T; ++k) paths[(size_t)i * T + k] = -1;
    plen[i] = node_path(parent, T, valid, i, paths + (size_t)i * T);
  }
  return valid ? 0 : ORC_BAD_TREE;
}

/* anc[b,i,w]: bit (j % 64) of word j / 64 is set iff node j is on path(i). */
void oracle_build_mask(const int32_t* parent, int B, int T, uint64_t* anc, int32_t* status) {
  int W = (T + 63) / 64;
  int32_t* path = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  for (int b = 0; b < B; ++b) {
    const int32_t* pb = parent + (size_t)b * T;
    int valid = tree_is_valid(pb, T);
    status[b] = valid ? 0 : ORC_BAD_TREE;
    for (int i = 0; i < T; ++i) {
      uint64_t* row = anc + ((size_t)b * T + i) * W;
      for (int w = 0; w < W; ++w) row[w] = 0;
      int n = node_path(pb, T, valid, i, path);
      for (int k = 0; k < n; ++k) row[path[k] / 64] |= (uint64_t)1 << (path[k] % 64);
    }
  }
  free(path);
}

/* ------------------------------------------------------------------------------------------ */
/* attention                                                                                   */
/* ------------------------------------------------------------------------------------------ */

static double load_elem(const void* base, size_t idx, int elem_bits) {
  if (elem_bits == 32) return (double)((const float*)base)[idx];
  uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef struct {
  int elem_bits;
  const void *q, *k_cache, *v_cache, *k_tree, *v_tree;
  const int32_t *cache_len, *parent;
  int B, T, Hq, Hkv, D, Lmax;
  double scale;
  const int32_t* rows; /* [n_rows*3] of (b, h, i), or NULL for every (b, i, h) in out's order */
  long n_rows;
  double *out, *lse;
  long next; /* work counter, protected by mu */
  pthread_mutex_t mu;
} attn_job;

/* One output row: softmax(scale * q . k_j) weighted sum of v_j over the prefix then path(i). */
static void attention_row(const attn_job* J, int b, int h, int i, double* o, double* lse_out,
                          double* s, int32_t* path) {
  const int D = J->D, G = J->Hq / J->Hkv, kvh = h / G;
  const int32_t* pb = J->parent + (size_t)b * J->T;
  int valid = tree_is_valid(pb, J->T);
  int npath = node_path(pb, J->T, valid, i, path);
  int L = J->cache_len[b];
  if (L < 0) L = 0;
  if (L > J->Lmax) L = J->Lmax;
  int nkeys = L + npath;
  size_t qoff = (((size_t)b * J->T + i) * J->Hq + h) * D;

  /* key j < L: prefix row j; key L + k: tree row path[k] */
  for (int j = 0; j < nkeys; ++j) {
    const void* kb;
    size_t koff;
    if (j < L) {
      kb = J->k_cache;
      koff = (((size_t)b * J->Hkv + kvh) * J->Lmax + j) * D;
    } else {
      kb = J->k_tree;
      koff = (((size_t)b * J->T + path[j - L]) * J->Hkv + kvh) * D;
    }
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += load_elem(J->q, qoff + d, J->elem_bits) * load_elem(kb, koff + d, J->elem_bits);
    s[j] = J->scale * dot;
  }
  double m = -INFINITY;
  for (int j = 0; j < nkeys; ++j)
    if (s[j] > m) m = s[j];
  double den = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    s[j] = exp(s[j] - m);
    den += s[j];
  }
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    const void* vb;
    size_t voff;
    if (j < L) {
      vb = J->v_cache;
      voff = (((size_t)b * J->Hkv + kvh) * J->Lmax + j) * D;
    } else {
      vb = J->v_tree;
      voff = (((size_t)b * J->T + path[j - L]) * J->Hkv + kvh) * D;
    }
    for (int d = 0; d < D; ++d) o[d] += s[j] * load_elem(vb, voff + d, J->elem_bits);
  }
  for (int d = 0; d < D; ++d) o[d] /= den;
  *lse_out = m + log(den);
}

static void* attention_worker(void* arg) {
  attn_job* J = (attn_job*)arg;
  double* s = (double*)malloc(sizeof(double) * ((size_t)J->Lmax + J->T));
  int32_t* path = (int32_t*)malloc(sizeof(int32_t) * (size_t)J->T);
  for (;;) {
    pthread_mutex_lock(&J->mu);
    long r = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (r >= J->n_rows) break;
    int b, h, i;
    if (J->rows) {
      b = J->rows[3 * r];
      h = J->rows[3 * r + 1];
      i = J->rows[3 * r + 2];
    } else { /* out is [B, T, Hq, D] */
      h = (int)(r % J->Hq);
      i = (int)((r / J->Hq) % J->T);
      b = (int)(r / ((long)J->Hq * J->T));
    }
    attention_row(J, b, h, i, J->out + (size_t)r * J->D, J->lse + r, s, path);
  }
  free(s);
  free(path);
  return NULL;
}

/* Tree attention of the selected rows (or of every row when rows == NULL, then out is
 * [B,T,Hq,D] and lse [B,T,Hq]).  Returns 0, or -1 on bad arguments. */
int oracle_attention(int elem_bits, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cache_len, const void* k_tree, const void* v_tree,
                     const int32_t* parent, int B, int T, int Hq, int Hkv, int D, int Lmax,
                     double scale, const int32_t* rows, long n_rows, double* out, double* lse,
                     int n_threads) {
  if ((elem_bits != 32 && elem_bits != 16) || B < 1 || T < 1 || Hkv < 1 ||
      Hq % Hkv != 0 || D < 1 || Lmax < 0)
    return -1;
  attn_job J;
  J.elem_bits = elem_bits;
  J.q = q;
  J.k_cache = k_cache;
  J.v_cache = v_cache;
  J.k_tree = k_tree;
  J.v_tree = v_tree;
  J.cache_len = cache_len;
  J.parent = parent;
  J.B = B;
  J.T = T;
  J.Hq = Hq;
  J.Hkv = Hkv;
  J.D = D;
  J.Lmax = Lmax;
  J.scale = scale;
  J.rows = rows;
  J.n_rows = rows ? n_rows : (long)B * T * Hq;
  J.out = out;
  J.lse = lse;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_t th[256];
  for (int t = 0; t < n_threads; ++t) pthread_create(&th[t], NULL, attention_worker, &J);
  for (int t = 0; t < n_threads; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* acceptance walk                                                                             */
/* ------------------------------------------------------------------------------------------ */

/* accept_path[b, :len] = path of the deepest accepted node (smallest index among equals),
 * -1 after it; accept_len[b] = its length (the root counts); bonus_tok[b] = target at it. */
void oracle_accept(const int32_t* parent, const int32_t* draft, const int32_t* target, int B,
                   int T, int32_t* accept_path, int32_t* accept_len, int32_t* bonus_tok) {
  char* acc = (char*)malloc((size_t)T);
  int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  for (int b = 0; b < B; ++b) {
    const int32_t* pb = parent + (size_t)b * T;
    const int32_t* db = draft + (size_t)b * T;
    const int32_t* tb = target + (size_t)b * T;
    int valid = tree_is_valid(pb, T);
    /* the root is the token the target model itself chose last step: always accepted */
    acc[0] = 1;
    depth[0] = 0;
    for (int c = 1; c < T; ++c) {
      if (!valid) {
        acc[c] = 0;
        depth[c] = 0;
        continue;
      }
      int p = pb[c]; /* p < c, so acc[p] and depth[p] are already known */
      acc[c] = acc[p] && db[c] == tb[p];
      depth[c] = depth[p] + 1;
    }
    int best = 0;
    for (int c = 1; c < T; ++c)
      if (acc[c] && depth[c] > depth[best]) best = c;
    int32_t* out = accept_path + (size_t)b * T;
    for (int k = 0; k < T; ++k) out[k] = -1;
    accept_len[b] = node_path(pb, T, valid, best, out);
    bonus_tok[b] = tb[best];
  }
  free(acc);
  free(depth);
}

/* ------------------------------------------------------------------------------------------ */
/* compaction                                                                                  */
/* ------------------------------------------------------------------------------------------ */

/* For each sequence b with L = cache_len[b] and n = accept_len[b]: cache rows L..L+n-1 of every
 * KV head receive tree rows accept_path[b, 0..n-1]; cache_len_out[b] = L + n.  Invalid lengths
 * or path entries, or L + n > Lmax, set status bits and commit nothing (cache_len_out[b] = L).
 * All source rows are read into a temporary before any row is written, so tree rows that live
 * inside the cache are handled too.  status bits are OR-ed in. */
void oracle_compact(int elem_bytes, void* k_cache, void* v_cache, const int32_t* cache_len,
                    int32_t* cache_len_out, const void* k_tree, const void* v_tree,
                    const int32_t* accept_path, const int32_t* accept_len, int B, int T, int Hkv,
                    int D, int Lmax, int32_t* status) {
  size_t row = (size_t)D * elem_bytes;
  unsigned char* tmp = (unsigned char*)malloc(row * 2 * (size_t)T * Hkv);
  for (int b = 0; b < B; ++b) {
    int L = cache_len[b];
    int n = accept_len[b];
    int bits = 0;
    if (L < 0 || L > Lmax) bits |= ORC_BAD_LEN;
    if (n < 0 || n > T) {
      bits |= ORC_BAD_PATH;
    } else {
      for (int k = 0; k < n; ++k) {
        int j = accept_path[(size_t)b * T + k];
        if (j < 0 || j >= T) bits |= ORC_BAD_PATH;
      }
    }
    if (!bits && (long)L + n > Lmax) bits |= ORC_OVERFLOW;
    status[b] |= bits;
    if (bits) {
      cache_len_out[b] = L;
      continue;
    }
    for (int h = 0; h < Hkv; ++h)
      for (int k = 0; k < n; ++k) {
        int j = accept_path[(size_t)b * T + k];
        size_t src = (((size_t)b * T + j) * Hkv + h) * row;
        memcpy(tmp + ((size_t)(h * n + k) * 2 + 0) * row, (const unsigned char*)k_tree + src, row);
        memcpy(tmp + ((size_t)(h * n + k) * 2 + 1) * row, (const unsigned char*)v_tree + src, row);
      }
    for (int h = 0; h < Hkv; ++h)
      for (int k = 0; k < n; ++k) {
        size_t dst = (((size_t)b * Hkv + h) * Lmax + L + k) * row;
        memcpy((unsigned char*)k_cache + dst, tmp + ((size_t)(h * n + k) * 2 + 0) * row, row);
        memcpy((unsigned char*)v_cache + dst, tmp + ((size_t)(h * n + k) * 2 + 1) * row, row);
      }
    cache_len_out[b] = L + n;
  }
  free(tmp);
}


/* ---- paged KV ------------------------------------------------------------------------------ */

/* Dense copies of the rows a paged cache names: k_cache/v_cache [B,Hkv,Lmax,D] receive rows
 * 0..L_b-1 of every sequence (other rows untouched), k_tree/v_tree [B,T,Hkv,D] the tree nodes'
 * rows.  Returns 0, or -1 if an entry names a slot outside the pool (nothing is read there). */
int oracle_paged_gather(int elem_bytes, const void* k_pool, const void* v_pool, int num_slots,
                        const int32_t* table, int max_pages, int page_size,
                        const int32_t* cache_len, const int32_t* tree_slot, int B, int T,
                        int Hkv, int D, int Lmax, void* k_cache, void* v_cache, void* k_tree,
                        void* v_tree) {
  size_t row = (size_t)D * elem_bytes;
  int rc = 0;
  for (int b = 0; b < B; ++b) {
    int L = cache_len[b];
    for (int p = 0; p < L && p < Lmax; ++p) {
      int page = table[(size_t)b * max_pages + p / page_size];
      long slot = (long)page * page_size + p % page_size;
      if (page < 0 || slot >= num_slots) {
        rc = -1;
        continue;
      }
      for (int h = 0; h < Hkv; ++h) {
        size_t src = ((size_t)slot * Hkv + h) * row;
        size_t dst = (((size_t)b * Hkv + h) * Lmax + p) * row;
        memcpy((unsigned char*)k_cache + dst, (const unsigned char*)k_pool + src, row);
        memcpy((unsigned char*)v_cache + dst, (const unsigned char*)v_pool + src, row);
      }
    }
    for (int j = 0; j < T; ++j) {
      int slot = tree_slot[(size_t)b * T + j];
      if (slot < 0 || slot >= num_slots) {
        rc = -1;
        continue;
      }
      for (int h = 0; h < Hkv; ++h) {
        size_t src = ((size_t)slot * Hkv + h) * row;
        size_t dst = (((size_t)b * T + j) * Hkv + h) * row;
        memcpy((unsigned char*)k_tree + dst, (const unsigned char*)k_pool + src, row);
        memcpy((unsigned char*)v_tree + dst, (const unsigned char*)v_pool + src, row);
      }
    }
  }
  return rc;
}

/* Commit of the accepted path by pointer swap, pages of one token.  For every sequence, in
 * order: the length, path and slots are checked (a failing sequence commits nothing and keeps
 * its length, as oracle_compact); then table[b][L + k] = tree_slot[b][path[k]] for k < n, and
 * the slots of the nodes not on the path are appended to free_slots in node order at
 * *free_top, which advances by their number; entries at or past num_slots are not written,
 * and a sequence with such an entry is flagged as having found the free list full. */
void oracle_commit_paged(int32_t* table, int max_pages, const int32_t* cache_len,
                         int32_t* cache_len_out, const int32_t* tree_slot,
                         const int32_t* accept_path, const int32_t* accept_len, int B, int T,
                         int num_slots, int32_t* free_slots, int32_t* free_top, int32_t* status) {
  unsigned char* on_path = (unsigned char*)malloc((size_t)T);
  for (int b = 0; b < B; ++b) {
    int L = cache_len[b];
    int n = accept_len[b];
    int bits = 0;
    if (L < 0 || L > max_pages) bits |= ORC_BAD_LEN;
    memset(on_path, 0, (size_t)T);
    if (n < 0 || n > T) {
      bits |= ORC_BAD_PATH;
    } else {
      for (int k = 0; k < n; ++k) {
        int j = accept_path[(size_t)b * T + k];
        if (j < 0 || j >= T || on_path[j]) bits |= ORC_BAD_PATH;
        else on_path[j] = 1;
      }
    }
    for (int j = 0; j < T; ++j) {
      int slot = tree_slot[(size_t)b * T + j];
      if (slot < 0 || slot >= num_slots) bits |= ORC_BAD_PATH;
    }
    if (!bits && (long)L + n > max_pages) bits |= ORC_OVERFLOW;
    status[b] |= bits;
    if (bits) {
      cache_len_out[b] = L;
      continue;
    }
    for (int k = 0; k < n; ++k)
      table[(size_t)b * max_pages + L + k] = tree_slot[(size_t)b * T + accept_path[(size_t)b * T + k]];
    for (int j = 0; j < T; ++j) {
      if (on_path[j]) continue;
      int at = (*free_top)++;
      if (at < num_slots) free_slots[at] = tree_slot[(size_t)b * T + j];
      else status[b] |= ORC_FREE_FULL;
    }
    cache_len_out[b] = L + n;
  }
  free(on_path);
}

/* ------------------------------------------------------------------------------------------ */
/* stochastic acceptance                                                                       */
/* ------------------------------------------------------------------------------------------ */

#define ORC_BAD_TOKEN 0x20

/* Inverse-CDF draw from the (unnormalised) distribution r[0..V-1]: the smallest y whose running
 * sum exceeds u times the total; the largest y with r[y] > 0 if none does; -1 if r has no mass. */
static int draw_token(const double* r, int V, double u) {
  double total = 0.0;
  for (int y = 0; y < V; ++y) total += r[y];
  const double thr = u * total;
  double run = 0.0;
  int last = -1;
  for (int y = 0; y < V; ++y) {
    if (r[y] > 0.0) last = y;
    run += r[y];
    if (run > thr && r[y] > 0.0) return y;
  }
  return last;
}

/* Rejection sampling over a draft tree (lesty.tech "EAGLE-2 vs. Medusa", section 4).
 *
 * p[b,u,:] is the target model's next-token distribution after node u and q[b,u,:] the draft
 * model's, from which u's children were drawn; the uniforms u_acc and u_res are fp64.  Starting
 * at the root (always kept), the walk
 * tries the children of the current node in index order.  A child with token x is accepted iff
 * u_acc[b,c] * q_j(x) < p_j(x), i.e. with probability min(1, p_j(x) / q_j(x)).  p_1 = p[b,u],
 * q_1 = q[b,u]; a rejection replaces p_j by the residual max(0, p_j - q_j) / sum(max(0, p_j - q_j))
 * for the next child, and with without_replacement != 0 also removes x from q_j and renormalises
 * it (q_{j+1} = q_j with q_j(x) set to zero, divided by 1 - q_j(x); all zero if that is not
 * positive).  An accepted child becomes the current node.  When no child is accepted, the bonus
 * token is drawn from the current p_j with u_res[b,u] (draw_token).  If a residual has no mass,
 * no further child is tried and the bonus is drawn from the p_j the rejected child faced.  A child
 * whose token lies outside [0, V) is skipped and ORC_BAD_TOKEN is OR-ed into status[b].
 * Outputs as oracle_accept. */
void oracle_accept_stochastic(const int32_t* parent, const int32_t* draft, const float* p,
                              const float* q, const double* u_acc, const double* u_res, int B,
                              int T, int V, int without_replacement, int32_t* accept_path,
                              int32_t* accept_len, int32_t* bonus_tok, int32_t* status) {
  double* pj = (double*)malloc(sizeof(double) * (size_t)V);
  double* qj = (double*)malloc(sizeof(double) * (size_t)V);
  double* res = (double*)malloc(sizeof(double) * (size_t)V);
  for (int b = 0; b < B; ++b) {
    const int32_t* pb = parent + (size_t)b * T;
    const int valid = tree_is_valid(pb, T);
    int32_t* out = accept_path + (size_t)b * T;
    for (int k = 0; k < T; ++k) out[k] = -1;
    int n = 0, u = 0;
    out[n++] = 0;
    for (;;) {
      const float* pu = p + ((size_t)b * T + u) * V;
      const float* qu = q + ((size_t)b * T + u) * V;
      for (int y = 0; y < V; ++y) {
        pj[y] = pu[y];
        qj[y] = qu[y];
      }
      int next = -1;
      for (int c = u + 1; c < T && valid; ++c) {
        if (pb[c] != u) continue;
        const int x = draft[(size_t)b * T + c];
        if (x < 0 || x >= V) {
          status[b] |= ORC_BAD_TOKEN;
          continue;
        }
        if (u_acc[(size_t)b * T + c] * qj[x] < pj[x]) {
          next = c;
          break;
        }
        double z = 0.0;
        for (int y = 0; y < V; ++y) {
          res[y] = pj[y] - qj[y] > 0.0 ? pj[y] - qj[y] : 0.0;
          z += res[y];
        }
        if (!(z > 0.0)) break; /* nothing left to resample from: draw from pj */
        for (int y = 0; y < V; ++y) pj[y] = res[y] / z;
        if (without_replacement) {
          const double keep = 1.0 - qj[x];
          qj[x] = 0.0;
          for (int y = 0; y < V; ++y) qj[y] = keep > 0.0 ? qj[y] / keep : 0.0;
        }
      }
      if (next < 0) {
        bonus_tok[b] = draw_token(pj, V, u_res[(size_t)b * T + u]);
        break;
      }
      out[n++] = next;
      u = next;
    }
    accept_len[b] = n;
  }
  free(pj);
  free(qj);
  free(res);
}

/* ------------------------------------------------------------------------------------------ */
/* EAGLE-2 dynamic draft tree: expansion, reranking, flattening                                */
/* ------------------------------------------------------------------------------------------ */

#define ORC_BAD_CONF 0x80

/* A drafter confidence used as a probability: NaN and negative values count as 0, values
 * above 1 as 1; anything outside [0, 1] is reported. */
static float conf_as_prob(float c, int32_t* st) {
  if (!(c >= 0.0f && c <= 1.0f)) *st |= ORC_BAD_CONF;
  return c > 0.0f ? (c < 1.0f ? c : 1.0f) : 0.0f;
}

/* A node value as it is ranked: NaN and negative values count as 0. */
static float rank_value(float v) { return v > 0.0f ? v : 0.0f; }

/* Node a outranks node b: a larger value, or the same value and a smaller id (created earlier,
 * hence never deeper). */
static int outranks(const float* value, int a, int b) {
  const float va = rank_value(value[a]), vb = rank_value(value[b]);
  return va > vb || (va == vb && a < b);
}

/* Reranking and flattening (rainlin.net "EAGLE 系列", section 7.2).
 *
 * The node table of sequence b holds n_nodes nodes (row stride n_max): node_parent[i] is the id
 * of i's parent (-1 for the root, node 0) and node_value[i] its global acceptance value.  The T
 * nodes that outrank all others are kept; when no child's value exceeds its parent's, the kept
 * set is a connected tree (a parent outranks its children).  The kept tree is flattened in level
 * order: by depth, then by the flattened index of the parent, then by node id (siblings are
 * created in the drafter's order).  Outputs per flattened position f: parent_out (flattened
 * index of the parent, -1 at the root), tok_out (node_tok), depth_out, node_out (node id).
 * A table that is not such a tree (node 0 not a root, a parent id not below the node's, a child
 * valued above its parent) sets ORC_BAD_TREE in status[b] (OR-ed) and gets parent -1, token -1,
 * depth 0 and node -1 at every position.  Requires 1 <= T <= n_nodes. */
void oracle_eagle2_rerank(const int32_t* node_tok, const int32_t* node_parent,
                          const float* node_value, int n_nodes, int n_max, int B, int T,
                          int32_t* parent_out, int32_t* tok_out, int32_t* depth_out,
                          int32_t* node_out, int32_t* status) {
  char* kept = (char*)malloc((size_t)n_nodes);
  int32_t* flat_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_nodes);
  int32_t* dep = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_nodes);
  for (int b = 0; b < B; ++b) {
    const int32_t* nt = node_tok + (size_t)b * n_max;
    const int32_t* np = node_parent + (size_t)b * n_max;
    const float* nv = node_value + (size_t)b * n_max;
    int32_t* po = parent_out + (size_t)b * T;
    int32_t* to = tok_out + (size_t)b * T;
    int32_t* dout = depth_out + (size_t)b * T;
    int32_t* no = node_out + (size_t)b * T;

    int valid = np[0] == -1 && T >= 1 && T <= n_nodes;
    for (int i = 1; i < n_nodes && valid; ++i) {
      const int p = np[i];
      if (p < 0 || p >= i || rank_value(nv[i]) > rank_value(nv[p])) valid = 0;
    }
    if (!valid) {
      status[b] |= ORC_BAD_TREE;
      for (int f = 0; f < T; ++f) {
        po[f] = -1;
        to[f] = -1;
        dout[f] = 0;
        no[f] = -1;
      }
      continue;
    }

    /* keep: T times, the best node not yet kept */
    memset(kept, 0, (size_t)n_nodes);
    for (int t = 0; t < T; ++t) {
      int best = -1;
      for (int i = 0; i < n_nodes; ++i)
        if (!kept[i] && (best < 0 || outranks(nv, i, best))) best = i;
      kept[best] = 1;
    }

    /* depth of every kept node: parent steps to the root */
    int max_depth = 0;
    for (int i = 0; i < n_nodes; ++i) {
      flat_of[i] = -1;
      if (!kept[i]) continue;
      int d = 0;
      for (int cur = i; np[cur] != -1; cur = np[cur]) ++d;
      dep[i] = d;
      if (d > max_depth) max_depth = d;
    }

    /* flatten level by level: within a level, smallest (parent's flattened index, id) first */
    int f = 0;
    for (int d = 0; d <= max_depth; ++d) {
      for (;;) {
        int best = -1;
        for (int i = 0; i < n_nodes; ++i) {
          if (!kept[i] || dep[i] != d || flat_of[i] >= 0) continue;
          if (best < 0) {
            best = i;
            continue;
          }
          const int pf_i = d == 0 ? -1 : flat_of[np[i]];
          const int pf_b = d == 0 ? -1 : flat_of[np[best]];
          if (pf_i < pf_b || (pf_i == pf_b && i < best)) best = i;
        }
        if (best < 0) break;
        flat_of[best] = f;
        po[f] = d == 0 ? -1 : flat_of[np[best]];
        to[f] = nt[best];
        dout[f] = d;
        no[f] = best;
        ++f;
      }
    }
  }
  free(kept);
  free(flat_of);
  free(dep);
}

/* Expansion (rainlin.net "EAGLE 系列", section 7.1) followed by reranking.
 *
 * The root (node 0, token root_tok[b]) has value 1.  Level l = 1 .. depth expands the frontier
 * of level l - 1 (the root alone for l = 1): the drafter gives frontier slot r the `branch`
 * candidate children child_tok / child_conf [l-1][b][r][c] (layout [depth, B, k, branch]).
 * Child c of slot r becomes node n_l + r * branch + c, where n_l counts the nodes of the levels
 * before; its value is its parent's value times its confidence, a float32 product (the
 * confidence taken as conf_as_prob; ORC_BAD_CONF is OR-ed in for one outside [0, 1]).  The
 * global acceptance value of a node is thus the product of the confidences on its root path.
 * The frontier of level l is the min(k, children of level l) children of that level that
 * outrank the others, best first; frontier_out [depth, B, k] (optional) receives it, padded
 * with -1.  The node table is written to node_tok / node_parent / node_value [B, n_max] and
 * reranked as oracle_eagle2_rerank.  Returns the node count, or -1 if it exceeds n_max. */
int oracle_eagle2_build(const int32_t* root_tok, const int32_t* child_tok,
                        const float* child_conf, int B, int depth, int k, int branch, int T,
                        int32_t* node_tok, int32_t* node_parent, float* node_value, int n_max,
                        int32_t* frontier_out, int32_t* parent_out, int32_t* tok_out,
                        int32_t* depth_out, int32_t* node_out, int32_t* status) {
  int n_nodes = 1;
  int32_t* front = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  char* picked = (char*)malloc((size_t)k * branch + 1);
  for (int b = 0; b < B; ++b) {
    int32_t* nt = node_tok + (size_t)b * n_max;
    int32_t* np = node_parent + (size_t)b * n_max;
    float* nv = node_value + (size_t)b * n_max;
    int32_t st = 0;
    nt[0] = root_tok[b];
    np[0] = -1;
    nv[0] = 1.0f;
    int n = 1, F = 1;
    front[0] = 0;
    for (int l = 1; l <= depth; ++l) {
      if (n + F * branch > n_max) {
        free(front);
        free(picked);
        return -1;
      }
      const int base = n;
      for (int r = 0; r < F; ++r)
        for (int c = 0; c < branch; ++c) {
          const size_t src = (((size_t)(l - 1) * B + b) * k + r) * branch + c;
          const int id = n++;
          const float prob = conf_as_prob(child_conf[src], &st);
          nt[id] = child_tok[src];
          np[id] = front[r];
          nv[id] = nv[front[r]] * prob;
        }
      const int Fn = n - base < k ? n - base : k;
      memset(picked, 0, (size_t)(n - base));
      for (int i = 0; i < Fn; ++i) {
        int best = -1;
        for (int j = base; j < n; ++j)
          if (!picked[j - base] && (best < 0 || outranks(nv, j, best))) best = j;
        picked[best - base] = 1;
        front[i] = best;
      }
      F = Fn;
      if (frontier_out)
        for (int i = 0; i < k; ++i)
          frontier_out[((size_t)(l - 1) * B + b) * k + i] = i < F ? front[i] : -1;
    }
    status[b] |= st;
    n_nodes = n;
  }
  free(front);
  free(picked);
  oracle_eagle2_rerank(node_tok, node_parent, node_value, n_nodes, n_max, B, T, parent_out,
                       tok_out, depth_out, node_out, status);
  return n_nodes;
}

/* ------------------------------------------------------------------------------------------ */
/* Two-stage drafter LM head (jialefu.github.io, "EAGLE-4: Notes on the Efficient LM Head")    */
/* ------------------------------------------------------------------------------------------ */
/*
 * Stage one scores the whole vocabulary with a low-rank head: u = B h, then A u, and keeps
 * candidates by a local top-k inside each tile of consecutive rows of A, whose rows were
 * shuffled beforehand (row_token[row] names the token of each row).  Stage two recomputes the
 * candidates' logits exactly from the full head's rows, W[token] . h.  The drafter's children
 * are the best of those candidates, with a softmax over the candidates as confidence.
 *
 * Everything here is the plain definition in fp64: each dot product is one loop in index order,
 * bfloat16 inputs widened exactly.  Ties at equal value go to the smaller row (screening) or
 * the smaller token (children).  The GPU kernels compute in float32; their choices are checked
 * for validity against these exact values and the float32 rounding bound, not bit for bit.
 */

static double bf16d(uint16_t b) {
  union {
    uint32_t u;
    float f;
  } x;
  x.u = (uint32_t)b << 16;
  return (double)x.f;
}

static double dot_bf16(const uint16_t* x, const uint16_t* y, int d) {
  double acc = 0.0;
  for (int i = 0; i < d; ++i) acc += bf16d(x[i]) * bf16d(y[i]);
  return acc;
}

/* u[m, i] = B[i, :] . h[m, :]; h [M, d], B [r, d] bfloat16 bits. */
void oracle_lm_project(const uint16_t* h, const uint16_t* Bm, int M, int r, int d, double* u) {
  for (int m = 0; m < M; ++m)
    for (int i = 0; i < r; ++i)
      u[(size_t)m * r + i] = dot_bf16(Bm + (size_t)i * d, h + (size_t)m * d, d);
}

/* Approximate score of every stored row of A [n, r] (bfloat16) for every hidden state:
 * s[m, row] = A[row, :] . u[m, :]. */
void oracle_lm_scores(const uint16_t* A, const double* u, int M, int r, int n, double* s) {
  for (int m = 0; m < M; ++m)
    for (int row = 0; row < n; ++row) {
      const uint16_t* a = A + (size_t)row * r;
      double acc = 0.0;
      for (int i = 0; i < r; ++i) acc += bf16d(a[i]) * u[(size_t)m * r + i];
      s[(size_t)m * n + row] = acc;
    }
}

/* Local top-k: tile t holds rows t*tile .. t*tile + tile - 1 (the last one may be shorter).
 * Its k_tile best rows by score (ties to the smaller row), best first, become candidates
 * cand[m, t * k_tile + j] = row_token[row] with score cand_score[m, t * k_tile + j]; a tile of
 * fewer rows pads with token -1 and score -inf.  s is oracle_lm_scores' output. */
void oracle_lm_screen(const double* s, const int32_t* row_token, int M, int n, int tile,
                      int k_tile, int32_t* cand, double* cand_score) {
  const int n_tiles = (n + tile - 1) / tile;
  const int C = n_tiles * k_tile;
  char* taken = (char*)malloc((size_t)tile);
  for (int m = 0; m < M; ++m) {
    const double* sm = s + (size_t)m * n;
    for (int t = 0; t < n_tiles; ++t) {
      const int r0 = t * tile, rows = n - r0 < tile ? n - r0 : tile;
      memset(taken, 0, (size_t)tile);
      for (int j = 0; j < k_tile; ++j) {
        int best = -1;
        for (int q = 0; q < rows; ++q)
          if (!taken[q] && (best < 0 || sm[r0 + q] > sm[r0 + best])) best = q;
        const size_t o = (size_t)m * C + (size_t)t * k_tile + j;
        if (best < 0) {
          cand[o] = -1;
          cand_score[o] = -INFINITY;
        } else {
          taken[best] = 1;
          cand[o] = row_token[r0 + best];
          cand_score[o] = sm[r0 + best];
        }
      }
    }
  }
  free(taken);
}

/* Exact logits of the candidates: logits[m, c] = W[cand[m, c], :] . h[m, :], W [V, d]
 * bfloat16 in token order.  A candidate outside [0, V) gets -inf, and one other than -1 (the
 * padding of a short tile) sets ORC_BAD_TOKEN in status[m]. */
void oracle_lm_rescore(const uint16_t* W, const uint16_t* h, const int32_t* cand, int M, int C,
                       int d, int V, double* logits, int32_t* status) {
  for (int m = 0; m < M; ++m)
    for (int c = 0; c < C; ++c) {
      const int tok = cand[(size_t)m * C + c];
      if (tok < 0 || tok >= V) {
        logits[(size_t)m * C + c] = -INFINITY;
        if (tok != -1) status[m] |= ORC_BAD_TOKEN;
        continue;
      }
      logits[(size_t)m * C + c] = dot_bf16(W + (size_t)tok * d, h + (size_t)m * d, d);
    }
}

/* Exact logit of every vocabulary token: logits[m, v] = W[v, :] . h[m, :] (the full head;
 * what stage two evaluates at the candidates).  Rows are split over n_threads threads. */
struct lm_all_job {
  const uint16_t *W, *h;
  int M, d, V, v0, v1;
  double* logits;
};

static void* lm_all_worker(void* arg) {
  const struct lm_all_job* J = (const struct lm_all_job*)arg;
  for (int m = 0; m < J->M; ++m)
    for (int v = J->v0; v < J->v1; ++v)
      J->logits[(size_t)m * J->V + v] =
          dot_bf16(J->W + (size_t)v * J->d, J->h + (size_t)m * J->d, J->d);
  return NULL;
}

void oracle_lm_logits_all(const uint16_t* W, const uint16_t* h, int M, int d, int V,
                          double* logits, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 64) n_threads = 64;
  pthread_t th[64];
  struct lm_all_job jobs[64];
  for (int k = 0; k < n_threads; ++k) {
    jobs[k].W = W;
    jobs[k].h = h;
    jobs[k].M = M;
    jobs[k].d = d;
    jobs[k].V = V;
    jobs[k].v0 = (int)((long)V * k / n_threads);
    jobs[k].v1 = (int)((long)V * (k + 1) / n_threads);
    jobs[k].logits = logits;
  }
  int started = 0;
  for (int k = 1; k < n_threads; ++k)
    if (pthread_create(&th[k], NULL, lm_all_worker, &jobs[k]) == 0) ++started;
    else lm_all_worker(&jobs[k]);
  lm_all_worker(&jobs[0]);
  for (int k = 1; k <= started; ++k) pthread_join(th[k], NULL);
}

/* The drafter's children: the K best valid candidates of hidden state m (by logit, ties to the
 * smaller token), best first, and their confidences, the softmax of the logits over all valid
 * candidates of m.  Fewer than K valid candidates pad with token -1, confidence 0.  A token
 * listed twice among the candidates counts twice, as two candidates. */
void oracle_lm_topk(const double* logits, const int32_t* cand, int M, int C, int K, int V,
                    int32_t* out_tok, double* out_conf) {
  char* taken = (char*)malloc((size_t)C);
  for (int m = 0; m < M; ++m) {
    const double* l = logits + (size_t)m * C;
    const int32_t* cm = cand + (size_t)m * C;
    double mx = -INFINITY;
    for (int c = 0; c < C; ++c) {
      taken[c] = !(cm[c] >= 0 && cm[c] < V);
      if (!taken[c] && l[c] > mx) mx = l[c];
    }
    double z = 0.0;
    for (int c = 0; c < C; ++c)
      if (!taken[c]) z += exp(l[c] - mx);
    for (int j = 0; j < K; ++j) {
      int best = -1;
      for (int c = 0; c < C; ++c) {
        if (taken[c]) continue;
        if (best < 0 || l[c] > l[best] || (l[c] == l[best] && cm[c] < cm[best])) best = c;
      }
      if (best < 0) {
        out_tok[(size_t)m * K + j] = -1;
        out_conf[(size_t)m * K + j] = 0.0;
      } else {
        taken[best] = 1;
        out_tok[(size_t)m * K + j] = cm[best];
        out_conf[(size_t)m * K + j] = exp(l[best] - mx) / z;
      }
    }
  }
  free(taken);
}
