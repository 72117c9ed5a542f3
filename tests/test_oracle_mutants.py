"""Plausible mistakes planted in copies of the oracle source must each fail at least one pin.

The oracle itself is never modified: each case copies ``oracle/tree_oracle.c``, replaces one
snippet, compiles the copy into a temporary library and runs every pin against it.  CPU only.
"""
import os

import pytest

import pins
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "tree_oracle.c")

MUTANTS = {
    # a node does not see itself
    "path_without_self": ("for (int cur = i; cur != -1; cur = parent[cur]) out[n++] = cur;",
                          "for (int cur = (i ? parent[i] : i); cur != -1; cur = parent[cur]) "
                          "out[n++] = cur;"),
    # path kept in walk order (node first) instead of root first
    "path_not_reversed": ("for (int a = 0, z = n - 1; a < z; ++a, --z) {",
                          "for (int a = 0, z = -1; a < z; ++a, --z) {"),
    # mask bits numbered from the top of the word
    "mask_bit_order": ("row[path[k] / 64] |= (uint64_t)1 << (path[k] % 64);",
                       "row[path[k] / 64] |= (uint64_t)1 << (63 - path[k] % 64);"),
    # one prefix row dropped
    "prefix_off_by_one": ("int nkeys = L + npath;", "int nkeys = (L > 0 ? L - 1 : 0) + npath;"),
    # query heads mapped round-robin instead of in contiguous groups
    "gqa_round_robin": ("kvh = h / G;", "kvh = h % J->Hkv;"),
    # scale ignored
    "no_scale": ("s[j] = J->scale * dot;", "s[j] = dot;"),
    # tree keys taken by position instead of by path node
    "tree_row_by_position": ("koff = (((size_t)b * J->T + path[j - L]) * J->Hkv + kvh) * D;",
                             "koff = (((size_t)b * J->T + (j - L)) * J->Hkv + kvh) * D;"),
    # values read from the key tensor for the tree part
    "tree_values_from_keys": ("vb = J->v_tree;", "vb = J->k_tree;"),
    # log-sum-exp without the running maximum
    "lse_without_max": ("*lse_out = m + log(den);", "*lse_out = log(den);"),
    # a draft compared with the target at its own position instead of its parent's
    "accept_own_target": ("acc[c] = acc[p] && db[c] == tb[p];", "acc[c] = acc[p] && db[c] == tb[c];"),
    # acceptance ignores whether the ancestors were accepted
    "accept_ignores_ancestors": ("acc[c] = acc[p] && db[c] == tb[p];", "acc[c] = db[c] == tb[p];"),
    # equal depth resolved towards the largest index
    "accept_tie_largest": ("if (acc[c] && depth[c] > depth[best]) best = c;",
                           "if (acc[c] && depth[c] >= depth[best]) best = c;"),
    # first accepted child rather than the longest path
    "accept_first_match": ("if (acc[c] && depth[c] > depth[best]) best = c;",
                           "if (acc[c] && depth[c] == depth[best] + 1 && pb[c] == best) best = c;"),
    # bonus token taken at the parent of the last kept node
    "bonus_at_parent": ("bonus_tok[b] = tb[best];", "bonus_tok[b] = tb[best ? pb[best] : 0];"),
    # compaction writes one row too far
    "compact_shifted": ("size_t dst = (((size_t)b * Hkv + h) * Lmax + L + k) * row;",
                        "size_t dst = (((size_t)b * Hkv + h) * Lmax + L + k + (k > 0)) * row;"),
    # compaction length excludes the root
    "compact_len": ("cache_len_out[b] = L + n;\n  }\n  free(tmp);",
                    "cache_len_out[b] = L + n - 1;\n  }\n  free(tmp);"),
    # pointer-swap commit length excludes the root
    "commit_len": ("cache_len_out[b] = L + n;\n  }\n  free(on_path);",
                   "cache_len_out[b] = L + n - 1;\n  }\n  free(on_path);"),
    # overflow check off by one
    "compact_overflow": ("if (!bits && (long)L + n > Lmax) bits |= ORC_OVERFLOW;",
                         "if (!bits && (long)L + n > Lmax + 1) bits |= ORC_OVERFLOW;"),
    # paged gather ignores the offset within a page
    "paged_no_offset": ("long slot = (long)page * page_size + p % page_size;",
                        "long slot = (long)page * page_size;"),
    # paged gather indexes the table by position instead of by page
    "paged_table_by_position": ("int page = table[(size_t)b * max_pages + p / page_size];",
                                "int page = table[(size_t)b * max_pages + p % max_pages];"),
    # tree rows read at the node's index instead of its slot
    "paged_tree_by_index": ("int slot = tree_slot[(size_t)b * T + j];\n      if (slot < 0 || slot >= num_slots) {\n        rc = -1;",
                            "int slot = j;\n      if (slot < 0 || slot >= num_slots) {\n        rc = -1;"),
    # commit adopts the slots in node order rather than path order (same set)
    "commit_node_order": ("table[(size_t)b * max_pages + L + k] = tree_slot[(size_t)b * T + accept_path[(size_t)b * T + k]];",
                          "table[(size_t)b * max_pages + L + k] = tree_slot[(size_t)b * T + accept_path[(size_t)b * T + (n - 1 - k)]];"),
    # accepted nodes' slots also returned to the free list
    "commit_frees_accepted": ("      if (on_path[j]) continue;\n", ""),
    # commit overflow check off by one
    "commit_overflow": ("if (!bits && (long)L + n > max_pages) bits |= ORC_OVERFLOW;",
                        "if (!bits && (long)L + n > max_pages + 1) bits |= ORC_OVERFLOW;"),
    # stochastic: residual without the clamp at zero
    "stoch_residual_no_max": ("res[y] = pj[y] - qj[y] > 0.0 ? pj[y] - qj[y] : 0.0;",
                              "res[y] = pj[y] - qj[y];"),
    # stochastic: residual not renormalised
    "stoch_residual_unnormalised": ("for (int y = 0; y < V; ++y) pj[y] = res[y] / z;",
                                    "for (int y = 0; y < V; ++y) pj[y] = res[y];"),
    # stochastic: ratio upside down
    "stoch_ratio_inverted": ("if (u_acc[(size_t)b * T + c] * qj[x] < pj[x]) {",
                             "if (u_acc[(size_t)b * T + c] * pj[x] < qj[x]) {"),
    # stochastic, without replacement: the rejected token stays in q
    "stoch_q_keeps_rejected": ("          qj[x] = 0.0;\n", ""),
    # stochastic, without replacement: q not renormalised after the removal
    "stoch_q_unnormalised": ("qj[y] = keep > 0.0 ? qj[y] / keep : 0.0;", "qj[y] = qj[y];"),
    # stochastic: bonus drawn from the target distribution instead of the residual
    "stoch_bonus_from_p": ("bonus_tok[b] = draw_token(pj, V, u_res[(size_t)b * T + u]);",
                           "for (int y = 0; y < V; ++y) res[y] = pu[y];\n"
                           "        bonus_tok[b] = draw_token(res, V, u_res[(size_t)b * T + u]);"),
    # stochastic: children tried from the last index down
    "stoch_children_reversed": ("for (int c = u + 1; c < T && valid; ++c) {",
                                "for (int c = T - 1; c > u && valid; --c) {"),
    # stochastic: the bonus uses the parent's uniform
    "stoch_uniform_of_parent": ("draw_token(pj, V, u_res[(size_t)b * T + u]);",
                                "draw_token(pj, V, u_res[(size_t)b * T + (u ? pb[u] : 0)]);"),
    # stochastic: no guard for a residual without mass
    "stoch_no_zero_guard": ("if (!(z > 0.0)) break; /* nothing left to resample from: draw from pj */",
                            ""),
    # stochastic: an out-of-vocabulary child is tested (as token 0) instead of skipped
    "stoch_bad_token_tested": ("          status[b] |= ORC_BAD_TOKEN;\n          continue;\n", ""),
    # draft tree: a node's value is its own confidence, not the path product
    "e2_value_not_product": ("nv[id] = nv[front[r]] * prob;", "nv[id] = prob;"),
    # draft tree: every child hung under the best frontier node
    "e2_parent_first_slot": ("np[id] = front[r];", "np[id] = front[0];"),
    # draft tree: equal values go to the larger id
    "e2_tie_larger_id": ("return va > vb || (va == vb && a < b);",
                         "return va > vb || (va == vb && a > b);"),
    # draft tree: the frontier keeps the worst children
    "e2_frontier_worst": ("if (!picked[j - base] && (best < 0 || outranks(nv, j, best))) best = j;",
                          "if (!picked[j - base] && (best < 0 || outranks(nv, best, j))) best = j;"),
    # draft tree: the rerank keeps the T earliest nodes whatever their values
    "e2_rerank_by_id": ("if (!kept[i] && (best < 0 || outranks(nv, i, best))) best = i;",
                        "if (!kept[i] && (best < 0 || i < best)) best = i;"),
    # draft tree: a level flattened by node id, ignoring the parents' flattened order
    "e2_flatten_by_id": ("if (pf_i < pf_b || (pf_i == pf_b && i < best)) best = i;",
                         "if (i < best) best = i;"),
    # draft tree: siblings flattened in reverse
    "e2_siblings_reversed": ("if (pf_i < pf_b || (pf_i == pf_b && i < best)) best = i;",
                             "if (pf_i < pf_b || (pf_i == pf_b && i > best)) best = i;"),
    # draft tree: confidences used unclamped
    "e2_conf_unclamped": ("return c > 0.0f ? (c < 1.0f ? c : 1.0f) : 0.0f;", "return c;"),
    # draft tree: bad confidences not reported
    "e2_conf_not_flagged": ("if (!(c >= 0.0f && c <= 1.0f)) *st |= ORC_BAD_CONF;", ""),
    # draft tree: a child valued above its parent accepted as a tree
    "e2_table_allows_growth": ("if (p < 0 || p >= i || rank_value(nv[i]) > rank_value(nv[p])) valid = 0;",
                               "if (p < 0 || p >= i) valid = 0;"),
    # draft tree: flattened depth counted from one
    "e2_depth_from_one": ("        dout[f] = d;\n", "        dout[f] = d + 1;\n"),
    # LM head: the projection uses h's row for B's index
    "lm_project_swapped": ("u[(size_t)m * r + i] = dot_bf16(Bm + (size_t)i * d, h + (size_t)m * d, d);",
                           "u[(size_t)m * r + i] = dot_bf16(Bm + (size_t)(i % r) * d, h + (size_t)(i % M) * d, d);"),
    # LM head: a dot product that skips its first element
    "lm_dot_skips_first": ("for (int i = 0; i < d; ++i) acc += bf16d(x[i]) * bf16d(y[i]);",
                           "for (int i = 1; i < d; ++i) acc += bf16d(x[i]) * bf16d(y[i]);"),
    # LM head: screening scores from the hidden state's first r elements instead of u = B h
    "lm_scores_skip_projection": ("for (int i = 0; i < r; ++i) acc += bf16d(a[i]) * u[(size_t)m * r + i];",
                                  "for (int i = 0; i < r; ++i) acc += bf16d(a[i]) * (double)(i == 0);"),
    # LM head: equal scores go to the larger row
    "lm_screen_tie_larger": ("if (!taken[q] && (best < 0 || sm[r0 + q] > sm[r0 + best])) best = q;",
                             "if (!taken[q] && (best < 0 || sm[r0 + q] >= sm[r0 + best])) best = q;"),
    # LM head: the last row of every tile never considered
    "lm_tile_drops_last_row": ("const int r0 = t * tile, rows = n - r0 < tile ? n - r0 : tile;",
                               "const int r0 = t * tile, rows = n - r0 < tile - 1 ? n - r0 : tile - 1;"),
    # LM head: candidates reported by row instead of token
    "lm_cand_is_row": ("cand[o] = row_token[r0 + best];", "cand[o] = r0 + best;"),
    # LM head: the exact logits read W's row by candidate slot instead of token
    "lm_rescore_by_slot": ("logits[(size_t)m * C + c] = dot_bf16(W + (size_t)tok * d, h + (size_t)m * d, d);",
                           "logits[(size_t)m * C + c] = dot_bf16(W + (size_t)(c % V) * d, h + (size_t)m * d, d);"),
    # LM head: the full head's logits one row off
    "lm_logits_all_shifted": ("dot_bf16(J->W + (size_t)v * J->d, J->h + (size_t)m * J->d, J->d);",
                              "dot_bf16(J->W + (size_t)((v + 1) % J->V) * J->d, J->h + (size_t)m * J->d, J->d);"),
    # LM head: equal logits go to the larger token
    "lm_topk_tie_larger": ("if (best < 0 || l[c] > l[best] || (l[c] == l[best] && cm[c] < cm[best])) best = c;",
                           "if (best < 0 || l[c] > l[best] || (l[c] == l[best] && cm[c] > cm[best])) best = c;"),
    # LM head: confidences normalised over the chosen children only
    "lm_conf_over_chosen": ("out_conf[(size_t)m * K + j] = exp(l[best] - mx) / z;",
                            "out_conf[(size_t)m * K + j] = exp(l[best] - mx) / (z > 0 ? 1.0 : z);"),
    # LM head: out-of-vocabulary candidates not reported
    "lm_bad_token_silent": ("if (tok != -1) status[m] |= ORC_BAD_TOKEN;", ""),
    # paged commit: a full free list not reported
    "commit_free_full_silent": ("else status[b] |= ORC_FREE_FULL;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site of {name} not found once in the oracle source"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new), encoding="utf-8")
    so = O.build(str(mutant_src), str(tmp_path / "libmutant.so"))
    lib = O.load(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
            break
        except Exception as e:  # a crash or bad value in the mutant also counts as caught
            caught.append(f"{pin.__name__}:{type(e).__name__}")
            break
    assert caught, f"mutant {name} passed every pin"
