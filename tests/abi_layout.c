/* Prints the size and every field offset of the public structs of
 * include/blockattn.h, one "struct field offset" line each, so that a test can
 * compare them with the Python binding's ctypes declarations. */
#include <stddef.h>
#include <stdio.h>

#include "blockattn.h"

#define F(s, f) printf("%s %s %zu\n", #s, #f, offsetof(s, f))
#define SZ(s) printf("%s sizeof %zu\n", #s, sizeof(s))

int main(void) {
  SZ(ba_problem);
  F(ba_problem, n_q_heads); F(ba_problem, n_kv_heads); F(ba_problem, head_dim); F(ba_problem, q_len);
  F(ba_problem, q_pos0); F(ba_problem, q_stride_token); F(ba_problem, q_stride_head); F(ba_problem, dtype);
  F(ba_problem, scale); F(ba_problem, causal); F(ba_problem, split_mode); F(ba_problem, batch);
  F(ba_problem, q_stride_batch);
  SZ(ba_kv_block);
  F(ba_kv_block, k); F(ba_kv_block, v); F(ba_kv_block, len); F(ba_kv_block, pos0);
  F(ba_kv_block, k_stride_token); F(ba_kv_block, k_stride_head); F(ba_kv_block, v_stride_token);
  F(ba_kv_block, v_stride_head); F(ba_kv_block, k_stride_batch); F(ba_kv_block, v_stride_batch);
  SZ(ba_state);
  F(ba_state, m); F(ba_state, l); F(ba_state, o);
  SZ(ba_fanout);
  F(ba_fanout, n_branches); F(ba_fanout, n_q_heads); F(ba_fanout, n_kv_heads); F(ba_fanout, head_dim);
  F(ba_fanout, prefix_len); F(ba_fanout, suffix_len); F(ba_fanout, scale);
  SZ(ba_fanout_prefill);
  F(ba_fanout_prefill, n_branches); F(ba_fanout_prefill, n_new); F(ba_fanout_prefill, n_q_heads);
  F(ba_fanout_prefill, n_kv_heads); F(ba_fanout_prefill, head_dim); F(ba_fanout_prefill, prefix_len);
  F(ba_fanout_prefill, suffix_len); F(ba_fanout_prefill, scale);
  SZ(ba_kv_pages);
  F(ba_kv_pages, prefix_pages); F(ba_kv_pages, suffix_pages); F(ba_kv_pages, page_len);
  F(ba_kv_pages, n_pool_pages);
  return 0;
}
