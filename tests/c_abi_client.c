/* A plain C99 client of the wavefront-round library: no Python, no torch.
 *
 * Builds a request through the C ABI alone (include/wf.h, include/wf_dit.h),
 * prints every round's plan as one JSON object per line, then the page
 * layout, the split the attention would make in a steady round, and the
 * status codes of calls that must fail.  Host-only calls: it needs no GPU.
 * tests/test_c_abi.py compiles it, runs it and compares what it prints with
 * the oracle.
 *
 * usage: c_abi_client S W W_store anchor n_chunk F Hh Ww heads head_dim layers dtype mask
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wf.h"
#include "wf_dit.h"

static int fail_if(int cond, const char* what) {
  if (cond) fprintf(stderr, "c_abi_client: %s (%s)\n", what, wf_last_error());
  return cond;
}

static void print_plan(const wf_plan* p) {
  int s, j;
  printf("{\"k\": %lld, \"n_active\": %d, \"evict\": %d, \"kv_tokens\": %lld, \"flops\": %.17g, ",
         (long long)p->k, p->n_active, p->evict_chunk, (long long)p->kv_tokens, p->flops);
  printf("\"anchor\": [%d, %d, %d, %d], \"cells\": [", p->anchor.present, p->anchor.slot,
         p->anchor.frame0, p->anchor.capture);
  for (s = 0; s <= p->S; ++s) {
    const wf_cell* c = &p->cells[s];
    printf("%s[%d, %d, %d, %d, %d]", s ? ", " : "", c->stage, c->chunk, c->active, c->slot, c->frame0);
  }
  printf("], \"groups\": [");
  for (s = 0; s <= p->S; ++s) {
    const wf_group* g = &p->groups[s];
    printf("%s[", s ? ", " : "");
    for (j = 0; j < g->n_pages; ++j)
      printf("%s[%d, %d, %d]", j ? ", " : "", g->kind[j], g->chunk[j], g->slot[j]);
    printf("]");
  }
  printf("]}\n");
}

int main(int argc, char** argv) {
  wf_config cfg;
  wf_handle* h = NULL;
  wf_handle* other = NULL;
  wf_layout lay;
  wf_plan plan;
  size_t pool = 0, anchor = 0, tables = 0;
  int32_t n_split = 0, stage[WF_MAX_SPLIT], at[WF_MAX_SPLIT];
  int64_t k, rounds;
  int i;

  if (argc != 14) {
    fprintf(stderr, "usage: %s S W W_store anchor n_chunk F Hh Ww heads head_dim layers dtype mask\n",
            argv[0]);
    return 2;
  }
  memset(&cfg, 0, sizeof(cfg));
  cfg.S = atoi(argv[1]);
  cfg.W = atoi(argv[2]);
  cfg.W_store = atoi(argv[3]);
  cfg.anchor = atoi(argv[4]);
  cfg.n_chunk = atoi(argv[5]);
  cfg.F = atoi(argv[6]);
  cfg.Hh = atoi(argv[7]);
  cfg.Ww = atoi(argv[8]);
  cfg.n_heads = atoi(argv[9]);
  cfg.head_dim = atoi(argv[10]);
  cfg.n_layers = atoi(argv[11]);
  cfg.dtype = atoi(argv[12]);
  cfg.mask = atoi(argv[13]);

  if (fail_if(wf_create(&cfg, &h) != WF_OK, "wf_create")) return 1;
  rounds = (int64_t)cfg.n_chunk + cfg.S;
  for (k = 0; k < rounds; ++k) {
    if (fail_if(wf_round_plan(h, k, &plan) != WF_OK, "wf_round_plan")) return 1;
    print_plan(&plan);
  }

  if (fail_if(wf_pool_bytes(&cfg, &pool, &anchor, &tables) != WF_OK, "wf_pool_bytes")) return 1;
  if (fail_if(wf_page_layout(&cfg, &lay) != WF_OK, "wf_page_layout")) return 1;
  printf("{\"layout\": [%lld, %lld, %lld, %lld, %lld], \"bytes\": [%zu, %zu, %zu]}\n",
         (long long)lay.n_slots, (long long)lay.page_bytes, (long long)lay.pool_bytes,
         (long long)lay.anchor_bytes, (long long)lay.table_bytes, pool, anchor, tables);

  /* the split of the last full-width round (fp32 requests never split) */
  k = rounds - cfg.S - 1;
  if (fail_if(wf_round_plan(h, k, &plan) != WF_OK, "wf_round_plan")) return 1;
  if (fail_if(wf_attention_split_choice(h, &plan, &n_split, stage, at) != WF_OK,
              "wf_attention_split_choice"))
    return 1;
  printf("{\"split_k\": %lld, \"split\": [", (long long)k);
  for (i = 0; i < n_split; ++i) printf("%s[%d, %d]", i ? ", " : "", stage[i], at[i]);
  printf("]}\n");

  /* calls that must fail, each before any device work */
  printf("{\"errors\": [%d, %d, %d, %d, %d, %d], \"text\": \"%s\"}\n",
         wf_round_plan(h, rounds, &plan),                 /* WF_ERANGE */
         wf_round_plan(NULL, 0, &plan),                   /* WF_EINVAL */
         wf_kv_publish(h, &plan, 0, NULL, NULL, NULL, NULL, NULL),   /* WF_EORDER: round k, not 0 */
         wf_set_attention_split(h, 7),                    /* WF_EINVAL */
         wf_next_round(h, NULL),                          /* WF_EINVAL */
         (wf_create(&cfg, &other) == WF_OK && other != h &&
          wf_attention_split_choice(other, &plan, &n_split, stage, at) == WF_OK) ? 0 : -100,
         wf_strerror(WF_ERANGE));
  wf_destroy(other);
  wf_destroy(h);
  return 0;
}
