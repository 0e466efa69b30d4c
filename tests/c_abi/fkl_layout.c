/*
 * Plain C99 client of include/fkl.h: compiles the header as C, links against
 * libfkl.so, and prints the layout of every struct the header declares (size,
 * then each field's offset) and the results of a few host-only calls, one
 * "key value..." line each, for comparison with the Python binding's mirrors.
 * Makes no device call.
 */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "fkl.h"

#define FIELD(T, f) printf(" %s=%zu", #f, offsetof(T, f))

int main(void) {
  printf("fkl_shape %zu", sizeof(fkl_shape));
  FIELD(fkl_shape, N); FIELD(fkl_shape, d); FIELD(fkl_shape, V); FIELD(fkl_shape, K);
  FIELD(fkl_shape, T); FIELD(fkl_shape, chunk); FIELD(fkl_shape, vslab); FIELD(fkl_shape, flags);
  printf("\n");
  printf("fkl_terms %zu", sizeof(fkl_terms));
  FIELD(fkl_terms, row_weight); FIELD(fkl_terms, label); FIELD(fkl_terms, label_weight);
  printf("\n");
  printf("fkl_topk_shape %zu", sizeof(fkl_topk_shape));
  FIELD(fkl_topk_shape, N); FIELD(fkl_topk_shape, d); FIELD(fkl_topk_shape, V); FIELD(fkl_topk_shape, K);
  FIELD(fkl_topk_shape, chunk); FIELD(fkl_topk_shape, flags);
  printf("\n");
  printf("fkl_plan %zu", sizeof(fkl_plan));
  FIELD(fkl_plan, fwd_rows); FIELD(fkl_plan, bwd_rows); FIELD(fkl_plan, vslab); FIELD(fkl_plan, fwd_passes);
  FIELD(fkl_plan, bwd_passes); FIELD(fkl_plan, slabs); FIELD(fkl_plan, fwd_bytes); FIELD(fkl_plan, bwd_bytes);
  printf("\n");
  printf("fkl_kernel_stat %zu", sizeof(fkl_kernel_stat));
  FIELD(fkl_kernel_stat, name); FIELD(fkl_kernel_stat, launches); FIELD(fkl_kernel_stat, total_ms);
  FIELD(fkl_kernel_stat, min_ms); FIELD(fkl_kernel_stat, max_ms); FIELD(fkl_kernel_stat, flops);
  FIELD(fkl_kernel_stat, bytes);
  printf("\n");

  fkl_shape s;
  memset(&s, 0, sizeof(s));
  s.N = 32768; s.d = 2880; s.V = 201088; s.K = 100; s.T = 1.0f; s.chunk = 4096;
  size_t fb = 0, bb = 0;
  fkl_status st = fkl_workspace_size(&s, &fb, &bb);
  printf("workspace %d %zu %zu\n", (int)st, fb, bb);
  fkl_plan pl;
  memset(&pl, 0, sizeof(pl));
  st = fkl_plan_info(&s, &pl);
  printf("plan %d %lld %lld %lld %lld %lld %lld %zu %zu\n", (int)st, (long long)pl.fwd_rows, (long long)pl.bwd_rows,
         (long long)pl.vslab, (long long)pl.fwd_passes, (long long)pl.bwd_passes, (long long)pl.slabs,
         pl.fwd_bytes, pl.bwd_bytes);
  fkl_topk_shape ts;
  memset(&ts, 0, sizeof(ts));
  ts.N = 16384; ts.d = 4096; ts.V = 128256; ts.K = 100;
  size_t tb = 0;
  st = fkl_topk_workspace_size(&ts, &tb);
  printf("topk_workspace %d %zu\n", (int)st, tb);
  st = fkl_workspace_size(NULL, &fb, &bb);
  printf("null_shape %d %s\n", (int)st, fkl_last_error()[0] ? "message" : "empty");
  printf("status_strings %s|%s\n", fkl_status_string(FKL_OK), fkl_status_string(FKL_EWORKSPACE));
  printf("version %d\n", fkl_version());
  return 0;
}
