/* A plain C99 caller of liblcsa's host-side plan functions: it includes only
 * include/lcsa.h and links liblcsa.so, with no C++ or Python in between.
 * Prints the plan of a workload given on the command line as
 *   batch heads grid_h grid_w q_frames cached_frames kv_ratio local_range topk_ratio
 * followed by the row-pointer checksum and the window of query block 0, one
 * "key value" pair per line, or "error <status> <detail>" and exit code 1. */
#include <stdio.h>
#include <stdlib.h>

#include "lcsa.h"

int main(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s batch heads grid_h grid_w q_frames cached kv_ratio local_range topk_ratio\n",
            argv[0]);
    return 2;
  }
  lcsa_desc d = {0};
  d.batch = atoi(argv[1]);
  d.heads = atoi(argv[2]);
  d.head_dim = 128;
  d.grid_h = atoi(argv[3]);
  d.grid_w = atoi(argv[4]);
  d.q_frames = atoi(argv[5]);
  d.cached_frames = atoi(argv[6]);
  d.kv_ratio = (float)atof(argv[7]);
  d.local_range = atoi(argv[8]);
  d.topk_ratio = atof(argv[9]);

  lcsa_plan_t plan = NULL;
  lcsa_status st = lcsa_plan_create(&d, &plan);
  if (st != LCSA_OK) {
    printf("error %d %s\n", (int)st, lcsa_last_error());
    return 1;
  }
  lcsa_plan_info in;
  st = lcsa_plan_get_info(plan, &in);
  if (st != LCSA_OK) {
    printf("error %d %s\n", (int)st, lcsa_last_error());
    lcsa_plan_destroy(plan);
    return 1;
  }
  printf("abi %d\n", (int)lcsa_abi_version());
  printf("kv_frames %d\nnqb %d\nnkb %d\nk %d\nblock_h %d\nblock_w %d\n", in.kv_frames, in.nqb, in.nkb,
         in.k, in.block_h, in.block_w);
  printf("rows %lld\nnnz %lld\nmax_window %d\n", (long long)in.rows, (long long)in.nnz, in.max_window);

  int32_t* rp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(in.rows + 1));
  if (!rp) return 3;
  st = lcsa_plan_row_ptr(plan, rp, in.rows + 1);
  if (st != LCSA_OK) {
    printf("error %d %s\n", (int)st, lcsa_last_error());
    free(rp);
    lcsa_plan_destroy(plan);
    return 1;
  }
  unsigned long long sum = 0;
  for (int64_t r = 0; r <= in.rows; ++r) sum = sum * 1000003ull + (unsigned long long)rp[r];
  printf("row_ptr_hash %llu\n", sum);
  free(rp);

  int32_t* win = (int32_t*)malloc(sizeof(int32_t) * (size_t)(in.max_window > 0 ? in.max_window : 1));
  int32_t count = 0;
  if (!win) return 3;
  st = lcsa_plan_window(plan, 0, win, in.max_window, &count);
  if (st != LCSA_OK) {
    printf("error %d %s\n", (int)st, lcsa_last_error());
    free(win);
    lcsa_plan_destroy(plan);
    return 1;
  }
  printf("window0");
  for (int32_t i = 0; i < count; ++i) printf(" %d", win[i]);
  printf("\n");
  free(win);
  printf("status_string %s\n", lcsa_status_string(LCSA_ERR_SHAPE));
  /* threshold calls reject a missing threshold array on the host, before any
     HIP call */
  st = lcsa_select_reuse(plan, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                         NULL, NULL, 0, NULL);
  printf("reuse_without_tau %d\n", (int)st);
  st = lcsa_select_steady(plan, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                          NULL, NULL, 0, NULL);
  printf("steady_without_kth %d\n", (int)st);
  lcsa_plan_destroy(plan);
  lcsa_plan_destroy(NULL);
  return 0;
}
