/* A C99 caller of the library: the three headers compile as plain C with
 * every warning an error, the exported symbols link from C, and the
 * host-side calls (parameter checks, status text, planning, host replays of
 * every kernel family, a null parameter block) answer without a GPU.
 * Built and run by tests/test_c_abi_from_c.py. */
#include <stdio.h>
#include "conv2d_bwd.h"
#include "rms_norm_matmul.h"
#include "mha_grad_v.h"

int main(void) {
  conv2d_params p = {32, 128, 56, 56, 256, 3, 3, 2, 1, 1, 28, 28};
  conv2d_params bad = p;
  conv2d_params small = {2, 9, 13, 11, 7, 3, 3, 2, 1, 1, 7, 6};
  conv2d_plan_info info;
  rms_matmul_params rp = {7, 19, 45, 1e-6f};
  mha_grad_v_params mp = {65, 65, 3, 3, 64, 5, 1};
  char msg[256];
  int rc;
  bad.out_h = 27;
  printf("check %d %d\n", conv2d_check_params(&p), conv2d_check_params(&bad));
  printf("status %s\n", conv2d_status_string(CONV2D_ERR_BAD_SHAPE));
  printf("variants %d\n", conv2d_num_variants());
  rc = conv2d_describe_plan(&p, 0, &info);
  printf("plan %d %lld %lld\n", rc, (long long)info.useful_macs, (long long)info.phases);
  printf("replay %d\n", conv2d_check_indexing(&small, 0, msg, sizeof msg));
  printf("replay_fwd %d\n", conv2d_check_indexing_forward(&small, 0, msg, sizeof msg));
  printf("replay_gw %d\n", conv2d_check_indexing_grad_weight(&small, msg, sizeof msg));
  printf("replay_rms %d\n", rms_norm_matmul_check_indexing(&rp, msg, sizeof msg));
  printf("replay_mha %d\n", mha_grad_v_check_indexing(&mp, msg, sizeof msg));
  printf("null %d\n", conv2d_grad_input(NULL, NULL, NULL, NULL, NULL));
  return 0;
}
