/* A plain C (C99) caller of the library's boundary, built and run by
   tests/test_c_abi.py without a GPU: the header compiles as C, and the
   host-only entry points (version, status strings, plan and workspace
   queries, argument checks) answer as documented. */
#include <stdio.h>
#include <string.h>

#include "sv.h"

static int failures = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                             \
    }                                                         \
  } while (0)

static sv_verify_params params(int32_t batch, int32_t q_len, int32_t max_kv_len, sv_kv_dtype dtype) {
  sv_verify_params p;
  memset(&p, 0, sizeof p);
  p.batch = batch;
  p.q_len = q_len;
  p.num_q_heads = 24;
  p.num_kv_heads = 4;
  p.head_dim = 256;
  p.page_size = 16;
  p.max_pages_per_req = (max_kv_len + 15) / 16;
  p.num_pages = p.max_pages_per_req * batch;
  p.max_kv_len = max_kv_len;
  p.kv_dtype = dtype;
  p.sm_scale = 0.0625f;
  return p;
}

int main(void) {
  int32_t splits = 0, chunk = 0, kernel = -1;
  sv_verify_params p = params(1, 8, 524296, SV_KV_FP16);

  CHECK(sv_version() > 0);
  CHECK(strcmp(sv_status_string(SV_OK), sv_status_string(SV_ERR_HIP)) != 0);

  /* the 512K single request: 64 chunks, row tiles, a workspace for the partials */
  CHECK(sv_verify_plan(&p, &splits, &chunk) == SV_OK);
  CHECK(splits == 64 && chunk % 64 == 0 && (long long)splits * chunk >= p.max_kv_len);
  CHECK(sv_verify_plan_kernel(&p, &kernel) == SV_OK && kernel == SV_KERNEL_ROW_TILES);
  CHECK(sv_verify_workspace_bytes(&p) > 0);

  /* 96 rows per KV head over the ragged batch's bound: the two-half kernel */
  p = params(32, 16, 131088, SV_KV_FP16);
  p.page_size = 64;
  p.max_pages_per_req = (131088 + 63) / 64;
  p.num_pages = p.max_pages_per_req * 32;
  CHECK(sv_verify_plan_kernel(&p, &kernel) == SV_OK && kernel == SV_KERNEL_TWO_HALVES);

  /* bad shapes are refused on the host, with a message */
  p = params(1, 8, 4104, SV_KV_FP16);
  p.head_dim = 128;
  CHECK(sv_verify_plan(&p, &splits, &chunk) == SV_ERR_UNSUPPORTED);
  CHECK(strstr(sv_last_error(), "head_dim") != NULL);
  p = params(1, 8, 4104, SV_KV_FP16);
  CHECK(sv_verify_plan_kernel(&p, NULL) == SV_ERR_INVALID_ARGUMENT);

  /* null device pointers are refused without a launch */
  CHECK(sv_verify_attention(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL) ==
        SV_ERR_INVALID_ARGUMENT);

  /* greedy accept's workspace query */
  CHECK(sv_greedy_accept_workspace_bytes(1, 8, 248320) > 0);

  if (failures == 0) printf("c abi ok\n");
  return failures == 0 ? 0 : 1;
}
