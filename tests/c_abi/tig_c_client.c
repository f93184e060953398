/*
 * A C99 client of the C ABI in include/tig.h: no Python, no torch, only the
 * HIP runtime for device memory.  Run without arguments it exercises the host
 * side (workspace queries, argument errors, the plan descriptor); with --gpu it
 * also runs tig_tree_gemm and tig_logprob_gather on the device and checks them
 * against values fixed by arithmetic:
 *   - A = 1, W row n = n + 1 (small integers, exact in bf16): C[m][n] = K (n + 1),
 *     exact in FP32 at every partial sum, for every leaf count;
 *   - H = 1 and every W entry 2^-10: all logits equal 1 (K = 1024), so every
 *     row's logprob is -ln V and its log-sum-exp is 1 + ln V
 *     ([BitRL, section 2]: the logprob of the sampled token under the softmax).
 * Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tig.h"

/* bf16 bits of a float that bf16 holds exactly (small integers, halves). */
static uint16_t bf16_exact(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      return 1;                           \
    }                                     \
  } while (0)

static int host_checks(void) {
  size_t bytes = 0;
  tig_plan plan;
  CHECK(tig_logprob_workspace_bytes(64, 512, 4096, 8, &bytes) == TIG_OK && bytes > 0, "workspace query");
  CHECK(tig_logprob_workspace_bytes(64, 500, 4096, 8, &bytes) == TIG_ERR_UNSUPPORTED,
        "K = 500 with 8 leaves must be refused (leaf of 62.5 columns)");
  CHECK(tig_tree_gemm(NULL, 512, NULL, 512, NULL, 64, TIG_OUT_F32, 4, 64, 512, 8, NULL) == TIG_ERR_INVALID_ARG,
        "NULL operands must be refused");
  CHECK(strlen(tig_last_error()) > 0, "a failing call leaves a message");
  CHECK(tig_plan_describe(4096, 8, &plan) == TIG_OK && plan.leaves == 8 && plan.leaf_len == 512 &&
            plan.mfma_m == 32 && plan.mfma_n == 32 && plan.mfma_k == 16,
        "plan of (K = 4096, 8 leaves)");
  CHECK(strcmp(tig_status_string(TIG_OK), tig_status_string(TIG_ERR_WORKSPACE)) != 0, "status strings");
  printf("host: workspace for 64 x 512 x 4096 at 8 leaves = %zu bytes; plan digest %02x%02x%02x%02x...\n", bytes,
         plan.digest[0], plan.digest[1], plan.digest[2], plan.digest[3]);
  return 0;
}

static int gpu_checks(void) {
  const int64_t M = 70, N = 130, K = 1024, V = 5000;
  const int32_t leaves[] = {1, 8, 16};
  uint16_t *hA = malloc((size_t)M * K * 2), *hW = malloc((size_t)N * K * 2), *hWv = malloc((size_t)V * K * 2);
  float *hC = malloc((size_t)M * N * 4), *hlp = malloc((size_t)M * 4), *hlse = malloc((size_t)M * 4);
  int64_t* hids = malloc((size_t)M * 8);
  void *dA, *dW, *dC, *dWv, *dids, *dlp, *dlse, *dws;
  size_t ws = 0;
  int li;
  int64_t m, n;
  CHECK(hA && hW && hWv && hC && hlp && hlse && hids, "host allocation");
  for (m = 0; m < M * K; ++m) hA[m] = bf16_exact(1.0f);
  for (n = 0; n < N; ++n)
    for (m = 0; m < K; ++m) hW[n * K + m] = bf16_exact((float)(n + 1));
  for (m = 0; m < V * K; ++m) hWv[m] = bf16_exact(1.0f / 1024.0f);
  for (m = 0; m < M; ++m) hids[m] = (m * 37) % V;
  CHECK(tig_logprob_workspace_bytes(M, K, V, 16, &ws) == TIG_OK, "workspace query");
  CHECK(hipMalloc(&dA, (size_t)M * K * 2) == hipSuccess && hipMalloc(&dW, (size_t)N * K * 2) == hipSuccess &&
            hipMalloc(&dC, (size_t)M * N * 4) == hipSuccess && hipMalloc(&dWv, (size_t)V * K * 2) == hipSuccess &&
            hipMalloc(&dids, (size_t)M * 8) == hipSuccess && hipMalloc(&dlp, (size_t)M * 4) == hipSuccess &&
            hipMalloc(&dlse, (size_t)M * 4) == hipSuccess && hipMalloc(&dws, ws) == hipSuccess,
        "device allocation");
  CHECK(hipMemcpy(dA, hA, (size_t)M * K * 2, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(dW, hW, (size_t)N * K * 2, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(dWv, hWv, (size_t)V * K * 2, hipMemcpyHostToDevice) == hipSuccess &&
            hipMemcpy(dids, hids, (size_t)M * 8, hipMemcpyHostToDevice) == hipSuccess,
        "uploads");
  for (li = 0; li < 3; ++li) {
    tig_status s = tig_tree_gemm(dA, K, dW, K, dC, N, TIG_OUT_F32, M, N, K, leaves[li], NULL);
    CHECK(s == TIG_OK, "tig_tree_gemm at %d leaves: %s", leaves[li], tig_last_error());
    CHECK(hipMemcpy(hC, dC, (size_t)M * N * 4, hipMemcpyDeviceToHost) == hipSuccess, "download");
    for (m = 0; m < M; ++m)
      for (n = 0; n < N; ++n)
        CHECK(hC[m * N + n] == (float)(K * (n + 1)), "C[%lld][%lld] = %.9g at %d leaves, expected %lld", (long long)m,
              (long long)n, hC[m * N + n], leaves[li], (long long)(K * (n + 1)));
    s = tig_logprob_gather(dA, dWv, (const int64_t*)dids, (float*)dlp, (float*)dlse, M, K, V, leaves[li], dws, ws,
                           NULL);
    CHECK(s == TIG_OK, "tig_logprob_gather at %d leaves: %s", leaves[li], tig_last_error());
    CHECK(hipMemcpy(hlp, dlp, (size_t)M * 4, hipMemcpyDeviceToHost) == hipSuccess &&
              hipMemcpy(hlse, dlse, (size_t)M * 4, hipMemcpyDeviceToHost) == hipSuccess,
          "download");
    for (m = 0; m < M; ++m) {
      const double want = -log((double)V), logit = (double)K / 1024.0;
      CHECK(fabs(hlp[m] - want) <= 1e-5, "logprob[%lld] = %.9g, expected %.9g", (long long)m, hlp[m], want);
      CHECK(fabs(hlse[m] - (logit - want)) <= 1e-4, "lse[%lld] = %.9g", (long long)m, hlse[m]);
    }
  }
  printf("gpu: tree GEMM exact at 1, 8 and 16 leaves; logprob -ln %lld = %.7f (first row %.7f)\n", (long long)V,
         -log((double)V), hlp[0]);
  hipFree(dA); hipFree(dW); hipFree(dC); hipFree(dWv); hipFree(dids); hipFree(dlp); hipFree(dlse); hipFree(dws);
  free(hA); free(hW); free(hWv); free(hC); free(hlp); free(hlse); free(hids);
  return 0;
}

int main(int argc, char** argv) {
  int r = host_checks();
  if (r == 0 && argc > 1 && strcmp(argv[1], "--gpu") == 0) r = gpu_checks();
  if (r == 0) printf("ok\n");
  return r;
}
