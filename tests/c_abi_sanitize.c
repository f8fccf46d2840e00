/* Host paths of the library under AddressSanitizer and UBSan: table builders
 * (Givens pair tables, fp16 angles, sign tables), their validation, and the
 * argument checks of every entry point.  No kernel is launched (every call
 * with placeholder pointers fails validation first): with no GPU
 * the table uploads fail with RW4_ERR_HIP (or NOMEM) after the host work;
 * with a GPU they succeed and the transforms are destroyed again.  Built
 * and run by tests/test_host_sanitizers.py; prints one line per failed
 * check. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rw4.h"

static int fails = 0;

static void expect(const char* what, rw4_status got, rw4_status want) {
  if (got != want) {
    printf("FAIL %s: %s, expected %s\n", what, rw4_status_str(got), rw4_status_str(want));
    ++fails;
  }
}
/* a transform with device tables: OK with a GPU, a HIP or memory error without */
static void expect_built(const char* what, rw4_status got, rw4_transform* t) {
  if (got == RW4_OK) {
    expect(what, rw4_transform_destroy(t), RW4_OK);
  } else if (got != RW4_ERR_HIP && got != RW4_ERR_NOMEM) {
    printf("FAIL %s: %s\n", what, rw4_status_str(got));
    ++fails;
  }
}

enum { K = 512, G = K / 128, L = 3 };

/* layer l of group g pairs channel 2 s + l % 2 with 2 s + 1 + l % 2 (a valid matching) */
static void fill_tables(uint8_t* pairs, float* theta, uint16_t* theta16, float* beta) {
  int g, l, s;
  for (g = 0; g < G; ++g)
    for (l = 0; l < L; ++l)
      for (s = 0; s < 64; ++s) {
        const int idx = (g * L + l) * 64 + s;
        const int i = 2 * s + (l & 1), j = i + 1;
        if (j < 128) {
          pairs[2 * idx] = (uint8_t)i;
          pairs[2 * idx + 1] = (uint8_t)j;
        } else {
          pairs[2 * idx] = pairs[2 * idx + 1] = 0xFF;
        }
        theta[idx] = 0.01f * (float)(idx % 97) - 0.4f;
        theta16[idx] = 0x3C00;  /* 1.0 */
      }
  for (s = 0; s < K; ++s) beta[s] = 0.001f * (float)(s % 31);
}

int main(void) {
  uint8_t* pairs = malloc(2 * G * L * 64);
  float* theta = malloc(sizeof(float) * G * L * 64);
  uint16_t* theta16 = malloc(sizeof(uint16_t) * G * L * 64);
  float* beta = malloc(sizeof(float) * K);
  int8_t* signs = malloc(K);
  rw4_transform* t = NULL;
  int i;
  if (!pairs || !theta || !theta16 || !beta || !signs) return 2;

  /* Givens: valid tables build (host LUT, padding, cos/sin/exp), then the upload */
  fill_tables(pairs, theta, theta16, beta);
  expect_built("givens valid", rw4_transform_givens(K, L, pairs, theta, beta, NULL, &t), t);
  expect_built("givens f16 valid", rw4_transform_givens_f16(K, L, pairs, theta16, beta, NULL, &t), t);
  /* invalid tables: rejected before any device work */
  pairs[2 * 5] = 9; pairs[2 * 5 + 1] = 9;               /* i == j */
  expect("givens i == j", rw4_transform_givens(K, L, pairs, theta, beta, NULL, &t), RW4_ERR_ARG);
  fill_tables(pairs, theta, theta16, beta);
  pairs[2 * 70 + 1] = 200;                                /* out of range */
  expect("givens range", rw4_transform_givens(K, L, pairs, theta, beta, NULL, &t), RW4_ERR_ARG);
  fill_tables(pairs, theta, theta16, beta);
  pairs[2 * 64] = 0; pairs[2 * 64 + 1] = 1; pairs[2 * 65] = 1; pairs[2 * 65 + 1] = 2;  /* channel reused */
  expect("givens reuse", rw4_transform_givens(K, L, pairs, theta, beta, NULL, &t), RW4_ERR_ARG);
  fill_tables(pairs, theta, theta16, beta);
  theta[7] = NAN;
  expect("givens nan angle", rw4_transform_givens(K, L, pairs, theta, beta, NULL, &t), RW4_ERR_ARG);
  fill_tables(pairs, theta, theta16, beta);
  beta[3] = INFINITY;
  expect("givens inf beta", rw4_transform_givens(K, L, pairs, theta, beta, NULL, &t), RW4_ERR_ARG);
  fill_tables(pairs, theta, theta16, beta);
  theta16[11] = 0x7E00;                                   /* fp16 NaN */
  expect("givens f16 nan", rw4_transform_givens_f16(K, L, pairs, theta16, beta, NULL, &t), RW4_ERR_ARG);
  expect("givens K", rw4_transform_givens(K + 1, L, pairs, theta, beta, NULL, &t), RW4_ERR_SHAPE);
  expect("givens layers", rw4_transform_givens(K, 0, pairs, theta, beta, NULL, &t), RW4_ERR_SHAPE);
  expect("givens null", rw4_transform_givens(K, L, NULL, theta, beta, NULL, &t), RW4_ERR_ARG);

  /* signed Hadamard: +-1 only, then the table upload */
  for (i = 0; i < K; ++i) signs[i] = (i % 3) ? 1 : -1;
  expect_built("signed valid", rw4_transform_hadamard_signed(K, 128, signs, NULL, &t), t);
  signs[17] = 0;
  expect("signed zero", rw4_transform_hadamard_signed(K, 128, signs, NULL, &t), RW4_ERR_ARG);

  /* plain Hadamard (no device tables): create, query, use in validation, destroy */
  expect("hadamard", rw4_transform_hadamard(K, 128, NULL, &t), RW4_OK);
  if (rw4_transform_k(t) != K) { printf("FAIL transform K\n"); ++fails; }
  expect("quantize ld", rw4_quantize_act(t, RW4_ACT_GROUP128, (void*)64, RW4_BF16, 4, 100, (uint8_t*)64,
                                         (float*)64, NULL, NULL), RW4_ERR_ARG);
  expect("quantize asym ld", rw4_quantize_act_asym(t, (void*)64, RW4_BF16, 4, 100, (uint8_t*)64, (float*)64,
                                                   (float*)64, NULL), RW4_ERR_ARG);
  expect("rotate empty", rw4_rotate_act(t, NULL, RW4_BF16, 0, K, NULL, RW4_F32, K, NULL), RW4_OK);
  expect("decode fused rows", rw4_decode_fused(t, (void*)64, RW4_BF16, 17, K, (uint8_t*)64, (float*)64, 64,
                                               (void*)64, RW4_BF16, 64, NULL), RW4_ERR_SHAPE);
  expect("static rrs K", rw4_quantize_act_static(t, RW4_ACT_RRS_PER_TOKEN, NULL, RW4_BF16, 0, K, NULL, NULL, NULL),
         RW4_OK);
  expect("reorder empty", rw4_quantize_act_rrs_reorder(t, NULL, RW4_BF16, 0, K, NULL, NULL, NULL, NULL, NULL),
         RW4_OK);
  expect("destroy", rw4_transform_destroy(t), RW4_OK);
  expect("hadamard 8192", rw4_transform_hadamard(8192, 8192, NULL, &t), RW4_OK);
  expect("reorder K", rw4_quantize_act_rrs_reorder(t, (void*)64, RW4_BF16, 4, 8192, (uint8_t*)64, (float*)64,
                                                   (int32_t*)64, (void*)64, NULL), RW4_ERR_UNSUPPORTED);
  expect("destroy 8192", rw4_transform_destroy(t), RW4_OK);

  /* entry points without a transform */
  expect("gemm asym K", rw4_w4a4_gemm_asym(NULL, NULL, NULL, NULL, NULL, NULL, 4, 4, 200, NULL, RW4_BF16, 4, NULL),
         RW4_ERR_SHAPE);
  expect("code sums K", rw4_weight_code_sums(NULL, 4, 100, NULL, NULL), RW4_ERR_SHAPE);
  expect("dequantize asym", rw4_dequantize_asym(NULL, NULL, NULL, 4, 128, NULL, RW4_F32, 128, NULL), RW4_ERR_ARG);
  expect("permute K", rw4_permute_codes((uint8_t*)64, 4, 100, (int32_t*)64, (uint8_t*)128, NULL), RW4_ERR_SHAPE);
  if (rw4_rrs_reorder_workspace_bytes(100) != 0) { printf("FAIL workspace bytes\n"); ++fails; }

  free(pairs); free(theta); free(theta16); free(beta); free(signs);
  if (fails == 0) printf("sanitized host ok\n");
  return fails != 0;
}
