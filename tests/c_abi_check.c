/* A C99 program against include/rw4.h: the header compiles as C, and the
 * library reports argument and shape errors through its status codes
 * before any device work (so this runs without a GPU).  Built and run by
 * tests/test_c_abi.py; prints one line per failed check. */
#include <stdio.h>
#include <string.h>

#include "rw4.h"

static int fails = 0;

static void expect(const char* what, rw4_status got, rw4_status want) {
  if (got != want) {
    printf("FAIL %s: %s, expected %s\n", what, rw4_status_str(got), rw4_status_str(want));
    ++fails;
  }
}

int main(void) {
  rw4_transform* t = (rw4_transform*)&fails; /* must be cleared on failure */
  const rw4_status all[] = {RW4_OK, RW4_ERR_ARG, RW4_ERR_SHAPE, RW4_ERR_UNSUPPORTED, RW4_ERR_HIP, RW4_ERR_NOMEM};
  size_t i, j;

  if (strlen(rw4_version()) == 0) { printf("FAIL empty version\n"); ++fails; }
  for (i = 0; i < sizeof all / sizeof all[0]; ++i)
    for (j = i + 1; j < sizeof all / sizeof all[0]; ++j)
      if (strcmp(rw4_status_str(all[i]), rw4_status_str(all[j])) == 0) { printf("FAIL status strings\n"); ++fails; }

  /* transforms: K a multiple of 128, block a power of two in [128, K] dividing K */
  expect("hadamard K=100", rw4_transform_hadamard(100, 128, NULL, &t), RW4_ERR_SHAPE);
  if (t != NULL) { printf("FAIL out not cleared\n"); ++fails; }
  expect("hadamard block=100", rw4_transform_hadamard(4096, 100, NULL, &t), RW4_ERR_SHAPE);
  expect("hadamard block>K", rw4_transform_hadamard(256, 512, NULL, &t), RW4_ERR_SHAPE);
  expect("hadamard null out", rw4_transform_hadamard(4096, 128, NULL, NULL), RW4_ERR_ARG);
  expect("destroy null", rw4_transform_destroy(NULL), RW4_OK);

  /* activations: a transform is required */
  expect("quantize null transform",
         rw4_quantize_act(NULL, RW4_ACT_GROUP128, NULL, RW4_BF16, 16, 4096, NULL, NULL, NULL, NULL), RW4_ERR_ARG);

  /* GEMM: shapes first, then empty products, then pointers */
  expect("gemm K=100", rw4_w4a4_gemm(NULL, NULL, NULL, NULL, 16, 16, 100, NULL, RW4_BF16, 16, NULL), RW4_ERR_SHAPE);
  expect("gemm M<0", rw4_w4a4_gemm(NULL, NULL, NULL, NULL, -1, 16, 128, NULL, RW4_BF16, 16, NULL), RW4_ERR_SHAPE);
  expect("gemm M=0", rw4_w4a4_gemm(NULL, NULL, NULL, NULL, 0, 16, 128, NULL, RW4_BF16, 16, NULL), RW4_OK);
  expect("gemm null", rw4_w4a4_gemm(NULL, NULL, NULL, NULL, 16, 16, 128, NULL, RW4_BF16, 16, NULL), RW4_ERR_ARG);
  expect("gemm group 96", rw4_w4a4_gemm_g(NULL, NULL, NULL, NULL, 16, 16, 384, 96, NULL, RW4_BF16, 16, NULL),
         RW4_ERR_ARG);
  expect("gemm group 256, K=384",
         rw4_w4a4_gemm_g(NULL, NULL, NULL, NULL, 16, 16, 384, 256, NULL, RW4_BF16, 16, NULL), RW4_ERR_SHAPE);

  /* dequantize */
  expect("dequantize M=0", rw4_dequantize(NULL, NULL, 0, 128, NULL, RW4_BF16, 128, NULL), RW4_OK);
  expect("dequantize K=100", rw4_dequantize(NULL, NULL, 4, 100, NULL, RW4_BF16, 128, NULL), RW4_ERR_SHAPE);
  expect("dequantize null", rw4_dequantize(NULL, NULL, 4, 128, NULL, RW4_F32, 128, NULL), RW4_ERR_ARG);

  if (fails == 0) printf("c abi ok\n");
  return fails != 0;
}
