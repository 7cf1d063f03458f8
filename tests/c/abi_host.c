/*
 * Host-only use of the C ABI from plain C: argument validation, status
 * strings, workspace sizes and the argument checks that entry points run
 * before any HIP call. Needs no GPU. Prints one line per check and exits
 * nonzero on the first unexpected result.
 */
#include <stdio.h>
#include <string.h>

#include "msda.h"

static int fails = 0;

static void expect(const char *what, msda_status got, msda_status want) {
  printf("%s: %s\n", what, msda_status_string(got));
  if (got != want) {
    printf("  expected %s\n", msda_status_string(want));
    ++fails;
  }
}

int main(void) {
  /* four levels of an 800x1333 image at strides 8, 16, 32, 64 */
  const int64_t shapes[4][2] = {{100, 167}, {50, 84}, {25, 42}, {13, 21}};
  const int64_t starts[4] = {0, 16700, 20900, 21950};
  const int64_t S = 22223, M = 8, D = 32, L = 4, K = 4, Lq = 22223;
  size_t bytes = 0;

  expect("validate encoder shape", msda_validate(&shapes[0][0], starts, 1, S, M, D, L, Lq, K, MSDA_F32),
         MSDA_SUCCESS);
  expect("validate K = 17", msda_validate(&shapes[0][0], starts, 1, S, M, D, L, Lq, 17, MSDA_F32),
         MSDA_ERROR_NOT_SUPPORTED);
  expect("validate S too small", msda_validate(&shapes[0][0], starts, 1, S - 1, M, D, L, Lq, K, MSDA_BF16),
         MSDA_ERROR_INVALID_VALUE);
  expect("validate unknown dtype", msda_validate(&shapes[0][0], starts, 1, S, M, D, L, Lq, K, 7),
         MSDA_ERROR_NOT_SUPPORTED);

  expect("workspace size", msda_backward_workspace_size(&shapes[0][0], starts, 2, S, M, D, L, Lq, K, MSDA_F32,
                                                        &bytes),
         MSDA_SUCCESS);
  printf("workspace bytes: %zu\n", bytes);
  if (bytes == 0 || bytes % 256 != 0) {
    printf("  expected a positive multiple of 256\n");
    ++fails;
  }

  /* null device pointers are rejected before anything is enqueued */
  expect("forward with null pointers",
         msda_forward(NULL, &shapes[0][0], starts, NULL, NULL, NULL, 1, S, M, D, L, Lq, K, MSDA_F32, 0),
         MSDA_ERROR_INVALID_VALUE);
  expect("backward without workspace",
         msda_backward((const void *)256, &shapes[0][0], starts, (const float *)256, (const float *)256,
                       (const void *)256, (float *)256, (float *)256, (float *)256, 1, S, M, D, L, Lq, K,
                       MSDA_F32, NULL, 0, 0),
         MSDA_ERROR_WORKSPACE);

  if (strlen(msda_status_string((msda_status)99)) == 0) {
    printf("unknown status has an empty string\n");
    ++fails;
  }
  printf("%s\n", fails ? "FAILED" : "OK");
  return fails ? 1 : 0;
}
