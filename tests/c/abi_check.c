/* Plain C client of libdhsa: size queries and host-side argument checks.
 * Built by tests/test_c_abi.py with gcc (no HIP headers, no C++); every call
 * below returns before touching a device. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dhsa.h"

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);        \
      return 1;                                                        \
    }                                                                  \
  } while (0)

int main(void) {
  const int32_t nc[2] = {3, 2};
  const int32_t offs[7] = {0, 10, 50, 100, 0, 60, 100};
  int32_t rows = 0;
  int64_t nnz = 0;
  size_t bytes = 0;

  EXPECT(dhsa_version() >= 100);
  EXPECT(strcmp(dhsa_status_string(DHSA_ERR_CAPACITY), "DHSA_ERR_CAPACITY") == 0);

  /* rows keep min(topk + recent, i + 1) chunks */
  EXPECT(dhsa_csr_size(2, nc, 4, 2, &rows, &nnz) == DHSA_OK);
  EXPECT(rows == 4 * 5 && nnz == 4 * ((1 + 2 + 2) + (1 + 2)));
  EXPECT(dhsa_csr_capacity(2, nc, 4, 1, 1, &rows, &nnz) == DHSA_OK);
  EXPECT(nnz == 4 * ((1 + 2 + 2) + (1 + 2)));
  EXPECT(dhsa_csr_capacity(2, nc, 4, 1, -1, &rows, &nnz) == DHSA_ERR_TOPK);
  EXPECT(strlen(dhsa_last_error()) > 0);

  EXPECT(dhsa_mask_workspace_size(2, nc, 4, 2, 128, &bytes) == DHSA_OK && bytes > 0);
  EXPECT(dhsa_mask_workspace_size(2, nc, 4, 3, 128, &bytes) == DHSA_ERR_SHAPE);
  EXPECT(dhsa_prefill_workspace_size(2, 100, nc, offs, &bytes) == DHSA_OK && bytes > 0);
  EXPECT(dhsa_layer_workspace_size(2, 100, 4, 2, 128, nc, offs, 2, 0, 1, &bytes) == DHSA_OK);
  EXPECT(dhsa_nms_offsets_stride(131072, 32, &rows) == DHSA_OK && rows == 4097);
  EXPECT(dhsa_nms_workspace_size(1, DHSA_NMS_MAX_LEN + 1, 8, &bytes) == DHSA_ERR_UNSUPPORTED);

  /* NULL device pointers are rejected on the host */
  EXPECT(dhsa_build_mask(NULL, NULL, 2, 100, 4, 2, 128, nc, offs, NULL, 2, NULL, NULL, 0, NULL,
                         NULL, 0, NULL) == DHSA_ERR_NULL_POINTER);
  EXPECT(dhsa_sparse_prefill(NULL, NULL, NULL, 2, 100, 4, 2, 128, nc, offs, NULL, NULL, NULL, 0,
                             0.f, NULL, NULL, NULL, 0, NULL) == DHSA_ERR_NULL_POINTER);
  EXPECT(dhsa_nms_boundaries(NULL, 1, 100, 4, 0.5f, NULL, 26, NULL, NULL, 0, NULL) ==
         DHSA_ERR_NULL_POINTER);
  printf("c abi ok\n");
  return 0;
}
