/* A plain C99 caller of the library's C ABI: it includes both public headers
 * and uses only what they declare.  It runs on a host without a GPU: every
 * call below is answered on the host (version, layout geometry, argument
 * checks that fail before any launch).  Exit status 0 when every answer is
 * the documented one. */
#include <stdio.h>
#include <string.h>

#include "kvc.h"
#include "kvc_ceiling.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

int main(void) {
  kvc_layout_info info;
  kvc_cache cache;
  int32_t status = 0;
  unsigned char fake[64];

  expect(kvc_version() == 3, "ABI version 3");

  expect(kvc_layout_query(KVC_LAYOUT_V4, &info) == KVC_OK, "V4 query");
  expect(info.data_bytes == 576 && info.scale_bytes == 8 && info.row_bytes == 584 &&
             info.group == 64 && info.quant_dims == 448,
         "V4 geometry");
  expect(kvc_layout_query(KVC_LAYOUT_V41, &info) == KVC_OK, "V41 query");
  expect(info.data_bytes == 512 && info.scale_bytes == 16 && info.row_bytes == 528 &&
             info.group == 32 && info.quant_dims == 512,
         "V41 geometry");
  expect(kvc_layout_query(KVC_LAYOUT_V41_FP4, &info) == KVC_OK, "V41_FP4 query");
  expect(info.data_bytes == 256 && info.scale_bytes == 32 && info.row_bytes == 288 &&
             info.group == 16 && info.quant_dims == 512,
         "V41_FP4 geometry");
  expect(kvc_layout_query(7, &info) == KVC_EUNSUPPORTED, "unknown layout rejected");

  /* a well-formed cache descriptor over host bytes: the calls below fail on
   * their own arguments before anything reaches the device */
  memset(&cache, 0, sizeof cache);
  cache.base = fake;
  cache.layout = KVC_LAYOUT_V41;
  cache.page_size = 1;
  cache.page_stride = 528;
  cache.num_pages = 1;
  expect(kvc_store_rows(&cache, NULL, 512, NULL, 1, &status, NULL) == KVC_EINVAL,
         "store with NULL rows rejected");
  expect(strstr(kvc_last_error(), "kvc_store_rows") != NULL, "error message names the call");
  expect(kvc_store_rows(&cache, NULL, 512, NULL, 0, &status, NULL) == KVC_OK, "empty store");
  expect(kvc_ceiling_gather_shape(NULL, NULL, -1, NULL) == -1, "yardstick argument check");

  if (failures == 0) printf("C ABI consumer: all checks passed\n");
  return failures == 0 ? 0 : 1;
}
