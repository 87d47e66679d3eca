// Exercises the host-side code of libmole under AddressSanitizer and
// UndefinedBehaviorSanitizer (built host-only; no GPU is touched): the
// dedupe and gather of the host-resident and file-backed tables, the
// training index, the staging and workspace sizes, the constant copies,
// the host state release, and the argument checks of the GPU entry points
// (every call below fails validation before any launch).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>
#include <fcntl.h>

#include <vector>

#include "../../include/mole.h"

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main(int argc, char** argv) {
  const char* dir = argc > 1 ? argv[1] : "/tmp";
  const int64_t V = 3000, N = 4, D = 256, T = 5000;
  const size_t crow = (size_t)N * 3 * D / 8, srow = (size_t)N * (D / 64);
  std::vector<uint8_t> codes((size_t)V * crow);
  std::vector<uint16_t> scales((size_t)V * srow);
  for (size_t i = 0; i < codes.size(); ++i) codes[i] = (uint8_t)(i * 2654435761u >> 24);
  for (size_t i = 0; i < scales.size(); ++i) scales[i] = (uint16_t)(i * 40503u);
  std::vector<int64_t> ids(T);
  for (int64_t t = 0; t < T; ++t) ids[t] = (t * 7919) % (V / 3);
  // host gather, single thread and pool
  for (int nt : {1, 8}) {
    std::vector<uint8_t> cs((size_t)T * crow);
    std::vector<uint16_t> ss((size_t)T * srow);
    std::vector<int64_t> remap(T);
    int64_t U = -1;
    CHECK(mole_gather_nf3_host(ids.data(), T, codes.data(), scales.data(), V, N, D, cs.data(), ss.data(),
                               remap.data(), &U, nt) == MOLE_OK);
    CHECK(U == V / 3);
    for (int64_t t = 0; t < T; ++t)
      CHECK(memcmp(cs.data() + remap[t] * crow, codes.data() + ids[t] * crow, crow) == 0);
  }
  ids[17] = V;  // bad id
  std::vector<uint8_t> cs((size_t)T * crow);
  std::vector<uint16_t> ss((size_t)T * srow);
  std::vector<int64_t> remap(T);
  int64_t U = 0;
  CHECK(mole_gather_nf3_host(ids.data(), T, codes.data(), scales.data(), V, N, D, cs.data(), ss.data(),
                             remap.data(), &U, 4) == MOLE_ERR_ID);
  ids[17] = 3;
  // training index
  std::vector<int64_t> uniq(T), row_ptr(T + 1), tok(T);
  CHECK(mole_train_index(ids.data(), T, V, uniq.data(), remap.data(), row_ptr.data(), tok.data(), &U) == MOLE_OK);
  CHECK(row_ptr[U] == T);
  // file tier
  char path[512];
  snprintf(path, sizeof path, "%s/mole_sanitize_table.bin", dir);
  CHECK(mole_nf3_file_write(path, codes.data(), scales.data(), V, N, D) == MOLE_OK);
  int fd = open(path, O_RDONLY);
  CHECK(fd >= 0);
  int64_t fV, fN, fD;
  CHECK(mole_nf3_file_shape(fd, &fV, &fN, &fD) == MOLE_OK && fV == V && fN == N && fD == D);
  CHECK(mole_gather_nf3_file(fd, ids.data(), T, V, N, D, cs.data(), ss.data(), remap.data(), &U, 8) == MOLE_OK);
  for (int64_t t = 0; t < T; ++t)
    CHECK(memcmp(cs.data() + remap[t] * crow, codes.data() + ids[t] * crow, crow) == 0);
  close(fd);
  unlink(path);
  // sizes, constants, release
  size_t bytes = 0, mn = 0, rec = 0;
  CHECK(mole_nf3_host_staging_size(T, N, D, &bytes) == MOLE_OK && bytes > 0);
  CHECK(mole_nf3_host_stack_staging_size(T, 3, N, D, &bytes) == MOLE_OK && bytes > 0);
  CHECK(mole_build_lut_workspace_size(50304, 2048, 8192, 16, MOLE_BF16, &mn, &rec) == MOLE_OK && rec >= mn);
  CHECK(mole_lookup_combine_grouped_workspace_size(T, &bytes) == MOLE_OK && bytes > 0);
  size_t fb = 0, bb = 0;
  CHECK(mole_train_workspace_size(T, U, D, 512, N, &fb, &bb) == MOLE_OK && fb > 0 && bb > 0);
  CHECK(mole_layer_workspace_size(T, D, 512, &bytes) == MOLE_OK && bytes > 0);
  float lv[16], coef[10], range = 0.f;
  CHECK(mole_nf3_levels(lv) == MOLE_OK && mole_nf3_midpoints(lv) == MOLE_OK && mole_nf4_levels(lv) == MOLE_OK &&
        mole_nf4_midpoints(lv) == MOLE_OK && mole_gelu_phi_coefficients(coef, 10, &range) == MOLE_OK);
  for (int s = 0; s >= -12; --s) CHECK(mole_status_string(s) != NULL);
  CHECK(mole_release_host_state() == MOLE_OK);
  // argument checks of the GPU entry points (rejected on the host)
  void* p = (void*)0x1000;
  CHECK(mole_lookup_combine((const int64_t*)p, p, p, p, (float*)p, 4, 10, 64, 65, MOLE_BF16, NULL) ==
        MOLE_ERR_UNSUPPORTED);
  CHECK(mole_lookup_combine_nf3((const int64_t*)p, p, p, (const uint8_t*)p, (const uint16_t*)p, (float*)p, 4, 10, 96,
                                4, MOLE_BF16, NULL) == MOLE_ERR_DIM);
  CHECK(mole_build_lut(p, p, p, p, 10, 64, 64, 4, MOLE_BF16, NULL, 0, NULL) == MOLE_ERR_NULL);
  CHECK(mole_lookup_combine_grouped_noalloc((const int64_t*)p, p, p, p, (float*)p, MOLE_GROUPED_NOALLOC_MAX_T + 1,
                                            10, 64, 4, MOLE_BF16, NULL) == MOLE_ERR_UNSUPPORTED);
  CHECK(mole_check_ids(NULL, 4, 10, NULL, NULL) == MOLE_ERR_NULL);
  printf("api host driver: ok\n");
  return 0;
}
