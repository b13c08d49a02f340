// Host-side argument validation of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer (built by weight_only_bit_02_amd/sanitize_host.py, run by tests/test_sanitize.py).
// Every call here is rejected on the host before anything is enqueued, so no GPU is needed;
// the sanitizers check the validation code itself (reads of the config structs, size
// arithmetic, the workspace layouts) on every status path.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>

#include "awq.h"
#include "awq_peaks.h"

static int failures = 0;
#define EXPECT(call, want)                                                               \
  do {                                                                                   \
    const int got = (int)(call);                                                         \
    if (got != (int)(want)) {                                                            \
      fprintf(stderr, "%s:%d: %s returned %d, want %d\n", __FILE__, __LINE__, #call, got, \
              (int)(want));                                                              \
      ++failures;                                                                        \
    }                                                                                    \
  } while (0)

int main() {
  // fake device pointers: 16-byte aligned, never dereferenced (every call fails validation)
  void* F = (void*)(uintptr_t)0x7F0000000000ull;
  void* ODD = (void*)(uintptr_t)0x7F0000000008ull;
  uint32_t* Fu = (uint32_t*)F;
  uint8_t* Fb = (uint8_t*)F;
  double* Fd = (double*)F;
  int32_t* Fi = (int32_t*)F;
  // heap-allocated configs, so a read past the struct would be caught
  awq_config* cfg = (awq_config*)malloc(sizeof(awq_config));
  *cfg = awq_config{4, 128, 1, 20};
  awq_config* bad = (awq_config*)malloc(sizeof(awq_config));

  for (int s = 0; s <= 8; ++s)
    if (!awq_status_string((awq_status)s)) ++failures;
  EXPECT(awq_gemv_max_m() >= 0, 1);

  // quantize + pack
  EXPECT(awq_quantize_pack(nullptr, 4, 256, nullptr, cfg, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_NULL_POINTER);
  EXPECT(awq_quantize_pack(F, 0, 256, nullptr, cfg, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_quantize_pack(F, 4, 200, nullptr, cfg, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_quantize_pack(ODD, 4, 256, nullptr, cfg, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_MISALIGNED);
  const int bad_cfgs[][4] = {{5, 128, 1, 20}, {4, 96, 1, 20}, {4, 128, 2, 20}, {4, 128, 1, 0}, {4, 128, 1, 65}};
  for (const auto& b : bad_cfgs) {
    *bad = awq_config{b[0], b[1], b[2], b[3]};
    EXPECT(awq_quantize_pack(F, 4, 256, nullptr, bad, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_UNSUPPORTED);
    EXPECT(awq_search_workspace_size(256, 64, 256, bad), 0);
  }
  EXPECT(awq_quantize_pack_clipped(F, 4, 256, nullptr, Fb, 0, cfg, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_quantize_pack_clipped(F, 4, 256, nullptr, Fb, 70000, cfg, Fu, F, Fb, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);

  // statistic and scales
  EXPECT(awq_activation_stats(F, 16, 256, Fd, F, 8, nullptr, nullptr), AWQ_ERR_WORKSPACE);
  EXPECT(awq_activation_stats(F, 9000, 256, Fd, F, 1 << 20, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_candidate_scales(Fd, 100, cfg, F, nullptr), AWQ_ERR_BAD_SHAPE);

  // search: workspace sizes over the supported range, then rejections
  for (int64_t T : {1, 17, 512, 8192})
    for (int64_t K : {128, 4096, 28672}) {
      const size_t ws = awq_search_workspace_size(T, 12288, K, cfg);
      if (ws == 0) ++failures;
      EXPECT(awq_search_scales(F, T, F, 12288, K, cfg, F, Fi, Fd, F, F, ws - 1, nullptr, nullptr),
             AWQ_ERR_WORKSPACE);
    }
  EXPECT(awq_search_workspace_size(8193, 64, 256, cfg), 0);
  EXPECT(awq_search_scales(F, 8193, F, 64, 256, cfg, F, Fi, Fd, F, F, 1 << 30, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_search_scales_noalloc(F, 8192, F, 4096, 28672, cfg, F, Fi, nullptr, nullptr, nullptr, nullptr),
         AWQ_ERR_SCRATCH_LIMIT);
  EXPECT(awq_search_scales_noalloc(nullptr, 512, F, 64, 256, cfg, F, Fi, nullptr, nullptr, nullptr, nullptr),
         AWQ_ERR_NULL_POINTER);

  // clip search
  for (int g : {128, 64, 32}) {
    *bad = awq_config{4, g, 1, 20};
    const size_t ws = awq_clip_search_workspace_size(512, 4096, 11008, 20, bad);
    if (ws == 0) ++failures;
    EXPECT(awq_clip_search(F, 512, F, 4096, 11008, nullptr, 200, 20, bad, Fb, Fd, F, ws - 1, nullptr, nullptr),
           AWQ_ERR_WORKSPACE);
  }
  EXPECT(awq_clip_search(F, 513, F, 64, 256, nullptr, 200, 20, cfg, Fb, Fd, F, 1 << 30, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_clip_search(F, 64, F, 64, 256, nullptr, 200, 300, cfg, Fb, Fd, F, 1 << 30, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);

  // linear: every kernel choice's shape limits, gated parity of N, the wide GEMM's formats
  for (int k = 0; k <= 5; ++k)
    EXPECT(awq_linear_w4a16_ex(nullptr, 1, Fu, F, Fb, 64, 256, cfg, F, nullptr, (awq_linear_kernel)k, nullptr),
           AWQ_ERR_NULL_POINTER);
  EXPECT(awq_linear_w4a16_ex(F, 9, Fu, F, Fb, 64, 256, cfg, F, nullptr, AWQ_LINEAR_GEMV, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_linear_w4a16_ex(F, 65, Fu, F, Fb, 64, 256, cfg, F, nullptr, AWQ_LINEAR_SKINNY, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_linear_w4a16_ex(F, 4, Fu, F, Fb, 64, 256, cfg, F, nullptr, (awq_linear_kernel)5, nullptr), AWQ_ERR_UNSUPPORTED);
  *bad = awq_config{8, 128, 1, 20};
  EXPECT(awq_linear_w4a16_gated_silu_ex(F, 512, Fu, F, Fb, 64, 256, bad, F, nullptr, AWQ_LINEAR_GEMM_WIDE, nullptr), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_linear_w4a16_gated_silu(F, 1, Fu, F, Fb, 65, 256, cfg, F, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_linear_w4a16(F, 1, Fu, F, Fb, 64, 256, cfg, ODD, nullptr, nullptr), AWQ_ERR_MISALIGNED);
  EXPECT(awq_linear_w4a16(F, 1, Fu, F, Fb, 64, 256, cfg, F, (uint32_t*)((char*)F + 2), nullptr), AWQ_ERR_MISALIGNED);

  // fold, probes
  EXPECT(awq_apply_inverse_scale(F, 4, 12, F, 1, F, nullptr, nullptr), AWQ_ERR_BAD_SHAPE);
  EXPECT(awq_apply_inverse_scale(F, 4, 16, F, 2, F, nullptr, nullptr), AWQ_ERR_UNSUPPORTED);
  EXPECT(awq_peak_read_stream(F, 4095, Fu, 4, nullptr), 2);
  EXPECT(awq_peak_mfma(0, (float*)F, 16, nullptr), 2);

  free(cfg);
  free(bad);
  if (failures) {
    fprintf(stderr, "%d host validation check(s) failed\n", failures);
    return 1;
  }
  printf("host validation ok under the sanitizers\n");
  return 0;
}
