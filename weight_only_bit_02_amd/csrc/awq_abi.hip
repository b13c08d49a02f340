// C ABI of libawq_mi355x: argument validation, workspace layout, kernel dispatch.
// The operations and their sources are documented in include/awq.h.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "awq.h"
#include "launch.hpp"

// Workspace of awq_search_scales_noalloc: a static device array, one copy per GPU for as
// long as the process lives. Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the symbol): its device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __attribute__((aligned(256))) unsigned char scratch[AWQ_NOALLOC_SCRATCH_BYTES];
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;

awq_config resolve(const awq_config* cfg) {
  if (cfg) return *cfg;
  return awq_config{4, 128, 1, 20};
}

bool supported(const awq_config& c) {
  return (c.w_bit == 3 || c.w_bit == 4 || c.w_bit == 8) &&
         (c.group_size == 128 || c.group_size == 64 || c.group_size == 32) &&
         (c.zero_point == 0 || c.zero_point == 1) && c.n_grid >= 1 && c.n_grid <= 64;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool good_nk(int64_t N, int64_t K) {
  return N >= 1 && K >= 128 && K % 128 == 0 && N < kMaxDim && K < kMaxDim;
}

awq_status hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Search workspace: [u: int64 K][act: fp64 K][s_grid: fp16 n_grid K]
// [partials: fp64 n_grid x row tiles x token chunks][errf: fp64 n_grid][cand: n_grid bytes]
// [xp: X in MFMA operand order, T rounded up to 64 tokens]
struct SearchLayout {
  size_t u, act, sgrid, partials, errf, cand, xp, total;
  int64_t n_partials;  // per grid point
};

SearchLayout search_layout(int64_t T, int64_t N, int64_t K, int n_grid) {
  SearchLayout L;
  const int64_t ntiles = (N + awq::search_row_tile() - 1) / awq::search_row_tile();
  const int64_t chunk = awq::search_token_chunk(T);
  L.n_partials = ntiles * ((T + chunk - 1) / chunk);
  L.u = 0;
  L.act = align256(L.u + (size_t)K * 8);
  L.sgrid = align256(L.act + (size_t)K * 8);
  L.partials = align256(L.sgrid + (size_t)n_grid * K * 2);
  L.errf = align256(L.partials + (size_t)n_grid * L.n_partials * 8);
  L.cand = align256(L.errf + (size_t)n_grid * 8);
  L.xp = align256(L.cand + (size_t)n_grid);
  L.total = align256(L.xp + awq::packed_x_bytes(T, K));
  return L;
}

// Clip-search workspace: [err: fp64 n_shrink x N x G]
// [xp: X in MFMA operand order, T rounded up to 64 tokens; or, in the Gram form, the
//  per-group G' and the channel scales]
struct ClipLayout {
  size_t err, xp, total;
};

ClipLayout clip_layout(int64_t T, int64_t N, int64_t K, int n_shrink, int group) {
  ClipLayout L;
  L.err = 0;
  L.xp = align256(L.err + awq::clip_err_bytes(T, N, K, n_shrink, group));
  L.total = align256(L.xp + awq::clip_scratch_bytes(T, K, group));
  return L;
}

// Largest M that AWQ_LINEAR_AUTO serves with a GEMV-class kernel (above it, the MFMA
// GEMM); AWQ_GEMV_MAX_M overrides it (0 .. 64) to measure the crossover.
int gemv_max_m_from_env() {
  const char* e = getenv("AWQ_GEMV_MAX_M");
  if (!e) return awq::kSkinnyMaxM;
  int v = atoi(e);
  if (v < 0) v = 0;
  if (v > awq::kSkinnyMaxM) v = awq::kSkinnyMaxM;
  return v;
}
const int g_gemv_max_m = gemv_max_m_from_env();

}  // namespace

extern "C" {

const char* awq_status_string(awq_status s) {
  // callers may pass any integer: read it as one (a value outside the enumerators is not a
  // valid awq_status in C++, so it must not be switched on as one)
  int v = 0;
  static_assert(sizeof(s) == sizeof(v), "awq_status is an int-sized enum");
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case AWQ_OK: return "ok";
    case AWQ_ERR_NULL_POINTER: return "a required pointer is NULL";
    case AWQ_ERR_BAD_SHAPE: return "bad shape (sizes must be >= 1, K a multiple of 128, T <= 8192)";
    case AWQ_ERR_UNSUPPORTED: return "unsupported config (w_bit 3, 4 or 8, group_size 128, 64 or 32, zero_point 0 or 1, 1 <= n_grid <= 64)";
    case AWQ_ERR_MISALIGNED: return "a base pointer is not 16-byte aligned";
    case AWQ_ERR_WORKSPACE: return "workspace missing or too small";
    case AWQ_ERR_HIP: return "HIP launch error";
    case AWQ_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the static AWQ_NOALLOC_SCRATCH_BYTES array";
  }
  return "unknown status";
}

int32_t awq_gemv_max_m(void) { return g_gemv_max_m; }

awq_status awq_quantize_pack(const void* W, int64_t N, int64_t K, const void* s,
                             const awq_config* cfg, uint32_t* qweight, void* scales,
                             uint8_t* zeros, uint32_t* flags, void* stream) {
  return awq_quantize_pack_clipped(W, N, K, s, nullptr, 0, cfg, qweight, scales, zeros, flags,
                                   stream);
}

awq_status awq_quantize_pack_clipped(const void* W, int64_t N, int64_t K, const void* s,
                                     const uint8_t* clip_idx, int32_t clip_steps,
                                     const awq_config* cfg, uint32_t* qweight, void* scales,
                                     uint8_t* zeros, uint32_t* flags, void* stream) {
  const awq_config c = resolve(cfg);
  if (!W || !qweight || !scales || !zeros) return AWQ_ERR_NULL_POINTER;
  if (!supported(c)) return AWQ_ERR_UNSUPPORTED;
  if (!good_nk(N, K)) return AWQ_ERR_BAD_SHAPE;
  if (clip_idx && (clip_steps < 1 || clip_steps > 65535)) return AWQ_ERR_BAD_SHAPE;
  if (!aligned16(W) || !aligned16(qweight) || !aligned16(scales) || !aligned16(zeros) ||
      (s && !aligned16(s)) || (flags && !aligned4(flags)))
    return AWQ_ERR_MISALIGNED;
  return hip_status(awq::launch_quant_pack((const uint16_t*)W, N, K, (const uint16_t*)s, qweight,
                                           (uint16_t*)scales, zeros, clip_idx, clip_steps,
                                           c.zero_point == 0, c.group_size, c.w_bit, flags,
                                           (hipStream_t)stream));
}

size_t awq_activation_stats_workspace_size(int64_t T, int64_t K) {
  (void)T;
  return K > 0 ? align256((size_t)K * 8) : 0;
}

awq_status awq_activation_stats(const void* X, int64_t T, int64_t K, double* act_mean,
                                void* workspace, size_t workspace_bytes, uint32_t* flags,
                                void* stream) {
  if (!X || !act_mean) return AWQ_ERR_NULL_POINTER;
  if (T < 1 || T > AWQ_MAX_CALIB_TOKENS || !good_nk(1, K)) return AWQ_ERR_BAD_SHAPE;
  if (!workspace || workspace_bytes < awq_activation_stats_workspace_size(T, K))
    return AWQ_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(act_mean) || !aligned16(workspace) ||
      (flags && !aligned4(flags)))
    return AWQ_ERR_MISALIGNED;
  hipStream_t st = (hipStream_t)stream;
  auto* u = (unsigned long long*)workspace;
  hipError_t e = awq::launch_zero_u64(u, K, st);
  if (e == hipSuccess) e = awq::launch_act_sums((const uint16_t*)X, T, K, u, flags, st);
  if (e == hipSuccess) e = awq::launch_act_finalize(u, T, K, act_mean, st);
  return hip_status(e);
}

awq_status awq_candidate_scales(const double* act_mean, int64_t K, const awq_config* cfg,
                                void* s_grid, void* stream) {
  const awq_config c = resolve(cfg);
  if (!act_mean || !s_grid) return AWQ_ERR_NULL_POINTER;
  if (!supported(c)) return AWQ_ERR_UNSUPPORTED;
  if (!good_nk(1, K)) return AWQ_ERR_BAD_SHAPE;
  if (!aligned16(act_mean) || !aligned16(s_grid)) return AWQ_ERR_MISALIGNED;
  return hip_status(
      awq::launch_scalegen(act_mean, K, c.n_grid, (uint16_t*)s_grid, (hipStream_t)stream));
}

size_t awq_search_workspace_size(int64_t T, int64_t N, int64_t K, const awq_config* cfg) {
  const awq_config c = resolve(cfg);
  if (!supported(c) || T < 1 || T > AWQ_MAX_CALIB_TOKENS || !good_nk(N, K)) return 0;
  return search_layout(T, N, K, c.n_grid).total;
}

awq_status awq_search_scales(const void* X, int64_t T, const void* W, int64_t N, int64_t K,
                             const awq_config* cfg, void* s_best, int32_t* best_idx,
                             double* err, void* s_grid, void* workspace,
                             size_t workspace_bytes, uint32_t* flags, void* stream) {
  const awq_config c = resolve(cfg);
  if (!X || !W || !s_best || !best_idx) return AWQ_ERR_NULL_POINTER;
  if (!supported(c)) return AWQ_ERR_UNSUPPORTED;
  if (T < 1 || T > AWQ_MAX_CALIB_TOKENS || !good_nk(N, K)) return AWQ_ERR_BAD_SHAPE;
  const SearchLayout L = search_layout(T, N, K, c.n_grid);
  if (!workspace || workspace_bytes < L.total) return AWQ_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(W) || !aligned16(s_best) || !aligned4(best_idx) ||
      (err && !aligned16(err)) || (s_grid && !aligned16(s_grid)) || !aligned16(workspace) ||
      (flags && !aligned4(flags)))
    return AWQ_ERR_MISALIGNED;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto* u = (unsigned long long*)(ws + L.u);
  auto* act = (double*)(ws + L.act);
  auto* sg = s_grid ? (uint16_t*)s_grid : (uint16_t*)(ws + L.sgrid);
  auto* partials = (double*)(ws + L.partials);
  const auto* Xh = (const uint16_t*)X;
  hipError_t e = awq::launch_zero_u64(u, K, st);
  if (e == hipSuccess) e = awq::launch_act_sums(Xh, T, K, u, flags, st);
  if (e == hipSuccess) e = awq::launch_act_finalize(u, T, K, act, st);
  if (e == hipSuccess) e = awq::launch_scalegen(act, K, c.n_grid, sg, st);
  const bool one_term = awq::search_one_term(T, N, K);
  auto* errf = (double*)(ws + L.errf);
  auto* cand = (uint8_t*)(ws + L.cand);
  if (e == hipSuccess)
    e = awq::launch_search_err(Xh, T, (const uint16_t*)W, N, K, sg, c.n_grid, c.zero_point == 0,
                               c.group_size, c.w_bit, (uint4*)(ws + L.xp), partials, errf, cand,
                               one_term, flags, st);
  if (e == hipSuccess)
    e = awq::launch_search_reduce(partials, c.n_grid, L.n_partials, one_term ? cand : nullptr,
                                  errf, sg, K, (uint16_t*)s_best, best_idx, err, flags, st);
  return hip_status(e);
}

awq_status awq_search_scales_noalloc(const void* X, int64_t T, const void* W, int64_t N,
                                     int64_t K, const awq_config* cfg, void* s_best,
                                     int32_t* best_idx, double* err, void* s_grid,
                                     uint32_t* flags, void* stream) {
  const awq_config c = resolve(cfg);
  if (!X || !W || !s_best || !best_idx) return AWQ_ERR_NULL_POINTER;
  if (!supported(c)) return AWQ_ERR_UNSUPPORTED;
  if (T < 1 || T > AWQ_MAX_CALIB_TOKENS || !good_nk(N, K)) return AWQ_ERR_BAD_SHAPE;
  if (search_layout(T, N, K, c.n_grid).total > (size_t)AWQ_NOALLOC_SCRATCH_BYTES)
    return AWQ_ERR_SCRATCH_LIMIT;
  // the current device's copy of the array (looked up on the first call on each device)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AWQ_ERR_HIP;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AWQ_ERR_HIP;
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return awq_search_scales(X, T, W, N, K, cfg, s_best, best_idx, err, s_grid, ws,
                           (size_t)AWQ_NOALLOC_SCRATCH_BYTES, flags, stream);
}

static awq_status linear_common(const void* X, int64_t M, const uint32_t* qweight,
                                const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                                const awq_config* cfg, void* Y, uint32_t* flags,
                                awq_linear_kernel kernel_arg, bool gated, void* stream) {
  // the caller may pass any integer: validate it as one before it is used as the enum
  int kv = 0;
  static_assert(sizeof(kernel_arg) == sizeof(kv), "awq_linear_kernel is an int-sized enum");
  memcpy(&kv, &kernel_arg, sizeof kv);
  const awq_config c = resolve(cfg);
  if (!X || !qweight || !scales || !zeros || !Y) return AWQ_ERR_NULL_POINTER;
  if (!supported(c)) return AWQ_ERR_UNSUPPORTED;
  if (M < 1 || M >= kMaxDim || !good_nk(N, K)) return AWQ_ERR_BAD_SHAPE;
  if (gated && (N < 2 || N % 2 != 0)) return AWQ_ERR_BAD_SHAPE;
  if (kv < AWQ_LINEAR_AUTO || kv > AWQ_LINEAR_GEMM_WIDE) return AWQ_ERR_UNSUPPORTED;
  awq_linear_kernel kernel = (awq_linear_kernel)kv;
  if (kernel == AWQ_LINEAR_GEMM_WIDE && !awq::gemm_wide_supported(K, c.group_size, c.w_bit, gated))
    return AWQ_ERR_UNSUPPORTED;
  if (kernel == AWQ_LINEAR_GEMV && M > awq::kGemvMaxM) return AWQ_ERR_BAD_SHAPE;
  if (kernel == AWQ_LINEAR_SKINNY && M > awq::kSkinnyMaxM) return AWQ_ERR_BAD_SHAPE;
  if (!aligned16(X) || !aligned16(qweight) || !aligned16(scales) || !aligned16(zeros) ||
      !aligned16(Y) || (flags && !aligned4(flags)))
    return AWQ_ERR_MISALIGNED;
  hipStream_t st = (hipStream_t)stream;
  if (flags) {
    // data conditions: a scan of X and the group scales ahead of the linear kernel
    const hipError_t e = awq::launch_nonfinite_scan((const uint16_t*)X, M * K,
                                                    (const uint16_t*)scales,
                                                    N * (K / c.group_size), flags, st);
    if (e != hipSuccess) return AWQ_ERR_HIP;
  }
  // AUTO, measured on the Llama-2-7B layer: the vector-ALU GEMV up to M = 3 (its dot cost
  // grows with M), the MFMA skinny GEMV up to g_gemv_max_m, the MFMA GEMM above.
  if (kernel == AWQ_LINEAR_AUTO && c.w_bit != 4) {
    kernel = M <= awq::kGemvMaxM ? AWQ_LINEAR_GEMV
             : M <= awq::kSkinnyMaxM ? AWQ_LINEAR_SKINNY : AWQ_LINEAR_GEMM;
    // the 256-row GEMM where it takes the format (8-bit: plain outputs on 128-column tiles;
    // 3-bit: 256-column tiles), by the 4-bit rule below
    if (kernel == AWQ_LINEAR_GEMM && awq::gemm_wide_supported(K, c.group_size, c.w_bit, gated) &&
        (gated ? awq::gemm_wide_tiles(M, N, true, c.w_bit) >= awq::kWideMinTilesGated
               : M >= awq::kWideMinM))
      kernel = AWQ_LINEAR_GEMM_WIDE;
  }
  if (kernel == AWQ_LINEAR_AUTO) {
    kernel = M <= awq::kVgemvAutoMaxM && M <= g_gemv_max_m ? AWQ_LINEAR_GEMV
             : M <= g_gemv_max_m                            ? AWQ_LINEAR_SKINNY
                                                            : AWQ_LINEAR_GEMM;
    // the 256-row tiling (measured on the Llama-2-7B shapes at M = 128..2048): plain outputs
    // from 128 rows, where its 128-column tiles already beat the 128-row GEMM on every shape;
    // fused gate|up (256-column tiles only) once it has 160 tiles (ahead from 172, behind at
    // 86 and below, where the 128-row tiles give twice as many CUs work)
    if (kernel == AWQ_LINEAR_GEMM && awq::gemm_wide_supported(K, c.group_size, c.w_bit, gated) &&
        (gated ? awq::gemm_wide_tiles(M, N, true, c.w_bit) >= awq::kWideMinTilesGated
               : M >= awq::kWideMinM))
      kernel = AWQ_LINEAR_GEMM_WIDE;
  }
  const auto* Xh = (const uint16_t*)X;
  const auto* sc = (const uint16_t*)scales;
  auto* Yh = (uint16_t*)Y;
  if (c.w_bit == 8) {
    // 8-bit codes: the vector GEMV (M <= 8), the skinny MFMA GEMV (M <= 64), the GEMMs
    if (kernel == AWQ_LINEAR_GEMM_WIDE)
      return hip_status(awq::launch_gemm_wide(Xh, M, qweight, sc, zeros, N, K, c.group_size, 8, Yh,
                                              gated, st));
    if (kernel == AWQ_LINEAR_GEMV)
      return hip_status(
          awq::launch_gemv8(Xh, M, qweight, sc, zeros, N, K, c.group_size, Yh, gated, st));
    if (kernel == AWQ_LINEAR_SKINNY)
      return hip_status(
          awq::launch_gemv_mfma8(Xh, M, qweight, sc, zeros, N, K, c.group_size, Yh, gated, st));
    return hip_status(
        awq::launch_gemm(Xh, M, qweight, sc, zeros, N, K, c.group_size, 8, Yh, gated, st));
  }
  if (c.w_bit == 3) {
    // 3-bit codes: the same kernels' 3-bit forms, with the same thresholds
    if (kernel == AWQ_LINEAR_GEMM_WIDE)
      return hip_status(awq::launch_gemm_wide(Xh, M, qweight, sc, zeros, N, K, c.group_size, 3, Yh,
                                              gated, st));
    if (kernel == AWQ_LINEAR_GEMV)
      return hip_status(
          awq::launch_gemv3(Xh, M, qweight, sc, zeros, N, K, c.group_size, Yh, gated, st));
    if (kernel == AWQ_LINEAR_SKINNY)
      return hip_status(
          awq::launch_gemv_mfma3(Xh, M, qweight, sc, zeros, N, K, c.group_size, Yh, gated, st));
    return hip_status(
        awq::launch_gemm(Xh, M, qweight, sc, zeros, N, K, c.group_size, 3, Yh, gated, st));
  }
  switch (kernel) {
    case AWQ_LINEAR_GEMM_WIDE:
      return hip_status(
          awq::launch_gemm_wide(Xh, M, qweight, sc, zeros, N, K, c.group_size, 4, Yh, gated, st));
    case AWQ_LINEAR_GEMV:
      return hip_status(
          awq::launch_gemv(Xh, M, qweight, sc, zeros, N, K, c.group_size, Yh, gated, st));
    case AWQ_LINEAR_SKINNY:
      return hip_status(
          awq::launch_gemv_mfma(Xh, M, qweight, sc, zeros, N, K, c.group_size, Yh, gated, st));
    default:
      return hip_status(
          awq::launch_gemm(Xh, M, qweight, sc, zeros, N, K, c.group_size, 4, Yh, gated, st));
  }
}

awq_status awq_linear_w4a16_ex(const void* X, int64_t M, const uint32_t* qweight,
                               const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                               const awq_config* cfg, void* Y, uint32_t* flags,
                               awq_linear_kernel kernel, void* stream) {
  return linear_common(X, M, qweight, scales, zeros, N, K, cfg, Y, flags, kernel, false, stream);
}

awq_status awq_linear_w4a16(const void* X, int64_t M, const uint32_t* qweight,
                            const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                            const awq_config* cfg, void* Y, uint32_t* flags, void* stream) {
  return awq_linear_w4a16_ex(X, M, qweight, scales, zeros, N, K, cfg, Y, flags, AWQ_LINEAR_AUTO,
                             stream);
}

awq_status awq_linear_w4a16_gated_silu_ex(const void* X, int64_t M, const uint32_t* qweight,
                                          const void* scales, const uint8_t* zeros, int64_t N,
                                          int64_t K, const awq_config* cfg, void* Y,
                                          uint32_t* flags, awq_linear_kernel kernel,
                                          void* stream) {
  return linear_common(X, M, qweight, scales, zeros, N, K, cfg, Y, flags, kernel, true, stream);
}

awq_status awq_linear_w4a16_gated_silu(const void* X, int64_t M, const uint32_t* qweight,
                                       const void* scales, const uint8_t* zeros, int64_t N,
                                       int64_t K, const awq_config* cfg, void* Y,
                                       uint32_t* flags, void* stream) {
  return awq_linear_w4a16_gated_silu_ex(X, M, qweight, scales, zeros, N, K, cfg, Y, flags,
                                        AWQ_LINEAR_AUTO, stream);
}

size_t awq_clip_search_workspace_size(int64_t T, int64_t N, int64_t K, int32_t n_shrink,
                                      const awq_config* cfg) {
  const awq_config c = resolve(cfg);
  if (!supported(c) || !good_nk(N, K) || n_shrink < 1) return 0;
  if (T < 1 || T > awq::kClipMaxTokens) return 0;
  return clip_layout(T, N, K, n_shrink, c.group_size).total;
}

awq_status awq_clip_search(const void* X, int64_t T, const void* W, int64_t N, int64_t K,
                           const void* s, int32_t clip_steps, int32_t n_shrink,
                           const awq_config* cfg, uint8_t* clip_idx, double* err,
                           void* workspace, size_t workspace_bytes, uint32_t* flags,
                           void* stream) {
  const awq_config c = resolve(cfg);
  if (!X || !W || !clip_idx) return AWQ_ERR_NULL_POINTER;
  if (!supported(c)) return AWQ_ERR_UNSUPPORTED;
  if (T < 1 || T > awq::kClipMaxTokens || !good_nk(N, K)) return AWQ_ERR_BAD_SHAPE;
  if (clip_steps < 1 || clip_steps > 65535 || n_shrink < 1 || n_shrink > clip_steps ||
      n_shrink > awq::kClipMaxShrink)
    return AWQ_ERR_BAD_SHAPE;
  if (!aligned16(X) || !aligned16(W) || (s && !aligned16(s)) || (err && !aligned16(err)) ||
      (flags && !aligned4(flags)))
    return AWQ_ERR_MISALIGNED;
  const ClipLayout L = clip_layout(T, N, K, n_shrink, c.group_size);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return AWQ_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  void* errs = ws + L.err;
  hipError_t e = awq::launch_clip_err((const uint16_t*)X, T, (const uint16_t*)W, N, K,
                                      (const uint16_t*)s, clip_steps, n_shrink, c.zero_point == 0,
                                      c.group_size, c.w_bit, (uint4*)(ws + L.xp), errs, flags, st);
  if (e == hipSuccess)
    e = awq::launch_clip_reduce(errs, T, n_shrink, N, K, c.group_size, clip_idx, err, flags, st);
  return hip_status(e);
}

awq_status awq_apply_inverse_scale(const void* A, int64_t rows, int64_t cols, const void* s,
                                   int32_t axis, void* out, uint32_t* flags, void* stream) {
  if (!A || !s || !out) return AWQ_ERR_NULL_POINTER;
  if (axis != 0 && axis != 1) return AWQ_ERR_UNSUPPORTED;
  if (rows < 1 || cols < 8 || cols % 8 != 0 || rows >= kMaxDim || cols >= kMaxDim)
    return AWQ_ERR_BAD_SHAPE;
  if (!aligned16(A) || !aligned16(s) || !aligned16(out) || (flags && !aligned4(flags)))
    return AWQ_ERR_MISALIGNED;
  return hip_status(awq::launch_inverse_scale((const uint16_t*)A, rows, cols, (const uint16_t*)s,
                                              axis, (uint16_t*)out, flags, (hipStream_t)stream));
}

}  // extern "C"
