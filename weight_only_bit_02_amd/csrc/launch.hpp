// Internal launchers: host functions that enqueue one kernel each on a stream.
// The C ABI (awq_abi.hip) validates arguments and calls these; nothing here checks
// arguments again.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

// a3 + a4: quantize W * diag(s) per group of 128 and pack codes / scales / zeros.
// clip_idx (nullable, [N][G]): group (n, j) shrinks its range by (steps - idx) / steps.
// sym: zero point off (sc = max|w'| / 7, zero fixed at 8, same stored format).
// group: 128 or 64 input channels per scale / zero.
hipError_t launch_quant_pack(const uint16_t* W, int64_t N, int64_t K, const uint16_t* s,
                             uint32_t* qweight, uint16_t* scales, uint8_t* zeros,
                             const uint8_t* clip_idx, int clip_steps, bool sym, int group,
                             int w_bit, uint32_t* flags, hipStream_t stream);

// f3: err[i][n][g] = sum_t (sum_{k in g} X_tk D_nk)^2 for the clip ratios i < n_shrink
// (T <= 512), then the first minimum per (n, g).
hipError_t launch_clip_err(const uint16_t* X, int64_t T, const uint16_t* W, int64_t N,
                           int64_t K, const uint16_t* s, int clip_steps, int n_shrink, bool sym,
                           int group, int w_bit, uint4* xp, void* err, uint32_t* flags,
                           hipStream_t stream);
// Bytes of the clip search's error array: fp64 [n_shrink][N][G] for 128-channel groups;
// for smaller ones the per-wave fp32 partials [n_shrink][G][waves][N] (4 or 8 waves by T).
size_t clip_err_bytes(int64_t T, int64_t N, int64_t K, int n_shrink, int group);
// Bytes of the MFMA-ordered copy of X (T tokens rounded up to 64, K channels) that the
// scale and clip searches read their activations from.
size_t packed_x_bytes(int64_t T, int64_t K);
// Bytes of the clip search's scratch: the copy of X above, or for the Gram form (128-channel
// groups, T > 256) the per-group Gram matrices G' in operand order and the channel scales,
// whichever is larger.
size_t clip_scratch_bytes(int64_t T, int64_t K, int group);
hipError_t launch_clip_reduce(const void* err, int64_t T, int n_shrink, int64_t N, int64_t K,
                              int group, uint8_t* clip_idx, double* err_best, uint32_t* flags,
                              hipStream_t stream);
constexpr int kClipMaxTokens = 512;
constexpr int kClipMaxShrink = 256;

// a1: u_k = sum_t |X_tk| in units of 2^-24 (int64, exact), then a_k = u_k 2^-24 / T.
hipError_t launch_zero_u64(unsigned long long* p, int64_t n, hipStream_t stream);
hipError_t launch_act_sums(const uint16_t* X, int64_t T, int64_t K, unsigned long long* u,
                           uint32_t* flags, hipStream_t stream);
hipError_t launch_act_finalize(const unsigned long long* u, int64_t T, int64_t K, double* act,
                               hipStream_t stream);

// a2: s_grid[i][k] = fp16_rne(pow(max(act_k, 2^-14), i / n_grid)).
hipError_t launch_scalegen(const double* act, int64_t K, int n_grid, uint16_t* s_grid,
                           hipStream_t stream);

// a5: per (alpha, row tile, token chunk) partial sums of the squared output error.
int search_row_tile();
int search_token_chunk(int64_t T);
// Whether a search of this size scores every grid point with one fp16 term of D first and
// re-scores only the near-minimal points with two (else two terms throughout).
bool search_one_term(int64_t T, int64_t N, int64_t K);
// xp: scratch for the copy of X in MFMA operand order (packed_x_bytes(T, K)). one_term:
// errf (fp64 n_grid) receives the one-term errors and cand (n_grid bytes) the points that
// the two-term pass re-scored into partials; both unused otherwise.
hipError_t launch_search_err(const uint16_t* X, int64_t T, const uint16_t* W, int64_t N,
                             int64_t K, const uint16_t* s_grid, int n_grid, bool sym, int group,
                             int w_bit, uint4* xp, double* partials, double* errf, uint8_t* cand,
                             bool one_term, uint32_t* flags, hipStream_t stream);
// a6: fixed-order sums of the partials (with cand: of the marked points only, errf for the
// rest), first-minimum argmin, s_best copy.
hipError_t launch_search_reduce(const double* partials, int n_grid, int64_t n_partials,
                                const uint8_t* cand, const double* errf, const uint16_t* s_grid,
                                int64_t K, uint16_t* s_best, int32_t* best_idx, double* err,
                                uint32_t* flags, hipStream_t stream);

// a7 / a8: Y = X deq(W)^T. gated (f1): W is gate|up stacked (N/2 rows each) and
// Y[M][N/2] = SiLU(X deq(W_gate)^T) * (X deq(W_up)^T); N is even.
// group: 128 or 64 (the layout of scales / zeros).
// 8-bit codes (qweight uint32 [N][K/4], byte j of word w = channel 4w + j; zeros uint8
// [N][G]): the vector GEMV for M <= 8, plain or gated.
hipError_t launch_gemv8(const uint16_t* X, int64_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                        int group, uint16_t* Y, bool gated, hipStream_t stream);
// 8-bit codes: the skinny MFMA GEMV (M <= kSkinnyMaxM), plain or gated.
hipError_t launch_gemv_mfma8(const uint16_t* X, int64_t M, const uint32_t* qweight,
                             const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                             int group, uint16_t* Y, bool gated, hipStream_t stream);
// 3-bit codes (two bit planes per 128-channel block): the vector GEMV (M <= 8) and the
// skinny MFMA GEMV (M <= kSkinnyMaxM), plain or gated.
hipError_t launch_gemv3(const uint16_t* X, int64_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                        int group, uint16_t* Y, bool gated, hipStream_t stream);
hipError_t launch_gemv_mfma3(const uint16_t* X, int64_t M, const uint32_t* qweight,
                             const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                             int group, uint16_t* Y, bool gated, hipStream_t stream);
hipError_t launch_gemv(const uint16_t* X, int64_t M, const uint32_t* qweight,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       int group, uint16_t* Y, bool gated, hipStream_t stream);
hipError_t launch_gemm(const uint16_t* X, int64_t M, const uint32_t* qweight,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       int group, int w_bit, uint16_t* Y, bool gated, hipStream_t stream);

// a8, 4- and 3-bit codes (and 8-bit codes, plain outputs), every group size: the GEMM
// with 256-row tiles (256 or 128 columns) and one wave per SIMD (gemm_wide.hip).
// gemm_wide_supported: the configs and sizes it takes; gemm_wide_tiles: its tile count for an
// M x N output (gated: N / 2 outputs).
bool gemm_wide_supported(int64_t K, int group, int w_bit, bool gated);
int64_t gemm_wide_tiles(int64_t M, int64_t N, bool gated, int w_bit);
constexpr int64_t kWideMinM = 128;         // AUTO: the wide GEMM from 128 rows (plain output)
constexpr int64_t kWideMinTilesGated = 160;  // and from 160 tiles (fused gate|up)
hipError_t launch_gemm_wide(const uint16_t* X, int64_t M, const uint32_t* qweight,
                            const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                            int group, int w_bit, uint16_t* Y, bool gated, hipStream_t stream);

// Data conditions of the linear path: OR AWQ_FLAG_NONFINITE_INPUT into *flags when a
// (n fp16 values, n % 8 == 0) or b (m fp16 values) holds an Inf or a NaN.
hipError_t launch_nonfinite_scan(const uint16_t* a, int64_t n, const uint16_t* b, int64_t m,
                                 uint32_t* flags, hipStream_t stream);

// f2: out = fp16(A / s) along columns (axis 1, len(s) = cols) or rows (axis 0,
// len(s) = rows); cols % 8 == 0; out may alias A.
hipError_t launch_inverse_scale(const uint16_t* A, int64_t rows, int64_t cols, const uint16_t* s,
                                int axis, uint16_t* out, uint32_t* flags, hipStream_t stream);

// a7 / a9 for small batches: 32-row MFMA tiles, K split over the waves of a block; one
// token tile up to M = 32, two up to 64.
constexpr int kSkinnyMaxM = 64;
hipError_t launch_gemv_mfma(const uint16_t* X, int64_t M, const uint32_t* qweight,
                            const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                            int group, uint16_t* Y, bool gated, hipStream_t stream);

constexpr int kGemvMaxM = 8;       // the vector-ALU GEMV serves M <= 8 when asked for
constexpr int kVgemvAutoMaxM = 3;  // and is the automatic choice up to M = 3

}  // namespace awq
