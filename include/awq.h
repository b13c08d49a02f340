/*
 * awq.h -- C ABI of the MI355X (gfx950) AWQ W4A16 hot-path library (libawq_mi355x.so).
 *
 * AWQ (activation-aware weight quantization) keeps activations in 16-bit and stores
 * weights as 4-bit integers, one fp16 scale and one 4-bit zero point per group of
 * 128 (or 64 or 32) consecutive input channels; before quantizing, input channel k of the weight is
 * multiplied by a scale s_k picked from offline activation magnitudes, and the
 * activation side carries 1/s_k (an equivalent transform).
 *
 * Sources (web pages, cited by title and section):
 *   "AWQ量化实战：无需重训，把大模型压进4bit显存" (xdnf.cn)            -- [PRACTICE]
 *   "AWQ量化技术Skill" (skillsbot.cn, awq-quantization usage page)  -- [SKILL]
 *   "大模型量化部署实战：GPTQ与AWQ算法" (yunthe.com)                 -- [GPTQ-AWQ]
 *   "什么是激活感知权重量化（AWQ）" (aiboss88.com)                   -- [WIKI]
 *   "AWQ技术概述：重新定义大语言模型量化" (nxmr.cn, untitled; its first heading) -- [NXMR]
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library never
 *     allocates, frees, copies to the host or synchronizes. Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and is complete when the
 *     stream reaches it.
 *   - fp16 = IEEE binary16, passed as void*. All matrices are dense row-major.
 *   - W is [N][K] (out features x in features), X is [rows][K], Y = X * W^T is [M][N]
 *     ([PRACTICE] §2.1: the weight is "output dim x input dim", channels are input dims).
 *   - Argument errors are detected on the host before anything is enqueued; the call
 *     then returns a non-zero status and touches no output. Launch failures return
 *     AWQ_ERR_HIP. Conditions that only the data reveals are OR-ed into the optional
 *     device word `flags` (never cleared by the library).
 *   - Identical inputs give bitwise-identical outputs (no floating-point atomics).
 *   - Base pointers must be 16-byte aligned.
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                          */
  AWQ_ERR_BAD_SHAPE = 2,     /* a size < 1, K % 128 != 0, T above 8192, ...          */
  AWQ_ERR_UNSUPPORTED = 3,   /* config outside w_bit 3,4,8 / group 128,64,32 / zp 0,1 */
  AWQ_ERR_MISALIGNED = 4,    /* a base pointer is not 16-byte aligned                */
  AWQ_ERR_WORKSPACE = 5,     /* workspace missing or smaller than the query returns  */
  AWQ_ERR_HIP = 6,           /* the HIP runtime reported an error on launch          */
  AWQ_ERR_SCRATCH_LIMIT = 7  /* a no-allocation call needs more than its static array */
} awq_status;

/* Quantization config ([SKILL] "如何使用该技能 / 步骤 2": quant_config zero_point, q_group_size,
 * w_bit; the page's "version" GEMM/GEMV switch becomes dispatch on M inside
 * awq_linear_w4a16). Supported: w_bit = 4, 8 ([PRACTICE] §3.3: near lossless; §5.2 / §5.3
 * raise w_bit when 4-bit accuracy falls short) or 3 ([PRACTICE] §4.3 names 3-bit weights as the extreme low
 * width), group_size = 128, 64 or 32 ([PRACTICE] §2.3:
 * 128 is the usual group, 64 and 32 also in use), zero_point = 1 or 0, 1 <= n_grid <= 64.
 * NULL config pointers mean {4, 128, 1, 20}. Every entry point takes the group size from
 * the config; K stays a multiple of 128 in every case, so a smaller group never straddles
 * a 128-channel step of the kernels. With 32-channel groups the skinny MFMA GEMV and the
 * GEMM round (q - z) sc to fp16 before the multiply (within the linear tolerance).
 * zero_point = 0 ([PRACTICE] §3.3 advises it; [GPTQ-AWQ] gives the signed range -8..7):
 * sc = max|w'| / 7, q - 8 = clamp(rint(w'/sc_h), -8, 7), stored offset by 8 with every
 * zero nibble 8 -- the same packed format, so the linear entry points are unchanged;
 * quantize, search and clip search honour the mode (8-bit: /127 and zero 128; 3-bit: /3
 * and zero 4). w_bit = 8 or 3: the same quantizer with 255 or 7 levels and its own packed
 * layout (see awq_quantize_pack); every entry point, linear kernels included, takes it
 * from the config.
 * The linear entry points need the config the weight was packed with. */
typedef struct awq_config {
  int32_t w_bit;
  int32_t group_size;
  int32_t zero_point;
  int32_t n_grid; /* number of alpha grid points: alpha_i = i / n_grid, i = 0 .. n_grid-1 */
} awq_config;

#define AWQ_FLAG_NONFINITE_INPUT 1u /* NaN or Inf met in W, s or X (outputs unspecified) */
#define AWQ_FLAG_SCALE_CLAMPED 2u   /* a group scale above 65504 was clamped to 65504   */
#define AWQ_FLAG_OVERFLOW 8u        /* a finite value folded by 1/s overflowed fp16      */

#define AWQ_MAX_CALIB_TOKENS 8192

/* Which linear kernel awq_linear_w4a16_ex runs. */
typedef enum awq_linear_kernel {
  AWQ_LINEAR_AUTO = 0, /* vector GEMV for M <= 3, skinny MFMA GEMV up to
                          awq_gemv_max_m(), MFMA GEMM above (8- and 3-bit
                          codes: vector GEMV up to 8, skinny up to 64)         */
  AWQ_LINEAR_GEMV = 1, /* wave-per-rows dequant-fused GEMV (any M <= 8)       */
  AWQ_LINEAR_GEMM = 2, /* MFMA dequant-GEMM (any M)                           */
  AWQ_LINEAR_SKINNY = 3, /* MFMA GEMV for small batches, split K (M <= 64)    */
  AWQ_LINEAR_GEMM_WIDE = 4 /* MFMA dequant-GEMM on 256-row tiles, one wave per SIMD
                              (4- and 3-bit codes, or 8-bit codes without the
                              gated epilogue; any group size; 256 K < 2^32;
                              else AWQ_ERR_UNSUPPORTED); AUTO takes
                              it over the GEMM from M = 128 (fused gate|up: from
                              160 tiles of 128 outputs)                        */
} awq_linear_kernel;

/*
 * awq_quantize_pack -- group-wise asymmetric 4-bit quantization of W * diag(s), packed.
 *   [PRACTICE] §2.3 (128 consecutive input channels share one step), §3.3 step 5;
 *   [GPTQ-AWQ] "大模型量化的核心原理与位宽选择" (4-bit integer + scale + zero point).
 *   Per row n and group j (g = group_size consecutive channels), in fp32 with
 *   round-to-nearest-even:
 *     w' = w * s_k;  sc = max((max w' - min w') / 15, 2^-14) (clamped at 65504);
 *     sc_h = fp16(sc);  z = clamp(rint(-min w' / sc_h), 0, 15);
 *     q = clamp(rint(w' / sc_h) + z, 0, 15).
 *   W        fp16 [N][K]          input, K % 128 == 0
 *   s        fp16 [K]             per-input-channel scale; NULL means s = 1 (plain RTN)
 *   qweight  uint32 [N][K/8]      out: word w holds the codes of k = 8w..8w+7; nibble j (bits
 *                                 4j..4j+3) holds k = 8w + (0,2,4,6,1,3,5,7)[j], so each byte
 *                                 holds one channel pair (2p low nibble, 2p+1 high nibble)
 *   scales   fp16 [N][G]          out: sc_h, G = K/g
 *   zeros    uint8 [N][ceil(G/2)] out: low nibble = even group, high = odd group
 *   flags    uint32 [1] or NULL   NONFINITE_INPUT, SCALE_CLAMPED
 *   w_bit = 8: 15 -> 255 above (codes 0..255); qweight uint32 [N][K/4], byte j of word w
 *   holds k = 4w + j; zeros uint8 [N][G], one byte per group; scales as above.
 *   w_bit = 3: 15 -> 7 above (codes 0..7); qweight uint32 [N][3K/32] in bit planes, 12
 *   words per 128-channel block b (words 12b .. 12b + 11): word 12b + i (i < 8) holds bits
 *   0-1 of the codes of k = 128b + 16i + 2f at bits 2f, 2f + 1 and of k + 1 at bits
 *   16 + 2f, 17 + 2f (f = 0..7); word 12b + 8 + j (j < 4) holds bit 2 of the codes of
 *   k = 128b + 32j + 2p at bit p and of k + 1 at bit 16 + p (p = 0..15); zeros and scales
 *   as for 4-bit.
 */
awq_status awq_quantize_pack(const void* W, int64_t N, int64_t K, const void* s,
                             const awq_config* cfg, uint32_t* qweight, void* scales,
                             uint8_t* zeros, uint32_t* flags, void* stream);

/*
 * awq_activation_stats -- per-input-channel mean absolute activation.
 *   [PRACTICE] §2.1 (accumulate calibration activations per input channel and take the
 *   mean absolute value); [WIKI] "工作机制" (offline activation statistics).
 *   a_k = (sum_t |X_tk|) / T, with the sum exact (fixed point) and one fp64 division.
 *   X         fp16 [T][K], 1 <= T <= 8192
 *   act_mean  fp64 [K]   out
 *   workspace device scratch of awq_activation_stats_workspace_size(T, K) bytes
 *   flags     NONFINITE_INPUT
 */
size_t awq_activation_stats_workspace_size(int64_t T, int64_t K);
awq_status awq_activation_stats(const void* X, int64_t T, int64_t K, double* act_mean,
                                void* workspace, size_t workspace_bytes, uint32_t* flags,
                                void* stream);

/*
 * awq_candidate_scales -- the per-channel scale of every alpha grid point.
 *   [PRACTICE] §2.2 (grid search over a candidate interval), §5.1 (one coefficient per
 *   layer); [WIKI] "工作机制" (scale set from offline activation statistics).
 *   s_grid[i][k] = fp16_rne(pow(max(act_mean[k], 2^-14), i / n_grid)) (fp64 pow), so row
 *   0 is all ones (plain RTN).
 *   act_mean fp64 [K];  s_grid fp16 [n_grid][K] out.
 */
awq_status awq_candidate_scales(const double* act_mean, int64_t K, const awq_config* cfg,
                                void* s_grid, void* stream);

/*
 * awq_search_scales -- activation-aware grid search of the per-channel scale.
 *   [PRACTICE] §2.2 / §3.3 step 4: pick, over the grid, the s whose quantized layer keeps
 *   the calibration outputs closest to the original ones; [WIKI] "工作机制" (equivalent
 *   transform W diag(s), X diag(1/s); no backpropagation).
 *     err_i = sum_t sum_n ( sum_k X_tk (W_nk - deq(Q(W diag(s_i)))_nk / s_ik) )^2
 *     best  = smallest i with err_i == min err
 *   Linears that share one input (q|k|v, gate|up) share one s: pass them concatenated
 *   along N.
 *   X         fp16 [T][K], 1 <= T <= 8192 (calibration activations)
 *   W         fp16 [N][K]
 *   s_best    fp16 [K]          out: s_{best}
 *   best_idx  int32 [1]         out: best
 *   err       fp64 [n_grid]     out (may be NULL)
 *   s_grid    fp16 [n_grid][K]  out (may be NULL): every candidate scale
 *   workspace device scratch of awq_search_workspace_size(T, N, K, cfg) bytes (statistics,
 *             candidate scales, partial errors and a copy of X in MFMA operand order)
 *   flags     NONFINITE_INPUT (a NaN or Inf in X or W, or a non-finite error), SCALE_CLAMPED
 *   Accuracy: the contraction runs on the matrix cores with D = W - deq / s split into
 *   fp16 hi + lo (22 significant bits) after scaling each (row, 128-channel step) of D by
 *   its own power of two, so the errors hold about 1e-6 relative whatever the spread of s
 *   across a row (a row whose |D| spans more than about 2^80 can overflow the fp32 running
 *   error: the error is then non-finite and NONFINITE_INPUT is raised).
 *   From N * K >= 2^22 weights and T >= 256 tokens every grid point is first scored with
 *   hi alone (half the matrix-core work; over that many terms the rounding moves an error
 *   by about 2e-6 relative at most), then every point whose error lies within 2^-12
 *   (relative) of the smallest is scored again with hi + lo: the chosen index is always
 *   decided by hi + lo errors, and err holds hi + lo errors for those points, hi-only
 *   errors for the others. No host synchronization: both passes and the choice of points
 *   run on the stream.
 *   Follow with awq_quantize_pack(W, s_best) to obtain the packed weights.
 */
size_t awq_search_workspace_size(int64_t T, int64_t N, int64_t K, const awq_config* cfg);
awq_status awq_search_scales(const void* X, int64_t T, const void* W, int64_t N, int64_t K,
                             const awq_config* cfg, void* s_best, int32_t* best_idx,
                             double* err, void* s_grid, void* workspace,
                             size_t workspace_bytes, uint32_t* flags, void* stream);

/*
 * awq_search_scales_noalloc -- awq_search_scales for callers that cannot allocate device
 *   memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc. Same arguments without the workspace, same kernels and bit-identical
 *   results. The workspace is a static device array of AWQ_NOALLOC_SCRATCH_BYTES that
 *   the library holds on every GPU it runs on until the process ends; its address is
 *   looked up on the first call on each device, so the current device must be the one
 *   `stream` belongs to. The call allocates nothing.
 *   Limit: awq_search_workspace_size(T, N, K, cfg) <= AWQ_NOALLOC_SCRATCH_BYTES (32 MiB:
 *   e.g. T = 512 calibration tokens up to K = 28672), else AWQ_ERR_SCRATCH_LIMIT before
 *   anything is enqueued. Every call on one GPU uses the same array (it keeps the last
 *   call's contents; each call clears what it needs): calls that overlap on one GPU
 *   (different streams or host threads) race and must be serialized by the caller.
 */
#define AWQ_NOALLOC_SCRATCH_BYTES (32u << 20)
awq_status awq_search_scales_noalloc(const void* X, int64_t T, const void* W, int64_t N,
                                     int64_t K, const awq_config* cfg, void* s_best,
                                     int32_t* best_idx, double* err, void* s_grid,
                                     uint32_t* flags, void* stream);

/*
 * awq_linear_w4a16 -- Y = X * deq(W)^T with 4-bit packed weights and fp16 activations.
 *   [PRACTICE] §3.4 (decode is memory-bound: smaller weights, faster tokens); [SKILL]
 *   "主要功能和特点" (GEMV kernel for single-token decode, GEMM kernel for batches).
 *   deq(W)_nk = (q_nk - z_nj) * sc_nj; products accumulate in fp32; Y is rounded to fp16.
 *   X fp16 [M][K]; qweight/scales/zeros as written by awq_quantize_pack; Y fp16 [M][N].
 *   flags uint32 [1] or NULL: NONFINITE_INPUT when X or the group scales hold an Inf or a
 *   NaN (Y is then unspecified where they reach). Only with a flags word does the call
 *   add a scan of X and the scales (2 bytes per element) ahead of the linear kernel.
 *   Dispatch: M <= 3 runs the vector-ALU dequant-fused GEMV, M <= 64 the skinny MFMA
 *   GEMV (dots on the matrix cores, K split over the waves of a block; two 32-token tiles
 *   above M = 32), larger M the MFMA dequant-GEMM (thresholds measured on the Llama-2-7B
 *   layer).
 */
awq_status awq_linear_w4a16(const void* X, int64_t M, const uint32_t* qweight,
                            const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                            const awq_config* cfg, void* Y, uint32_t* flags, void* stream);

/* Same as awq_linear_w4a16 with an explicit kernel choice (GEMV requires M <= 8,
 * SKINNY M <= 64, otherwise AWQ_ERR_BAD_SHAPE; GEMM_WIDE a config it supports, otherwise
 * AWQ_ERR_UNSUPPORTED). */
awq_status awq_linear_w4a16_ex(const void* X, int64_t M, const uint32_t* qweight,
                               const void* scales, const uint8_t* zeros, int64_t N, int64_t K,
                               const awq_config* cfg, void* Y, uint32_t* flags,
                               awq_linear_kernel kernel, void* stream);

/*
 * awq_linear_w4a16_gated_silu -- fused MLP module of a packed gate|up weight:
 *   Y = SiLU(X * deq(W_gate)^T) * (X * deq(W_up)^T), SiLU(v) = v / (1 + e^-v).
 *   [SKILL] "主要功能和特点" (fused attention/MLP modules lower decode latency); [WIKI]
 *   TinyChat (kernel fusion). Reading: Llama's gated MLP, with gate and up packed as one
 *   weight so one launch streams both.
 *   qweight/scales/zeros: one packed weight of N rows (awq_quantize_pack of the stacked
 *   [W_gate; W_up]): rows [0, N/2) are the gate projection, rows [N/2, N) the up
 *   projection. N must be even (else AWQ_ERR_BAD_SHAPE). X fp16 [M][K]; Y fp16 [M][N/2].
 *   g and u are accumulated in fp32 exactly as in awq_linear_w4a16, SiLU(g) * u is formed
 *   in fp32 and rounded once to fp16. Kernel choice, errors and alignment as for
 *   awq_linear_w4a16 / awq_linear_w4a16_ex.
 */
awq_status awq_linear_w4a16_gated_silu(const void* X, int64_t M, const uint32_t* qweight,
                                       const void* scales, const uint8_t* zeros, int64_t N,
                                       int64_t K, const awq_config* cfg, void* Y,
                                       uint32_t* flags, void* stream);
awq_status awq_linear_w4a16_gated_silu_ex(const void* X, int64_t M, const uint32_t* qweight,
                                          const void* scales, const uint8_t* zeros, int64_t N,
                                          int64_t K, const awq_config* cfg, void* Y,
                                          uint32_t* flags, awq_linear_kernel kernel,
                                          void* stream);

/*
 * awq_clip_search -- weight clipping: per group, the shrink of its quantization range
 *   that best preserves its share of the calibration outputs.
 *   [NXMR] §5.1 "精度下降严重" (tune clip_steps, 200 suggested, when accuracy drops).
 *   Reading: with s fixed (the scale search's choice; NULL = 1), group (n, g) of W diag(s)
 *   tries r_i = (clip_steps - i) / clip_steps, i = 0 .. n_shrink - 1 (r_0 = 1: plain
 *   min/max), quantized from the extremes r_i max and r_i min (fp32), scored by
 *     err_i(n, g) = sum_t ( sum_{k in g} X_tk D_nk )^2,  D = W - Q_{r_i}(W diag(s)) diag(1/s),
 *   and keeps the first minimum. Contraction as in awq_search_scales (D as fp16 hi + lo
 *   against fp16 X on the matrix cores, fp32 accumulation, fp64 reduction). For
 *   128-channel groups and T > 256 the same score is formed as d^T G d with the group's
 *   Gram matrix G = X_g^T X_g (fp64 sums, channels balanced by exact powers of two, kept
 *   as fp16 hi + lo): 2 * 128 instead of 2 * T flop per weight and ratio.
 *   X fp16 [T][K], 1 <= T <= 512 (else AWQ_ERR_BAD_SHAPE: one block scores all tokens);
 *   W fp16 [N][K]; s fp16 [K] or NULL; 1 <= n_shrink <= min(clip_steps, 256).
 *   clip_idx uint8 [N][G] out (pass to awq_quantize_pack_clipped); err fp64 [N][G]
 *   out, the chosen error, or NULL; G = K / group_size. workspace: device,
 *   awq_clip_search_workspace_size bytes (the errors: n_shrink N G doubles for
 *   128-channel groups, n_shrink N G w floats for smaller ones, w = 4 per-wave partials
 *   for T <= 256, else 8; and a copy of X in MFMA operand order, T rounded up to 64
 *   tokens, or the Gram matrices (512 B per channel) and channel scales, whichever is
 *   larger; 0 for an unsupported config or shape, T included), 16-byte aligned. Accuracy: each group's D is scaled by a power of two
 *   from its own largest |D| before the fp16 hi + lo split, so every group keeps 22
 *   significant bits whatever its magnitude or the code width.
 *   flags: NONFINITE_INPUT (a NaN or Inf in W or s, or in X through a non-finite error).
 */
size_t awq_clip_search_workspace_size(int64_t T, int64_t N, int64_t K, int32_t n_shrink,
                                      const awq_config* cfg);
awq_status awq_clip_search(const void* X, int64_t T, const void* W, int64_t N, int64_t K,
                           const void* s, int32_t clip_steps, int32_t n_shrink,
                           const awq_config* cfg, uint8_t* clip_idx, double* err,
                           void* workspace, size_t workspace_bytes, uint32_t* flags,
                           void* stream);

/*
 * awq_quantize_pack_clipped -- awq_quantize_pack with per-group clipping: group (n, g)
 *   quantizes from its extremes times r = (clip_steps - clip_idx[n][g]) / clip_steps
 *   (fp32); weights beyond the shrunk range take the end codes. clip_idx uint8 [N][K/g]
 *   (awq_clip_search's output) or NULL (plain awq_quantize_pack); 1 <= clip_steps <= 65535.
 */
awq_status awq_quantize_pack_clipped(const void* W, int64_t N, int64_t K, const void* s,
                                     const uint8_t* clip_idx, int32_t clip_steps,
                                     const awq_config* cfg, uint32_t* qweight, void* scales,
                                     uint8_t* zeros, uint32_t* flags, void* stream);

/*
 * awq_apply_inverse_scale -- fold 1/s into the producer of a linear's input (the other
 *   half of the equivalent transform): out = fp16(A / s), correctly rounded.
 *   [PRACTICE] §2.2 (W's salient channels are multiplied by s, the other side divided by
 *   s); [WIKI] "工作机制" (equivalent transformation: X W^T = (X diag(1/s)) (W diag(s))^T).
 *   A, out: fp16 [rows][cols], cols % 8 == 0 (else AWQ_ERR_BAD_SHAPE); out may equal A
 *   (in place). s: fp16, the scales awq_search_scales chose.
 *   axis = 1: out[r][k] = A[r][k] / s_k, len(s) = cols -- the activations themselves or
 *     a norm weight (rows = 1) that produces them;
 *   axis = 0: out[k][j] = A[k][j] / s_k, len(s) = rows -- the previous linear's weight,
 *     whose output row k feeds input channel k.
 *   Any other axis: AWQ_ERR_UNSUPPORTED. flags: AWQ_FLAG_OVERFLOW (a finite value became
 *   infinite), AWQ_FLAG_NONFINITE_INPUT (NaN or Inf in A or s).
 */
awq_status awq_apply_inverse_scale(const void* A, int64_t rows, int64_t cols, const void* s,
                                   int32_t axis, void* out, uint32_t* flags, void* stream);

/* Largest M served by a GEMV-class kernel under AWQ_LINEAR_AUTO with 4-bit codes (64, or
 * the value of the AWQ_GEMV_MAX_M environment variable clamped to 0..64, read at library
 * load). */
int32_t awq_gemv_max_m(void);

/* Human-readable text of a status code (static storage). */
const char* awq_status_string(awq_status status);

#ifdef __cplusplus
}
#endif
#endif /* AWQ_MI355X_H */
