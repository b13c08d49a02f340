"""Plain, slow CPU oracle of the AWQ (Activation-aware Weight Quantization) hot path.

TEST INFRASTRUCTURE ONLY: used by the tests, by the smoke check and by the
``cpu_baseline`` leg of the benchmark. The product path never imports it, and it
imports nothing from the product path.

Sources (web pages; cited by title and section):

* [AWQ-PRACTICE] "AWQ量化实战：无需重训，把大模型压进4bit显存" (xdnf.cn), the
  practitioner's walk-through: §1.1 (RTN baseline), §1.3 (scale salient channels
  by s > 1 before uniform low-bit quantization), §2.1 (weight is out x in,
  channels are input channels, statistic = mean absolute activation), §2.2 (grid
  search of s so that outputs before/after quantization agree; 1/s undone on the
  other side), §2.3 (128 consecutive input channels share one step), §3.3 (the
  per-layer steps: statistics -> search s -> 4-bit g128 quantize -> save scales).
* [AWQ-SKILL] "AWQ量化技术Skill" (skillsbot.cn awq-quantization usage page),
  "如何使用该技能 / 步骤 2": quant_config zero_point=True, q_group_size=128,
  w_bit=4; "主要功能和特点": 70B model 140 GB -> 35 GB.
* [GPTQ-VS-AWQ] "大模型量化部署实战：GPTQ与AWQ算法" (yunthe.com), section
  "大模型量化的核心原理与位宽选择": a 4-bit integer plus a scale and a zero point
  for dequantization; per-group (128) quantization.
* [NXMR] the nxmr.cn article (no title; first heading "AWQ技术概述：重新定义大语言模型
  量化"), §5.1 "精度下降严重": tune clip_steps (200 suggested) against accuracy loss.
* [AWQ-WIKI] "什么是激活感知权重量化（AWQ）" (aiboss88.com), section "工作机制":
  the protection is an equivalent transformation whose scale comes from offline
  activation statistics; no backpropagation or reconstruction.

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository):

* codes are unsigned 0..15 with a zero point (asymmetric), dequant = (q - z) * scale;
  the symmetric variant (zero_point False) uses sc = max|w'| / 7 and z = 8; 8- and 3-bit
  codes take the same steps with 255 / 7 levels;
* min/max affine group quantizer, computed in fp32 with IEEE round-to-nearest-even;
  the codes are rounded against the stored fp16 scale;
* scale floored at 2^-14, clamped to 65504 (flagged);
* group size 128 by default, 64 as the smaller size the practice page names;
* statistic = plain mean of |x| over all calibration tokens;
* s = (max(mean|x|, 2^-14))^alpha, alpha_i = i / n_grid, i = 0..n_grid-1, s stored as fp16;
* packed word: channels 0, 2, 4, 6 in the low nibbles of its bytes, 1, 3, 5, 7 in the high;
  3-bit codes in two bit planes per 128-channel block (see :func:`pack`);
* error = sum of squares of X * D^T with D = W - Q(W diag(s)) diag(1/s), ties -> smallest i;
* weight clipping: per group, ratios r_i = (clip_steps - i) / clip_steps, i < n_shrink
  (default 200 and 100), shrink the group's min/max; score = the group's own output
  contribution error; first minimum;
* the equivalent transform divides the producer of X by s (activations or a norm weight
  along columns, a previous linear's weight along rows), fp16 correctly rounded;
* the fused MLP module ([AWQ-SKILL] "主要功能和特点", fused attention/MLP; [AWQ-WIKI]
  TinyChat kernel fusion) is Llama's gated MLP: h = SiLU(x W_gate^T) * (x W_up^T) with
  SiLU(v) = v / (1 + e^-v), gate and up stacked as one packed weight (gate rows first).

Every function spells out the steps in order; numpy supplies only elementwise IEEE
operations, reductions and (fp64) matrix products.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "GROUP", "QMAX", "N_GRID", "ACT_FLOOR", "SCALE_FLOOR", "SCALE_MAX",
    "FLAG_NONFINITE_INPUT", "FLAG_SCALE_CLAMPED",
    "activation_mean_abs", "candidate_scales", "quantize_groups", "pack", "unpack",
    "quantize_pack", "dequantize", "NIBBLE_CHANNEL", "search_errors", "search_scales", "linear_reference",
    "linear_within_tolerance", "fp16_midpoint_distance", "relative_gap", "packed_bytes",
    "silu", "SILU_DMAX", "gated_silu_reference", "gated_silu_within_tolerance",
    "apply_inverse_scale", "FLAG_OVERFLOW",
    "CLIP_STEPS", "clip_ratios", "clip_errors", "clip_search", "W_BITS",
]

GROUP = 128                       # [AWQ-PRACTICE] §2.3; [AWQ-SKILL] q_group_size
QMAX = 15                         # 4-bit unsigned codes 0..15 with a zero point
W_BITS = (3, 4, 8)                # code widths: 4 (the format measured), 8 ([AWQ-PRACTICE] §3.3, §5.2, §5.3) and 3 (§4.3)
N_GRID = 20                       # alpha grid: 20 points in [0, 1)
ACT_FLOOR = 2.0 ** -14            # floor of the activation statistic (smallest normal fp16)
SCALE_FLOOR = np.float32(2.0 ** -14)
SCALE_MAX = np.float32(65504.0)   # largest finite fp16
MAX_CALIB_TOKENS = 8192           # keeps the |x| column sums exact in fp64

FLAG_NONFINITE_INPUT = 1
FLAG_SCALE_CLAMPED = 2
FLAG_OVERFLOW = 8                 # a finite input whose folded fp16 value is infinite

_F32 = np.float32
_F64 = np.float64


# --------------------------------------------------------------------------- a1
def activation_mean_abs(X16: np.ndarray) -> tuple[np.ndarray, int]:
    """Per-input-channel mean absolute activation, a_k = (1/T) sum_t |X_tk|.

    [AWQ-PRACTICE] §2.1: accumulate the calibration activations per input channel and
    take the mean absolute value ("激活强度"); a plain mean over all tokens.

    Every fp16 value is an integer multiple of 2^-24 and below 2^16, so for
    T <= 8192 every partial sum is a multiple of 2^-24 below 2^29 and is exact in
    fp64: the summation order cannot matter, and the only rounding is the final
    division by T (fp64, round-to-nearest-even).
    Returns (a fp64 [K], flags).
    """
    X16 = np.asarray(X16)
    assert X16.dtype == np.float16 and X16.ndim == 2
    T = X16.shape[0]
    assert 1 <= T <= MAX_CALIB_TOKENS
    Xd = X16.astype(_F64)
    flags = 0 if np.all(np.isfinite(Xd)) else FLAG_NONFINITE_INPUT
    col_sum = np.abs(Xd).sum(axis=0)
    a = col_sum / _F64(T)
    return a, flags


# --------------------------------------------------------------------------- a2
def candidate_scales(a: np.ndarray, n_grid: int = N_GRID) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Candidate per-channel scales for each grid point.

    [AWQ-PRACTICE] §1.3/§2.2 and [AWQ-WIKI] "工作机制": the scale comes from the
    offline activation statistic and is picked by a grid search over a candidate
    interval, one coefficient per layer (§5.1). Reading: s_ik = a_k^alpha_i with
    alpha_i = i / n_grid, a floored at 2^-14; pow in fp64, then one
    round-to-nearest-even conversion to fp16. alpha_0 = 0 gives s = 1 (plain RTN).
    Returns (alpha fp64 [n_grid], s fp16 [n_grid][K], s_exact fp64 [n_grid][K]).
    """
    a = np.maximum(np.asarray(a, dtype=_F64), _F64(ACT_FLOOR))
    alpha = np.arange(n_grid, dtype=_F64) / _F64(n_grid)
    s64 = np.empty((n_grid, a.shape[0]), dtype=_F64)
    for i in range(n_grid):
        s64[i] = np.power(a, alpha[i])
    s16 = s64.astype(np.float16)          # numpy converts fp64 -> fp16 in one RNE step
    return alpha, s16, s64


# --------------------------------------------------------------------------- a3
def quantize_groups(W16: np.ndarray, s16: np.ndarray | None = None, clip_ratio: np.ndarray | None = None,
                    zero_point: bool = True, group: int = GROUP, w_bit: int = 4) -> dict:
    """Group-wise asymmetric 4-bit quantization of W * diag(s).

    [AWQ-PRACTICE] §2.3 (128 consecutive input channels share one step) and §2.1
    (W is out x in, groups run along the input dimension); [GPTQ-VS-AWQ] (a 4-bit
    integer with a scale and a zero point, dequant = (q - z) * scale);
    [AWQ-SKILL] step 2 (w_bit 4, q_group_size 128, zero_point True).

    Steps per row n and group j (k in [g j, g j + g), g = group: 128, or 64 or 32 as
    [AWQ-PRACTICE] §2.3 also names), all in fp32, RNE:
      1. w' = f32(w) * f32(s)                  (exact: 11 + 11 significant bits)
      2. mx, mn = max / min of the g values w'
      3. sc = (mx - mn) / 15
      4. sc = max(sc, 2^-14); if sc > 65504 then sc = 65504 (flag SCALE_CLAMPED)
      5. sc_h = fp16(sc)                        (the stored scale)
      6. z = clamp(rint(-mn / f32(sc_h)), 0, 15)
      7. q = clamp(rint(w' / f32(sc_h)) + z, 0, 15)
    With ``clip_ratio`` (fp32 [N][G], the weight-clipping search), step 2 is followed by
    mx = f32(r mx), mn = f32(r mn): the group's range shrinks toward 0 by r and the
    weights beyond it take the end codes through the clamp of step 7.
    Symmetric (zero_point=False; [AWQ-PRACTICE] §3.3 advises zero_point False,
    [GPTQ-VS-AWQ] gives the signed range -8..7): steps 3 and 6 become
      3'. sc = max(|mx|, |mn|) / 7             6'. z = 8
    so q - 8 = clamp(rint(w' / sc_h), -8, 7) is the signed code, stored offset by 8 in the
    same format (every zero nibble 8).
    8-bit codes (w_bit = 8; [AWQ-PRACTICE] §3.3 offers it as the near-lossless setting, §5.2 / §5.3 raise w_bit when accuracy drops): the same
    steps with 15 -> 255 (codes 0..255) and, symmetric, 7 -> 127 and z = 128. 3-bit codes
    (w_bit = 3, the extreme low width [AWQ-PRACTICE] §4.3 names): 15 -> 7 (codes 0..7) and,
    symmetric, 7 -> 3 and z = 4 (signed range -4..3).
    Returns dict(q uint8 [N][K], z uint8 [N][G], scale fp16 [N][G], flags int).
    """
    W16 = np.asarray(W16)
    assert W16.dtype == np.float16 and W16.ndim == 2
    N, K = W16.shape
    assert group in (GROUP, 64, 32) and K % group == 0 and w_bit in W_BITS
    qmax = _F32(2 ** w_bit - 1)
    half = _F32(2 ** (w_bit - 1))
    G = K // group
    w = W16.astype(_F32)
    if s16 is not None:
        s16 = np.asarray(s16)
        assert s16.dtype == np.float16 and s16.shape == (K,)
        w = w * s16.astype(_F32)[None, :]
    flags = 0
    if not np.all(np.isfinite(w)):
        flags |= FLAG_NONFINITE_INPUT
    wg = w.reshape(N, G, group)
    mx = wg.max(axis=2)
    mn = wg.min(axis=2)
    if clip_ratio is not None:
        r = np.asarray(clip_ratio, dtype=_F32)
        assert r.shape == (N, G)
        mx = (r * mx).astype(_F32)
        mn = (r * mn).astype(_F32)
    if zero_point:
        sc = (mx - mn) / qmax
    else:
        sc = np.maximum(np.abs(mx), np.abs(mn)) / (half - _F32(1))
    sc = np.maximum(sc, SCALE_FLOOR)
    if np.any(sc > SCALE_MAX):
        flags |= FLAG_SCALE_CLAMPED
    sc = np.minimum(sc, SCALE_MAX)
    sc_h = sc.astype(np.float16)
    sc_f = sc_h.astype(_F32)
    with np.errstate(invalid="ignore"):
        if zero_point:
            z = np.clip(np.rint(-mn / sc_f), _F32(0), qmax)
        else:
            z = np.full(sc_f.shape, half)
        q = np.clip(np.rint(wg / sc_f[:, :, None]) + z[:, :, None], _F32(0), qmax)
    q = np.nan_to_num(q, nan=0.0).astype(np.uint8).reshape(N, K)
    z = np.nan_to_num(z, nan=0.0).astype(np.uint8)
    return {"q": q, "z": z, "scale": sc_h, "flags": flags}


# --------------------------------------------------------------------------- a4
# Channel held by nibble j (bits 4j..4j+3) of a packed word, relative to the word's first
# channel: the low halves of the word's four bytes hold channels 0, 2, 4, 6 and the high
# halves 1, 3, 5, 7, so masking bits {4p..4p+3, 16+4p..19+4p} of the word (p = 0..3)
# yields the adjacent channel pair (2p, 2p+1).
NIBBLE_CHANNEL = (0, 2, 4, 6, 1, 3, 5, 7)


def pack(q: np.ndarray, z: np.ndarray, scale: np.ndarray, w_bit: int = 4) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Packing of codes and zero points.

    The pages give no layout ([AWQ-WIKI] only names "platform-aware weight packing").
    Reading, 4-bit: qweight uint32 [N][K/8]; word w covers input channels 8w..8w+7 and
    nibble j (bits 4j..4j+3) holds the code of channel 8w + NIBBLE_CHANNEL[j]; zeros uint8
    [N][ceil(G/2)] where the low nibble holds the even group and the high nibble the
    odd group; scales fp16 [N][G].
    8-bit: qweight uint32 [N][K/4]; byte j of word w holds the code of channel 4w + j;
    zeros uint8 [N][G], one byte per group; scales fp16 [N][G].
    3-bit: qweight uint32 [N][3K/32], 12 words per 128-channel block b (words 12b ..
    12b + 11), split into bit planes: low-plane word i (i < 8) holds bits 0-1 of the codes
    of channels 16i + 2f (bits 2f, 2f + 1 of the word) and 16i + 2f + 1 (bits 16 + 2f,
    17 + 2f), f = 0..7; high-plane word 8 + j (j < 4) holds bit 2 of the codes of channels
    32j + 2p (bit p) and 32j + 2p + 1 (bit 16 + p), p = 0..15 (channels relative to the
    block). Zeros and scales as for 4-bit.
    """
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    G = np.asarray(z).shape[1]                  # groups per row (128, 64 or 32 channels each)
    if w_bit == 8:
        qweight = np.zeros((N, K // 4), dtype=np.uint32)
        for j in range(4):
            qweight |= q[:, j::4].astype(np.uint32) << np.uint32(8 * j)
        return qweight, np.asarray(scale, dtype=np.float16).copy(), np.asarray(z, dtype=np.uint8).copy()
    if w_bit == 3:
        assert K % 128 == 0
        qweight = np.zeros((N, 3 * K // 32), dtype=np.uint32)
        for k in range(K):
            b, c = divmod(k, 128)                 # block, channel within the block
            code = q[:, k].astype(np.uint32)
            lo_word = 12 * b + c // 16
            lo_shift = 2 * ((c % 16) // 2) + 16 * (c % 2)
            qweight[:, lo_word] |= (code & np.uint32(3)) << np.uint32(lo_shift)
            hi_word = 12 * b + 8 + c // 32
            hi_shift = (c % 32) // 2 + 16 * (c % 2)
            qweight[:, hi_word] |= (code >> np.uint32(2)) << np.uint32(hi_shift)
    else:
        assert w_bit == 4
        qweight = np.zeros((N, K // 8), dtype=np.uint32)
        for j in range(8):
            qweight |= q[:, NIBBLE_CHANNEL[j]::8].astype(np.uint32) << np.uint32(4 * j)
    zeros = np.zeros((N, (G + 1) // 2), dtype=np.uint8)
    zeros |= z[:, 0::2].astype(np.uint8)
    zeros[:, : G // 2] |= (z[:, 1::2].astype(np.uint8) << np.uint8(4))
    return qweight, np.asarray(scale, dtype=np.float16).copy(), zeros


def unpack(qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int):
    """Inverse of :func:`pack` (the code width follows from qweight's shape): returns
    (q uint8 [N][K], z uint8 [N][G], scale fp16 [N][G])."""
    N = qweight.shape[0]
    G = np.asarray(scales).shape[1]             # groups per row (128, 64 or 32 channels each)
    q = np.empty((N, K), dtype=np.uint8)
    if qweight.shape[1] == K // 4:              # 8-bit
        for j in range(4):
            q[:, j::4] = ((qweight >> np.uint32(8 * j)) & np.uint32(0xFF)).astype(np.uint8)
        return q, np.asarray(zeros, dtype=np.uint8)[:, :G].copy(), np.asarray(scales, dtype=np.float16)
    if qweight.shape[1] == 3 * K // 32:         # 3-bit bit planes
        for k in range(K):
            b, c = divmod(k, 128)
            lo = (qweight[:, 12 * b + c // 16] >> np.uint32(2 * ((c % 16) // 2) + 16 * (c % 2))) & np.uint32(3)
            hi = (qweight[:, 12 * b + 8 + c // 32] >> np.uint32((c % 32) // 2 + 16 * (c % 2))) & np.uint32(1)
            q[:, k] = (lo | (hi << np.uint32(2))).astype(np.uint8)
    else:
        assert qweight.shape[1] == K // 8
        for j in range(8):
            q[:, NIBBLE_CHANNEL[j]::8] = ((qweight >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)
    z = np.empty((N, G), dtype=np.uint8)
    z[:, 0::2] = zeros[:, : (G + 1) // 2] & np.uint8(0xF)
    z[:, 1::2] = zeros[:, : G // 2] >> np.uint8(4)
    return q, z, np.asarray(scales, dtype=np.float16)


def quantize_pack(W16: np.ndarray, s16: np.ndarray | None = None, clip_ratio: np.ndarray | None = None,
                  zero_point: bool = True, group: int = GROUP, w_bit: int = 4):
    """a3 + a4: returns (qweight, scales, zeros, flags)."""
    r = quantize_groups(W16, s16, clip_ratio, zero_point, group, w_bit)
    qweight, scales, zeros = pack(r["q"], r["z"], r["scale"], w_bit)
    return qweight, scales, zeros, r["flags"]


def dequantize(q: np.ndarray, z: np.ndarray, scale: np.ndarray, s16: np.ndarray | None = None) -> np.ndarray:
    """(q - z) * scale in fp64, divided by s when given: the weight the quantized layer stands for.

    [GPTQ-VS-AWQ]: dequant = (q - z) * scale; [AWQ-PRACTICE] §2.2: the 1/s is undone.
    """
    N, K = q.shape
    group = K // z.shape[1]
    zz = np.repeat(z.astype(_F64), group, axis=1)
    ss = np.repeat(scale.astype(_F64), group, axis=1)
    w = (q.astype(_F64) - zz) * ss
    if s16 is not None:
        w = w / s16.astype(_F64)[None, :]
    return w


# --------------------------------------------------------------------------- a5/a6
def search_errors(X16: np.ndarray, W16: np.ndarray, n_grid: int = N_GRID, grid_points=None,
                  zero_point: bool = True, group: int = GROUP, w_bit: int = 4) -> dict:
    """Output error of every candidate scale.

    [AWQ-PRACTICE] §2.2 and §3.3 step 4: grid search over a candidate interval so
    that the layer output on the calibration set before and after quantization
    agrees as closely as possible; [AWQ-WIKI] "工作机制": applied as the equivalent
    transform W diag(s), X diag(1/s).

      err_i = sum_t sum_n ( sum_k X_tk * D_nk )^2,
      D     = W - Q(W diag(s_i)) diag(1/s_i)            (fp64)

    ``grid_points`` restricts the evaluation to some indices (for bounded timing);
    the other entries of ``err`` are NaN.
    Returns dict(alpha, a, s16, s64, err fp64 [n_grid], flags).
    """
    a, flags = activation_mean_abs(X16)
    alpha, s16, s64 = candidate_scales(a, n_grid)
    Xd = X16.astype(_F64)
    Wd = W16.astype(_F64)
    err = np.full(n_grid, np.nan, dtype=_F64)
    points = range(n_grid) if grid_points is None else grid_points
    for i in points:
        r = quantize_groups(W16, s16[i], zero_point=zero_point, group=group, w_bit=w_bit)
        flags |= r["flags"]
        What = dequantize(r["q"], r["z"], r["scale"], s16[i])
        D = Wd - What
        E = Xd @ D.T
        err[i] = np.sum(E * E)
    return {"alpha": alpha, "a": a, "s16": s16, "s64": s64, "err": err, "flags": flags}


def search_scales(X16: np.ndarray, W16: np.ndarray, n_grid: int = N_GRID, zero_point: bool = True,
                  group: int = GROUP, w_bit: int = 4) -> dict:
    """a1..a6: the chosen grid index (first minimum), its scale and its packed weights.

    [AWQ-PRACTICE] §3.3 steps 4-5: pick the s with the smallest error, then
    quantize with it and keep the scale. Ties go to the smallest index (closest to
    plain RTN).
    """
    r = search_errors(X16, W16, n_grid, zero_point=zero_point, group=group, w_bit=w_bit)
    err = r["err"]
    best = 0
    for i in range(1, n_grid):
        if err[i] < err[best]:
            best = i
    s_best = r["s16"][best].copy()
    qweight, scales, zeros, f = quantize_pack(W16, s_best, zero_point=zero_point, group=group, w_bit=w_bit)
    r.update(best_idx=best, s_best=s_best, qweight=qweight, scales=scales, zeros=zeros,
             gap=relative_gap(err), flags=r["flags"] | f)
    return r


# --------------------------------------------------------------------------- weight clipping
CLIP_STEPS = 200  # [NXMR] §5.1: the suggested clip_steps


def clip_ratios(clip_steps: int = CLIP_STEPS, n_shrink: int = CLIP_STEPS // 2) -> np.ndarray:
    """Shrink ratios of the clipping grid: r_i = f32((clip_steps - i) / clip_steps),
    i = 0 .. n_shrink - 1 (r_0 = 1 is plain min/max quantization)."""
    assert 1 <= n_shrink <= clip_steps
    return np.array([(clip_steps - i) / clip_steps for i in range(n_shrink)], dtype=_F64).astype(_F32)


def clip_errors(X16: np.ndarray, W16: np.ndarray, s16: np.ndarray | None = None,
                clip_steps: int = CLIP_STEPS, n_shrink: int = CLIP_STEPS // 2,
                zero_point: bool = True, group: int = GROUP, w_bit: int = 4) -> np.ndarray:
    """Per-group output error of every shrink ratio, fp64 [n_shrink][N][G].

    Weight-clipping search ([NXMR] §5.1 "精度下降严重": tune clip_steps, 200 suggested,
    against accuracy loss). Reading: after the scale search, every group
    (row n, group g) of W diag(s) tries the ratios r_i of clip_ratios(), quantized with its
    range shrunk by r_i (quantize_groups' clip_ratio); the score is that group's own
    contribution to the calibration outputs,
        err[i, n, g] = sum_t ( sum_{k in g} X_tk D_nk )^2,  D = W - Q_r(W diag(s)) diag(1/s).
    """
    N, K = W16.shape
    G = K // group
    Xd = X16.astype(_F64)
    Wd = W16.astype(_F64)
    ratios = clip_ratios(clip_steps, n_shrink)
    err = np.empty((n_shrink, N, G), dtype=_F64)
    for i, r in enumerate(ratios):
        qz = quantize_groups(W16, s16, np.full((N, G), r, dtype=_F32), zero_point, group, w_bit)
        D = Wd - dequantize(qz["q"], qz["z"], qz["scale"], s16)
        for g in range(G):
            E = Xd[:, g * group:(g + 1) * group] @ D[:, g * group:(g + 1) * group].T
            err[i, :, g] = np.sum(E * E, axis=0)
    return err


def clip_search(X16: np.ndarray, W16: np.ndarray, s16: np.ndarray | None = None,
                clip_steps: int = CLIP_STEPS, n_shrink: int = CLIP_STEPS // 2,
                zero_point: bool = True, group: int = GROUP, w_bit: int = 4) -> dict:
    """Per group, the first ratio index with the smallest error, and the weight packed
    with those ratios. Returns dict(idx uint8 [N][G], ratio fp32 [N][G], err fp64
    [n_shrink][N][G], qweight, scales, zeros, flags)."""
    err = clip_errors(X16, W16, s16, clip_steps, n_shrink, zero_point, group, w_bit)
    idx = np.zeros(err.shape[1:], dtype=np.int64)
    best = err[0].copy()
    for i in range(1, n_shrink):
        better = err[i] < best
        idx[better] = i
        best[better] = err[i][better]
    ratio = clip_ratios(clip_steps, n_shrink)[idx]
    qweight, scales, zeros, flags = quantize_pack(W16, s16, ratio, zero_point, group, w_bit)
    return {"idx": idx.astype(np.uint8), "ratio": ratio, "err": err, "qweight": qweight,
            "scales": scales, "zeros": zeros, "flags": flags}


# --------------------------------------------------------------------------- a7/a8
def linear_reference(X16: np.ndarray, qweight: np.ndarray, scales: np.ndarray, zeros: np.ndarray, K: int):
    """W4A16 linear, y = X deq(W)^T, in fp64, with its error bound.

    [AWQ-PRACTICE] §3.4 / [AWQ-WIKI]: weight-only quantization, activations stay in
    16-bit. y_mn = sum_k x_mk (q_nk - z) sc, and bound_mn = sum_k |x_mk| |(q_nk - z) sc|.
    Returns (y fp64 [M][N], bound fp64 [M][N]).
    """
    q, z, sc = unpack(qweight, scales, zeros, K)
    Wdeq = dequantize(q, z, sc)
    Xd = np.asarray(X16).astype(_F64)
    return Xd @ Wdeq.T, np.abs(Xd) @ np.abs(Wdeq).T


def linear_within_tolerance(y, y_ref, bound, rel: float = 2e-3) -> np.ndarray:
    """Per-element check |y - y_ref| <= rel * bound (returns a boolean mask)."""
    y = np.asarray(y, dtype=_F64)
    return np.abs(y - y_ref) <= rel * bound


# --------------------------------------------------------------------------- equivalent transform
def apply_inverse_scale(A16: np.ndarray, s16: np.ndarray, axis: int) -> tuple[np.ndarray, int]:
    """Fold 1/s into the producer of a linear's input: fp16(A / s), correctly rounded.

    [AWQ-PRACTICE] §2.2: the salient input channels of W are multiplied by s before
    quantization and the other side is divided by s; [AWQ-WIKI] "工作机制": an equivalent
    transformation, X W^T = (X diag(1/s)) (W diag(s))^T. The division goes where X is
    made: the activations themselves or a norm weight (axis 1: A[r][k] / s_k, len(s) =
    columns), or the rows of the previous linear's weight (axis 0: A[k][j] / s_k,
    len(s) = rows). Returns (fp16 array, flags); FLAG_OVERFLOW when a finite input
    becomes infinite, FLAG_NONFINITE_INPUT when A or s holds NaN or inf.
    """
    A = np.asarray(A16, dtype=np.float16)
    s = np.asarray(s16, dtype=np.float16).astype(_F64)
    sb = s[None, :] if axis == 1 else s[:, None]
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        q = A.astype(_F64) / sb      # exact operands; fp64 quotient, then one rounding to fp16
        out = q.astype(np.float16)
    flags = 0
    if not (np.isfinite(A).all() and np.isfinite(s).all()):
        flags |= FLAG_NONFINITE_INPUT
    if np.any(np.isfinite(A) & np.isfinite(sb) & ~np.isfinite(out)):
        flags |= FLAG_OVERFLOW
    return out, flags


# --------------------------------------------------------------------------- fused MLP
SILU_DMAX = 1.1  # bound on |SiLU'(v)| over all v (the maximum is about 1.0998, near v = 2.40)


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v / (1 + e^-v) in fp64 (large negative v: e^-v overflows to inf, SiLU -> -0)."""
    v = np.asarray(v, dtype=_F64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def gated_silu_reference(X16: np.ndarray, qweight: np.ndarray, scales: np.ndarray,
                         zeros: np.ndarray, K: int):
    """Fused MLP module of a packed gate|up weight: h = SiLU(g) * u, in fp64.

    [AWQ-SKILL] "主要功能和特点": fused attention/MLP modules cut decode latency;
    [AWQ-WIKI] TinyChat: kernel fusion. The packed weight holds the N/2 gate rows first,
    then the N/2 up rows; g = x W_gate^T and u = x W_up^T are both W4A16 linears
    (linear_reference). Returns (h, g, u, bound_g, bound_u), each [M][N/2].
    """
    y, bound = linear_reference(X16, qweight, scales, zeros, K)
    nh = y.shape[1] // 2
    g, u = y[:, :nh], y[:, nh:2 * nh]
    return silu(g) * u, g, u, bound[:, :nh], bound[:, nh:2 * nh]


def gated_silu_within_tolerance(h, g, u, bound_g, bound_u, rel: float = 2e-3) -> np.ndarray:
    """Per-element check of a fused gate|up result against the fp64 reference.

    With |g' - g| <= rel * bound_g and |u' - u| <= rel * bound_u (the linear tolerance),
    |SiLU(g') u' - SiLU(g) u| <= SILU_DMAX |g' - g| |u| + |SiLU(g)| |u' - u|
    + SILU_DMAX |g' - g| |u' - u|; one fp16 rounding of the result adds at most 2^-11 |h|
    (2^-10 allowed, which also covers the fp32 evaluation of SiLU).
    """
    h = np.asarray(h, dtype=_F64)
    h_ref = silu(g) * u
    tol = (rel * (SILU_DMAX * bound_g * np.abs(u) + np.abs(silu(g)) * bound_u)
           + SILU_DMAX * rel * rel * bound_g * bound_u + 2.0 ** -10 * np.abs(h_ref))
    return np.abs(h - h_ref) <= tol


# --------------------------------------------------------------------------- hazards
def fp16_midpoint_distance(v: np.ndarray) -> np.ndarray:
    """Relative distance of fp64 values from the nearest fp16 rounding midpoint.

    Where a pow result lies within a few fp64 ulps of such a midpoint, two
    faithful pow implementations may round to different fp16 values; parity of s is
    then not decidable from the pages, and a test must treat that case as unpinned.
    """
    v = np.abs(np.asarray(v, dtype=_F64))
    h = v.astype(np.float16)
    hf = h.astype(_F64)
    up = np.nextafter(h, np.float16(np.inf)).astype(_F64)
    dn = np.nextafter(h, np.float16(0)).astype(_F64)
    mid_up = (hf + up) / 2.0
    mid_dn = (hf + dn) / 2.0
    d = np.minimum(np.abs(v - mid_up), np.abs(v - mid_dn))
    return d / np.maximum(v, np.finfo(_F64).tiny)


def relative_gap(err: np.ndarray) -> float:
    """(second smallest - smallest) / smallest over the finite errors (inf when unique and 0)."""
    e = np.sort(np.asarray(err, dtype=_F64)[np.isfinite(err)])
    if e.size < 2:
        return float("inf")
    if e[0] == 0.0:
        return float("inf") if e[1] > 0.0 else 0.0
    return float((e[1] - e[0]) / e[0])


def packed_bytes(N: int, K: int, group: int = GROUP, w_bit: int = 4) -> int:
    """Bytes of the packed format for one [N][K] weight: codes + fp16 scales + zero points."""
    G = K // group
    if w_bit == 8:
        return N * K + N * G * 2 + N * G
    return N * K * w_bit // 8 + N * G * 2 + N * ((G + 1) // 2)
