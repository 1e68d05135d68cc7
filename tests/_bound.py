"""Per-element error bound of a paged-attention result against the fp64 oracle.

Paging must not change the attention result (wiblog.cn, "AI 推理系列（十六）：
PagedAttention", section "非连续 KV 为什么需要专门的 Attention Kernel"), so the
device output is compared with the oracle's exact value element by element.
Next to the fixed absolute tolerance, every element must also lie within the
bound below, which scales with the data: on long contexts |out| is small (a
weighted mean over many N(0,1) rows) and an absolute 2e-2 alone would accept
an all-zero output.

Derivation (the device arithmetic: fp32 logits from exact products, base-2
online softmax, weights rounded to the element type before the PV product,
the running sum taken over the same rounded weights, fp32 accumulation, one
final rounding to the output type).  Write pi_t = w_t / W for the exact
weights and let the device use w~_t = w_t (1 + e_t) + a_t, |e_t| <= rho,
|a_t| <= alpha, in both the numerator and the sum.  Because
sum_t w_t (v_t - out) = 0,

    out~ - out = sum_t w~_t (v_t - out) / W~
               = sum_t (w_t e_t + a_t)(v_t - out) / W~,

and with W >= 1 (the device's reference maximum never exceeds the true one,
so its largest weight is at least 1),

    |out~ - out| <= (rho * spread + n * alpha * devmax) / (1 - rho - n * alpha),

spread = sum_t pi_t |v_t - out|, devmax = max_t |v_t - out|, n keys.  Common
factors of a group of weights (a rescale by a new maximum, a wave or
partition merge) cancel between numerator and sum; only their exp2
approximation error enters rho.

    rho   = u_w + (D + 8) 2^-24 lam + 2^-16
            u_w: unit roundoff of the weight's type (bf16 2^-8, f16 2^-11,
            fp32 kernels 0); (D + 8) 2^-24 lam: fp32 error of a logit,
            lam = max_t |scale| sum_d |q_d k_t,d| (the products are exact
            in fp32 for 16-bit inputs; D roundings of the sum plus the
            scale multiplications), which perturbs a weight by the same
            relative amount; 2^-16: the exp2 approximations of a weight and
            of up to 2^7 rescales / merges above it (each <= 2^-23).
    alpha = the absolute rounding floor of a weight: half the smallest f16
            subnormal (2^-25) for f16 weights; 2^-126 for bf16 and fp32
            weights (an fp32 value that small may be flushed to zero before
            it is rounded), divided by the smallest INT8 scale for INT8
            caches (the rounded quantity there is weight * scale).
    + kappa (spread + 2 |out|), kappa = 2^-13: fp32 accumulation of the
            numerator and of the sum over chains of at most 2^11 additions
            (chunks per wave, waves, partitions), sum_t pi_t |v_t| <=
            spread + |out|, and the final division.
    + u_o (|out| + bound) + the output type's floor (as alpha): the final
            round to nearest even.

This module holds no attention arithmetic: it combines the oracle's own
spread / devmax / lam outputs.
"""
import numpy as np

UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# Absolute rounding floor of a value of each type: half the smallest f16
# subnormal; 2^-126 for bf16 and fp32 (computed in fp32 first, where a value
# that small may be flushed to zero).
FLOOR = {"f32": 2.0 ** -126, "f16": 2.0 ** -25, "bf16": 2.0 ** -126}
KAPPA = 2.0 ** -13


def attention_bound(want, dtype, D, kv_scale_min=None):
    """Per-element bound |device - oracle| for an oracle Attention `want`
    (out, spread, devmax, lam, keys).  dtype is the query / output type;
    kv_scale_min is the smallest INT8 scale for INT8 caches (None for
    16-bit and fp32 caches)."""
    out = np.abs(want.out)
    u_w = 0.0 if dtype == "f32" else UNIT_ROUNDOFF[dtype]
    alpha = FLOOR[dtype]
    if kv_scale_min is not None:
        alpha = alpha / kv_scale_min
    rho = u_w + (D + 8) * 2.0 ** -24 * want.lam[..., None] + 2.0 ** -16
    na = want.keys.reshape((-1,) + (1,) * (want.out.ndim - 1)) * alpha
    denom = 1.0 - rho - na
    if np.any(denom <= 0):
        raise ValueError("bound undefined: rho + n * alpha >= 1")
    tol = (rho * want.spread + na * want.devmax) / denom
    tol = tol + KAPPA * (want.spread + 2.0 * out)
    u_o = UNIT_ROUNDOFF[dtype]
    return tol + u_o * (out + tol) + FLOOR[dtype]


def bound_violations(got64, want, dtype, D, kv_scale_min=None):
    """(number of elements outside the bound, largest |err| / bound)."""
    tol = attention_bound(want, dtype, D, kv_scale_min)
    err = np.abs(got64 - want.out)
    bad = err > tol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    return int(np.count_nonzero(bad)), float(ratio.max()) if ratio.size else 0.0
