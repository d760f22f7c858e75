"""Parity bars shared by the GPU tests (reading 16, with the output-rounding term below).

Per-token outputs stored in bf16 (y, dx): |got - ref| <= 2e-2 + ulp_bf16(ref) / 2 element-wise.
The flat 2e-2 is the bar stated for the bf16 path; the half unit in the last place is the
rounding of the output itself to bf16 (8 significant bits), which no kernel can avoid: at
|ref| in [1, 2) it is 2^-8 = 0.0039, at [4, 8) 2^-6 = 0.0156, at [8, 16) 2^-5 = 0.031. Reduced gradients (dW, db, dT), whose
magnitude grows with the token count, keep 2e-2 * max(1, |ref|_inf); the fp32 path keeps a
flat 1e-5."""
import numpy as np

TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_REDUCED = 2e-2


def half_ulp_bf16(ref):
    """Half a bf16 unit in the last place at |ref|: 2^(floor(log2 |ref|) - 8)."""
    a = np.maximum(np.abs(np.asarray(ref, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 8).astype(np.int64))


def token_excess(got, ref):
    """Largest |got - ref| - (2e-2 + ulp_bf16(ref) / 2), and the largest |got - ref|."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return -TOL_BF16, 0.0
    err = np.abs(got - ref)
    return float((err - (TOL_BF16 + half_ulp_bf16(ref))).max()), float(err.max())


def token_ok(got, ref):
    return token_excess(got, ref)[0] <= 0.0


def reduced_bound(ref):
    return TOL_REDUCED * max(1.0, float(np.abs(np.asarray(ref)).max()))


# Reduced gradients are sums over tokens (or windows and pairs) of products whose factors carry
# bf16 rounding: the per-token gradient (stored in bf16 after a few roundings upstream) and the
# activation. The standard forward error bound of such a sum is gamma * sum |terms|, with gamma a
# few bf16 unit roundoffs; GAMMA_REDUCED = 2^-6 allows four of 2^-8. When the terms cancel (for
# instance dW_k with N(0,1) query biases, where dk carries a large component along b_q that the
# token sum nearly cancels), that bound, not |ref|, sets what bf16 storage can resolve.
GAMMA_REDUCED = 2.0 ** -6


def reduced_excess(got, ref, absum=None):
    """Largest |got - ref| - (2e-2 max(1, |ref|_inf) + GAMMA_REDUCED * absum), element-wise (the
    second term only when the oracle's absolute-term sums are given), and the largest |got - ref|."""
    got, ref = np.asarray(got, dtype=np.float64).reshape(-1), np.asarray(ref, dtype=np.float64).reshape(-1)
    err = np.abs(got - ref)
    bound = reduced_bound(ref) + (0.0 if absum is None else GAMMA_REDUCED * np.asarray(absum).reshape(-1))
    return float((err - bound).max()), float(err.max())
