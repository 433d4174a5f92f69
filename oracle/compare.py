"""Error metric for comparing a float32 result g against the oracle's y.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A plain elementwise relative error |g - y| / |y| is not usable for a dot
product: an output near zero has an unbounded relative condition number, so
even an exact-order float32 sum fails it on random data.  The guarded metric
divides instead by the larger of |y_i| and D_i, the first-order magnitude
through which rounding in the dot product reaches the output:

    err_i = |g_i - y_i| / max(|y_i|, D_i, 2^-126)

with a = acc_i, A = sum_j |w_ij x_j| (the oracle's absacc), s = sigmoid(a):

    none      D = A
    sigmoid   D = s (1 - s) A                    (1 - s evaluated as sigmoid(-a))
    silu      D = |s (1 + a (1 - s))| A          (|silu'(a)| A)
    silu_mul  D = |m_i| |silu'(a)| A
    mul       D = |m_i| A
    add       D = A + |r_i|

The floor 2^-126 (the smallest normal float32) applies only to outputs in the
subnormal range, where float32 carries absolute, not relative, precision.

Any rounding of the float32 dot product obeys |acc_f32 - acc| <= c u A for a
modest c, so a correct kernel gives err of order c * 2^-24 whatever the data;
an indexing or layout mistake gives err of order 1.  The tolerances that gate
parity are per weight format: 1e-5 (f32), 2e-3 (f16, bf16) and 1e-4 (8-bit
and 4-bit block formats, whose dequantised values are exact).
"""
import numpy as np

FLT32_MIN_NORMAL = 2.0 ** -126

# Health ratio: err / (depth u) with u = 2^-24 and depth the longest chain of
# float32 roundings a correct implementation puts between the exact products
# and an output (its per-lane sequential length plus log2 of the reduction
# width).  The textbook bound for a recursive sum, |fl(sum) - sum| <=
# gamma_n sum |terms| with gamma_n ~ n u, puts a correct kernel at a ratio of
# O(1) on any data; a dropped or doubled weight, a wrong row or a layout slip
# lands orders of magnitude above it.  HEALTH_C is the constant of that bound
# the gate allows (the per-format tolerances stay the gate of record).
HEALTH_C = 4.0
UNIT_ROUNDOFF_F32 = 2.0 ** -24


def health_bound(depth):
    """Largest guarded error a correct float32 evaluation of depth chained
    roundings may show: HEALTH_C * depth * 2^-24."""
    return HEALTH_C * float(depth) * UNIT_ROUNDOFF_F32


TOLERANCE = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "q8b32": 1e-4, "q4b32": 1e-4}

# The signed Hadamard transform in float32: each output is reached through the
# sign multiply (exact for signs +-1), log2(n) <= 10 add/subtract stages and
# one scaling, each rounding by at most u = 2^-24 relative to the running
# magnitude, so |g - y| <= (log2(n) + 2) u d (d = n^-1/2 sum |x s|), under
# 7.2e-7 for n = 1024.  The gate is err = |g - y| / max(|y|, d) <= 1e-6.
FWHT_TOLERANCE = 1e-6


def _sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def error_scale(act, acc, absacc, m=None, r=None):
    a = np.asarray(acc, dtype=np.float64).reshape(-1)
    A = np.asarray(absacc, dtype=np.float64).reshape(-1)
    if act == "none":
        return A.copy()
    # 1 - sigmoid(a) taken as sigmoid(-a): the subtraction would cancel for
    # large positive a (1 - s is then below the spacing of doubles near 1)
    s, sm = _sigmoid(a), _sigmoid(-a)
    dsilu = np.abs(s * (1.0 + a * sm))
    if act == "sigmoid":
        return s * sm * A
    if act == "silu":
        return dsilu * A
    if act == "silu_mul":
        return np.abs(np.asarray(m, dtype=np.float64).reshape(-1)) * dsilu * A
    if act == "mul":
        return np.abs(np.asarray(m, dtype=np.float64).reshape(-1)) * A
    if act == "add":
        return A + np.abs(np.asarray(r, dtype=np.float64).reshape(-1))
    raise ValueError(f"unknown act {act}")


def compare(g, y, acc, absacc, act, m=None, r=None):
    """Return a dict: 'max_err' (guarded, the gate), 'argmax', 'max_plain_rel'
    and 'normwise' (for information), 'n'."""
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    if g.shape != y.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {y.shape}")
    if g.size == 0:
        return {"max_err": 0.0, "argmax": -1, "max_plain_rel": 0.0, "normwise": 0.0, "n": 0}
    D = error_scale(act, acc, absacc, m, r)
    diff = np.abs(g - y)
    denom = np.maximum(np.maximum(np.abs(y), D), FLT32_MIN_NORMAL)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(diff == 0.0, 0.0, diff / denom)
        plain = np.where(diff == 0.0, 0.0, diff / np.abs(y))
    err = np.where(np.isnan(err), np.inf, err)
    i = int(np.argmax(err))
    ymax = float(np.max(np.abs(y)))
    return {
        "max_err": float(err[i]),
        "argmax": i,
        "max_plain_rel": float(np.max(plain)),
        "normwise": float(np.max(diff) / ymax) if ymax > 0 else float(np.max(diff)),
        "n": int(g.size),
    }


def glu_error_scale(act, g, absg, u, absu):
    """D for y = f(g) u: |f'(g) u| A_g + |f(g)| A_u (first-order propagation of
    the two row sums' rounding), f = silu or sigmoid."""
    g = np.asarray(g, dtype=np.float64).reshape(-1)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    s, sm = _sigmoid(g), _sigmoid(-g)
    if act == "silu":
        f, df = g * s, s * (1.0 + g * sm)
    elif act == "sigmoid":
        f, df = s, s * sm
    else:
        raise ValueError(act)
    return np.abs(df * u) * np.asarray(absg, dtype=np.float64).reshape(-1) + np.abs(f) * np.asarray(absu, dtype=np.float64).reshape(-1)


def compare_glu(gout, y, act, g, absg, u, absu):
    """The guarded metric for the gated pair (same form as compare())."""
    gout = np.asarray(gout, dtype=np.float64).reshape(-1)
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    D = glu_error_scale(act, g, absg, u, absu)
    diff = np.abs(gout - y)
    denom = np.maximum(np.maximum(np.abs(y), D), FLT32_MIN_NORMAL)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(diff == 0.0, 0.0, diff / denom)
    err = np.where(np.isnan(err), np.inf, err)
    i = int(np.argmax(err)) if err.size else -1
    return {"max_err": float(err[i]) if err.size else 0.0, "argmax": i, "n": int(gout.size)}
