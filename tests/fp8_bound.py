"""The error of the 8-bit prefill against the exact attention, predicted from
the formats alone (test infrastructure, fp64).

Each rounding of the 8-bit path is to nearest, so its error is zero-mean and
bounded by half the step of the format at that value:
  * E4M3 (3 mantissa bits): step 2^(floor(log2 |y|) - 3) for |y| >= 2^-6, 2^-9
    below (subnormals), on the weights y = 2^(x - G) (G = ceil of the 32-token
    group's largest score) and on the values c s 2^-F (F from the block's
    largest V scale over the group);
  * INT8 queries: step sigma = 2^(e - 7) with max |q| < 2^e, i.e. at most
    max |q| / 64;
  * INT8 keys: step tau = 2^(E - 4) with the token's largest block scale below
    2^E, i.e. at most that scale / 8.
A rounding error of step u has variance u^2 / 12 when the residue is spread
evenly; a value that can only fall on the grid or half-way between two grid
points (a bf16 query near its row maximum, a key on a coarse grid) has at
most u^2 / 8: that bound is used for the INT8 steps.

To first order in these errors, with p_t the exact weights (normalised), o the
exact output and x the scores in log2 units:
  * weight errors enter the numerator only (the denominator takes the
    unquantised weights):  sum_t p_t v_tj eps_t;
  * value errors:          sum_t p_t dv_tj;
  * score errors move numerator and denominator together:
    sum_t p_t (v_tj - o_j) ln2 dx_t, with dx_t = sm log2(e) (dq . k_t + q . dk_t);
    the query's errors dq are shared by all tokens (a sum over channels d of
    dq_d C_dj, C = K^T diag(p) (V - o)), the keys' are independent per token.
The variances add; `predicted_sd` returns the standard deviation of the error
of every output channel.  The errors are sums of many independent bounded
terms, so the measured error divided by it behaves like a standard normal
variable: RMS about 1 or below (the bounds are upper bounds) and no value
beyond ~6 in a few hundred thousand.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634


def _step_e4m3(y):
    """E4M3 step at |y| (0 where y == 0, which rounds exactly)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    out = np.zeros_like(a)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    out[nz] = np.where(a[nz] >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    return out


def _exp_bound(a):
    """Smallest integer e with a < 2^e (a > 0), elementwise; -14 below fp16's normals."""
    a = np.asarray(a, dtype=np.float64)
    e = np.where(a > 0, np.frexp(np.where(a > 0, a, 1.0))[1], -14)
    return np.maximum(e, -14)


def predicted_sd(q, K, V, ks, vs, sm):
    """Standard deviation of each output channel's error, [H, D], for query
    rows q [H, D] (exact values) over the seen tokens' exact keys K [n, D] and
    values V [n, D] (token 0 first, groups of 32 aligned to it), the tokens'
    fp16 K block scales ks [n, D/32] and V scales vs ([n, D/32], or [n] for
    one per token), and the softmax scale sm."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, D = K.shape
    ng = (n + 31) // 32
    # INT8 key step of each token: at most its largest block scale / 8 (tau = 2^(E - 4))
    tau = np.ldexp(1.0, _exp_bound(np.asarray(ks, np.float64).max(axis=1)) - 4)
    # E4M3 value steps: per 32-token group and 32-channel block, 2^F with F = E' - 5
    vs = np.asarray(vs, dtype=np.float64)
    grp = np.arange(n) // 32
    if vs.ndim == 1:
        vmax = np.zeros(ng)
        np.maximum.at(vmax, grp, vs)
        F = np.repeat((_exp_bound(vmax) - 5)[:, None], D, axis=1)             # [ng, D]
    else:
        vmax = np.zeros((ng, vs.shape[1]))
        np.maximum.at(vmax, grp, vs)
        F = np.repeat(_exp_bound(vmax) - 5, 32, axis=1)                         # [ng, D]
    f2 = np.ldexp(1.0, F[grp])                                                   # [n, D]
    var_v = (_step_e4m3(V / f2) * f2) ** 2 / 12.0                                # [n, D]
    out = np.zeros_like(q)
    for h in range(q.shape[0]):
        x = sm * LOG2E * (K @ q[h])
        M = x.max()
        p = np.exp2(x - M)
        p /= p.sum()
        o = p @ V
        # weights: y = 2^(x - G) in each group, relative E4M3 error
        xg = np.full(ng * 32, -np.inf)
        xg[:n] = x
        G = np.ceil(xg.reshape(ng, 32).max(axis=1))
        y = np.exp2(x - G[grp])
        rel_w = (_step_e4m3(y) / y) ** 2 / 12.0                                  # [n]
        var = (p ** 2 * rel_w) @ (V ** 2)
        var += (p ** 2) @ var_v
        # scores: keys (independent per token) ...
        amax = np.abs(q[h]).max()
        sigma = math.ldexp(1.0, int(np.frexp(amax)[1]) - 7) if amax > 0 else 0.0
        dev = V - o
        var += sm ** 2 * float(q[h] @ q[h]) * ((p ** 2 * tau ** 2 / 8.0) @ (dev ** 2))
        # ... and the query's (shared by every token)
        C = K.T @ (p[:, None] * dev)                                             # [D (d), D (j)]
        var += sm ** 2 * (sigma ** 2 / 8.0) * (C ** 2).sum(axis=0)
        out[h] = np.sqrt(var)
    return out


def normalised_errors(got, exact, sd, floor_rel=1e-5):
    """(got - exact) / sd with sd floored at floor_rel x RMS(exact) (the fp32
    arithmetic of the products and sums)."""
    exact = np.asarray(exact, np.float64)
    rms = math.sqrt(float(np.mean(exact ** 2)))
    return (np.asarray(got, np.float64) - exact) / np.sqrt(sd ** 2 + (floor_rel * rms) ** 2)
