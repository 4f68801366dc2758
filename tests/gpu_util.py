"""Helpers of the GPU tests: host <-> device copies and the parity bar."""

import sys

import numpy as np
import torch

# Attention outputs: fp16 result of fp32 arithmetic against the fp64 oracle.
MAX_ABS = 5e-3
MEAN_ABS = 5e-4
# Stricter bar of our own, per output row (one query row of one head): at long contexts
# outputs are small (RMS ~ 1/sqrt(L)), so the absolute bound alone would pass a kernel
# that drops whole partitions; rows of one batch differ in scale, so each row is held to
# its own RMS.
MAX_OVER_ROW_RMS = 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def check_attention(got_f16, ref_f64, label=""):
    got = np.asarray(got_f16).astype(np.float64)
    ref = np.asarray(ref_f64, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    err = np.abs(got - ref)
    D = ref.shape[-1]
    row_rms = np.sqrt(np.mean(ref.reshape(-1, D) ** 2, axis=1))
    row_err = err.reshape(-1, D).max(axis=1)
    live = row_rms > 0
    worst = float((row_err[live] / row_rms[live]).max()) if live.any() else 0.0
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 rms=float(np.sqrt(np.mean(ref * ref))), max_over_row_rms=worst)
    note(f"  {label}: {stats}")
    assert stats["max_abs"] <= MAX_ABS, (label, stats)
    assert stats["mean_abs"] <= MEAN_ABS, (label, stats)
    assert worst <= MAX_OVER_ROW_RMS, (label, stats)
    # rows whose reference is exactly zero (empty contexts) must come out zero
    assert np.all(err.reshape(-1, D)[~live] == 0), label
    return stats


# ---------------------------------------------------------------------------------------
# rounding of the fp16 output store
# ---------------------------------------------------------------------------------------

def tie_base(rng, shape):
    """fp16 values x with |x| in [0.5, 2) away from binade edges, and u, the spacing of
    fp16 at x. x + k u is an fp16 value for |k| <= 8, and x + u / 2 lies exactly halfway
    between the two fp16 values x and x + u."""
    e = rng.integers(-1, 1, shape)           # binade 2^e
    f = rng.integers(8, 1000, shape)         # mantissa field
    sign = np.where(rng.integers(0, 2, shape) == 1, -1.0, 1.0)
    x = sign * (1.0 + f / 1024.0) * np.exp2(e)
    u = np.exp2(e - 10.0)
    return x, u


def tie_extra(n):
    """Multiples of u added to token t of a context of n tokens (n = 2 or 32) so that the
    mean over the n tokens is x + u / 2: token 0 gets u (n = 2), tokens 0 and 16 get 8 u
    each (n = 32, so each 16-token block or partition holds one)."""
    k = np.zeros(n)
    if n == 2:
        k[0] = 1
    elif n == 32:
        k[0] = k[16] = 8
    else:
        raise ValueError(n)
    return k


def write_tie_values(pool, table_row, n, x, u):
    """Value rows of logical tokens 0..n-1 of one sequence: x + tie_extra(n)[t] u per
    element (x, u: [Hkv, D]). Every value is an exact fp16 number."""
    for t, k in enumerate(tie_extra(n)):
        v = x + k * u
        v16 = v.astype(np.float16)
        assert np.array_equal(v16.astype(np.float64), v)
        pool[table_row[t // 16], t % 16, 1] = v16


def tie_expectations(x, u):
    """For a mean of exactly x + u / 2: (round to nearest even, truncation toward zero,
    half away from zero) as fp16."""
    mean = x + u / 2
    rne = mean.astype(np.float16)  # NumPy's fp64 -> fp16 conversion rounds to nearest even
    toward0 = np.where(x > 0, x, x + u).astype(np.float16)
    away = np.where(x > 0, x + u, x).astype(np.float16)
    return rne, toward0, away
