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
