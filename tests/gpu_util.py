"""Helpers of the GPU tests: host <-> device copies and the parity bar."""

import sys

import numpy as np
import torch

# Attention outputs: fp16 result of fp32 arithmetic against the fp64 oracle.
MAX_ABS = 5e-3
MEAN_ABS = 5e-4
# Stricter bar of our own: at long contexts outputs are small (RMS ~ 1/sqrt(L)), so the
# absolute bound alone would pass a kernel that drops whole partitions.
MAX_OVER_RMS = 1e-2


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
    rms = float(np.sqrt(np.mean(ref * ref)))
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), rms=rms,
                 max_over_rms=float(err.max() / rms) if rms > 0 else 0.0)
    note(f"  {label}: {stats}")
    assert stats["max_abs"] <= MAX_ABS, (label, stats)
    assert stats["mean_abs"] <= MEAN_ABS, (label, stats)
    if rms > 0:
        assert stats["max_over_rms"] <= MAX_OVER_RMS, (label, stats)
    return stats
