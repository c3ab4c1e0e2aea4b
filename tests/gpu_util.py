"""Helpers shared by the GPU parity tests (host/device transfers, tolerances)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O

# Output tolerances for attention results (max-abs; plus mean-abs for bf16).
TOL_F32_MAX = 1e-5
TOL_BF16_MAX = 1e-2
TOL_BF16_MEAN = 1e-3


def say(*a):
    """Progress line, flushed, so a GPU step names its case before it runs."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def to_dev(x: np.ndarray) -> torch.Tensor:
    """Host storage array -> device tensor (uint16 bf16 bits -> bfloat16)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if t.dtype == torch.uint16:
        t = t.view(torch.bfloat16)
    return t.to(dev())


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host numpy array in storage format."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy()
    return t.numpy()


def check_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    err = np.abs(got.astype(np.float64) - want)
    mx, mean = float(err.max()), float(err.mean())
    if dtype == "f32":
        assert mx <= TOL_F32_MAX, "%s: max-abs %.3g > %.1g" % (what, mx, TOL_F32_MAX)
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, \
            "%s: max-abs %.3g mean-abs %.3g" % (what, mx, mean)
    return mx, mean


def score_tol(want: np.ndarray) -> float:
    """fp32 scoring of a d-term dot product against fp64: 1e-5 relative to the
    row's largest magnitude (the fp32 sum of <= 128 exact products errs by a
    few units of 2^-24 of the partial sums)."""
    return 1e-5 * (1.0 + float(np.max(np.abs(want))))


def verdicts(s64_rows, got_rows, k):
    counts = {"exact": 0, "excused": 0, "failed": 0}
    fails = []
    for i, (s, g) in enumerate(zip(s64_rows, got_rows)):
        v = O.index_set_verdict(s, g, k)
        key = v.split(":")[0]
        counts[key] += 1
        if key == "failed":
            fails.append((i, v))
    return counts, fails
