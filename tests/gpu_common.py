"""Shared helpers of the GPU parity tests (not collected by pytest).

The tolerance is the one fixed for this path: per element
    |y - y_ref| <= 1e-2 + 5e-3 * |y_ref|
with y_ref the binary64 oracle value. Max-abs and max-rel (over |y_ref| >= 1)
errors are reported in the assertion message.
"""
from __future__ import annotations

import numpy as np

ATOL = 1e-2
RTOL = 5e-3


def err_report(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(y - ref)
    big = np.abs(ref) >= 1
    rel = (d[big] / np.abs(ref[big])).max() if big.any() else 0.0
    bad = d > ATOL + RTOL * np.abs(ref)
    return d.max() if d.size else 0.0, rel, int(bad.sum())


def within(y, ref):
    return err_report(y, ref)[2] == 0


def assert_within(y, ref, what=""):
    mabs, mrel, nbad = err_report(y, ref)
    assert nbad == 0, "%s: %d elements out of tolerance (max abs %.3g, max rel %.3g)" % (
        what, nbad, mabs, mrel)
    return mabs, mrel


def dev_tensor(a, device="cuda"):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def host(t):
    import torch
    a = t.detach().cpu().numpy()
    if a.dtype == np.int32:
        a = a.view(np.uint32)
    return a


def bits(t):
    """binary16 tensor -> its uint16 bit patterns on the host."""
    return host(t).view(np.uint16)


def assert_within_scaled(y, ref, scale, what=""):
    """|y - ref| <= 1e-2 + 5e-3 * scale, element by element. For a value that is a
    sum of stored binary16 terms, `scale` is the sum of the terms' magnitudes."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(y - ref)
    bad = d > ATOL + RTOL * np.asarray(scale, dtype=np.float64)
    assert not bad.any(), "%s: %d elements out of tolerance (max abs %.3g)" % (
        what, int(bad.sum()), d.max())
