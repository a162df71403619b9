"""Helpers shared by the GPU parity tests (host-side comparison only)."""
import numpy as np

TOL = {"f32": 1e-5, "bf16": 1e-2}


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_y(y_gpu, y_ref, out):
    """Element-wise |y - y_ref| <= tol |y_ref|; outputs of a zero accumulator are exactly 0."""
    import torch
    y = y_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape
    zero = y_ref == 0
    assert (y[zero] == 0).all(), "zero accumulator must give exactly 0"
    bad = np.abs(y - y_ref) > TOL[out] * np.abs(y_ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} outputs out of tolerance {TOL[out]}; first "
                             f"{[(tuple(i), y[tuple(i)], y_ref[tuple(i)]) for i in idx]}")
    del torch


def assert_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        diff = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(diff)} mismatches, first at {diff[:5].tolist()}: "
                             f"got {got[tuple(diff[0])]}, want {want[tuple(diff[0])]}")
