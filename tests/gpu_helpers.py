"""Helpers shared by the GPU parity tests (comparison rules, device copies)."""
import numpy as np

from oracle import oracle as O

# Requests the oracle flags as near ties (or with an unreachable zero residual)
# are excused from bit-exact comparison of their token decisions.
EXCUSE = O.NEAR_MASK | O.RESIDUAL_ZERO
RTOL = 1e-5          # probabilities / survivals / Q, relative, fp32
ATOL = 1e-37         # below the smallest normal fp32


def dev(a, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def ok_rows(flags):
    return (np.asarray(flags).astype(np.uint32) & EXCUSE) == 0


def assert_rows_equal(gpu, ref, ok, name):
    gpu, ref = np.asarray(gpu), np.asarray(ref)
    bad = [r for r in range(len(ref)) if ok[r] and not np.array_equal(gpu[r], ref[r])]
    assert not bad, f"{name}: {len(bad)} requests differ, first {bad[:5]}: gpu={gpu[bad[0]]} ref={ref[bad[0]]}"


def assert_close(gpu, ref, name, rtol=RTOL, atol=ATOL, mask=None):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref) - (rtol * np.abs(ref) + atol)
    if mask is not None:
        err = np.where(mask, err, -1.0)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err.max() <= 0, \
        f"{name}: |gpu-ref| beyond {rtol} rel at {worst}: gpu={gpu[worst]!r} ref={ref[worst]!r}"


def excused_fraction(flags):
    return float(np.mean(~ok_rows(flags)))
