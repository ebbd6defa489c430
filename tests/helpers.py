"""Shared helpers for the GPU parity tests: conversions and the tolerance check."""

import sys

import numpy as np
import torch

# Tolerance for bf16 outputs with fp32 accumulation: elementwise
# |gpu - oracle| <= ATOL + RTOL * |oracle|.
ATOL = 1e-2
RTOL = 2e-2


def np64(t):
    """fp64 numpy copy of a (CPU or GPU) tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits16(t):
    """uint16 bit patterns of a bf16 tensor."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    """Elementwise tolerance check; returns (max_abs, rel_l2, worst_ratio)."""
    g = np64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    ratio = float((err / (atol + rtol * np.abs(r))).max()) if err.size else 0.0
    max_abs = float(err.max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} worst_ratio={ratio:.3f}")
    if ratio > 1.0:
        bad = err > (atol + rtol * np.abs(r))
        idx = np.argwhere(bad)
        worst = np.unravel_index(np.argmax(err / (atol + rtol * np.abs(r))), err.shape)
        say(f"    {int(bad.sum())} elements out of tolerance; worst at {tuple(int(i) for i in worst)}"
            f" gpu={g[worst]:.5f} ref={r[worst]:.5f}")
        for ax in range(bad.ndim - 1):
            vals, cnt = np.unique(idx[:, ax], return_counts=True)
            say(f"    axis {ax}: {len(vals)} distinct, first {vals[:12].tolist()} counts {cnt[:12].tolist()}")
    assert ratio <= 1.0, f"{what}: tolerance exceeded (worst ratio {ratio:.3f}, max abs {max_abs:.3e})"
    return max_abs, rel_l2, ratio
