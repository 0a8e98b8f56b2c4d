"""Shared helpers of the GPU parity tests (host side only)."""
import sys

import numpy as np
import torch

# Tolerance for float outputs, as stated for this path: relative L2 error
# <= 1e-3 and max abs error <= 1e-2 * max|y| against the oracle's fp64 result.
REL_L2 = 1e-3
MAX_ABS_FRAC = 1e-2


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(h: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(h, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_same_bits(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.ascontiguousarray(gpu)
    ref = np.ascontiguousarray(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if gpu.dtype.itemsize == 4:
        g, r = gpu.view(np.uint32), ref.view(np.uint32)
    else:
        g, r = gpu.view(np.uint8), ref.view(np.uint8)
    bad = np.nonzero(g != r)
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} mismatches, first at {idx}: gpu {gpu[idx]!r} "
                             f"oracle {ref[idx]!r}")


def float_errors(y_gpu: np.ndarray, y_ref: np.ndarray):
    d = y_gpu.astype(np.float64) - y_ref
    nref = np.linalg.norm(y_ref)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mx = np.abs(y_ref).max() if y_ref.size else 0.0
    return rel, np.abs(d).max() if d.size else 0.0, mx


def assert_close(y_gpu: np.ndarray, y_ref: np.ndarray, what: str):
    assert y_gpu.shape == y_ref.shape, (what, y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), what
    rel, mabs, mx = float_errors(y_gpu, y_ref)
    say(f"  {what}: rel_l2 {rel:.2e} max_abs {mabs:.2e} (max|y| {mx:.3e})")
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mabs <= MAX_ABS_FRAC * mx + 1e-30, f"{what}: max abs {mabs:.3e} > {MAX_ABS_FRAC} * {mx:.3e}"
