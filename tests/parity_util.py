"""Element-by-element comparison of HIP outputs with the fp64 oracle.

Bound (per element): |gpu - ref| <= ATOL + RTOL * |ref|, with ATOL = 1e-2 and
RTOL = 8e-3.  bf16 has unit roundoff 2^-8 = 3.9e-3, so a single
round-to-nearest-even of an fp32 result lands within RTOL with about a factor
two to spare for the fp32 arithmetic before it; ATOL covers outputs near zero
whose fp32 rounding is relative to larger intermediates.
"""
import numpy as np
import torch

ATOL = 1e-2
RTOL = 8e-3


def to_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float64 host array (exact widening)."""
    return t.detach().float().cpu().double().numpy()


def worst(gpu: np.ndarray, ref: np.ndarray):
    """(max excess over the bound, flat index, gpu value, ref value)."""
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if gpu.size == 0:
        return -np.inf, -1, 0.0, 0.0
    ex = np.abs(gpu - ref) - (ATOL + RTOL * np.abs(ref))
    ex = np.where(np.isnan(ex), np.inf, ex)
    i = int(np.argmax(ex))
    return float(ex[i]), i, float(gpu[i]), float(ref[i])


def worst_ratio(gpu, ref) -> float:
    """Largest |gpu - ref| / (ATOL + RTOL |ref|); <= 1 means every element is within the bound."""
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if gpu.size == 0:
        return 0.0
    r = np.abs(gpu - ref) / (ATOL + RTOL * np.abs(ref))
    return float(np.inf) if np.isnan(r).any() else float(r.max())


def assert_close(gpu, ref, what: str = ""):
    """Fail with the worst element if any element breaks the bound or is not finite.

    Returns the worst |gpu - ref| / bound over the elements (<= 1 when it passes).
    """
    g = to_f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs oracle {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    ex, i, gv, rv = worst(g, r)
    assert ex <= 0.0, (f"{what}: element {np.unravel_index(i, g.shape)} gpu={gv!r} oracle={rv!r} "
                       f"|err|={abs(gv - rv):.3e} > bound {ATOL + RTOL * abs(rv):.3e}")
    return worst_ratio(g, r)


def worst_ratio_threaded(gpu, ref, threads: int = 8) -> float:
    """worst_ratio over large arrays, computed on row slices in parallel threads (numpy releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    gpu = np.asarray(gpu).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    n = gpu.size
    if n == 0:
        return 0.0
    parts = max(1, min(threads, n // (1 << 16)))
    bounds = [n * i // parts for i in range(parts + 1)]
    with ThreadPoolExecutor(max_workers=parts) as pool:
        return max(pool.map(lambda i: worst_ratio(gpu[bounds[i]:bounds[i + 1]], ref[bounds[i]:bounds[i + 1]]),
                            range(parts)))
