"""Bounds and validity checks for SubBlock routing outputs against the fp64 oracle.

Shared by the GPU parity tests and the smoke check; the derivations are in the
docstring of tests/test_gpu_subblock.py.  Every function takes host numpy
arrays (oracle outputs, and GPU outputs already copied to the host).
"""
import numpy as np
import torch

import oracle

U = 2.0 ** -24


# --------------------------------------------------------------------------- bounds and checks

def pool_bound(q_bits, ref):
    """Per-element bound on |gpu mean - exact mean| for token-major bf16 bits q_bits [B,N,H,Dh]."""
    mean_abs = oracle.subblock_pool(q_bits & np.uint16(0x7FFF))
    return 2.0 * (64.0 * U * mean_abs + U * np.abs(ref)) + 1e-38


def bf16_round(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()


def flip_room(mean, bound):
    """Largest change of bf16(mean') over |mean' - mean| <= bound."""
    r = bf16_round(mean)
    return np.maximum(np.abs(bf16_round(mean + bound) - r), np.abs(bf16_round(mean - bound) - r))


def score_bound(qp, kp, dq=None, dk=None):
    """Bound on |gpu score - oracle score| for oracle means qp [B,H,nq,Dh], kp [B,H,nk,Dh]."""
    qa, ka = np.abs(bf16_round(qp)), np.abs(bf16_round(kp))
    Dh = qp.shape[-1]
    e = Dh * U * np.matmul(qa, np.swapaxes(ka, -1, -2))
    if dq is not None:
        e = e + np.matmul(dq, np.swapaxes(ka, -1, -2)) + np.matmul(qa, np.swapaxes(dk, -1, -2)) \
            + np.matmul(dq, np.swapaxes(dk, -1, -2))
    return 2.0 * e + 1e-30


def check_kept_lists(kept, nb, keep):
    """Every row: keep distinct indices in [0, nb), ascending."""
    assert kept.shape[-1] == keep
    if keep == 0:
        return
    assert kept.min() >= 0 and kept.max() < nb
    if keep > 1:
        assert np.all(np.diff(kept, axis=-1) > 0), "kept lists not strictly ascending"


def kept_mask(kept, nb):
    mask = np.zeros(kept.shape[:-1] + (nb,), dtype=bool)
    np.put_along_axis(mask, kept.astype(np.int64), True, axis=-1)
    return mask


def check_valid_against_oracle(kept, s_ref, e):
    """Every kept block can outrank every dropped one within the bounds e."""
    nb = s_ref.shape[-1]
    keep = kept.shape[-1]
    if keep in (0, nb):
        return
    mask = kept_mask(kept, nb)
    lo_kept = np.where(mask, s_ref + e, np.inf).min(axis=-1)
    hi_dropped = np.where(mask, -np.inf, s_ref - e).max(axis=-1)
    bad = lo_kept < hi_dropped
    assert not bad.any(), f"{bad.sum()} rows keep a block that is outranked beyond the bounds"


def check_top_set_of_own_scores(kept, s_gpu):
    """Under the kernel's own scores, the kept set is a top-keep set with ties to the lower index.

    kept [B,H,nq,keep], s_gpu [B,H,nq,nb] (any float dtype); checked one head at a time.
    """
    nb = s_gpu.shape[-1]
    keep = kept.shape[-1]
    if keep in (0, nb):
        if keep == nb:
            assert np.array_equal(kept, np.broadcast_to(np.arange(nb), kept.shape))
        return
    idx = np.arange(nb)
    for b in range(kept.shape[0]):
        for h in range(kept.shape[1]):
            sk, kk = s_gpu[b, h], kept[b, h]
            mask = kept_mask(kk, nb)
            t = np.where(mask, sk, np.inf).min(axis=-1, keepdims=True)  # smallest kept score
            assert not np.any(~mask & (sk > t)), f"({b},{h}): a dropped block outscores a kept one"
            last_tied_kept = np.where(mask & (sk == t), idx, -1).max(axis=-1)
            first_tied_dropped = np.where(~mask & (sk == t), idx, nb).min(axis=-1)
            assert np.all(last_tied_kept < first_tied_dropped), f"({b},{h}): a tie went to a higher index"


def set_agreement(kept, kept_ref, nb):
    """Mean share of each row's kept blocks that the oracle keeps too."""
    keep = kept.shape[-1]
    if keep == 0:
        return 1.0
    both = kept_mask(kept, nb) & kept_mask(kept_ref, nb)
    return float(both.sum(axis=-1).mean() / keep)
