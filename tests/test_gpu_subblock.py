"""GPU parity of the SubBlock routing front-end against the fp64 oracle.

Pooled means: fp32 sums of at most 64 bf16 values and one division, so each
mean is within 64 u mean|x| + u |mean| of the exact one (u = 2^-24); the test
allows twice that.

Scores: the kernel multiplies the bf16-rounded fp32 means with fp32
accumulation.  Against the oracle (bf16 rounding of the exact fp64 means, exact
products, fp64 sum) two errors remain: the fp32 accumulation, at most
Dh u sum_d |q~_d k~_d|, and a bf16 rounding that the pooling error can flip
where a mean lies within its own bound of a rounding boundary.  The test
computes both per score from the oracle's means and allows twice their sum.
Where the pooled inputs are given exactly (route-only cases), no flip is
possible.

Kept blocks: several selections are correct where scores fall within their
bounds of the keep-th largest.  Each selection must be keep distinct ascending
in-range indices; every kept block must be able to outrank every dropped one
within the bounds (so every block whose oracle score clears the boundary by
more than the bounds is decided exactly as the oracle decides it); and under
the kernel's own scores the selection must be a top-keep set with ties to the
lower index.  On inputs whose products and sums are exact in fp32 the scores
equal the oracle's and the kept lists must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_dit_amd as dit
from parity_util import assert_close
from subblock_checks import (check_kept_lists, check_top_set_of_own_scores, check_valid_against_oracle,
                             flip_room, pool_bound, score_bound, set_agreement)
from synthetic_inputs import WORKLOADS, bits, correlated_heads, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def to_host(t):
    return t.cpu().numpy()


# --------------------------------------------------------------------------- pooling

POOL_SHAPES = [
    # B, N, H, Dh
    (1, 200, 2, 64),
    (2, 321, 3, 16),    # ragged last block of 1 token; 6 vectors per token
    (1, 130, 2, 256),
    (1, 64, 1, 32),     # exactly one block
    (1, 1, 4, 128),     # one token
    (1, 100, 5, 128),   # 80 vectors per token: a partial second column chunk
    (2, 1000, 4, 32),
    (1, 4096 * 64, 1, 16),  # the largest sequence: 4096 blocks
]


@pytest.mark.parametrize("head_major", [False, True], ids=["token_major", "head_major"])
@pytest.mark.parametrize("shape", POOL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_pool_matches_oracle(shape, head_major):
    B, N, H, Dh = shape
    q = correlated_heads(shape, seed=11 + N, device=DEV)
    k = correlated_heads(shape, seed=12 + N, device=DEV)
    qin = q.permute(0, 2, 1, 3).contiguous() if head_major else q
    kin = k.permute(0, 2, 1, 3).contiguous() if head_major else k
    qp, kp = dit.dit_subblock_pool(qin, kin, head_major=head_major)
    torch.cuda.synchronize()
    for got, src in ((qp, q), (kp, k)):
        ref = oracle.subblock_pool(bits(src))
        err = np.abs(to_host(got).astype(np.float64) - ref)
        bound = pool_bound(bits(src), ref)
        assert np.all(err <= bound), f"worst err/bound {(err / bound).max():.3g}"


def test_pool_layouts_and_repeats_agree():
    shape = (2, 515, 4, 64)
    q = correlated_heads(shape, seed=21, device=DEV)
    k = correlated_heads(shape, seed=22, device=DEV)
    a = dit.dit_subblock_pool(q, k)
    b = dit.dit_subblock_pool(q, k)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])  # deterministic
    # q and k may be the same buffer
    c = dit.dit_subblock_pool(q, q)
    torch.cuda.synchronize()
    assert torch.equal(c[0], a[0]) and torch.equal(c[1], a[0])


# --------------------------------------------------------------------------- route on given pooled means

ROUTE_SHAPES = [
    # B, H, nb, Dh
    (1, 1, 1, 16),
    (1, 2, 5, 32),
    (2, 3, 64, 64),
    (1, 2, 65, 128),
    (1, 1, 130, 256),
    (1, 2, 700, 128),
    (1, 1, 2100, 64),   # more than 2048 blocks
    (1, 1, 4096, 16),   # the largest block count
    (1, 1, 4096, 256),  # the largest block count at the largest head (64 x 64 score tiles)
]


def fused_kept(qd, kd, keep=None, sparsity=None):
    """Kept lists from the fused route (no score matrix written)."""
    kept, scores = dit.dit_subblock_route(qd, kd, keep=keep, sparsity=sparsity, write_scores=False)
    assert scores is None
    return kept


def route_inputs(shape, seed):
    g = torch.Generator().manual_seed(seed)
    qp = torch.randn(shape, generator=g) * 0.25
    kp = torch.randn(shape, generator=g) * 0.25
    return qp, kp


@pytest.mark.parametrize("shape", ROUTE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_route_matches_oracle(shape):
    B, H, nb, Dh = shape
    qp, kp = route_inputs(shape, seed=31 + nb)
    s_ref = oracle.subblock_scores(qp.double().numpy(), kp.double().numpy())
    e = score_bound(qp.double().numpy(), kp.double().numpy())
    qd, kd = qp.to(DEV), kp.to(DEV)
    for keep in sorted({0, 1, max(1, nb // 4), nb - 1, nb} - {-1}):
        if keep > nb or keep < 0:
            continue
        kept, scores = dit.dit_subblock_route(qd, kd, keep=keep)
        torch.cuda.synchronize()
        s_gpu = to_host(scores)[..., :nb].astype(np.float64)
        err = np.abs(s_gpu - s_ref)
        assert np.all(err <= e), f"keep {keep}: worst score err/bound {(err / e).max():.3g}"
        kh = to_host(kept)
        check_kept_lists(kh, nb, keep)
        check_valid_against_oracle(kh, s_ref, e)
        check_top_set_of_own_scores(kh, s_gpu)
        # scores kept on chip: the same lists, bit for bit
        kf = fused_kept(qd, kd, keep=keep)
        torch.cuda.synchronize()
        assert torch.equal(kf, kept), f"keep {keep}: fused route differs from scores + top-k"


@pytest.mark.parametrize("nb", [7, 64, 200, 2100])
def test_route_exact_scores_and_ties_bit_exact(nb):
    # Means on a 1/8 grid: every product is a multiple of 1/64 and every sum of
    # Dh of them stays below 2^10, so fp32 holds all scores exactly and the
    # kernel's scores equal the oracle's.  Key blocks repeat a few rows, so
    # most scores tie and the tie rule decides.
    B, H, Dh = 1, 2, 32
    rng = np.random.default_rng(nb)
    qp = rng.integers(-16, 17, size=(B, H, nb, Dh)) / 8.0
    rows = rng.integers(-16, 17, size=(B, H, 5, Dh)) / 8.0
    kp = np.ascontiguousarray(rows[:, :, rng.integers(0, 5, size=nb)])
    s_ref = oracle.subblock_scores(qp, kp)
    qd = torch.from_numpy(qp).float().to(DEV)
    kd = torch.from_numpy(kp).float().to(DEV)
    for sparsity in (0.0, 0.5, 0.75, 0.8, 0.95):
        keep = oracle.subblock_keep(nb, sparsity)
        assert keep == dit.dit_subblock_keep(nb, sparsity)
        kept, scores = dit.dit_subblock_route(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(scores)[..., :nb].astype(np.float64), s_ref)
        assert np.array_equal(to_host(kept), oracle.subblock_topk(s_ref, keep)), sparsity
        kf = fused_kept(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(kf), oracle.subblock_topk(s_ref, keep)), f"fused, sparsity {sparsity}"


@pytest.mark.parametrize("nb", [300, 1953, 2100])
@pytest.mark.parametrize("first_rare", [False, True])
def test_route_crowded_first_digit_bit_exact(nb, first_rare):
    # Scores crowded into the magnitudes [0.5, 2) with both signs, i.e. one
    # first-digit bin and its mirror, on a 1/64 grid (exact in bf16 means and
    # fp32 sums).  With the first key in the crowded pair the top-k counts that
    # pair by ballots; with a rare first key (magnitude 8) it counts every key
    # by atomics.  Either way the lists must equal the oracle's.
    B, H, Dh = 1, 2, 16
    rng = np.random.default_rng(1000 + nb + first_rare)
    qp = np.zeros((B, H, nb, Dh))
    qp[..., 0] = rng.choice([-1.0, 1.0], size=(B, H, nb))
    qp[..., 1] = rng.choice([0.0, 0.125], size=(B, H, nb))
    kp = np.zeros((B, H, nb, Dh))
    crowd = rng.integers(4, 16, size=(B, H, nb)) / 8.0 * rng.choice([-1.0, 1.0], size=(B, H, nb))
    spread = rng.choice([0.0, 0.0625, 0.25, 4.0, -3.0], size=(B, H, nb))
    kp[..., 0] = np.where(rng.random((B, H, nb)) < 0.8, crowd, spread)
    kp[..., 1] = rng.integers(-2, 3, size=(B, H, nb)) / 8.0
    kp[..., 2:] = rng.integers(-8, 9, size=(B, H, nb, Dh - 2)) / 8.0  # multiplied by the zero q means
    if first_rare:
        kp[:, :, 0, 0] = 8.0
    else:
        kp[:, :, 0, 0] = 1.0
    s_ref = oracle.subblock_scores(qp, kp)
    qd = torch.from_numpy(qp).float().to(DEV)
    kd = torch.from_numpy(kp).float().to(DEV)
    for sparsity in (0.5, 0.75, 0.95):
        keep = oracle.subblock_keep(nb, sparsity)
        kept, scores = dit.dit_subblock_route(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(scores)[..., :nb].astype(np.float64), s_ref)
        assert np.array_equal(to_host(kept), oracle.subblock_topk(s_ref, keep)), sparsity
        kf = fused_kept(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(kf), oracle.subblock_topk(s_ref, keep)), f"fused, sparsity {sparsity}"


@pytest.mark.parametrize("nb", [5, 300, 1953, 2100])
@pytest.mark.parametrize("sign,centre", [(1.0, 16.0), (1.0, 16.5), (-1.0, 16.0), (-1.0, 16.5)])
def test_route_narrow_range_bit_exact(nb, sign, centre):
    # Every score of a row within half a unit of +-16 or +-16.5: one sign and
    # one or two binary magnitudes, so the keys agree in most of their top
    # bits and the selection's first digit must come from the bits below the
    # ones they share.  On a 1/64 grid, exact in bf16 means and fp32 sums; the
    # lists must equal the oracle's bit for bit.
    B, H, Dh = 1, 2, 16
    rng = np.random.default_rng(3000 + nb + int(4 * centre) + (sign < 0))
    qp = np.zeros((B, H, nb, Dh))
    qp[..., 0] = sign
    qp[..., 1] = rng.integers(-4, 5, size=(B, H, nb)) / 8.0
    kp = np.zeros((B, H, nb, Dh))
    kp[..., 0] = centre
    kp[..., 1] = rng.integers(-8, 9, size=(B, H, nb)) / 8.0
    kp[..., 2:] = rng.integers(-8, 9, size=(B, H, nb, Dh - 2)) / 8.0  # multiplied by the zero q means
    s_ref = oracle.subblock_scores(qp, kp)
    assert np.all(np.abs(np.abs(s_ref) - centre) <= 0.5)
    qd = torch.from_numpy(qp).float().to(DEV)
    kd = torch.from_numpy(kp).float().to(DEV)
    for sparsity in (0.0, 0.5, 0.75, 0.95):
        keep = oracle.subblock_keep(nb, sparsity)
        kept, scores = dit.dit_subblock_route(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(scores)[..., :nb].astype(np.float64), s_ref)
        assert np.array_equal(to_host(kept), oracle.subblock_topk(s_ref, keep)), sparsity
        kf = fused_kept(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(kf), oracle.subblock_topk(s_ref, keep)), f"fused, sparsity {sparsity}"


@pytest.mark.parametrize("nb", [5, 700, 1953, 2100])
@pytest.mark.parametrize("levels", [1, 2, 8, "one_apart"])
def test_route_few_distinct_scores_bit_exact(nb, levels):
    # Rows whose scores take one, two or eight values (or all one value but
    # for a single larger one): the selection ends on candidates that are all
    # equal, so the tie rule (lowest index first) decides.  Exact scores; the
    # lists must equal the oracle's bit for bit.
    B, H, Dh = 1, 2, 16
    rng = np.random.default_rng(4000 + nb + (9 if levels == "one_apart" else levels))
    qp = np.ones((B, H, nb, Dh))
    kp = np.zeros((B, H, nb, Dh))
    if levels == "one_apart":
        kp[..., 0] = 0.5
        kp[:, :, rng.integers(0, nb), 0] = 0.625
    else:
        kp[..., 0] = rng.integers(0, levels, size=(B, H, nb)) / 8.0
    s_ref = oracle.subblock_scores(qp, kp)
    qd = torch.from_numpy(qp).float().to(DEV)
    kd = torch.from_numpy(kp).float().to(DEV)
    for sparsity in (0.0, 0.5, 0.75, 0.95):
        keep = oracle.subblock_keep(nb, sparsity)
        kept, scores = dit.dit_subblock_route(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(scores)[..., :nb].astype(np.float64), s_ref)
        assert np.array_equal(to_host(kept), oracle.subblock_topk(s_ref, keep)), sparsity
        kf = fused_kept(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(kf), oracle.subblock_topk(s_ref, keep)), f"fused, sparsity {sparsity}"


@pytest.mark.parametrize("nb", [1953, 4096])
def test_route_shared_component_valid(nb):
    # Block means with a component shared by every block of a head (as when
    # a head's queries and keys share a mean direction): the scores crowd
    # into a narrow band of one sign.  Lists must be valid top-keep sets of
    # the oracle's scores, and both routes must agree bit for bit.
    B, H, Dh = 1, 2, 64
    g = torch.Generator().manual_seed(nb)
    base = torch.randn((B, H, 1, Dh), generator=g)
    qp = base + 0.125 * torch.randn((B, H, nb, Dh), generator=g)
    kp = base + 0.125 * torch.randn((B, H, nb, Dh), generator=g)
    s_ref = oracle.subblock_scores(qp.double().numpy(), kp.double().numpy())
    e = score_bound(qp.double().numpy(), kp.double().numpy())
    qd, kd = qp.to(DEV), kp.to(DEV)
    for sparsity in (0.75, 0.95):
        kept, scores = dit.dit_subblock_route(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        keep = kept.shape[-1]
        kh = to_host(kept)
        check_kept_lists(kh, nb, keep)
        check_valid_against_oracle(kh, s_ref, e)
        check_top_set_of_own_scores(kh, to_host(scores)[..., :nb].astype(np.float64))
        kf = fused_kept(qd, kd, sparsity=sparsity)
        torch.cuda.synchronize()
        assert torch.equal(kf, kept), f"sparsity {sparsity}: fused route differs from scores + top-k"


def test_route_special_values():
    # all-zero means: every score is +0 or -0, all tie, the lowest indices are kept
    B, H, nb, Dh = 1, 1, 9, 16
    z = torch.zeros((B, H, nb, Dh), device=DEV)
    zn = z.clone()
    zn[0, 0, ::2] = -0.0
    kept, scores = dit.dit_subblock_route(z, zn, keep=4)
    torch.cuda.synchronize()
    assert to_host(kept).tolist() == [[[list(range(4)) for _ in range(nb)]]]
    kf = fused_kept(z, zn, keep=4)
    torch.cuda.synchronize()
    assert to_host(kf).tolist() == [[[list(range(4)) for _ in range(nb)]]]
    # NaN in one key block: kept lists stay keep distinct ascending in-range indices
    kn = torch.randn((B, H, nb, Dh), device=DEV)
    kn[0, 0, 3, 5] = float("nan")
    qn = torch.randn((B, H, nb, Dh), device=DEV)
    kept, _ = dit.dit_subblock_route(qn, kn, keep=4)
    kf = fused_kept(qn, kn, keep=4)
    torch.cuda.synchronize()
    check_kept_lists(to_host(kept), nb, 4)
    check_kept_lists(to_host(kf), nb, 4)
    assert torch.equal(kf, kept)
    # neither output asked for: a no-op
    assert fused_kept(qn, kn, keep=0).shape[-1] == 0


# the workloads' routing shapes, and the largest block count with two rows per wave and with one
@pytest.mark.parametrize("shape", [(1, 32, 1953, 128), (2, 32, 1953, 128), (1, 32, 3851, 128), (1, 4, 2048, 128),
                                   (1, 2, 2049, 256), (3, 5, 513, 16)], ids=lambda s: "x".join(map(str, s)))
def test_route_fused_equals_scores_then_topk(shape):
    B, H, nb, Dh = shape
    qp, kp = route_inputs(shape, seed=81 + nb)
    qd, kd = qp.to(DEV), kp.to(DEV)
    for sparsity in (0.75, 0.8):
        kept, _ = dit.dit_subblock_route(qd, kd, sparsity=sparsity)
        kf = torch.full_like(kept, -3)
        dit.dit_subblock_route(qd, kd, sparsity=sparsity, kept=kf, write_scores=False)
        torch.cuda.synchronize()
        assert torch.equal(kf, kept), f"sparsity {sparsity}"
    check_kept_lists(to_host(kf), nb, dit.dit_subblock_keep(nb, 0.8))


# The top-k and the fused route pick their register slots per nb (S = 4, 8,
# 16, 32 or 64 slots of 64 blocks) and skip the nb test on the first half of
# the slots, which is whole for every nb a bucket serves; these are the
# bucket edges, where the last slot is either full or holds a single block.
@pytest.mark.parametrize("nb", [256, 257, 512, 513, 1024, 1025, 2048, 2049, 4096])
def test_route_slot_bucket_edges(nb):
    B, H, Dh = 1, 2, 32
    qp, kp = route_inputs((B, H, nb, Dh), seed=500 + nb)
    s_ref = oracle.subblock_scores(qp.double().numpy(), kp.double().numpy())
    e = score_bound(qp.double().numpy(), kp.double().numpy())
    qd, kd = qp.to(DEV), kp.to(DEV)
    for keep in sorted({1, nb // 4, nb - 1, nb}):
        kept, scores = dit.dit_subblock_route(qd, kd, keep=keep)
        kf = fused_kept(qd, kd, keep=keep)
        torch.cuda.synchronize()
        s_gpu = to_host(scores)[..., :nb].astype(np.float64)
        kh = to_host(kept)
        check_kept_lists(kh, nb, keep)
        check_valid_against_oracle(kh, s_ref, e)
        check_top_set_of_own_scores(kh, s_gpu)
        assert torch.equal(kf, kept), f"nb {nb}, keep {keep}: fused route differs from scores + top-k"


def test_route_deterministic_and_buffers_reused():
    shape = (1, 3, 300, 128)
    qp, kp = route_inputs(shape, seed=41)
    qd, kd = qp.to(DEV), kp.to(DEV)
    kept, scores = dit.dit_subblock_route(qd, kd, sparsity=0.75)
    kept2 = torch.full_like(kept, -7)
    scores2 = torch.full_like(scores, 3.0)
    dit.dit_subblock_route(qd, kd, sparsity=0.75, scores=scores2, kept=kept2)
    torch.cuda.synchronize()
    assert torch.equal(kept, kept2) and torch.equal(scores[..., :300], scores2[..., :300])
    # self-routing: q and k pooled from one buffer
    k_self, _ = dit.dit_subblock_route(qd, qd, keep=10)
    torch.cuda.synchronize()
    check_kept_lists(to_host(k_self), 300, 10)


# --------------------------------------------------------------------------- end to end: q', k' -> kept blocks

def end_to_end(B, N, H, Dh, sparsity, seed, head_major=False, sample_rows=None):
    shape = (B, N, H, Dh)
    q = correlated_heads(shape, seed=seed, device=DEV)
    k = correlated_heads(shape, seed=seed + 1, device=DEV)
    qin = q.permute(0, 2, 1, 3).contiguous() if head_major else q
    kin = k.permute(0, 2, 1, 3).contiguous() if head_major else k
    qp, kp = dit.dit_subblock_pool(qin, kin, head_major=head_major)
    kept, scores = dit.dit_subblock_route(qp, kp, sparsity=sparsity)
    torch.cuda.synchronize()
    nb = qp.shape[2]
    keep = dit.dit_subblock_keep(nb, sparsity)
    del qin, kin

    qb, kb = bits(q), bits(k)
    del q, k
    kp_ref = oracle.subblock_pool(kb)
    dk = flip_room(kp_ref, pool_bound(kb, kp_ref))
    err_k = np.abs(to_host(kp).astype(np.float64) - kp_ref)
    assert np.all(err_k <= pool_bound(kb, kp_ref)), "k pooling"
    rows = np.arange(nb) if sample_rows is None else np.unique(sample_rows)
    # Tokens of the sampled query blocks only, in block order: each sampled
    # block is a whole 64-token slice and only the sample's last block can be
    # shorter (it sorts last), so pooling the concatenation pools each block.
    qb_rows = np.concatenate([qb[:, 64 * i:64 * i + 64] for i in rows], axis=1)
    qp_ref = oracle.subblock_pool(qb_rows)
    q_bound = pool_bound(qb_rows, qp_ref)
    dq = flip_room(qp_ref, q_bound)
    qp_gpu = to_host(qp)[:, :, rows].astype(np.float64)
    assert np.all(np.abs(qp_gpu - qp_ref) <= q_bound), "q pooling"

    s_ref = oracle.subblock_scores(qp_ref, kp_ref)
    e = score_bound(qp_ref, kp_ref, dq, dk)
    s_all = to_host(scores)[..., :nb]
    s_gpu = s_all[:, :, rows].astype(np.float64)
    err = np.abs(s_gpu - s_ref)
    assert np.all(err <= e), f"worst score err/bound {(err / e).max():.3g}"
    kh = to_host(kept)
    check_kept_lists(kh, nb, keep)
    check_valid_against_oracle(kh[:, :, rows], s_ref, e)
    check_top_set_of_own_scores(kh, s_all)
    kf = fused_kept(qp, kp, sparsity=sparsity)
    torch.cuda.synchronize()
    assert torch.equal(kf, kept), "fused route differs from scores + top-k"
    return set_agreement(kh[:, :, rows], oracle.subblock_topk(s_ref, keep), nb)


@pytest.mark.parametrize("head_major", [False, True], ids=["token_major", "head_major"])
def test_end_to_end_small(head_major):
    agree = end_to_end(2, 64 * 37 + 29, 4, 64, 0.75, seed=51, head_major=head_major)
    assert agree > 0.95


@pytest.mark.parametrize("name", ["lowres", "full5s", "full10s", "batch2"])
def test_end_to_end_workload(name):
    wl = WORKLOADS[name]
    nb = -(-wl.N // 64)
    rows = np.random.default_rng(61).choice(nb, size=12, replace=False)
    rows = np.concatenate([rows, [0, nb - 1]])  # first and (short) last block
    print(f"[subblock] {name}: N={wl.N} nb={nb} H={wl.H} Dh={wl.Dh}", flush=True)
    agree = end_to_end(wl.B, wl.N, wl.H, wl.Dh, 0.75, seed=71, sample_rows=rows)
    print(f"[subblock] {name}: kept-set agreement with the oracle {agree:.4f}", flush=True)
    assert agree > 0.95


# --------------------------------------------------------------------------- QK RMSNorm + RoPE fused with pooling

QK_POOL_SHAPES = [
    # B, N, H, Dh, bands
    (1, 200, 2, 64, (16, 24, 24)),
    (2, 321, 3, 16, (4, 6, 6)),        # ragged last block of 1 token
    (1, 130, 2, 256, (32, 112, 112)),  # 128 rotary pairs: two per lane
    (1, 64, 1, 32, (8, 12, 12)),
    (1, 1, 4, 128, (16, 56, 56)),
    (1, 100, 5, 128, (16, 56, 56)),    # a partial second column chunk
]


def qk_pool_inputs(B, N, H, Dh, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((B, N, H, Dh), generator=g) * 1.5).to(torch.bfloat16).to(DEV)
    k = (torch.randn((B, N, H, Dh), generator=g) * 0.7).to(torch.bfloat16).to(DEV)
    wq = (1.0 + 0.02 * torch.randn(Dh, generator=g)).to(torch.bfloat16).to(DEV)
    wk = (1.0 + 0.02 * torch.randn(Dh, generator=g)).to(torch.bfloat16).to(DEV)
    grid = (max(1, N // 30), 5, 6)
    extra = N - grid[0] * 30 if N >= 30 else N
    if N < 30:
        grid = (0, 5, 6)
    pos = dit.dit_packed_positions(*grid, extra, device=DEV)
    return q, k, wq, wk, pos


@pytest.mark.parametrize("shape", QK_POOL_SHAPES, ids=lambda s: "x".join(map(str, s[:4])))
def test_qk_pool_matches_parts_and_oracle(shape):
    B, N, H, Dh, bands = shape
    q, k, wq, wk, pos = qk_pool_inputs(B, N, H, Dh, seed=N + Dh)
    qo, ko, qp, kp = dit.dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, pos, bands)
    qr, kr = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, pos, bands)
    qpr, kpr = dit.dit_subblock_pool(qr, kr)
    torch.cuda.synchronize()
    # the same outputs as the two separate kernels, bit for bit
    assert torch.equal(qo, qr) and torch.equal(ko, kr)
    assert torch.equal(qp, qpr) and torch.equal(kp, kpr)
    # Against the oracle: outputs within the bf16 bound.  The oracle's means are
    # of bf16(exact q'), the kernel's of its stored q' (each within
    # 1e-2 + 8e-3|q'| of exact q'), and bf16 rounding moves a value by at most
    # 2^-9 of it, so each mean is within 1e-2 + (8e-3 + 2^-9) * mean|q'|, plus
    # the fp32 sum's own error.
    o_q, o_k, o_qp, o_kp = oracle.qk_rmsnorm_rope3d_pool(bits(q), bits(k), bits(wq), bits(wk), to_host(pos), bands)
    assert_close(qo, o_q, "q'")
    assert_close(ko, o_k, "k'")
    for got, ref_out, ref in ((qp, o_q, o_qp), (kp, o_k, o_kp)):
        mean_abs = oracle.subblock_pool(bits(torch.from_numpy(np.abs(ref_out)).float().to(torch.bfloat16)))
        bound = 1e-2 + (8e-3 + 2.0 ** -9) * 1.01 * mean_abs + 64 * 2.0 ** -24 * mean_abs
        err = np.abs(to_host(got).astype(np.float64) - ref)
        assert np.all(err <= bound), f"pooled: worst err/bound {(err / bound).max():.3g}"


def test_qk_pool_in_place():
    B, N, H, Dh, bands = 1, 257, 4, 128, (16, 56, 56)
    q, k, wq, wk, pos = qk_pool_inputs(B, N, H, Dh, seed=3)
    qr, kr, qpr, kpr = dit.dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, pos, bands)
    qi, ki = q.clone(), k.clone()
    dit.dit_qk_rmsnorm_rope3d_pool(qi, ki, wq, wk, pos, bands, q_out=qi, k_out=ki)
    torch.cuda.synchronize()
    assert torch.equal(qi, qr) and torch.equal(ki, kr)


@pytest.mark.parametrize("name", ["full5s", "full10s"])
def test_qk_pool_full_workload_equals_parts(name):
    wl = WORKLOADS[name]
    ins = make_inputs(wl, device=DEV, names=("q", "k", "wq", "wk"))
    pos = dit.dit_packed_positions(*wl.grid, wl.n_extra, device=DEV)
    qo, ko, qp, kp = dit.dit_qk_rmsnorm_rope3d_pool(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands,
                                                    theta=wl.theta, eps=wl.eps)
    qr, kr = dit.dit_qk_rmsnorm_rope3d(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands, theta=wl.theta,
                                       eps=wl.eps)
    assert torch.equal(qo, qr) and torch.equal(ko, kr)
    del ins
    qpr, kpr = dit.dit_subblock_pool(qr, kr)
    torch.cuda.synchronize()
    assert torch.equal(qp, qpr) and torch.equal(kp, kpr)


@pytest.mark.parametrize("head_major", [False, True], ids=["token_major", "head_major"])
@pytest.mark.parametrize("shape", [QK_POOL_SHAPES[0], QK_POOL_SHAPES[1], QK_POOL_SHAPES[2], QK_POOL_SHAPES[5]],
                         ids=lambda s: "x".join(map(str, s[:4])))
def test_qk_pool_from_fused_projection(shape, head_major):
    # q and k read out of a fused [B, N, 3*H*Dh] projection, q', k' in either layout: the same
    # outputs as the layout QK kernel and the same means as the contiguous token-major call
    B, N, H, Dh, bands = shape
    q, k, wq, wk, pos = qk_pool_inputs(B, N, H, Dh, seed=7 + N)
    HD = H * Dh
    qkv = torch.cat([q.reshape(B, N, HD), k.reshape(B, N, HD), torch.full((B, N, HD), float("nan"), device=DEV,
                                                                          dtype=torch.bfloat16)], dim=-1).contiguous()
    qo, ko, qp, kp = dit.dit_qk_rmsnorm_rope3d_pool(qkv, None, wq, wk, pos, bands, head_major=head_major, heads=(H, Dh))
    ql, kl = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, pos, bands, head_major=head_major)
    _, _, qp_ref, kp_ref = dit.dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, pos, bands)
    torch.cuda.synchronize()
    assert torch.equal(qo, ql) and torch.equal(ko, kl)
    assert torch.equal(qp, qp_ref) and torch.equal(kp, kp_ref)


def test_every_entry_point_accepts_empty_inputs():
    # zero tokens (or zero samples) is a no-op for every entry point, through the binding
    bf = dict(dtype=torch.bfloat16, device=DEV)
    D, H, Dh, bands = 256, 4, 64, (16, 24, 24)
    x = torch.empty((1, 0, D), **bf)
    v = torch.zeros((1, D), **bf)
    w = torch.ones((Dh,), **bf)
    pos = torch.empty((0, 3), dtype=torch.int32, device=DEV)
    q = torch.empty((1, 0, H, Dh), **bf)
    assert dit.dit_adaln_modulate(x, v, v).shape == (1, 0, D)
    assert dit.dit_gated_residual(x, x, v).shape == (1, 0, D)
    xo, z = dit.dit_gated_residual_adaln(x, x, v, v, v)
    assert xo.shape == z.shape == (1, 0, D)
    assert dit.dit_swiglu(torch.empty((0, 2 * D), **bf)).shape == (0, D)
    qo, ko = dit.dit_qk_rmsnorm_rope3d(q, q, w, w, pos, bands)
    assert qo.shape == (1, 0, H, Dh)
    ql, kl = dit.dit_qk_rmsnorm_rope3d_layout(torch.empty((1, 0, 3 * H * Dh), **bf), H, Dh, w, w, pos, bands)
    assert ql.shape == (1, H, 0, Dh)
    assert dit.dit_packed_positions(0, 4, 4, 0, device=DEV).shape == (0, 3)
    qp, kp = dit.dit_subblock_pool(q, q)
    assert qp.shape == (1, H, 0, Dh)
    kept, scores = dit.dit_subblock_route(qp, kp, sparsity=0.75)
    assert kept.shape == (1, H, 0, 0)
    outs = dit.dit_qk_rmsnorm_rope3d_pool(q, q, w, w, pos, bands)
    assert outs[2].shape == (1, H, 0, Dh)
    change = dit.dit_residual_change(x, x)
    dit.dit_copy16(torch.empty(0, dtype=torch.uint8, device=DEV), torch.empty(0, dtype=torch.uint8, device=DEV))
    # zero samples
    qp0, kp0 = dit.dit_subblock_pool(torch.empty((0, 100, H, Dh), **bf), torch.empty((0, 100, H, Dh), **bf))
    assert qp0.shape == (0, H, 2, Dh)
    torch.cuda.synchronize()
    assert torch.all(change == 0)
