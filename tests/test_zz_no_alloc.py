"""The allocation-free residual-change entry point against the one with a workspace.

dit_residual_change_noalloc keeps its per-tile partials in the library's static
scratch array instead of a caller workspace.  Called through the C ABI, it must
give exactly the sums dit_residual_change gives on the same inputs (the same
kernels in the same order), on two calls in a row with the second smaller (the
array still holds the first call's partials), and both must agree with the
fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_dit_amd as dit
from synthetic_inputs import bits

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    dit.load_library()  # raises if libdit_ops.so is missing: no fallback path exists
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def draw(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


def noalloc_c_abi(r, rc, out):
    """Call the C entry point directly (raw device pointers, torch's current stream)."""
    B, N, D = r.shape
    stream = torch.cuda.current_stream().cuda_stream
    return dit.load_library().dit_residual_change_noalloc(r.data_ptr(), rc.data_ptr(), out.data_ptr(), B, N, D,
                                                          stream)


def check_against_oracle(got, r, rc, what):
    ref = oracle.residual_change(bits(r), bits(rc))
    g = got.cpu().numpy()
    rel = np.abs(g - ref) / np.maximum(np.abs(ref), 1e-300)
    assert np.all(rel <= 2e-6), f"{what}: relative error {rel.max():.3g} against the oracle"


# (B, N, D): several tiles with a ragged last tile, then a smaller call that
# reads fewer partials than the first one left in the array.
CALLS = [(2, 4099, 4096), (1, 333, 1032)]


def test_noalloc_equals_workspace_entry_point_two_calls():
    for i, (B, N, D) in enumerate(CALLS):
        print(f"[no-alloc] call {i}: B={B} N={N} D={D}", flush=True)
        r = draw((B, N, D), seed=100 + i)
        rc = draw((B, N, D), seed=200 + i)
        want = dit.dit_residual_change(r, rc)
        got = torch.full((B, 3), float("nan"), dtype=torch.float64, device=DEV)
        assert noalloc_c_abi(r, rc, got) == dit.DIT_OK
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {i}: {got.cpu().numpy()} != {want.cpu().numpy()}"
        check_against_oracle(got, r, rc, f"call {i}")


def test_noalloc_at_the_largest_shipped_sequence():
    # 246,432 tokens x 4096 channels: 61,608 partials of the 131,072 the array holds
    B, N, D = 1, 246_432, 4096
    print(f"[no-alloc] B={B} N={N} D={D}", flush=True)
    r = draw((B, N, D), seed=7)
    rc = draw((B, N, D), seed=8)
    want = dit.dit_residual_change(r, rc)
    got = torch.empty((B, 3), dtype=torch.float64, device=DEV)
    assert noalloc_c_abi(r, rc, got) == dit.DIT_OK
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # then a small call right after, on another shape
    r2, rc2 = r[:, :1000, :1024].contiguous(), rc[:, :1000, :1024].contiguous()
    want2 = dit.dit_residual_change(r2, rc2)
    got2 = torch.empty((1, 3), dtype=torch.float64, device=DEV)
    dit.dit_residual_change_noalloc(r2, rc2, got2)
    torch.cuda.synchronize()
    assert torch.equal(got2, want2)
    check_against_oracle(got2, r2, rc2, "small call after the large one")


def test_noalloc_special_cases():
    # N == 0 writes zeros; r == r_cached gives a zero change; beyond the capacity the call is refused
    out = torch.full((2, 3), 7.0, dtype=torch.float64, device=DEV)
    empty = torch.empty((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    assert noalloc_c_abi(empty, empty, out) == dit.DIT_OK
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))
    r = draw((1, 64, 256), seed=9)
    same = torch.empty((1, 3), dtype=torch.float64, device=DEV)
    dit.dit_residual_change_noalloc(r, r, same)
    torch.cuda.synchronize()
    s = same.cpu().numpy()[0]
    assert s[0] == 0.0 and s[1] > 0.0 and s[2] == 0.0
    big = torch.empty((1, 3), dtype=torch.float64, device=DEV)
    # NULL inputs: the capacity check comes first, and a call that got past it would stop at DIT_ERR_NULL
    status = dit.load_library().dit_residual_change_noalloc(None, None, big.data_ptr(), 2, 524_288, 4096, None)
    assert status == dit.DIT_ERR_SCRATCH
