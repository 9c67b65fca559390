"""Entry points enqueued on two streams at once give the same bits as one by one.

The library keeps no state between calls and enqueues only on the stream it
is given, so independent calls on two streams may run concurrently.  Each
stream here gets its own outputs (and its own residual-change workspace);
after both are drained every output must equal the same call made alone on
the default stream.  The arithmetic itself is checked against the oracle
elsewhere.
"""
import pytest
import torch

import video_diffusion_transformer_dit_amd as dit

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _randn(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def _calls(seed):
    """One set of inputs and a function that runs every entry point on them into fresh outputs."""
    B, T, Hg, Wg, extra = 2, 3, 8, 12, 13
    N = T * Hg * Wg + extra  # 301 tokens
    D, H, Dh, F, bands = 512, 4, 64, 1024, (16, 24, 24)
    x, yr = _randn((B, N, D), seed), _randn((B, N, D), seed + 1)
    shift, scale, gate = (_randn((B, D), seed + i, 0.1) for i in (2, 3, 4))
    sw_in = _randn((B * N, 2 * F), seed + 5)
    q, k = _randn((B, N, H, Dh), seed + 6), _randn((B, N, H, Dh), seed + 7)
    qkv = _randn((B, N, 3 * H * Dh), seed + 8)
    wq, wk = 1 + _randn((Dh,), seed + 9, 0.02), 1 + _randn((Dh,), seed + 10, 0.02)
    workspace = torch.empty(max(dit.dit_residual_change_workspace_bytes(B, N, D), 16), dtype=torch.uint8,
                            device=DEV)

    def run(stream):
        out = {}
        out["pos"] = dit.dit_packed_positions(T, Hg, Wg, extra, stream=stream)
        out["y"] = dit.dit_adaln_modulate(x, shift, scale, stream=stream)
        out["res"] = dit.dit_gated_residual(x, yr, gate, stream=stream)
        out["x_out"], out["z"] = dit.dit_gated_residual_adaln(x, yr, gate, shift, scale, stream=stream)
        out["sw"] = dit.dit_swiglu(sw_in, stream=stream)
        out["qo"], out["ko"] = dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, out["pos"], bands, stream=stream)
        out["qh"], out["kh"] = dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, out["pos"], bands,
                                                                stream=stream)
        out["change"] = dit.dit_residual_change(out["res"], x, workspace=workspace, stream=stream)
        _, _, qp, kp = dit.dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, out["pos"], bands, stream=stream)
        out["kept"], scores = dit.dit_subblock_route(qp, kp, sparsity=0.75, stream=stream)
        out["scores"] = scores[..., :qp.shape[2]]  # the row padding past nb is unspecified
        return out

    return run


def test_two_streams_equal_one_by_one():
    run_a, run_b = _calls(100), _calls(200)
    ref_a = run_a(None)
    torch.cuda.synchronize()
    ref_b = run_b(None)
    torch.cuda.synchronize()

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(3):
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        # the outputs are allocated on the current stream inside run(); tie them to the side streams
        with torch.cuda.stream(sa):
            out_a = run_a(sa)
        with torch.cuda.stream(sb):
            out_b = run_b(sb)
        torch.cuda.synchronize()
        for name in ref_a:
            assert torch.equal(out_a[name], ref_a[name]), f"repeat {rep}: stream A {name}"
            assert torch.equal(out_b[name], ref_b[name]), f"repeat {rep}: stream B {name}"
