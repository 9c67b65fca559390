"""Every entry point captured in one HIP graph and replayed.

The library's calls only enqueue kernels on the caller's stream (no
allocation, memset or synchronisation), so a caller can capture them.  The
graph holds one call of each entry point on shapes with ragged tiles.  It is
replayed three times, each time after eager work on the same outputs (zeroing
them, then a synchronisation), and every output of every replay must equal the
eager calls' bit for bit.  That equality is the test: the arithmetic is checked
against the oracle elsewhere.
"""
import pytest
import torch

import video_diffusion_transformer_dit_amd as dit

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _randn(shape, seed, scale=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(DEV)


def test_graph_replays_equal_eager_calls():
    B, T, Hg, Wg, extra = 2, 2, 10, 14, 20
    N = T * Hg * Wg + extra  # 300 tokens: 4 full 64-token blocks and a ragged one
    D, H, Dh, F, bands = 256, 4, 64, 512, (16, 24, 24)
    nb = (N + dit.DIT_SUBBLOCK_TOKENS - 1) // dit.DIT_SUBBLOCK_TOKENS
    keep = dit.dit_subblock_keep(nb, 0.75)
    print(f"[graph] B={B} N={N} D={D} H={H} Dh={Dh} F={F} nb={nb} keep={keep}", flush=True)

    x, yr = _randn((B, N, D), 1), _randn((B, N, D), 2)
    shift, scale, gate = _randn((B, D), 3, 0.1), _randn((B, D), 4, 0.1), _randn((B, D), 5, 0.1)
    sw_in = _randn((B * N, 2 * F), 6)
    q, k = _randn((B, N, H, Dh), 7), _randn((B, N, H, Dh), 8)
    qkv = _randn((B, N, 3 * H * Dh), 9)
    wq, wk = 1 + _randn((Dh,), 10, 0.02), 1 + _randn((Dh,), 11, 0.02)

    out = {
        "pos": torch.empty((N, 3), dtype=torch.int32, device=DEV),
        "y": torch.empty_like(x), "res": torch.empty_like(x), "x_out": torch.empty_like(x), "z": torch.empty_like(x),
        "sw": torch.empty((B * N, F), dtype=torch.bfloat16, device=DEV),
        "qo": torch.empty_like(q), "ko": torch.empty_like(k),
        "qh": torch.empty((B, H, N, Dh), dtype=torch.bfloat16, device=DEV),
        "kh": torch.empty((B, H, N, Dh), dtype=torch.bfloat16, device=DEV),
        "change": torch.empty((B, 3), dtype=torch.float64, device=DEV),
        "qp_out": torch.empty_like(q), "kp_out": torch.empty_like(k),
        "qp": torch.empty((B, H, nb, Dh), dtype=torch.float32, device=DEV),
        "kp": torch.empty((B, H, nb, Dh), dtype=torch.float32, device=DEV),
        "scores": torch.empty((B, H, nb, dit.dit_subblock_scores_ld(nb)), dtype=torch.float32, device=DEV),
        "kept": torch.empty((B, H, nb, keep), dtype=torch.int32, device=DEV),
    }
    workspace = torch.empty(max(dit.dit_residual_change_workspace_bytes(B, N, D), 16), dtype=torch.uint8,
                            device=DEV)

    def calls():
        dit.dit_packed_positions(T, Hg, Wg, extra, pos=out["pos"])
        dit.dit_adaln_modulate(x, shift, scale, y=out["y"])
        dit.dit_gated_residual(x, yr, gate, out=out["res"])
        dit.dit_gated_residual_adaln(x, yr, gate, shift, scale, x_out=out["x_out"], z=out["z"])
        dit.dit_swiglu(sw_in, out=out["sw"])
        dit.dit_qk_rmsnorm_rope3d(q, k, wq, wk, out["pos"], bands, q_out=out["qo"], k_out=out["ko"])
        dit.dit_qk_rmsnorm_rope3d_layout(qkv, H, Dh, wq, wk, out["pos"], bands, head_major=True,
                                         q_out=out["qh"], k_out=out["kh"])
        dit.dit_residual_change(out["res"], x, out=out["change"], workspace=workspace)
        dit.dit_qk_rmsnorm_rope3d_pool(q, k, wq, wk, out["pos"], bands, q_out=out["qp_out"], k_out=out["kp_out"],
                                       q_pooled=out["qp"], k_pooled=out["kp"])
        dit.dit_subblock_route(out["qp"], out["kp"], keep=keep, scores=out["scores"], kept=out["kept"])

    def zero_outputs():
        for t in out.values():
            t.zero_()

    zero_outputs()  # the score rows' padding past nb is never written: start it at zero on both sides
    calls()
    torch.cuda.synchronize()
    eager = {name: t.clone() for name, t in out.items()}

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for replay in range(3):
        zero_outputs()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            assert torch.equal(t, eager[name]), f"replay {replay}: {name} differs from the eager calls"
    del graph
