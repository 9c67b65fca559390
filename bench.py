#!/usr/bin/env python3
"""Benchmark of the fused DiT non-GEMM operator chain on one MI355X.

A step is one pass of the whole chain over one batch of synthetic tokens
already resident in HBM: packed positions, AdaLN modulate, gated residual,
SwiGLU and QK RMSNorm + 3D RoPE, each a kernel of libdit_ops.so launched on
torch's current stream.  After W untimed steps, K steps are timed between two
device synchronisations (wall clock), with HIP events around every kernel of
every timed step on the launch stream.  The step is then captured once as a
HIP graph; three replays are checked bit for bit against the eager step, and
after W untimed replays K replays are timed between two device
synchronisations.  When every checked replay matches, `ms_per_step`, `value`
and `tokens_per_s` are the replayed step's (the same kernels on the same
buffers, launched as one graph); `eager_ms_per_step` keeps the eager figure.

The printed JSON line reports:
  value          whole-chain algorithmic HBM bytes / step time (GB/s)
  tokens_per_s   tokens / step time
  ops            per-kernel average duration, bytes and GB/s from the events
  roofline       the dominant kernel against the 8 TB/s HBM peak; `traffic`
                 is the counter-measured HBM bytes per launch from the
                 committed counter summary when it was taken on the current
                 kernel source, else null
  copy_ceiling   a plain 16-byte-vector copy on the same device
  graph_replay   the same step captured once as a HIP graph and replayed
                 (replays checked bit for bit against the eager step); not
                 part of `value`
  next_fused_residual_adaln
                 the gated residual fused with the AdaLN that follows it,
                 timed on its own after the chain (not part of `value`)
  next_qk_layout QK read from a fused QKV buffer, written head-major, timed
                 on its own after the chain (not part of `value`)
  next_residual_change
                 the Cache-DiT residual-change statistic over the sequence,
                 timed on its own after the chain (not part of `value`)
  cpu_baseline   the fp64 oracle on a bounded sample of the same workload,
                 on the host cores (and the GPU outputs of that sample checked
                 against it)

Algorithmic bytes are compulsory traffic: each input read once, each output
written once, small per-sample vectors and weights counted once.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + tokens/s for fused DiT op chain, 1344x768 5s"
HBM_PEAK_GBPS = 8000.0
OPS = ("positions", "adaln", "residual", "swiglu", "qk")
KERNEL_SOURCES = {
    "positions": "positions.hip",
    "adaln": "adaln.hip",
    "residual": "residual.hip",
    "swiglu": "swiglu.hip",
    "qk": "qk_rope.hip",
    "residual_adaln": "residual_adaln.hip",
    "qk_layout": "qk_rope.hip",
    "change": "residual_change.hip",
    "change_final": "residual_change.hip",
    "qk_pool": "qk_rope.hip",
    "qk_pool_layout": "qk_rope.hip",
    "pool": "subblock.hip",
    "pool_hm": "subblock.hip",
    "scores": "subblock.hip",
    "topk": "subblock.hip",
    "route_fused": "subblock.hip",
    "copy": "copy.hip",
    **{p: "patterns.hip" for p in ("p_read", "p_write", "p_swiglu", "p_residual", "p_adaln", "p_residual_adaln",
                                   "p_head_major", "p_score_tiles", "p_topk_rows")},
}
# Kernels of the next rows, measured after the chain (see main()).
NEXT_OPS = ("residual_adaln", "qk_layout", "qk_pool_layout", "change", "change_final", "qk_pool", "pool", "pool_hm",
            "scores", "topk", "route_fused")
ROUTE_SPARSITY = 0.75
# std of the per-head component added to the block means for the second route timing
SHARED_OFFSET_STD = 0.3
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "{op}_{workload}_counters.md")


def op_bytes(wl, next_rows: bool = False) -> dict:
    """Compulsory HBM bytes of one launch of each op on workload ``wl`` (the chain's five, and with
    ``next_rows`` the kernels of the next rows as the benchmark runs them)."""
    B, N, R, D, F, H, Dh = wl.B, wl.N, wl.R, wl.D, wl.F, wl.H, wl.Dh
    out = {
        "positions": 12 * N,                                   # write (t, h, w) int32
        "adaln": 2 * R * D * 2 + 2 * B * D * 2,                # x in, y out, shift + scale
        "residual": 3 * R * D * 2 + B * D * 2,                 # x, y in, out, gate
        "swiglu": R * 2 * F * 2 + R * F * 2,                   # [a|b] in, out
        "qk": 4 * R * H * Dh * 2 + 12 * N + 2 * Dh * 2,        # q, k in, q', k' out, pos, wq, wk
    }
    if next_rows:
        nb = -(-N // 64)
        keep = dit_keep(nb)
        pooled = 2 * B * H * nb * Dh * 4
        out.update({
            "residual_adaln": 4 * R * D * 2 + 3 * B * D * 2,   # x, y in, x_out, z out, gate + shift + scale
            "qk_layout": out["qk"],                            # same bytes, strided in, head-major out
            "change": 2 * R * D * 2,                           # r, r_cached in (partials: 16 B per 2048 vectors)
            "qk_pool": out["qk"] + pooled,                     # QK's bytes plus the block means out
            "qk_pool_layout": out["qk"] + pooled,              # the same from a fused QKV buffer, head-major out
            "pool": 2 * R * H * Dh * 2 + pooled,               # q', k' in, fp32 block means out
            "pool_hm": 2 * R * H * Dh * 2 + pooled,
            "scores": pooled + B * H * nb * nb * 4,            # means in, fp32 scores out
            "topk": B * H * nb * nb * 4 + B * H * nb * keep * 4,  # scores in, kept indices out
            "route_fused": pooled + B * H * nb * keep * 4,     # means in, kept indices out (no score matrix)
            # access-pattern streams (one launch each; the head-major copy moves one of q, k)
            "p_read": R * 4 * F,
            "p_write": R * 2 * F,
            "p_swiglu": R * 6 * F,
            "p_residual": R * 6 * D,
            "p_adaln": R * 4 * D,
            "p_residual_adaln": R * 8 * D,
            "p_head_major": R * 4 * H * Dh,
            "p_score_tiles": pooled + B * H * nb * nb * 4,   # the score kernel's bytes (head dim 128)
            "p_topk_rows": B * H * nb * nb * 4 + B * H * nb * (-(-nb // 4)) * 4,  # top-k's bytes at keep = nb / 4
        })
    return out


def dit_keep(nb: int) -> int:
    from video_diffusion_transformer_dit_amd import dit_subblock_keep

    return dit_subblock_keep(nb, ROUTE_SPARSITY)


def source_digest(op: str) -> str:
    """sha256 of the kernel source a counter summary was taken on (plus the shared header)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "video_diffusion_transformer_dit_amd", "csrc")
    for name in (KERNEL_SOURCES[op], "device_common.hpp"):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(op: str, workload: str):
    """Counter-measured HBM bytes per launch from profiles/, if taken on the current source."""
    path = COUNTER_SUMMARY.format(op=op, workload=workload)
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as fh:
        text = fh.read()
    digest = re.search(r"kernel source sha256:\s*([0-9a-f]{64})", text)
    traffic = re.search(r"HBM bytes per launch \(calibrated\):\s*([0-9.eE+]+)", text)
    if not digest or not traffic or digest.group(1) != source_digest(op):
        return None
    return float(traffic.group(1))


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="full5s", help="full5s (default), lowres, full10s, batch2, tiny")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for the CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replayed chain")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run three 1 GiB dit_copy16 calls after warm-up (known-size work for counter calibration)")
    p.add_argument("--summarize-rocprof", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="write profiles/ summaries from rocprofv3 CSV output of a kernel-trace run and of "
                        "FETCH_SIZE and WRITE_SIZE counter runs of this benchmark, then exit")
    p.add_argument("--summarize-stalls", nargs=2, metavar=("TRACE_DIR", "STALL_DIR"),
                   help="write the profiles/ summary of the shader-sequencer stall counter run (wave time waiting, "
                        "issuing VALU, VMEM latency) next to the kernel trace, then exit")
    p.add_argument("--summarize-sq", nargs=2, metavar=("TRACE_DIR", "SQ_DIR"),
                   help="write the profiles/ summary of the shader-sequencer counter run (instruction mix, LDS "
                        "waits, VALU issue rate, MFMA work) next to the kernel trace, then exit")
    return p.parse_args(argv)


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.summarize_rocprof:
        return summarize_rocprof(*args.summarize_rocprof, workload=args.workload)
    if args.summarize_sq:
        return summarize_sq(*args.summarize_sq, workload=args.workload)
    if args.summarize_stalls:
        return summarize_stalls(*args.summarize_stalls, workload=args.workload)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the chain on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the operators are row-local, so more GPUs would each run this same benchmark on their own "
              "share of the tokens.", file=sys.stderr)
        return 2

    import torch

    import synthetic_inputs as si
    import video_diffusion_transformer_dit_amd as dit

    dit.load_library()  # raises if libdit_ops.so is not built: there is no other path
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = si.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    ins = si.make_inputs(wl, device=dev)
    pos = torch.empty((wl.N, 3), dtype=torch.int32, device=dev)
    y = torch.empty_like(ins["x_mod"])
    out = torch.empty_like(ins["res_x"])
    sw = torch.empty((wl.R, wl.F), dtype=torch.bfloat16, device=dev)
    qo = torch.empty_like(ins["q"])
    ko = torch.empty_like(ins["k"])
    torch.cuda.synchronize()
    print(f"[bench] workload {wl.name}: {wl.R} tokens, inputs drawn in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def launch(op, st=None):
        st = stream if st is None else st
        if op == "positions":
            dit.dit_packed_positions(*wl.grid, wl.n_extra, pos=pos, stream=st)
        elif op == "adaln":
            dit.dit_adaln_modulate(ins["x_mod"], ins["shift"], ins["scale"], y=y, eps=wl.eps, stream=st)
        elif op == "residual":
            dit.dit_gated_residual(ins["res_x"], ins["res_y"], ins["gate"], out=out, stream=st)
        elif op == "swiglu":
            dit.dit_swiglu(ins["swiglu_in"], out=sw, stream=st)
        else:
            dit.dit_qk_rmsnorm_rope3d(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands, q_out=qo, k_out=ko,
                                      theta=wl.theta, eps=wl.eps, stream=st)

    def step(events=None):
        for i, op in enumerate(OPS):
            if events is not None:
                events[i][0].record(stream)
            launch(op)
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dit.dit_copy16(src, dst, stream=stream)
        del src, dst
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in OPS]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] {args.steps} timed steps done", file=sys.stderr, flush=True)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nbytes = op_bytes(wl)
    chain_bytes = sum(nbytes.values())
    ops = {}
    for i, op in enumerate(OPS):
        ms = sum(events[s][i][0].elapsed_time(events[s][i][1]) for s in range(args.steps)) / args.steps
        ops[op] = {"avg_ms": round(ms, 5), "bytes": nbytes[op], "GB_s": round(nbytes[op] / (ms * 1e-3) / 1e9, 1),
                   "pct_of_peak": round(100.0 * nbytes[op] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
    kernel_ms = sum(o["avg_ms"] for o in ops.values())
    dominant = max(ops, key=lambda o: ops[o]["avg_ms"])
    achieved = ops[dominant]["GB_s"]
    traffic = committed_traffic(dominant, wl.name)
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "algorithmic_bytes": nbytes[dominant]}

    # The same step captured once as a HIP graph and replayed: the five
    # launches then cost one graph launch, which matters where they are
    # launch-bound (the tiny workload).  Replays are checked against the eager
    # step bit for bit, three times, with eager work between the replays; K
    # replays are then timed between two device synchronisations, as the
    # eager steps are.  When the replays match, the headline step time is the
    # replayed one (the same kernels on the same buffers).
    graph_replay = None
    if not args.no_graph and not args.copy_calibration:
        outs = {"positions": pos, "adaln": y, "residual": out, "swiglu": sw, "q": qo, "k": ko}
        try:
            step()
            torch.cuda.synchronize()
            eager = {k: v.clone() for k, v in outs.items()}
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream(dev)  # default priority
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for op in OPS:
                    launch(op, side)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                cap = torch.cuda.current_stream(dev)
                for op in OPS:
                    launch(op, cap)
            torch.cuda.synchronize()
            equal = True
            for _ in range(3):
                for v in outs.values():
                    v.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                equal = equal and all(torch.equal(outs[k], eager[k]) for k in outs)
            del eager
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            g0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            gms = (time.perf_counter() - g0) * 1e3 / args.steps
            graph_replay = {"ms_per_step": round(gms, 4), "GB_s": round(chain_bytes / (gms * 1e-3) / 1e9, 1),
                            "pct_of_peak": round(100.0 * chain_bytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                            "tokens_per_s": round(wl.R / (gms * 1e-3)),
                            "replays_equal_eager": bool(equal), "replays_checked": 3}
            del g
        except RuntimeError as e:  # capture unsupported here: the eager figure stands
            graph_replay = {"error": str(e)[:200]}
        print(f"[bench] graph replay: {graph_replay}", file=sys.stderr, flush=True)

    # Per-op medians under a flush protocol: every timed call is preceded,
    # outside its events, by a 1 GiB scratch write that evicts the 4 MB L2 of
    # each XCD and the 256 MB last-level cache, so no op starts with warm data.
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flushed = {}
    reps = max(20, args.steps)
    for op in OPS:
        pairs = []
        for i in range(args.warmup + reps):
            flush_buf.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch(op)
            e1.record(stream)
            if i >= args.warmup:
                pairs.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in pairs)
        med = t[len(t) // 2]
        flushed[op] = {"median_ms": round(med, 5), "min_ms": round(t[0], 5),
                       "GB_s_median": round(nbytes[op] / (med * 1e-3) / 1e9, 1),
                       "pct_of_peak_median": round(100.0 * nbytes[op] / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
    del flush_buf

    # One GPU's share of an 8-way sequence split (row-local ops: each GPU runs
    # this same chain on N/8 tokens, with the matching slice of the positions).
    share = None
    if wl.B == 1:
        ns = wl.N // 8
        sl = {"x_mod": ins["x_mod"][:, :ns], "res_x": ins["res_x"][:, :ns], "res_y": ins["res_y"][:, :ns],
              "swiglu_in": ins["swiglu_in"][:ns], "q": ins["q"][:, :ns], "k": ins["k"][:, :ns]}
        outs_s = {"y": y[:, :ns], "out": out[:, :ns], "sw": sw[:ns], "qo": qo[:, :ns], "ko": ko[:, :ns]}
        pos_s = pos[:ns]

        def share_step():
            dit.dit_adaln_modulate(sl["x_mod"], ins["shift"], ins["scale"], y=outs_s["y"], eps=wl.eps, stream=stream)
            dit.dit_gated_residual(sl["res_x"], sl["res_y"], ins["gate"], out=outs_s["out"], stream=stream)
            dit.dit_swiglu(sl["swiglu_in"], out=outs_s["sw"], stream=stream)
            dit.dit_qk_rmsnorm_rope3d(sl["q"], sl["k"], ins["wq"], ins["wk"], pos_s, wl.bands, q_out=outs_s["qo"],
                                      k_out=outs_s["ko"], theta=wl.theta, eps=wl.eps, stream=stream)

        for _ in range(args.warmup):
            share_step()
        torch.cuda.synchronize()
        t_s0 = time.perf_counter()
        for _ in range(args.steps):
            share_step()
        torch.cuda.synchronize()
        share_ms = (time.perf_counter() - t_s0) * 1e3 / args.steps
        share_bytes = (chain_bytes - nbytes["positions"]) * ns // wl.N
        share = {"rows": ns, "of": "1/8 of the tokens (sequence split), positions sliced, not rebuilt",
                 "ms_per_step": round(share_ms, 4), "bytes": share_bytes,
                 "GB_s": round(share_bytes / (share_ms * 1e-3) / 1e9, 1),
                 "pct_of_peak": round(100.0 * share_bytes / (share_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                 "tokens_per_s": round(ns / (share_ms * 1e-3))}
        # (the slices receive the same values the full chain wrote there: same inputs, per-row kernels)

    # The next fusion, measured on its own after the chain: gated residual ->
    # AdaLN in one kernel (x and y read once, x_out and z written once).
    fused_bytes = 4 * wl.R * wl.D * 2 + 3 * wl.B * wl.D * 2
    # Own output buffers: the chain's outputs stay intact for the oracle check.
    fused_x = torch.empty_like(out)
    fused_z = torch.empty_like(y)
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        if i >= args.warmup:
            fev[i - args.warmup][0].record(stream)
        dit.dit_gated_residual_adaln(ins["res_x"], ins["res_y"], ins["gate"], ins["shift"], ins["scale"],
                                     x_out=fused_x, z=fused_z, eps=wl.eps, stream=stream)
        if i >= args.warmup:
            fev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    fused_ms = sum(a.elapsed_time(b) for a, b in fev) / args.steps
    unfused_ms = ops["residual"]["avg_ms"] + ops["adaln"]["avg_ms"]
    fused = {"op": "dit_gated_residual_adaln", "avg_ms": round(fused_ms, 5), "bytes": fused_bytes,
             "GB_s": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1),
             "pct_of_peak": round(100.0 * fused_bytes / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
             "unfused_ms": round(unfused_ms, 5), "unfused_bytes": nbytes["residual"] + nbytes["adaln"],
             "time_saved_pct": round(100.0 * (1.0 - fused_ms / unfused_ms), 1),
             "traffic": committed_traffic("residual_adaln", wl.name)}

    # QK with the layouts around attention: q and k read straight out of a fused
    # [B, N, 3*H*Dh] projection buffer, q' and k' written head-major [B, H, N, Dh].
    HD = wl.H * wl.Dh
    qkv = torch.empty((wl.B, wl.N, 3 * HD), dtype=torch.bfloat16, device=dev)
    qkv[..., :HD].copy_(ins["q"].reshape(wl.B, wl.N, HD))
    qkv[..., HD:2 * HD].copy_(ins["k"].reshape(wl.B, wl.N, HD))
    qkv[..., 2 * HD:].zero_()
    qo_hm = torch.empty((wl.B, wl.H, wl.N, wl.Dh), dtype=torch.bfloat16, device=dev)
    ko_hm = torch.empty_like(qo_hm)
    lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        if i >= args.warmup:
            lev[i - args.warmup][0].record(stream)
        dit.dit_qk_rmsnorm_rope3d_layout(qkv, wl.H, wl.Dh, ins["wq"], ins["wk"], pos, wl.bands, head_major=True,
                                         q_out=qo_hm, k_out=ko_hm, theta=wl.theta, eps=wl.eps, stream=stream)
        if i >= args.warmup:
            lev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    layout_ms = sum(a.elapsed_time(b) for a, b in lev) / args.steps
    # the same, also writing the SubBlock block means (one pass prepares attention and routing)
    nb_r = -(-wl.N // 64)
    qo_hm2, ko_hm2 = torch.empty_like(qo_hm), torch.empty_like(ko_hm)
    qp_r = torch.empty((wl.B, wl.H, nb_r, wl.Dh), dtype=torch.float32, device=dev)
    kp_r = torch.empty_like(qp_r)
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        if i >= args.warmup:
            pev[i - args.warmup][0].record(stream)
        dit.dit_qk_rmsnorm_rope3d_pool(qkv, None, ins["wq"], ins["wk"], pos, wl.bands, head_major=True,
                                       heads=(wl.H, wl.Dh), q_out=qo_hm2, k_out=ko_hm2, q_pooled=qp_r, k_pooled=kp_r,
                                       theta=wl.theta, eps=wl.eps, stream=stream)
        if i >= args.warmup:
            pev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    layout_pool_ms = sum(a.elapsed_time(b) for a, b in pev) / args.steps
    layout_pool_same = bool(torch.equal(qo_hm2, qo_hm) and torch.equal(ko_hm2, ko_hm))
    del qkv, qo_hm2, ko_hm2, qp_r, kp_r
    layout_pool_bytes = nbytes["qk"] + 2 * wl.B * wl.H * nb_r * wl.Dh * 4
    layout = {"op": "dit_qk_rmsnorm_rope3d_layout (fused QKV in, head-major out)", "avg_ms": round(layout_ms, 5),
              "bytes": nbytes["qk"], "GB_s": round(nbytes["qk"] / (layout_ms * 1e-3) / 1e9, 1),
              "pct_of_peak": round(100.0 * nbytes["qk"] / (layout_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
              "token_major_ms": ops["qk"]["avg_ms"],
              "passes_avoided": "splitting q, k out of the QKV buffer and transposing q', k' to head-major: "
                                "each a further read and write of q and k (2 x 4.1 GB here)",
              "traffic": committed_traffic("qk_layout", wl.name),
              "with_block_means": {
                  "op": "dit_qk_rmsnorm_rope3d_pool (same layouts, also the SubBlock block means)",
                  "avg_ms": round(layout_pool_ms, 5), "bytes": layout_pool_bytes,
                  "GB_s": round(layout_pool_bytes / (layout_pool_ms * 1e-3) / 1e9, 1),
                  "pct_of_peak": round(100.0 * layout_pool_bytes / (layout_pool_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}}

    # Cache-DiT residual-change statistic over the packed sequence (the two
    # residual inputs stand in for the current and cached boundary residuals).
    change_bytes = 2 * wl.R * wl.D * 2
    change_out = torch.empty((wl.B, 3), dtype=torch.float64, device=dev)
    change_ws = torch.empty(max(16, dit.dit_residual_change_workspace_bytes(wl.B, wl.N, wl.D)), dtype=torch.uint8,
                            device=dev)
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.warmup + args.steps):
        if i >= args.warmup:
            cev[i - args.warmup][0].record(stream)
        dit.dit_residual_change(ins["res_x"], ins["res_y"], out=change_out, workspace=change_ws, stream=stream)
        if i >= args.warmup:
            cev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    change_ms = sum(a.elapsed_time(b) for a, b in cev) / args.steps
    change = {"op": "dit_residual_change (two launches: partials, fixed-order reduce)", "avg_ms": round(change_ms, 5),
              "bytes": change_bytes, "GB_s": round(change_bytes / (change_ms * 1e-3) / 1e9, 1),
              "pct_of_peak": round(100.0 * change_bytes / (change_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
              "traffic_partial_kernel": committed_traffic("change", wl.name)}

    # SubBlock routing front-end on the chain's q', k' at sparsity 0.75: block
    # means (both input layouts), block scores alone (keep = 0 runs only the
    # score kernel), then scores plus the kept blocks (top-k = the difference,
    # both timed in the same context).
    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.warmup + args.steps):
            if i >= args.warmup:
                ev[i - args.warmup][0].record(stream)
            fn()
            if i >= args.warmup:
                ev[i - args.warmup][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / args.steps

    def rate(nbytes_, ms, op):
        return {"avg_ms": round(ms, 5), "bytes": nbytes_, "GB_s": round(nbytes_ / (ms * 1e-3) / 1e9, 1),
                "pct_of_peak": round(100.0 * nbytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                "traffic": committed_traffic(op, wl.name)}

    sparsity = ROUTE_SPARSITY
    nb = -(-wl.N // 64)
    keep = dit.dit_subblock_keep(nb, sparsity)
    ld = dit.dit_subblock_scores_ld(nb)
    qp_s = torch.empty((wl.B, wl.H, nb, wl.Dh), dtype=torch.float32, device=dev)
    kp_s = torch.empty_like(qp_s)
    sc = torch.empty((wl.B, wl.H, nb, ld), dtype=torch.float32, device=dev)
    kept = torch.empty((wl.B, wl.H, nb, keep), dtype=torch.int32, device=dev)
    kept0 = torch.empty((wl.B, wl.H, nb, 0), dtype=torch.int32, device=dev)
    pool_ms = timed(lambda: dit.dit_subblock_pool(qo, ko, q_pooled=qp_s, k_pooled=kp_s, stream=stream))
    # the same bytes read as head-major [B, H, N, Dh] (timing only)
    qo_as_hm = qo.view(wl.B, wl.H, wl.N, wl.Dh)
    ko_as_hm = ko.view(wl.B, wl.H, wl.N, wl.Dh)
    pool_hm_ms = timed(lambda: dit.dit_subblock_pool(qo_as_hm, ko_as_hm, head_major=True, q_pooled=qp_s,
                                                     k_pooled=kp_s, stream=stream))
    # Scores alone (keep = 0 runs only the score kernel) and the full route,
    # each timed right after a full route: the score kernel's time depends on
    # what ran before it (after a top-k has read the whole score matrix it is
    # not the same as back to back), so top-k = route - scores compares like
    # with like.  Per step: the route (timed), scores alone (timed), the route
    # (untimed, so that the next timed route also follows one).
    def route_call():
        dit.dit_subblock_route(qp_s, kp_s, keep=keep, scores=sc, kept=kept, stream=stream)

    def scores_call():
        dit.dit_subblock_route(qp_s, kp_s, keep=0, scores=sc, kept=kept0, stream=stream)

    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    route_call()
    for i in range(args.warmup + args.steps):
        e = rev[i - args.warmup] if i >= args.warmup else None
        if e:
            e[0].record(stream)
        route_call()
        if e:
            e[1].record(stream)
            e[2].record(stream)
        scores_call()
        if e:
            e[3].record(stream)
        route_call()
    torch.cuda.synchronize()
    route_ms = sum(e[0].elapsed_time(e[1]) for e in rev) / args.steps
    scores_ms = sum(e[2].elapsed_time(e[3]) for e in rev) / args.steps

    # The two kernels' traffic with no arithmetic, each where its kernel runs:
    # the score tiles (DIT_STREAM_SCORE_TILES, head dim 128 only) right after a
    # full route, the top-k rows (DIT_STREAM_TOPK_ROWS, ceil(nb / 4) words per
    # row: the kept count at this sparsity) right after the score tiles have
    # written the matrix, and a route after both, so that every score kernel
    # launch still follows a full pass over the matrix.
    has_pattern = wl.Dh == 128 and keep == -(-nb // 4)
    score_pattern_ms = topk_pattern_ms = None
    if has_pattern:
        kept_p = torch.empty((wl.B * wl.H * nb * keep,), dtype=torch.int32, device=dev)
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        route_call()
        for i in range(args.warmup + args.steps):
            e = pev[i - args.warmup] if i >= args.warmup else None
            if e:
                e[0].record(stream)
            dit.dit_stream_pattern(dit.DIT_STREAM_SCORE_TILES, wl.B * wl.H * nb, 4 * ld, in0=qp_s, in1=kp_s, out0=sc,
                                   heads=nb, stream=stream)
            if e:
                e[1].record(stream)
                e[2].record(stream)
            dit.dit_stream_pattern(dit.DIT_STREAM_TOPK_ROWS, wl.B * wl.H * nb, 4 * ld, in0=sc, out0=kept_p, heads=nb,
                                   stream=stream)
            if e:
                e[3].record(stream)
            route_call()
        torch.cuda.synchronize()
        score_pattern_ms = sum(e[0].elapsed_time(e[1]) for e in pev) / args.steps
        topk_pattern_ms = sum(e[2].elapsed_time(e[3]) for e in pev) / args.steps
        del kept_p
    # the same kept lists with the scores kept on chip (one fused kernel, no score matrix)
    kept_f = torch.empty_like(kept)
    fused_route_ms = timed(lambda: dit.dit_subblock_route(qp_s, kp_s, keep=keep, kept=kept_f, write_scores=False,
                                                          stream=stream))
    # QK RMSNorm + RoPE that also writes the block means (no second read of q', k')
    qo_f, ko_f = torch.empty_like(qo), torch.empty_like(ko)
    qk_pool_ms = timed(lambda: dit.dit_qk_rmsnorm_rope3d_pool(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands,
                                                              q_out=qo_f, k_out=ko_f, q_pooled=qp_s, k_pooled=kp_s,
                                                              theta=wl.theta, eps=wl.eps, stream=stream))
    del qo_f, ko_f
    dit.dit_subblock_pool(qo, ko, q_pooled=qp_s, k_pooled=kp_s, stream=stream)
    pooled_bytes = 2 * wl.B * wl.H * nb * wl.Dh * 4
    score_elems = wl.B * wl.H * nb * nb
    pool_bytes = 2 * wl.R * wl.H * wl.Dh * 2 + pooled_bytes
    scores_bytes = pooled_bytes + score_elems * 4
    topk_bytes = score_elems * 4 + wl.B * wl.H * nb * keep * 4
    score_flops = 2 * score_elems * wl.Dh
    topk_ms = route_ms - scores_ms
    fused_route_bytes = pooled_bytes + wl.B * wl.H * nb * keep * 4
    # the fused route's strips: 32 query blocks (16 past 2048 blocks), each reading its head's key means
    strip_blocks = 32 if nb <= 2048 else 16
    l2_key_bytes = wl.B * wl.H * (-(-nb // strip_blocks)) * nb * wl.Dh * 4
    subblock = {
        "sparsity": sparsity, "blocks": nb, "keep": keep,
        "pool": rate(pool_bytes, pool_ms, "pool"),
        "pool_head_major": rate(pool_bytes, pool_hm_ms, "pool_hm"),
        "qk_with_pool": {**rate(nbytes["qk"] + pooled_bytes, qk_pool_ms, "qk_pool"),
                         "op": "dit_qk_rmsnorm_rope3d_pool (QK writing the block means too)",
                         "separate_ms": round(ops["qk"]["avg_ms"] + pool_ms, 5)},
        "scores": {**rate(scores_bytes, scores_ms, "scores"),
                   "TFLOP_s": round(score_flops / (scores_ms * 1e-3) / 1e12, 1),
                   "pct_of_bf16_mfma_peak": round(100.0 * score_flops / (scores_ms * 1e-3) / 2.5e15, 2)},
        "topk": rate(topk_bytes, topk_ms, "topk"),
        "route_fused": {**rate(fused_route_bytes, fused_route_ms, "route_fused"),
                        "op": "dit_subblock_route with scores = NULL (scores and selection in one kernel)",
                        "TFLOP_s": round(score_flops / (fused_route_ms * 1e-3) / 1e12, 1),
                        "bound": "L2 reads of the key means: each strip of query blocks reads its head's fp32 key "
                                 "means again (strip_blocks per strip), then selects from registers",
                        "strip_blocks": strip_blocks,
                        "l2_key_read_bytes": l2_key_bytes,
                        "l2_key_read_GB_s": round(l2_key_bytes / (fused_route_ms * 1e-3) / 1e9, 1),
                        "two_kernel_ms": round(route_ms, 5)},
        "total_ms": round(pool_ms + route_ms, 5),
        "total_after_fused_qk_ms": round(qk_pool_ms - ops["qk"]["avg_ms"] + route_ms, 5),
        "total_after_fused_qk_and_route_ms": round(qk_pool_ms - ops["qk"]["avg_ms"] + fused_route_ms, 5),
    }
    route_fused_same = bool(torch.equal(kept_f, kept))
    # The same two routes on means that share a component per head: a seeded
    # N(0, SHARED_OFFSET_STD^2) vector added to every block mean of a head's q
    # and k.  Each query block's scores then crowd into a narrow band of one
    # sign, which the selection has to resolve below the key bits they share.
    g_off = torch.Generator(device=dev).manual_seed(7)
    offset = torch.randn((wl.B, wl.H, 1, wl.Dh), generator=g_off, device=dev) * SHARED_OFFSET_STD
    qp_s.add_(offset)
    kp_s.add_(offset)
    shared_route_ms = timed(route_call)
    shared_fused_ms = timed(lambda: dit.dit_subblock_route(qp_s, kp_s, keep=keep, kept=kept_f, write_scores=False,
                                                           stream=stream))
    shared_same = bool(torch.equal(kept_f, kept))
    subblock["shared_component"] = {"offset_std": SHARED_OFFSET_STD, "route_ms": round(shared_route_ms, 5),
                                    "route_fused_ms": round(shared_fused_ms, 5),
                                    "fused_equals_two_kernel": shared_same}
    route_fused_same = route_fused_same and shared_same
    del qp_s, kp_s, sc, kept, kept0, kept_f, offset

    # A plain streaming copy on the same device: the practical ceiling.
    cbytes = 2 << 30
    src = torch.empty(cbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dit.dit_copy16(src, dst, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        dit.dit_copy16(src, dst, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    # the runtime's device-to-device copy of the same buffers (torch issues hipMemcpyAsync for it)
    for _ in range(3):
        dst.copy_(src)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    memcpy_ms = e0.elapsed_time(e1) / reps
    copy_ceiling = {"bytes": 2 * cbytes, "avg_ms": round(copy_ms, 4),
                    "GB_s": round(2 * cbytes / (copy_ms * 1e-3) / 1e9, 1),
                    "memcpy_dtod_ms": round(memcpy_ms, 4),
                    "memcpy_dtod_GB_s": round(2 * cbytes / (memcpy_ms * 1e-3) / 1e9, 1)}
    del src, dst

    # Access-pattern ceilings: each kernel's traffic with no arithmetic, in that
    # kernel's own launch shape (dit_stream_pattern), on buffers of the same
    # sizes; the chain's outputs are left intact for the oracle check below.
    ceilings = pattern_ceilings(dit, wl, ins, ops, fused_ms, layout_ms, timed, dev)
    if score_pattern_ms:
        ceilings["scores_shape"] = {
            "avg_ms": round(score_pattern_ms, 5), "bytes": scores_bytes,
            "GB_s": round(scores_bytes / (score_pattern_ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100.0 * scores_bytes / (score_pattern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "kernel_over_pattern": round(scores_ms / score_pattern_ms, 4),
            "timing": "each call right after a full route, as the score kernel's"}
    if topk_pattern_ms:
        ceilings["topk_shape"] = {
            "avg_ms": round(topk_pattern_ms, 5), "bytes": topk_bytes,
            "GB_s": round(topk_bytes / (topk_pattern_ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100.0 * topk_bytes / (topk_pattern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "kernel_over_pattern": round(topk_ms / topk_pattern_ms, 4),
            "timing": "each call right after the score tiles have written the matrix, as top-k follows the score "
                      "kernel inside the route"}

    mix_ms = 2 * ops["adaln"]["avg_ms"] + ops["qk"]["avg_ms"] + 2 * ops["residual"]["avg_ms"] + ops["swiglu"]["avg_ms"]
    mix_bytes = 2 * nbytes["adaln"] + nbytes["qk"] + 2 * nbytes["residual"] + nbytes["swiglu"]
    block_mix = {"ops": "2 adaln + qk + 2 residual + swiglu (kernel-time sum)", "ms": round(mix_ms, 4),
                 "GB_s": round(mix_bytes / (mix_ms * 1e-3) / 1e9, 1), "tokens_per_s": round(wl.R / (mix_ms * 1e-3))}

    fused_mix_ms = ops["qk"]["avg_ms"] + 2 * fused_ms + ops["swiglu"]["avg_ms"]
    fused_mix_bytes = nbytes["qk"] + 2 * fused_bytes + nbytes["swiglu"]
    block_mix_fused = {"ops": "qk + 2 fused residual->adaln + swiglu (kernel-time sum; each residual feeds "
                              "the next AdaLN)", "ms": round(fused_mix_ms, 4),
                       "GB_s": round(fused_mix_bytes / (fused_mix_ms * 1e-3) / 1e9, 1),
                       "tokens_per_s": round(wl.R / (fused_mix_ms * 1e-3))}

    # The next-row outputs against the chain's own: the fused residual is the
    # plain residual bit for bit, and the head-major q', k' are the token-major
    # ones transposed (the oracle check below covers the fused z).
    consistency = {
        "fused_x_out_equals_residual": bool(torch.equal(fused_x, out)),
        "fused_pool_head_major_equals_layout_qk": layout_pool_same,
        "fused_route_equals_scores_then_topk": route_fused_same,
        "head_major_equals_token_major": bool(
            torch.equal(qo_hm.permute(0, 2, 1, 3), qo.view(wl.B, wl.N, wl.H, wl.Dh))
            and torch.equal(ko_hm.permute(0, 2, 1, 3), ko.view(wl.B, wl.N, wl.H, wl.Dh))),
    }
    del qo_hm, ko_hm, fused_x

    eager_ms_per_step = ms_per_step
    graph_ok = bool(graph_replay and graph_replay.get("replays_equal_eager"))
    if graph_ok:
        ms_per_step = graph_replay["ms_per_step"]
    value = chain_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timing": ("HIP graph of the step, K replays between two device synchronisations (replays equal the eager "
                   "step bit for bit)" if graph_ok else "K eager steps between two device synchronisations"),
        "eager_ms_per_step": round(eager_ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "fp32",
        "data": "synthetic: seeded N(0,1) bf16 activations, per-sample modulation N(0,0.1), "
                "RMSNorm weights 1+N(0,0.02), inputs resident in HBM",
        "config": {"workload": wl.description, "tokens": wl.R, "batch": wl.B, "latent_grid": list(wl.grid),
                   "extra_tokens": wl.n_extra, "hidden": wl.D, "heads": [wl.H, wl.Dh], "swiglu_width": wl.F,
                   "rope_bands": list(wl.bands), "theta": wl.theta, "eps": wl.eps},
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(wl.R / (ms_per_step * 1e-3)),
        "chain_bytes": chain_bytes,
        "kernel_ms_sum": round(kernel_ms, 4),
        "ops": ops,
        "ops_flushed": flushed,
        "roofline": roofline,
        "copy_ceiling": copy_ceiling,
        "ceilings": ceilings,
        "graph_replay": graph_replay,
        "block_mix": block_mix,
        "next_fused_residual_adaln": fused,
        "next_qk_layout": layout,
        "next_residual_change": change,
        "next_subblock_routing": subblock,
        "block_mix_fused": block_mix_fused,
        "next_consistency": consistency,
        "one_gpu_share_of_8": share,
        "env": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                "device": torch.cuda.get_device_name(dev)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, ins, {"y": y, "out": out, "sw": sw, "qo": qo, "ko": ko,
                                                        "fz": fused_z}, args.cpu_seconds)
    ok = gate_on_parity(result, consistency)
    if not ok:
        print("[bench] FAILED: GPU outputs disagree with the oracle or with each other; value withheld",
              file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)
    return 0 if ok else 3


def gate_on_parity(result: dict, consistency: dict) -> bool:
    """Credit a figure only to kernels whose outputs were checked.

    Sets `parity_checked` (the oracle leg ran) and `parity_ok` (null when unchecked).  When the oracle check
    or a consistency check fails, `value` becomes null (the figure moves to `value_if_parity_held`) and the
    return is False, which main() turns into a non-zero exit status.
    """
    checked = "cpu_baseline" in result
    ok = all(consistency.values()) and (not checked or bool(result["cpu_baseline"]["parity_ok"]))
    result["parity_checked"] = checked
    result["parity_ok"] = ok if checked else None
    if not ok:
        result["value_if_parity_held"] = result["value"]
        result["value"] = None
    return ok


def pattern_ceilings(dit, wl, ins, ops, fused_ms: float, layout_ms: float, timed, dev) -> dict:
    """Each kernel's memory traffic with no arithmetic, in its own launch shape, timed as the kernels are.

    `kernel_over_pattern` is the kernel's average duration over its pattern's: 1.0 means the kernel moves
    its bytes as fast as a stream of the same shape with nothing to compute.
    """
    import torch

    R, D, F, H, Dh = wl.R, wl.D, wl.F, wl.H, wl.Dh
    HD = H * Dh
    swiglu_out = torch.empty((R, F), dtype=torch.bfloat16, device=dev)
    o1 = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty_like(o1)
    sink = torch.empty(16, dtype=torch.uint8, device=dev)
    q, k = ins["q"].reshape(R, HD), ins["k"].reshape(R, HD)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    a, b = ins["res_x"].reshape(R, D), ins["res_y"].reshape(R, D)
    sp = dit.dit_stream_pattern
    cases = {
        # name: (launch, bytes, kernel ms it bounds or None)
        "read": (lambda: sp(dit.DIT_STREAM_READ, R, 4 * F, in0=ins["swiglu_in"], out0=sink), R * 4 * F, None),
        "write": (lambda: sp(dit.DIT_STREAM_WRITE, R, 2 * F, out0=swiglu_out), R * 2 * F, None),
        "swiglu_shape": (lambda: sp(dit.DIT_STREAM_SPLIT_ROWS, R, 2 * F, in0=ins["swiglu_in"], out0=swiglu_out),
                         R * 6 * F, ops["swiglu"]["avg_ms"]),
        "residual_shape": (lambda: sp(dit.DIT_STREAM_TWO_IN, R, 2 * D, in0=a, in1=b, out0=o1), R * 6 * D,
                           ops["residual"]["avg_ms"]),
        "adaln_shape": (lambda: sp(dit.DIT_STREAM_ROW_GROUP, R, 2 * D, in0=ins["x_mod"], out0=o1), R * 4 * D,
                        ops["adaln"]["avg_ms"]),
        "fused_residual_adaln_shape": (
            lambda: sp(dit.DIT_STREAM_ROW_GROUP_2X2, R, 2 * D, in0=a, in1=b, out0=o1, out1=o2), R * 8 * D, fused_ms),
        "qk_token_major_copy": (lambda: (dit.dit_copy16(q, qo), dit.dit_copy16(k, ko)), R * 8 * HD,
                                ops["qk"]["avg_ms"]),
        "qk_head_major_copy": (lambda: (sp(dit.DIT_STREAM_HEAD_MAJOR, R, 2 * HD, in0=q, out0=qo, heads=H),
                                        sp(dit.DIT_STREAM_HEAD_MAJOR, R, 2 * HD, in0=k, out0=ko, heads=H)),
                               R * 8 * HD, layout_ms),
    }
    out = {}
    for name, (fn, nbytes, kernel_ms) in cases.items():
        ms = timed(fn)
        entry = {"avg_ms": round(ms, 5), "bytes": nbytes, "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                 "pct_of_peak": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
        if kernel_ms:
            entry["kernel_over_pattern"] = round(kernel_ms / ms, 4)
        out[name] = entry
    out["note"] = ("qk copies are two launches (q, then k) where the QK kernel is one; the head-major copy reads "
                   "separate q, k and is compared with QK from a fused QKV buffer (next_qk_layout)")
    del swiglu_out, o1, o2, qo, ko
    return out


def cpu_baseline(wl, ins, outs, target_s: float) -> dict:
    """Time the fp64 oracle on evenly spaced tokens of the workload and check the GPU rows against it."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: used only by this leg of the benchmark
    from synthetic_inputs import bits
    from tests.parity_util import worst_ratio

    threads = max(1, min(16, os.cpu_count() or 1))
    R, N, B = wl.R, wl.N, wl.B
    pos_ref = oracle.packed_positions(*wl.grid, wl.n_extra)
    nbytes = op_bytes(wl)
    per_token = (nbytes["adaln"] + nbytes["residual"] + nbytes["swiglu"] + nbytes["qk"]) / R + 12 * N / R

    def chunk_rows(rows):
        idx = torch.as_tensor(rows, device=ins["x_mod"].device)
        host = {
            "x": bits(ins["x_mod"].reshape(R, -1).index_select(0, idx)),
            "rx": bits(ins["res_x"].reshape(R, -1).index_select(0, idx)),
            "ry": bits(ins["res_y"].reshape(R, -1).index_select(0, idx)),
            "sw": bits(ins["swiglu_in"].index_select(0, idx)),
            "q": bits(ins["q"].reshape(R, -1).index_select(0, idx)),
            "k": bits(ins["k"].reshape(R, -1).index_select(0, idx)),
        }
        gpu = {k: outs[k].reshape(R, -1).index_select(0, idx).float().cpu().double().numpy()
               for k in ("y", "out", "sw", "qo", "ko", "fz")}
        return host, gpu

    shift, scale, gate = bits(ins["shift"]), bits(ins["scale"]), bits(ins["gate"])
    wq, wk = bits(ins["wq"]), bits(ins["wk"])

    op_seconds = {"adaln": 0.0, "residual": 0.0, "swiglu": 0.0, "qk": 0.0}

    def run_oracle(rows, host, nthreads=threads, timing=op_seconds):
        """All four ops on the given rows (each row is one token of one sample); per-op oracle time into timing."""
        res = {"y": [], "out": [], "sw": [], "qo": [], "ko": []}
        samples = np.asarray(rows) // N
        tokens = np.asarray(rows) % N
        for b in range(B):
            sel = np.nonzero(samples == b)[0]
            if sel.size == 0:
                continue
            n = sel.size
            t0 = time.perf_counter()
            res["y"].append((sel, oracle.adaln_modulate(host["x"][sel].reshape(1, n, -1), shift[b:b + 1],
                                                        scale[b:b + 1], eps=wl.eps, threads=nthreads).reshape(n, -1)))
            t1 = time.perf_counter()
            res["out"].append((sel, oracle.gated_residual(host["rx"][sel].reshape(1, n, -1),
                                                          host["ry"][sel].reshape(1, n, -1), gate[b:b + 1],
                                                          threads=nthreads).reshape(n, -1)))
            t2 = time.perf_counter()
            qr, kr = oracle.qk_rmsnorm_rope3d(host["q"][sel].reshape(1, n, wl.H, wl.Dh),
                                              host["k"][sel].reshape(1, n, wl.H, wl.Dh), wq, wk,
                                              pos_ref[tokens[sel]], wl.bands, wl.theta, wl.eps, threads=nthreads)
            t3 = time.perf_counter()
            timing["adaln"] += t1 - t0
            timing["residual"] += t2 - t1
            timing["qk"] += t3 - t2
            res["qo"].append((sel, qr.reshape(n, -1)))
            res["ko"].append((sel, kr.reshape(n, -1)))
        t0 = time.perf_counter()
        res["sw"].append((np.arange(len(rows)), oracle.swiglu(host["sw"], threads=nthreads)))
        timing["swiglu"] += time.perf_counter() - t0
        return res

    fused_seconds = [0.0]

    def fused_check(rows, host, gpu):
        """Fused residual -> AdaLN z on the same rows (timed apart from the four ops' oracle work)."""
        samples = np.asarray(rows) // N
        ratio = 0.0
        for b in range(B):
            sel = np.nonzero(samples == b)[0]
            if sel.size == 0:
                continue
            n = sel.size
            t0 = time.perf_counter()
            _, z = oracle.gated_residual_adaln(host["rx"][sel].reshape(1, n, -1), host["ry"][sel].reshape(1, n, -1),
                                               gate[b:b + 1], shift[b:b + 1], scale[b:b + 1], eps=wl.eps,
                                               threads=threads)
            fused_seconds[0] += time.perf_counter() - t0
            ratio = max(ratio, worst_ratio(gpu["fz"][sel], z.reshape(n, -1)))
        return ratio

    def check(res, gpu):
        """Largest |gpu - oracle| / bound over the chunk (<= 1 passes)."""
        ratio = 0.0
        for key, parts in res.items():
            for sel, ref in parts:
                ratio = max(ratio, worst_ratio(gpu[key][sel], ref))
        return ratio

    # Seeded random tokens, in chunks, until about target_s seconds of oracle time.
    order = np.random.default_rng(0).permutation(R)
    chunk = 1024
    elapsed, done, max_ratio = 0.0, 0, 0.0
    for c0 in range(0, R, chunk):
        rows = np.sort(order[c0:c0 + chunk]).tolist()
        host, gpu = chunk_rows(rows)
        t = time.perf_counter()
        res = run_oracle(rows, host)
        elapsed += time.perf_counter() - t
        done += len(rows)
        max_ratio = max(max_ratio, check(res, gpu), fused_check(rows, host, gpu))
        if elapsed >= target_s:
            break
    tokens_per_s = done / elapsed
    # the same oracle on one thread, over one chunk of the same tokens
    rows = np.sort(order[:chunk]).tolist()
    host, _ = chunk_rows(rows)
    single = {k: 0.0 for k in op_seconds}
    t = time.perf_counter()
    run_oracle(rows, host, nthreads=1, timing=single)
    single_tokens_per_s = len(rows) / (time.perf_counter() - t)
    next_rows = next_row_oracle_rates(wl, ins, pos_ref, done, fused_seconds[0], threads)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(tokens_per_s * per_token / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(tokens_per_s, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {R} tokens (seeded uniform random rows) of the {wl.name} workload; all four ops "
                  f"in the fp64 C oracle on {threads} host threads; {elapsed:.1f} s of oracle time (the same "
                  f"tokens' GPU outputs, and the fused residual->AdaLN z, are checked against it)",
        "tokens_per_s_per_op": {k: round(done / v, 1) for k, v in op_seconds.items() if v > 0},
        "single_thread_tokens_per_s": round(single_tokens_per_s, 1),
        "single_thread_tokens_per_s_per_op": {k: round(len(rows) / v, 1) for k, v in single.items() if v > 0},
        "host_cpu": cpu_model,
        "host_logical_cpus": os.cpu_count(),
        "parity_rows_checked": done,
        "parity_max_err_over_bound": round(max_ratio, 4),
        "parity_ok": bool(max_ratio <= 1.0),
        "next_rows": next_rows,
    }


def next_row_oracle_rates(wl, ins, pos_ref, fused_tokens: int, fused_seconds: float, threads: int) -> dict:
    """The oracle's rate on each next row, from a bounded sample of the workload's own inputs.

    Fused residual -> AdaLN: the calls made to check the GPU's z above (``threads`` threads).  The
    rest run single-threaded (the oracle has no threaded form of them) on a sample: 2048 tokens
    for QK from a fused buffer to head-major, 16,384 tokens for the residual-change statistic and
    for the block means (256 blocks), 256 query blocks of one head against all key blocks for the
    scores, and the kept blocks of those 256 rows.  Inputs are the workload's seeded tensors (the
    means are seeded normal values); nothing is taken from the GPU's outputs.
    """
    import numpy as np

    import oracle
    from synthetic_inputs import bits

    R, N, D, H, Dh = wl.R, wl.N, wl.D, wl.H, wl.Dh
    HD = H * Dh
    out = {}
    if fused_seconds > 0:
        rate = fused_tokens / fused_seconds
        out["fused_residual_adaln"] = {"tokens_per_s": round(rate, 1),
                                       "GB_s": round(rate * 8 * D / 1e9, 4), "threads": threads,
                                       "sample": f"{fused_tokens} tokens"}
    n = min(2048, N)
    q = bits(ins["q"].reshape(R, HD)[:n])
    k = bits(ins["k"].reshape(R, HD)[:n])
    qk = np.ascontiguousarray(np.concatenate([q, k], axis=1)).reshape(-1)
    wq, wk = bits(ins["wq"]), bits(ins["wk"])
    t = time.perf_counter()
    oracle.qk_rmsnorm_rope3d_layout(qk, qk[HD:], wq, wk, pos_ref[:n], wl.bands, 1, n, H, Dh, 2 * HD, 1,
                                    wl.theta, wl.eps)
    dt = time.perf_counter() - t
    out["qk_layout"] = {"tokens_per_s": round(n / dt, 1), "GB_s": round(n * (8 * HD + 12) / dt / 1e9, 4),
                        "threads": 1, "sample": f"{n} tokens, fused q|k buffer in, head-major out"}
    n = min(16384, N)
    r = bits(ins["res_x"].reshape(R, D)[:n]).reshape(1, n, D)
    rc = bits(ins["res_y"].reshape(R, D)[:n]).reshape(1, n, D)
    t = time.perf_counter()
    oracle.residual_change(r, rc)
    dt = time.perf_counter() - t
    out["residual_change"] = {"tokens_per_s": round(n / dt, 1), "GB_s": round(n * 4 * D / dt / 1e9, 4),
                              "threads": 1, "sample": f"{n} tokens"}
    t = time.perf_counter()
    oracle.subblock_pool(bits(ins["q"].reshape(R, HD)[:n]).reshape(1, n, H, Dh))
    dt = time.perf_counter() - t
    out["subblock_pool"] = {"tokens_per_s": round(n / dt, 1), "GB_s": round(n * 2 * HD / dt / 1e9, 4),
                            "threads": 1, "sample": f"{n} tokens ({-(-n // 64)} blocks) of q"}
    nb = -(-N // 64)
    nq = min(256, nb)
    g = np.random.default_rng(0)
    qp = g.standard_normal((1, 1, nq, Dh)) * 0.125
    kp = g.standard_normal((1, 1, nb, Dh)) * 0.125
    t = time.perf_counter()
    s = oracle.subblock_scores(qp, kp)
    dt = time.perf_counter() - t
    out["subblock_scores"] = {"scores_per_s": round(nq * nb / dt, 1), "GFLOP_s": round(2 * nq * nb * Dh / dt / 1e9, 4),
                              "threads": 1, "sample": f"{nq} query blocks x {nb} key blocks, Dh {Dh}"}
    keep = oracle.subblock_keep(nb, 0.75)
    t = time.perf_counter()
    oracle.subblock_topk(s, keep)
    dt = time.perf_counter() - t
    out["subblock_topk"] = {"rows_per_s": round(nq / dt, 1), "GB_s": round(nq * (4 * nb + 4 * keep) / dt / 1e9, 4),
                            "threads": 1, "sample": f"{nq} rows of {nb} scores, keep {keep}"}
    return out

# --------------------------------------------------------------------------- rocprofv3 summaries

# Kernel name pattern -> op, most specific first (names carry template arguments).
KERNEL_OPS = (
    (r"pattern_read_kernel", "p_read"),
    (r"pattern_write_kernel", "p_write"),
    (r"pattern_split_rows_kernel", "p_swiglu"),
    (r"pattern_two_in_kernel", "p_residual"),
    (r"pattern_row_group_kernel<false,", "p_adaln"),
    (r"pattern_row_group_kernel<true,", "p_residual_adaln"),
    (r"pattern_head_major_kernel", "p_head_major"),
    (r"pattern_score_tiles_kernel", "p_score_tiles"),
    (r"pattern_topk_rows_kernel", "p_topk_rows"),
    (r"gated_residual_adaln_kernel", "residual_adaln"),
    (r"adaln_modulate_kernel", "adaln"),
    (r"gated_residual_kernel", "residual"),
    (r"swiglu_kernel", "swiglu"),
    (r"qk_rmsnorm_rope3d_pool_kernel<\d+, true>", "qk_pool_layout"),
    (r"qk_rmsnorm_rope3d_pool_kernel", "qk_pool"),
    (r"qk_rmsnorm_rope3d_head_major_kernel", "qk_layout"),
    (r"qk_rmsnorm_rope3d_kernel", "qk"),
    (r"residual_change_partial_kernel", "change"),
    (r"residual_change_final_kernel", "change_final"),
    (r"subblock_pool_token_major_kernel", "pool"),
    (r"subblock_pool_head_major_kernel", "pool_hm"),
    (r"subblock_scores_persistent_kernel", "scores"),
    (r"subblock_scores_kernel", "scores"),
    (r"subblock_topk_kernel", "topk"),
    (r"subblock_route_fused_kernel", "route_fused"),
    (r"packed_positions_kernel", "positions"),
    (r"copy16_kernel", "copy"),
)

PROFILE_COMMANDS = """\
cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_trace -o trace -- \\
    python $REPO/bench.py --workload {wl} --steps 10 --warmup 2 --no-cpu-baseline
rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/prof_fetch -o fetch -- \\
    python $REPO/bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline --copy-calibration
rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/prof_write -o write -- \\
    python $REPO/bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline --copy-calibration
cd $REPO && python bench.py --workload {wl} --summarize-rocprof $OUT/prof_trace $OUT/prof_fetch $OUT/prof_write"""

SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_VMEM_RD",
               "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")

SQ_COMMANDS = """\
cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_trace -o trace -- \\
    python $REPO/bench.py --workload {wl} --steps 10 --warmup 2 --no-cpu-baseline
rocprofv3 --pmc {counters} --output-format csv -d $OUT/prof_sq -o sq -- \\
    python $REPO/bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline --no-graph
cd $REPO && python bench.py --workload {wl} --summarize-sq $OUT/prof_trace $OUT/prof_sq"""

# wave64 VALU instructions the chip can issue per second: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64
# instruction per SIMD every 4 cycles (16 lanes wide)
VALU_ISSUE_PEAK = 256 * 4 * 2.4e9 / 4
MFMA_16X16X16_FLOPS = 2 * 16 * 16 * 16


def _kernel_op(name: str):
    for pattern, op in KERNEL_OPS:
        if re.search(pattern, name):
            return op
    return None


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        with open(f, newline="", encoding="utf-8") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_rocprof(trace_dir: str, fetch_dir: str, write_dir: str, workload: str = "full5s") -> int:
    """Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    Counter calibration: every dit_copy16 dispatch in the counter runs moves a
    known number of bytes (one 16-byte vector per work-item, read once and
    written once), so FETCH_SIZE and WRITE_SIZE are each scaled by
    known bytes / counter bytes summed over those dispatches.
    """
    import synthetic_inputs as si

    wl = si.WORKLOADS[workload]
    nbytes = op_bytes(wl, next_rows=True)
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    commands = PROFILE_COMMANDS.format(wl=workload)

    # Per-dispatch durations; each op keeps only its full-size launches (the
    # largest grid it ran with): the benchmark also runs the chain's kernels on
    # one GPU's share of the tokens, and those smaller launches are left out.
    by_grid = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        op = _kernel_op(r["Kernel_Name"])
        if not op:
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        m = re.search(r"::(\w+(?:<[^()]*>)?)\(", r["Kernel_Name"])
        entry = by_grid.setdefault(op, {}).setdefault(grid, {"name": m.group(1) if m else r["Kernel_Name"][:60],
                                                             "us": []})
        entry["us"].append(us)
    stats = {}
    for op, grids in by_grid.items():
        full = grids[max(grids)]
        t = full["us"]
        stats[op] = {"name": full["name"], "calls": len(t), "avg_us": sum(t) / len(t), "min_us": min(t),
                     "max_us": max(t), "smaller_launches": sum(len(g["us"]) for g in grids.values()) - len(t)}

    counters = {"FETCH_SIZE": {}, "WRITE_SIZE": {}}
    calib = {"FETCH_SIZE": [0.0, 0.0], "WRITE_SIZE": [0.0, 0.0]}  # known bytes, counter bytes
    for directory in (fetch_dir, write_dir):
        for r in _csv_rows(directory, "counter_collection.csv"):
            op = _kernel_op(r["Kernel_Name"])
            name = r["Counter_Name"]
            if op is None or name not in counters:
                continue
            kib = float(r["Counter_Value"])
            if op == "copy":
                calib[name][0] += 16.0 * int(r["Grid_Size"])
                calib[name][1] += kib * 1024.0
            else:
                counters[name].setdefault(op, {}).setdefault(int(r["Grid_Size"]), []).append(kib)
    for name in counters:  # full-size launches only, as for the durations
        counters[name] = {op: grids[max(grids)] for op, grids in counters[name].items()}
    factor = {k: (v[0] / v[1] if v[1] else None) for k, v in calib.items()}

    lines = [f"# Kernel durations: {wl.description}", "",
             "rocprofv3 kernel trace of the benchmark (10 timed + 2 warm-up steps of the chain, then the "
             "flushed per-op calls, the same counts of each next-row kernel and the copy-ceiling copies). "
             "Each kernel's figures cover its full-size launches only; `smaller` counts the launches on one "
             "GPU's share of the tokens, left out. Bytes are the compulsory (algorithmic) HBM bytes of one "
             "launch; GB/s uses the average duration.", "", "Commands (REPO = the repository root, OUT = an output directory for the raw rocprofv3 files):", "", "```",
             commands, "```", "",
             "| kernel | calls | smaller | avg us | min us | max us | algorithmic bytes | GB/s at avg | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for op in (*OPS, *NEXT_OPS, "copy"):
        if op not in stats:
            continue
        st = stats[op]
        b = nbytes.get(op)
        gbs = f"{b / (st['avg_us'] * 1e-6) / 1e9:.1f}" if b else "-"
        pct = f"{100 * b / (st['avg_us'] * 1e-6) / 1e9 / HBM_PEAK_GBPS:.1f}" if b else "-"
        lines.append(f"| `{st['name']}` | {st['calls']} | {st['smaller_launches']} | {st['avg_us']:.2f} "
                     f"| {st['min_us']:.2f} | {st['max_us']:.2f} | {b if b else '-'} | {gbs} | {pct} |")
    with open(os.path.join(out_dir, f"kernels_{workload}_trace.md"), "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")

    for op in (*OPS[1:], *NEXT_OPS):
        if op not in counters["FETCH_SIZE"] or op not in counters["WRITE_SIZE"] or op not in nbytes:
            continue
        f_kib = sum(counters["FETCH_SIZE"][op]) / len(counters["FETCH_SIZE"][op])
        w_kib = sum(counters["WRITE_SIZE"][op]) / len(counters["WRITE_SIZE"][op])
        hbm = f_kib * 1024 * factor["FETCH_SIZE"] + w_kib * 1024 * factor["WRITE_SIZE"]
        body = [
            f"# HBM traffic of `{op}` on {wl.description}", "",
            "rocprofv3 counters, one counter per run (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch averaged "
            "over the timed and warm-up launches of the run; each scaled by the same counter's reading for "
            "dit_copy16 calls of known size in the same run.", "",
            "Commands (REPO = the repository root, OUT = an output directory for the raw rocprofv3 files):", "", "```", commands, "```", "",
            f"- dispatches: {len(counters['FETCH_SIZE'][op])} (FETCH_SIZE run), "
            f"{len(counters['WRITE_SIZE'][op])} (WRITE_SIZE run)",
            f"- FETCH_SIZE per launch: {f_kib:.1f} KiB (raw)",
            f"- WRITE_SIZE per launch: {w_kib:.1f} KiB (raw)",
            f"- copy calibration factor FETCH_SIZE: {factor['FETCH_SIZE']:.4f} "
            f"({calib['FETCH_SIZE'][0]:.0f} known bytes read / {calib['FETCH_SIZE'][1]:.0f} counted)",
            f"- copy calibration factor WRITE_SIZE: {factor['WRITE_SIZE']:.4f} "
            f"({calib['WRITE_SIZE'][0]:.0f} known bytes written / {calib['WRITE_SIZE'][1]:.0f} counted)",
            f"- HBM bytes per launch (calibrated): {hbm:.6e}",
            f"- algorithmic bytes per launch: {nbytes[op]:.6e}",
            f"- calibrated / algorithmic: {hbm / nbytes[op]:.4f}",
            f"- kernel source sha256: {source_digest(op)}",
        ]
        if op in stats:
            body.append(f"- kernel-trace average duration: {stats[op]['avg_us']:.2f} us "
                        f"({nbytes[op] / (stats[op]['avg_us'] * 1e-6) / 1e9:.1f} GB/s algorithmic)")
        with open(os.path.join(out_dir, f"{op}_{workload}_counters.md"), "w", encoding="utf-8") as fh:
            fh.write("\n".join(body) + "\n")
    write_ceilings_summary(stats, nbytes, wl, workload, commands, out_dir)
    print(f"wrote profiles/ summaries for {workload}; calibration factors {factor}")
    return 0


# pattern -> (kernel it bounds, launches of the pattern per kernel launch)
PATTERN_BOUNDS = {"p_read": (None, 1), "p_write": (None, 1), "p_swiglu": ("swiglu", 1),
                  "p_residual": ("residual", 1), "p_adaln": ("adaln", 1), "p_residual_adaln": ("residual_adaln", 1),
                  "p_head_major": ("qk_layout", 2), "p_score_tiles": ("scores", 1),
                  "p_topk_rows": ("topk", 1)}


def write_ceilings_summary(stats: dict, nbytes: dict, wl, workload: str, commands: str, out_dir: str):
    """profiles/ceilings_<workload>.md: each access-pattern stream against the kernel whose traffic it carries."""
    lines = [f"# Access-pattern ceilings: {wl.description}", "",
             "Each stream (dit_stream_pattern) carries one kernel's loads and stores with no arithmetic, in that "
             "kernel's launch shape; durations from the same rocprofv3 kernel trace as the kernels "
             "(kernels_<workload>_trace.md), full-size launches only. `kernel / pattern` is the kernel's average "
             "duration over its pattern's (the head-major copy moves one of q and k per launch, so QK with "
             "head-major output is set against two of its launches; that kernel also reads q, k out of a fused "
             "QKV buffer). The SubBlock patterns run where their kernels run: the score tiles right after a full "
             "route, the top-k rows right after the score tiles have written the matrix.", "",
             "Commands (REPO = the repository root, OUT = an output directory for the raw rocprofv3 files):", "",
             "```", commands, "```", "",
             "| pattern | kernel | calls | avg us | bytes | GB/s | % of 8 TB/s | kernel avg us | kernel / pattern |",
             "|---|---|---|---|---|---|---|---|---|"]
    for pat, (kernel, per) in PATTERN_BOUNDS.items():
        if pat not in stats:
            continue
        st = stats[pat]
        b = nbytes[pat]
        gbs = b / (st["avg_us"] * 1e-6) / 1e9
        k_us = stats[kernel]["avg_us"] if kernel in stats else None
        ratio = f"{k_us / (per * st['avg_us']):.3f}" if k_us else "-"
        lines.append(f"| `{st['name']}` | {kernel or '-'} | {st['calls']} | {st['avg_us']:.2f} | {b} | {gbs:.1f} "
                     f"| {100 * gbs / HBM_PEAK_GBPS:.1f} | {f'{k_us:.2f}' if k_us else '-'} | {ratio} |")
    if "copy" in stats:
        cb = 2 * (2 << 30)
        lines += ["", f"- `copy16_kernel` (2 GiB read + 2 GiB written): {stats['copy']['avg_us']:.2f} us, "
                      f"{cb / (stats['copy']['avg_us'] * 1e-6) / 1e9:.1f} GB/s"]
    with open(os.path.join(out_dir, f"ceilings_{workload}.md"), "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")


def _full_size_durations(trace_dir: str) -> dict:
    """op -> average duration (us) of its full-size launches in a kernel-trace run."""
    by_grid = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        op = _kernel_op(r["Kernel_Name"])
        if op:
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            by_grid.setdefault(op, {}).setdefault(grid, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {op: sum(g[max(g)]) / len(g[max(g)]) for op, g in by_grid.items()}


def summarize_sq(trace_dir: str, sq_dir: str, workload: str = "full5s", out_dir: str | None = None) -> int:
    """Shader-sequencer counters per kernel (full-size launches, averaged per dispatch) as a profiles/ summary.

    VALU issue is SQ_INSTS_VALU over the kernel-trace average duration, against VALU_ISSUE_PEAK; the
    LDS wait share is SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES (both in quad-cycles); MFMA work is
    SQ_INSTS_MFMA x 8192 flops (v_mfma_f32_16x16x16_bf16) against the algorithmic flops of the scores.
    """
    import synthetic_inputs as si

    wl = si.WORKLOADS[workload]
    avg_us = _full_size_durations(trace_dir)
    per = {}  # op -> grid -> dispatch id -> counter -> value
    for r in _csv_rows(sq_dir, "counter_collection.csv"):
        op = _kernel_op(r["Kernel_Name"])
        if op is None or r["Counter_Name"] not in SQ_COUNTERS:
            continue
        d = per.setdefault(op, {}).setdefault(int(r["Grid_Size"]), {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    nb = -(-wl.N // 64)
    score_flops = 2.0 * wl.B * wl.H * nb * nb * wl.Dh
    lines = [f"# Shader-sequencer counters per kernel: {wl.description}", "",
             "One rocprofv3 counter run of the benchmark with the eight SQ counters below, next to the "
             "kernel-trace run that gives each kernel's average duration. Full-size launches only, averaged "
             "per dispatch. Per-wave figures divide by SQ_WAVES. VALU issue = SQ_INSTS_VALU per second of "
             "the traced average duration, as a share of the chip's wave64 issue limit (256 CUs x 4 SIMDs x "
             f"2.4 GHz / 4 cycles = {VALU_ISSUE_PEAK:.3e} per second). LDS wait = SQ_WAIT_INST_LDS / "
             "SQ_WAVE_CYCLES (both in quad-cycles). MFMA flops = SQ_INSTS_MFMA x 8192.", "",
             f"Counters: {' '.join(SQ_COUNTERS)}", "",
             "Commands (REPO = the repository root, OUT = an output directory for the raw rocprofv3 files):", "",
             "```", SQ_COMMANDS.format(wl=workload, counters=" ".join(SQ_COUNTERS)), "```", "",
             "| kernel | dispatches | waves | VALU / wave | SALU / wave | LDS / wave | MFMA / wave | "
             "VMEM reads / wave | LDS wait % | avg us | VALU issue % of limit |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    extra = []
    for op in (*OPS, *NEXT_OPS, "copy"):
        if op not in per:
            continue
        grids = per[op]
        ds = list(grids[max(grids)].values())
        mean = {c: sum(d.get(c, 0.0) for d in ds) / len(ds) for c in SQ_COUNTERS}
        waves = mean["SQ_WAVES"]
        if waves <= 0:
            continue
        pw = {c: mean[c] / waves for c in SQ_COUNTERS}
        wait = 100.0 * mean["SQ_WAIT_INST_LDS"] / mean["SQ_WAVE_CYCLES"] if mean["SQ_WAVE_CYCLES"] else 0.0
        us = avg_us.get(op)
        issue = f"{100.0 * mean['SQ_INSTS_VALU'] / (us * 1e-6) / VALU_ISSUE_PEAK:.1f}" if us else "-"
        us_s = f"{us:.2f}" if us else "-"
        lines.append(f"| {op} | {len(ds)} | {waves:.0f} | {pw['SQ_INSTS_VALU']:.1f} | {pw['SQ_INSTS_SALU']:.1f} "
                     f"| {pw['SQ_INSTS_LDS']:.1f} | {pw['SQ_INSTS_MFMA']:.1f} | {pw['SQ_INSTS_VMEM_RD']:.1f} "
                     f"| {wait:.1f} | {us_s} | {issue} |")
        if op == "scores" and mean["SQ_INSTS_MFMA"] > 0:
            mf = mean["SQ_INSTS_MFMA"] * MFMA_16X16X16_FLOPS
            extra.append(f"- scores: MFMA flops per launch {mf:.4e} against {score_flops:.4e} algorithmic "
                         f"({mf / score_flops:.3f}x: tiles padded to 128 blocks)"
                         + (f"; {mf / (us * 1e-6) / 1e12:.1f} TFLOP/s issued at the traced average" if us else ""))
    sources = {}
    for op in per:
        if op in KERNEL_SOURCES:
            sources.setdefault(KERNEL_SOURCES[op], source_digest(op))
    lines += [""] + extra + [f"- kernel source sha256 ({name} and device_common.hpp): {digest}"
                             for name, digest in sorted(sources.items())]
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"kernels_{workload}_sq_counters.md")
    with open(out, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}")
    return 0


STALL_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_INST_LEVEL_VMEM", "SQ_INSTS_VMEM", "SQ_INSTS_SMEM")

STALL_COMMANDS = """\
cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_trace -o trace -- \\
    python $REPO/bench.py --workload {wl} --steps 10 --warmup 2 --no-cpu-baseline
rocprofv3 --pmc {counters} --output-format csv -d $OUT/prof_stall -o stall -- \\
    python $REPO/bench.py --workload {wl} --steps 2 --warmup 1 --no-cpu-baseline --no-graph
cd $REPO && python bench.py --workload {wl} --summarize-stalls $OUT/prof_trace $OUT/prof_stall"""


def summarize_stalls(trace_dir: str, stall_dir: str, workload: str = "full5s", out_dir: str | None = None) -> int:
    """Where each kernel's waves spend their time (full-size launches, averaged per dispatch).

    SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_VALU count quad-cycles summed over
    waves: their ratios are shares of wave residency spent waiting on a dependency (a memory counter
    or a barrier), waiting to be issued, and issuing VALU work.  SQ_INST_LEVEL_VMEM accumulates the
    vector-memory instructions in flight every cycle, so over SQ_INSTS_VMEM it is their average latency.
    """
    import synthetic_inputs as si

    wl = si.WORKLOADS[workload]
    avg_us = _full_size_durations(trace_dir)
    per = {}
    for r in _csv_rows(stall_dir, "counter_collection.csv"):
        op = _kernel_op(r["Kernel_Name"])
        if op is None or r["Counter_Name"] not in STALL_COUNTERS:
            continue
        d = per.setdefault(op, {}).setdefault(int(r["Grid_Size"]), {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = [f"# Where the waves' time goes: {wl.description}", "",
             "One rocprofv3 counter run of the benchmark with the eight SQ counters below, next to the "
             "kernel-trace run that gives each kernel's average duration. Full-size launches only, averaged "
             "per dispatch. Shares are of SQ_WAVE_CYCLES (wave residency, quad-cycles): `waiting` = "
             "SQ_WAIT_ANY (a wave held by a dependency: s_waitcnt on memory or LDS, or a barrier), `issue "
             "wait` = SQ_WAIT_INST_ANY (ready but not issued), `VALU` = SQ_ACTIVE_INST_VALU. VMEM latency = "
             "SQ_INST_LEVEL_VMEM / SQ_INSTS_VMEM (cycles a vector-memory instruction is in flight, on "
             "average). Wave life = 4 x SQ_WAVE_CYCLES / SQ_WAVES cycles.", "",
             f"Counters: {' '.join(STALL_COUNTERS)}", "",
             "Commands (REPO = the repository root, OUT = an output directory for the raw rocprofv3 files):", "",
             "```", STALL_COMMANDS.format(wl=workload, counters=" ".join(STALL_COUNTERS)), "```", "",
             "| kernel | waves | wave life (cycles) | waiting % | issue wait % | VALU % | VMEM / wave | "
             "VMEM latency (cycles) | SMEM / wave | avg us |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for op in (*OPS, *NEXT_OPS, *PATTERN_BOUNDS, "copy"):
        if op not in per:
            continue
        grids = per[op]
        ds = list(grids[max(grids)].values())
        mean = {c: sum(d.get(c, 0.0) for d in ds) / len(ds) for c in STALL_COUNTERS}
        waves, cyc = mean["SQ_WAVES"], mean["SQ_WAVE_CYCLES"]
        if waves <= 0 or cyc <= 0:
            continue
        lat = mean["SQ_INST_LEVEL_VMEM"] / mean["SQ_INSTS_VMEM"] if mean["SQ_INSTS_VMEM"] else 0.0
        us = avg_us.get(op)
        lines.append(f"| {op} | {waves:.0f} | {4 * cyc / waves:.0f} | {100 * mean['SQ_WAIT_ANY'] / cyc:.1f} "
                     f"| {100 * mean['SQ_WAIT_INST_ANY'] / cyc:.1f} | {100 * mean['SQ_ACTIVE_INST_VALU'] / cyc:.1f} "
                     f"| {mean['SQ_INSTS_VMEM'] / waves:.1f} | {lat:.0f} | {mean['SQ_INSTS_SMEM'] / waves:.1f} "
                     f"| {f'{us:.2f}' if us else '-'} |")
    sources = {}
    for op in per:
        if op in KERNEL_SOURCES:
            sources.setdefault(KERNEL_SOURCES[op], source_digest(op))
    lines += [""] + [f"- kernel source sha256 ({name} and device_common.hpp): {digest}"
                     for name, digest in sorted(sources.items())]
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"kernels_{workload}_stalls.md")
    with open(out, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
