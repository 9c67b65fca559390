#!/usr/bin/env python3
"""Benchmark of the fused DiT non-GEMM operator chain on one MI355X.

A step is one pass of the whole chain over one batch of synthetic tokens
already resident in HBM: packed positions, AdaLN modulate, gated residual,
SwiGLU and QK RMSNorm + 3D RoPE, each a kernel of libdit_ops.so launched on
torch's current stream.  After W untimed steps, K steps are timed between two
device synchronisations (wall clock), with HIP events around every kernel of
every timed step on the launch stream.

The printed JSON line reports:
  value          whole-chain algorithmic HBM bytes / step time (GB/s)
  tokens_per_s   tokens / step time
  ops            per-kernel average duration, bytes and GB/s from the events
  roofline       the dominant kernel against the 8 TB/s HBM peak; `traffic`
                 is the counter-measured HBM bytes per launch from the
                 committed counter summary when it was taken on the current
                 kernel source, else null
  copy_ceiling   a plain 16-byte-vector copy on the same device
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
    "copy": "copy.hip",
}
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "{op}_{workload}_counters.md")


def op_bytes(wl) -> dict:
    """Compulsory HBM bytes of one launch of each op on workload ``wl``."""
    B, N, R, D, F, H, Dh = wl.B, wl.N, wl.R, wl.D, wl.F, wl.H, wl.Dh
    return {
        "positions": 12 * N,                                   # write (t, h, w) int32
        "adaln": 2 * R * D * 2 + 2 * B * D * 2,                # x in, y out, shift + scale
        "residual": 3 * R * D * 2 + B * D * 2,                 # x, y in, out, gate
        "swiglu": R * 2 * F * 2 + R * F * 2,                   # [a|b] in, out
        "qk": 4 * R * H * Dh * 2 + 12 * N + 2 * Dh * 2,        # q, k in, q', k' out, pos, wq, wk
    }


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
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one 1 GiB dit_copy16 per timed step's warm-up (counter calibration runs)")
    return p.parse_args(argv)


def main(argv=None) -> int:
    args = parse_args(argv)
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

    def launch(op):
        if op == "positions":
            dit.dit_packed_positions(*wl.grid, wl.n_extra, pos=pos, stream=stream)
        elif op == "adaln":
            dit.dit_adaln_modulate(ins["x_mod"], ins["shift"], ins["scale"], y=y, eps=wl.eps, stream=stream)
        elif op == "residual":
            dit.dit_gated_residual(ins["res_x"], ins["res_y"], ins["gate"], out=out, stream=stream)
        elif op == "swiglu":
            dit.dit_swiglu(ins["swiglu_in"], out=sw, stream=stream)
        else:
            dit.dit_qk_rmsnorm_rope3d(ins["q"], ins["k"], ins["wq"], ins["wk"], pos, wl.bands, q_out=qo, k_out=ko,
                                      theta=wl.theta, eps=wl.eps, stream=stream)

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
    copy_ceiling = {"bytes": 2 * cbytes, "avg_ms": round(copy_ms, 4),
                    "GB_s": round(2 * cbytes / (copy_ms * 1e-3) / 1e9, 1)}
    del src, dst

    mix_ms = 2 * ops["adaln"]["avg_ms"] + ops["qk"]["avg_ms"] + 2 * ops["residual"]["avg_ms"] + ops["swiglu"]["avg_ms"]
    mix_bytes = 2 * nbytes["adaln"] + nbytes["qk"] + 2 * nbytes["residual"] + nbytes["swiglu"]
    block_mix = {"ops": "2 adaln + qk + 2 residual + swiglu (kernel-time sum)", "ms": round(mix_ms, 4),
                 "GB_s": round(mix_bytes / (mix_ms * 1e-3) / 1e9, 1), "tokens_per_s": round(wl.R / (mix_ms * 1e-3))}

    value = chain_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
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
        "roofline": roofline,
        "copy_ceiling": copy_ceiling,
        "block_mix": block_mix,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, ins, {"y": y, "out": out, "sw": sw, "qo": qo, "ko": ko},
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline(wl, ins, outs, target_s: float) -> dict:
    """Time the fp64 oracle on evenly spaced tokens of the workload and check the GPU rows against it."""
    import numpy as np
    import torch

    import oracle  # test infrastructure: used only by this leg of the benchmark
    from synthetic_inputs import bits
    from tests.parity_util import worst

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
               for k in ("y", "out", "sw", "qo", "ko")}
        return host, gpu

    shift, scale, gate = bits(ins["shift"]), bits(ins["scale"]), bits(ins["gate"])
    wq, wk = bits(ins["wq"]), bits(ins["wk"])

    def run_oracle(rows, host):
        """All four ops on the given rows (each row is one token of one sample)."""
        res = {"y": [], "out": [], "sw": [], "qo": [], "ko": []}
        samples = np.asarray(rows) // N
        tokens = np.asarray(rows) % N
        for b in range(B):
            sel = np.nonzero(samples == b)[0]
            if sel.size == 0:
                continue
            n = sel.size
            res["y"].append((sel, oracle.adaln_modulate(host["x"][sel].reshape(1, n, -1), shift[b:b + 1],
                                                        scale[b:b + 1], eps=wl.eps, threads=threads).reshape(n, -1)))
            res["out"].append((sel, oracle.gated_residual(host["rx"][sel].reshape(1, n, -1),
                                                          host["ry"][sel].reshape(1, n, -1), gate[b:b + 1],
                                                          threads=threads).reshape(n, -1)))
            qr, kr = oracle.qk_rmsnorm_rope3d(host["q"][sel].reshape(1, n, wl.H, wl.Dh),
                                              host["k"][sel].reshape(1, n, wl.H, wl.Dh), wq, wk,
                                              pos_ref[tokens[sel]], wl.bands, wl.theta, wl.eps, threads=threads)
            res["qo"].append((sel, qr.reshape(n, -1)))
            res["ko"].append((sel, kr.reshape(n, -1)))
        res["sw"].append((np.arange(len(rows)), oracle.swiglu(host["sw"], threads=threads)))
        return res

    def check(res, gpu):
        ex = -np.inf
        for key, parts in res.items():
            for sel, ref in parts:
                ex = max(ex, worst(gpu[key][sel], ref)[0])
        return ex

    # Calibrate on one small chunk, then size the sample for about target_s seconds.
    chunk = 64
    rows_all = np.linspace(0, R - 1, num=min(R, 1 << 20)).astype(np.int64)
    probe = rows_all[:: max(1, len(rows_all) // chunk)][:chunk].tolist()
    host, gpu = chunk_rows(probe)
    t = time.perf_counter()
    res = run_oracle(probe, host)
    per_row = (time.perf_counter() - t) / len(probe)
    max_excess = check(res, gpu)
    total = min(R, max(chunk, int(target_s / max(per_row, 1e-9))))
    sample = np.unique(np.linspace(0, R - 1, num=total).astype(np.int64))
    elapsed, done = 0.0, 0
    for c0 in range(0, len(sample), 512):
        rows = sample[c0:c0 + 512].tolist()
        host, gpu = chunk_rows(rows)
        t = time.perf_counter()
        res = run_oracle(rows, host)
        elapsed += time.perf_counter() - t
        done += len(rows)
        max_excess = max(max_excess, check(res, gpu))
    tokens_per_s = done / elapsed
    return {
        "value": round(tokens_per_s * per_token / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(tokens_per_s, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {R} tokens, evenly spaced over the sequence, of the {wl.name} workload; all four "
                  f"ops in the fp64 C oracle on {threads} host threads; {elapsed:.1f} s of oracle time "
                  f"(the same tokens' GPU outputs are checked against it)",
        "parity_rows_checked": done + len(probe),
        "parity_max_excess": max_excess,
        "parity_ok": bool(max_excess <= 0.0),
    }


if __name__ == "__main__":
    sys.exit(main())
