#!/usr/bin/env python3
"""Benchmark of the TileQ fused MoE-layer forward on one MI355X.

Default workload: a Mixtral-8x7B-shaped MoE layer at decode, B = 32 tokens
(8 experts on a 2 x 4 grid, SwiGLU 4096 -> 14336 -> 4096, rank 64 per
projection, 2-bit group-128 residuals, top-2 softmax gating, fp16), synthetic
seeded weights and tokens.  One step = one full forward (routing, column
stages, residual GEMMs with the low-rank row stage, SwiGLU, combine) over the
batch, inputs resident in HBM.  Four independently placed copies of the layer
weights (about 1.6 GB) are used in rotation so the 256 MB Infinity Cache
cannot serve repeated reads.

Prints one JSON line.  `value` is tokens/s of the whole forward; `roofline`
gives the dominant kernel's achieved algorithmic bandwidth (or MFMA rate)
from HIP events recorded around that kernel on its own stream, in a second
pass over the same steps; `cpu_baseline` times the CPU oracle on a bounded
sample of the same batch.  Other workloads (--workload) are for the builder's
own measurements; the default line is the reported one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE-layer tokens/sec at decode (B=1..64) & prefill; "
          "achieved HBM GB/s / MFMA %")
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0

WORKLOADS = {
    "mixtral_decode": ("mixtral8x7b_decode", 32),
    "mixtral_decode_b1": ("mixtral8x7b_decode", 1),
    "mixtral_decode_b8": ("mixtral8x7b_decode", 8),
    "mixtral_decode_b64": ("mixtral8x7b_decode", 64),
    "qwen15_prefill512": ("qwen15_moe_prefill512", 512),
    "fine64_mixed4160": ("fine64_zipf_mixed4160", 4160),
    "mixtral_prefill16k": ("mixtral8x7b_prefill16k_bf16", 16384),
    "tiny": ("tiny", 64),
}

# sources of the dominant kernel of each path (the traffic summary is only
# used while it was taken on these exact sources)
KERNEL_SOURCES = {
    "decode": ["bit_rank_post_amd/csrc/gemm_decode.hip", "bit_rank_post_amd/csrc/tq_device.h",
               "bit_rank_post_amd/csrc/tq_internal.h"],
    "prefill": ["bit_rank_post_amd/csrc/gemm_prefill.hip", "bit_rank_post_amd/csrc/tq_device.h",
                "bit_rank_post_amd/csrc/tq_internal.h"],
}
KERNEL_NAMES = {
    "decode": "gemm_dec_kernel (gate+up streaming 2-bit residual GEMV/MFMA with low-rank "
              "row stage and SwiGLU epilogue)",
    "prefill": "gemm_pre_kernel (gate+up grouped 2-bit dequant MFMA GEMM with low-rank "
               "K-extension and SwiGLU epilogue)",
}


def kernel_hash(path_name):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path_name]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, path_name):
    """HBM bytes per launch of the dominant kernel from a committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_dominant_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_hash(path_name):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None

# ---------------------------------------------------------------------------
# algorithmic work (what the method must move / compute), from the routing


def proj_work(p, rows_used, cols_used, slots, col_rows):
    """Bytes and flops of one projection: residual codes + scales/zeros of
    the active experts, U blocks of active grid rows, V blocks of active grid
    columns; flops of the residual and both low-rank products."""
    d_in, d_out, r, G = p["d_in"], p["d_out"], p["rank"], p["group"]
    res_bytes = d_out * d_in / 4 + 4.0 * d_out * d_in / G
    return dict(res_bytes=res_bytes, u_bytes=d_out * r * 2.0 * len(rows_used),
                v_bytes=d_in * r * 2.0 * len(cols_used),
                res_flops=2.0 * d_in * d_out * slots, col_flops=2.0 * r * d_in * col_rows)


def algorithmic(layer, ids, T):
    K = layer["K"]
    flat = ids.reshape(-1)
    active = sorted(set(int(e) for e in flat if 0 <= e < K))
    S = len(flat)
    out = {}
    act_b = 2
    if layer["kind"] == "single":
        names = ["single"]
    else:
        names = ["gate", "up", "down"]
    tot_bytes = 0.0
    tot_flops = 0.0
    per = {}
    for n in names:
        p = layer["proj"][n]
        m_of = p["tile_of_expert"] // p["N"]
        n_of = p["tile_of_expert"] % p["N"]
        rows = sorted(set(int(m_of[e]) for e in active))
        cols = sorted(set(int(n_of[e]) for e in active))
        if n == "down":
            col_rows = S
            row_flops = 2.0 * p["rank"] * p["d_out"] * T * len(rows)
        else:
            pairs = {(int(n_of[e]), t) for t in range(T) for e in ids[t] if 0 <= e < K}
            col_rows = len(pairs)
            row_flops = 2.0 * p["rank"] * p["d_out"] * S
        w = proj_work(p, rows, cols, S, col_rows)
        w["bytes"] = w["res_bytes"] * len(active) + w["u_bytes"] + w["v_bytes"]
        w["flops"] = w["res_flops"] + w["col_flops"] + row_flops
        per[n] = w
        tot_bytes += w["bytes"]
        tot_flops += w["flops"]
    d_in0 = layer["proj"][names[0]]["d_in"]
    d_out_last = layer["proj"][names[-1]]["d_out"]
    io_bytes = T * d_in0 * act_b + T * d_out_last * act_b + S * 8
    tot_bytes += io_bytes
    if layer.get("shared") is not None:
        sh = layer["shared"]
        tot_bytes += 3 * sh["d_ff"] * layer["d_model"] * 2
        tot_flops += 2.0 * T * 3 * sh["d_ff"] * layer["d_model"]
    # dominant kernel: the residual GEMM of the input projection(s)
    if layer["kind"] == "single":
        p = per["single"]
        dom_bytes = p["res_bytes"] * len(active) + p["u_bytes"] * 0 + T * d_in0 * act_b \
            + S * layer["proj"]["single"]["d_out"] * 4
        dom_flops = p["res_flops"]
    else:
        g, u = per["gate"], per["up"]
        dom_bytes = (g["res_bytes"] + u["res_bytes"]) * len(active) + g["u_bytes"] + u["u_bytes"] \
            + T * d_in0 * act_b + S * layer["d_ff"] * act_b
        r = layer["proj"]["gate"]["rank"]
        dom_flops = g["res_flops"] + u["res_flops"] + 2 * 2.0 * r * layer["d_ff"] * S
    out.update(total_bytes=tot_bytes, total_flops=tot_flops, dom_bytes=dom_bytes,
               dom_flops=dom_flops, active_experts=len(active))
    return out

# ---------------------------------------------------------------------------


def cpu_baseline(layer, x, ids, gates, n_tok, min_s=10.0):
    """Time the fp64 CPU oracle (as it stands) on consecutive n_tok-token
    chunks of the batch, from the first token, until at least min_s seconds
    of CPU work (or the whole batch)."""
    from oracle import tileq_ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [os.cpu_count() or 1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    T = x.shape[0]
    done = 0
    t0 = time.perf_counter()
    while done < T:
        tok = np.arange(done, min(T, done + n_tok))
        tileq_ref.forward(layer, x, ids, gates, tokens=tok, keep_weights=False)
        done += len(tok)
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"first {done} tokens of the batch in chunks of {n_tok}; fp64 oracle "
                       f"building each used expert weight explicitly per chunk ({dt:.1f} s wall)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--scheme", default="tileq",
                    choices=("tileq", "rank0", "per_expert", "shared_u", "shared_v"),
                    help="weight-sharing scheme of the low-rank part (as a tile map); "
                         "the others are comparisons: rank0, per_expert, shared_u, shared_v")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB elementwise copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the forward runs on one GPU only; --gpus {args.gpus} is not "
              "supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_rank_post_amd as tq
    import synth
    from bit_rank_post_amd import io as tqio

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg_name, T = WORKLOADS[args.workload]
    cfg = synth.CONFIG_BY_NAME[cfg_name]
    print(f"[bench] generating {cfg_name} (T={T})", file=sys.stderr, flush=True)
    layer = synth.make_layer(cfg, scheme=args.scheme)
    pg = layer["proj"]["single" if cfg.kind == "single" else "gate"]
    x, ids, gates = synth.make_tokens(cfg, T)
    copies = max(1, args.copies)
    Ls = [tqio.upload_layer(layer) for _ in range(copies)]
    xd, idd, gd = tqio.tokens_to_device(x, ids, gates, cfg.act)
    k = cfg.topk
    d_out = cfg.d_ff if cfg.kind == "single" else cfg.d_model
    y = torch.empty((T, d_out), dtype=torch.float16 if cfg.act == "f16" else torch.bfloat16,
                    device="cuda")
    ydt = tq.TQ_F16 if cfg.act == "f16" else tq.TQ_BF16
    ws = tqio.workspace(Ls[0], T, k)
    path = 1 if T * k <= 16 * cfg.K else 2
    print(f"[bench] uploaded {copies} copies; path={'decode' if path == 1 else 'prefill'}",
          file=sys.stderr, flush=True)

    def step(i):
        Ls[i % copies].forward(xd, T, idd, gd, k, y, ydt, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step",
          file=sys.stderr, flush=True)

    # the same steps replayed from HIP graphs (one captured forward per weight
    # copy): removes the host launch path and most inter-kernel gaps
    graph_ms = None
    try:
        graphs = []
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        graph_ms = 1e3 * (time.perf_counter() - t0) / args.steps
        print(f"[bench] graph replay: {graph_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        del graphs
    except Exception as exc:  # noqa: BLE001 - report eager numbers only
        print(f"[bench] graph capture unavailable: {exc}", file=sys.stderr, flush=True)

    # second pass: stage durations from HIP events on the forward's stream
    for L in Ls:
        L.profile_enable(True)
    acc = None
    for i in range(args.steps):
        step(i)
        st = Ls[i % copies].profile_read()
        acc = st if acc is None else {kk: acc[kk] + st[kk] for kk in acc}
    for L in Ls:
        L.profile_enable(False)
    stages_ms = {kk: v / args.steps for kk, v in acc.items()}

    if args.calibrate_copy:
        # one elementwise kernel of known traffic (reads 256 MiB, writes
        # 256 MiB): scales the FETCH_SIZE / WRITE_SIZE counters to bytes
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.abs(a, out=b)
        torch.cuda.synchronize()
        del a, b

    work = algorithmic(layer, ids, T)
    dom_ms = stages_ms["gemm_in"]
    decode = path == 1
    if decode:
        achieved = work["dom_bytes"] / (dom_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    else:
        achieved = work["dom_flops"] / (dom_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_F16_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_F16_TFLOPS, 4))
    path_name = "decode" if decode else "prefill"
    # (the counter summaries are taken with the grid of the configuration)
    tr = traffic_from_profile(args.workload, path_name) if args.scheme == "tileq" else None
    roof["traffic"] = tr
    roof["kernel"] = KERNEL_NAMES[path_name]
    roof["kernel_ms"] = round(dom_ms, 5)
    roof["algorithmic_bytes_per_launch"] = work["dom_bytes"]
    roof["algorithmic_flops_per_launch"] = work["dom_flops"]

    cpu = None
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens or min(T, 4)
        print(f"[bench] cpu baseline: oracle on {n_tok}-token chunks for about 10 s", file=sys.stderr, flush=True)
        cpu = cpu_baseline(layer, x, ids, gates, n_tok)

    # both loops time the same steps of the same forward; the faster execution
    # mode is reported, the other one beside it
    eager_ms = ms_per_step
    use_graph = graph_ms is not None and graph_ms < eager_ms
    if use_graph:
        ms_per_step = graph_ms
    value = T / (ms_per_step * 1e-3)
    whole_gbs = work["total_bytes"] / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{cfg_name}: {cfg.K} experts on {pg['M']}x{pg['N']} grid"
                               f"{'' if args.scheme == 'tileq' else ' (' + args.scheme + ')'}, "
                               f"d_model {cfg.d_model}, d_ff {cfg.d_ff}, rank {pg['rank']}, "
                               f"2-bit group-{cfg.group} residual, top-{cfg.topk}, "
                               f"{cfg.act} activations, T={T} tokens, "
                               f"{'decode' if decode else 'prefill'} path",
                   "global_batch": T, "seq_len": 1, "parallelism": "single GPU",
                   "weight_copies_rotated": copies},
        "roofline": roof,
        "cpu_baseline": cpu,
        "execution": "hip_graph_replay" if use_graph else "eager",
        "eager_ms_per_step": round(eager_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
        "stages_ms": {kk: round(v, 5) for kk, v in stages_ms.items()},
        "whole_forward": {"algorithmic_bytes": work["total_bytes"],
                          "algorithmic_flops": work["total_flops"],
                          "achieved_GBps": round(whole_gbs, 1),
                          "active_experts": work["active_experts"]},
        "kernel_source_sha256": kernel_hash(path_name),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
