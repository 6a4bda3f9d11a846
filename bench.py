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
sample of the same batch.  The prefill half of the metric is measured in the
same run and reported in the `prefill` object: the Mixtral-shaped layer at
rank 128 with 16384 bf16 tokens and 70/30 expert imbalance (ms per step,
tokens/s, the gate/up kernel's MFMA rate against the dense fp16/bf16 peak).
Other workloads (--workload) are single measurements without that object.
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
    "mixtral_decode_3bit": ("mixtral8x7b_decode", 32, 3),
    "mixtral_prefill16k_3bit": ("mixtral8x7b_prefill16k_bf16", 16384, 3),
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
    res_bytes = d_out * d_in * p.get("bits", 2) / 8 + 4.0 * d_out * d_in / G
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


def measure(workload, steps, warmup, copies, scheme="tileq", log=None, keep=None):
    """Time `steps` forwards of a workload (eager launches, then the same steps
    replayed from HIP graphs), then a profiled pass for the stage durations.
    Returns the fields of a bench record (without the CPU baseline) and the
    generated arrays.  `keep` (a dict) holds the generated layer and its
    uploaded copies for the next call with the same configuration (then the
    copies are not freed here)."""
    import torch

    import bit_rank_post_amd as tq
    import synth
    from bit_rank_post_amd import io as tqio

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg_name, T = WORKLOADS[workload][:2]
    bits = WORKLOADS[workload][2] if len(WORKLOADS[workload]) > 2 else 2
    cfg = synth.CONFIG_BY_NAME[cfg_name]
    copies = max(1, copies)
    key = (cfg_name, bits, scheme, copies)
    if keep is not None and keep.get("key") == key:
        layer, Ls = keep["layer"], keep["Ls"]
        say(f"reusing {cfg_name} (T={T}, {bits}-bit residuals)")
    else:
        say(f"generating {cfg_name} (T={T}, {bits}-bit residuals)")
        layer = synth.make_layer(cfg, scheme=scheme, bits=bits)
        Ls = [tqio.upload_layer(layer) for _ in range(copies)]
        if keep is not None:
            for L in keep.get("Ls", []):
                L.close()
            keep.update(key=key, layer=layer, Ls=Ls)
    pg = layer["proj"]["single" if cfg.kind == "single" else "gate"]
    x, ids, gates = synth.make_tokens(cfg, T)
    xd, idd, gd = tqio.tokens_to_device(x, ids, gates, cfg.act)
    k = cfg.topk
    d_out = cfg.d_ff if cfg.kind == "single" else cfg.d_model
    y = torch.empty((T, d_out), dtype=torch.float16 if cfg.act == "f16" else torch.bfloat16,
                    device="cuda")
    ydt = tq.TQ_F16 if cfg.act == "f16" else tq.TQ_BF16
    ws = tqio.workspace(Ls[0], T, k)
    decode = Ls[0].forward_path(T, k) == 1
    say(f"uploaded {copies} copies; path={'decode' if decode else 'prefill'}")

    def step(i):
        Ls[i % copies].forward(xd, T, idd, gd, k, y, ydt, ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms = 1e3 * (time.perf_counter() - t0) / steps
    say(f"timed {steps} steps: {eager_ms * 1e3:.1f} us/step")

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
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        graph_ms = 1e3 * (time.perf_counter() - t0) / steps
        say(f"graph replay: {graph_ms * 1e3:.1f} us/step")
        del graphs
    except Exception as exc:  # noqa: BLE001 - report eager numbers only
        say(f"graph capture unavailable: {exc}")

    # the router in front: router logits -> top-k -> forward, as two calls
    # (tq_router_topk, then tq_forward) and as one (tq_forward_from_logits,
    # where at decode the router runs inside the forward's first launch);
    # logits N(0,1), so the routing is uniform like the workload's
    router = None
    if cfg.K <= 256 and k <= min(cfg.K, 32):
        lg = torch.from_numpy(np.random.default_rng(7).standard_normal(
            (T, cfg.K)).astype(np.float32)).cuda()
        ids2 = torch.empty((T, k), dtype=torch.int32, device="cuda")
        g2 = torch.empty((T, k), dtype=torch.float32, device="cuda")

        def two_calls(i):
            tq.router_topk(lg, k, ids2, g2)
            Ls[i % copies].forward(xd, T, ids2, g2, k, y, ydt, ws)

        def one_call(i):
            Ls[i % copies].forward_from_logits(xd, T, lg, k, ids2, g2, y, ydt, ws)

        rt = {}
        for name, fn in (("router_then_forward_ms", two_calls), ("forward_from_logits_ms", one_call)):
            for i in range(warmup):
                fn(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                fn(i)
            torch.cuda.synchronize()
            rt[name] = round(1e3 * (time.perf_counter() - t0) / steps, 5)
        router = rt
        say(f"router + forward: {rt}")

    # second pass: stage durations from HIP events on the forward's stream
    for L in Ls:
        L.profile_enable(True)
    acc = None
    for i in range(steps):
        step(i)
        st = Ls[i % copies].profile_read()
        acc = st if acc is None else {kk: acc[kk] + st[kk] for kk in acc}
    for L in Ls:
        L.profile_enable(False)
    stages_ms = {kk: v / steps for kk, v in acc.items()}

    work = algorithmic(layer, ids, T)
    dom_ms = stages_ms["gemm_in"]
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
    tr = traffic_from_profile(workload, path_name) if scheme == "tileq" else None
    roof["traffic"] = tr
    roof["kernel"] = KERNEL_NAMES[path_name]
    roof["kernel_ms"] = round(dom_ms, 5)
    roof["algorithmic_bytes_per_launch"] = work["dom_bytes"]
    roof["algorithmic_flops_per_launch"] = work["dom_flops"]

    # both loops time the same steps of the same forward; the faster execution
    # mode is reported, the other one beside it
    use_graph = graph_ms is not None and graph_ms < eager_ms
    ms = graph_ms if use_graph else eager_ms
    rec = {
        "workload": f"{cfg_name}: {cfg.K} experts on {pg['M']}x{pg['N']} grid"
                    f"{'' if scheme == 'tileq' else ' (' + scheme + ')'}, "
                    f"d_model {cfg.d_model}, d_ff {cfg.d_ff}, rank {pg['rank']}, "
                    f"{bits}-bit group-{cfg.group} residual, top-{cfg.topk}, "
                    f"{cfg.act} activations, T={T} tokens, {path_name} path",
        "T": T, "dtype": cfg.act, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "roofline": roof, "execution": "hip_graph_replay" if use_graph else "eager",
        "eager_ms_per_step": round(eager_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
        "stages_ms": {kk: round(v, 5) for kk, v in stages_ms.items()},
        "router_eager": router,
        "whole_forward": {"algorithmic_bytes": work["total_bytes"],
                          "algorithmic_flops": work["total_flops"],
                          "achieved_GBps": round(work["total_bytes"] / (ms * 1e-3) / 1e9, 1),
                          "achieved_TFLOPs": round(work["total_flops"] / (ms * 1e-3) / 1e12, 2),
                          "active_experts": work["active_experts"]},
        "kernel_source_sha256": kernel_hash(path_name),
        "grid": (pg["M"], pg["N"]),
    }
    if keep is None:
        for L in Ls:
            L.close()
    return rec, (layer, x, ids, gates)


def attainable_read(nbytes, copies=4, iters=40):
    """GB/s of a plain streaming read of nbytes (tq_calibrate_read: 16-byte
    loads over the whole grid), over `copies` buffers in rotation so that the
    Infinity Cache cannot serve them: the read rate this device attains, the
    practical ceiling beside the nominal HBM peak."""
    import torch
    import bit_rank_post_amd as tq
    nbytes = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(copies)]
    scratch = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(2 * copies):
        tq.calibrate_read(bufs[i % copies], scratch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        tq.calibrate_read(bufs[i % copies], scratch)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / iters
    del bufs
    return {"GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "us_per_read": round(us, 2),
            "bytes": nbytes,
            "how": f"plain streaming read of the kernel's algorithmic bytes (tq_calibrate_read, "
                   f"{copies} buffers rotated), mean of {iters} launches"}


def with_attainable(roof, cal):
    """The roofline dict with the attainable-read rate and the fraction of it."""
    r = dict(roof)
    r["attainable"] = dict(cal, frac=round(roof["achieved"] / cal["GBps"], 4))
    return r


def bench_pack(steps, warmup):
    """The offline packer on the Mixtral-shaped gate projection: 8 experts on
    the 2 x 4 grid, d_out 14336, d_in 4096, rank 64 with a sketch of 72
    columns, one power iteration, 2-bit group-128 residuals, fp16 weights in.
    Returns a record with the pack time and its fp64 rate against the
    published fp64 peak (78.6 TFLOP/s)."""
    import torch

    import bit_rank_post_amd as tq
    import synth
    K, M, N, d_out, d_in, r, l, G, q = 8, 2, 4, 14336, 4096, 64, 72, 128, 1
    print("[bench] generating dense Mixtral-shaped gate experts", file=sys.stderr, flush=True)
    W, tiles = synth.make_dense_experts(K, M, N, d_out, d_in, r, seed=31)
    Wd = torch.from_numpy(W).cuda()
    omega = torch.from_numpy(np.random.default_rng(32).standard_normal((N * d_in, l))).cuda()
    m, n = M * d_out, N * d_in
    out = dict(U=torch.empty((m, r), dtype=torch.float16, device="cuda"),
               sigma=torch.empty(r, dtype=torch.float32, device="cuda"),
               V=torch.empty((n, r), dtype=torch.float16, device="cuda"),
               codes=torch.empty((K, d_out, d_in // 16), dtype=torch.int32, device="cuda"),
               scales=torch.empty((K, d_out, d_in // G), dtype=torch.float16, device="cuda"),
               zeros=torch.empty((K, d_out, d_in // G), dtype=torch.float16, device="cuda"))
    ws = None
    args = dict(K=K, M=M, N=N, d_in=d_in, d_out=d_out, rank=r, group=G, bits=2, sketch=l,
                power_iters=q, act=tq.TQ_F16, tile_of_expert=tiles, W=Wd, w_dtype=tq.TQ_F16,
                omega=omega, **out)
    for _ in range(warmup):
        tq.pack_proj(**args, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        tq.pack_proj(**args, ws=ws)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    flops = (2.0 * m * n * l * (2 + 2 * q)          # W_big products: sketch, power, Z
             + 8.0 * m * l * l * (1 + q) + 2.0 * n * l * l   # Gram matrices and whitening
             + 2.0 * m * l * r + 2.0 * n * l * r             # U, V
             + 2.0 * K * d_out * d_in * r)                   # each expert's low-rank block
    wbytes = K * d_out * d_in * 2.0
    return {"workload": f"offline packer, Mixtral-shaped gate projection: {K} experts on "
                        f"{M}x{N}, d_out {d_out}, d_in {d_in}, rank {r}, sketch {l}, "
                        f"{q} power iteration, 2-bit group-{G} residual, fp16 weights",
            "ms_per_pack": round(ms, 3), "steps": steps,
            "fp64_flops_per_pack": flops,
            "achieved_fp64_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
            "peak_fp64_TFLOPs": 78.6,
            "frac": round(flops / (ms * 1e-3) / 1e12 / 78.6, 4),
            "weight_bytes_read_per_W_pass": wbytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral_decode",
                    choices=sorted(WORKLOADS) + ["pack_mixtral_gate"])
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--scheme", default="tileq",
                    choices=("tileq", "rank0", "per_expert", "shared_u", "shared_v"),
                    help="weight-sharing scheme of the low-rank part (as a tile map); "
                         "the others are comparisons: rank0, per_expert, shared_u, shared_v")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill half of the metric (the 16k-token bf16 "
                         "Mixtral-shaped prefill measured beside the decode line)")
    ap.add_argument("--cpu-tokens", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB elementwise copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the forward runs on one GPU only; --gpus {args.gpus} is not "
              "supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload == "pack_mixtral_gate":
        print(json.dumps(bench_pack(min(args.steps, 5), min(args.warmup, 1))))
        return
    keep = {}
    rec, (layer, x, ids, gates) = measure(args.workload, args.steps, args.warmup, args.copies,
                                          args.scheme, keep=keep)
    # the other decode batch sizes of the metric (B = 1 .. 64), same layer
    # and weight copies, each its own timing
    batches = None
    if not args.no_prefill and args.workload == "mixtral_decode" and args.scheme == "tileq":
        batches = {}
        for b, wl in ((1, "mixtral_decode_b1"), (8, "mixtral_decode_b8"), (64, "mixtral_decode_b64")):
            r, _ = measure(wl, min(args.steps, 100), min(args.warmup, 10), args.copies, keep=keep)
            batches[str(b)] = {"ms_per_step": round(r["ms_per_step"], 5),
                               "tokens_per_s": round(r["tokens_per_s"], 1),
                               "execution": r["execution"],
                               "roofline": {kk: r["roofline"][kk] for kk in
                                            ("bound", "achieved", "peak", "unit", "frac",
                                             "kernel_ms", "algorithmic_bytes_per_launch")}}
    for L in keep.get("Ls", []):
        L.close()
    keep.clear()
    if rec["roofline"]["bound"] == "hbm":
        rec["roofline"] = with_attainable(rec["roofline"],
                                          attainable_read(rec["roofline"]["algorithmic_bytes_per_launch"]))
        for b in (batches or {}).values():
            b["roofline"] = with_attainable(
                b["roofline"], attainable_read(b["roofline"]["algorithmic_bytes_per_launch"]))

    if args.calibrate_copy:
        # one elementwise kernel of known traffic (reads 256 MiB, writes
        # 256 MiB): scales the FETCH_SIZE / WRITE_SIZE counters to bytes
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.abs(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # the prefill half of the metric, in the same run: the Mixtral-shaped
    # 16k-token bf16 prefill (compute bound; one weight copy)
    prefill = None
    if not args.no_prefill and args.workload == "mixtral_decode" and args.scheme == "tileq":
        psteps = min(args.steps, 20)
        pre, _ = measure("mixtral_prefill16k", psteps, min(args.warmup, 3), 1)
        prefill = {"workload": pre["workload"], "steps": psteps, "dtype": pre["dtype"],
                   "ms_per_step": round(pre["ms_per_step"], 5),
                   "tokens_per_s": round(pre["tokens_per_s"], 1),
                   "roofline": pre["roofline"], "execution": pre["execution"],
                   "eager_ms_per_step": pre["eager_ms_per_step"],
                   "graph_ms_per_step": pre["graph_ms_per_step"],
                   "stages_ms": pre["stages_ms"], "whole_forward": pre["whole_forward"],
                   "kernel_source_sha256": pre["kernel_source_sha256"]}

    cpu = None
    if not args.no_cpu_baseline:
        T = rec["T"]
        n_tok = args.cpu_tokens or min(T, 4)
        print(f"[bench] cpu baseline: oracle on {n_tok}-token chunks for about 10 s",
              file=sys.stderr, flush=True)
        cpu = cpu_baseline(layer, x, ids, gates, n_tok)

    T = rec["T"]
    ms_per_step = rec["ms_per_step"]
    out = {
        "metric": METRIC, "value": round(rec["tokens_per_s"], 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
        "data": "synthetic",
        "config": {"workload": rec["workload"], "global_batch": T, "seq_len": 1,
                   "parallelism": "single GPU",
                   "weight_copies_rotated": max(1, args.copies)},
        "roofline": rec["roofline"],
        "cpu_baseline": cpu,
        "execution": rec["execution"],
        "eager_ms_per_step": rec["eager_ms_per_step"],
        "graph_ms_per_step": rec["graph_ms_per_step"],
        "stages_ms": rec["stages_ms"],
        "router_eager": rec["router_eager"],
        "whole_forward": rec["whole_forward"],
        "kernel_source_sha256": rec["kernel_source_sha256"],
        "prefill": prefill,
        "decode_batches": batches,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
