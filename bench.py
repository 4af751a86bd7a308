#!/usr/bin/env python3
"""Benchmark of the whole speculative-decoding step on one MI355X.

One step = n-gram draft over every request's context -> chain selection and
budget allocation -> rejection-sampling verification of the chosen chains ->
commit of the emitted tokens, on the batch-allocation workload: BS 128,
V = 151,936, a 7-token model chain and a 15-token n-gram chain per request,
budget 256 verified draft slots, bf16 target rows, T = 1.0, 8,192-token
contexts (synthetic, seeded; see workloads/synth.py).

The commit appends each request's emitted tokens after its context and writes
the new lengths to a separate buffer, so every one of the K timed steps reads
the same contexts and does the same work.  Two timed regions on one stream:
K eager steps with an event pair attached to the dispatch of every
verification statistics kernel (that kernel's live average duration, and an
eager throughput), then the K steps captured in one HIP
graph (checked against the eager step first) replayed once between two
events, which gives the reported throughput.  Prints one JSON line.
"""
import argparse
import ctypes as C
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify+draft steps/sec at BS128, V=151936, B=7; achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, AMD's published figure
STATS_KERNEL = "k_stats_flat"   # the HBM-bound pass of the step
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "verify_stats_bs128_v151936_bf16_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "draft_verification_spec_amd", "csrc", f)
                  for f in ("verify.hip", "common.hpp")]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true", help="skip the dense verify + draft measurement")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


class Hip:
    """HIP events through the runtime library (timing only)."""

    def __init__(self):
        self.lib = C.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [C.c_void_p]

    def event(self):
        e = C.c_void_p()
        assert self.lib.hipEventCreate(C.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(C.c_void_p(e), C.c_void_p(stream)) == 0

    def ms(self, a, b):
        self.lib.hipEventSynchronize(C.c_void_p(b))
        out = C.c_float()
        assert self.lib.hipEventElapsedTime(C.byref(out), C.c_void_p(a), C.c_void_p(b)) == 0
        return out.value


def sources_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch of the statistics kernel from committed counter
    runs, or None when absent or taken on different kernel sources."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    text = open(PROFILE_COUNTERS).read()
    m = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != sources_digest():
        return None
    return float(t.group(1))


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 10}), flush=True)


def cpu_baseline(c, budget_s=12.0):
    """The oracle, as it stands, on the same inputs: whole steps over the full
    batch, repeated until about budget_s seconds of CPU work."""
    import numpy as np
    from oracle import oracle as O
    O.build()
    n, t0 = 0, time.perf_counter()
    while True:
        O.step_chain(c["ctx"], c["ctx_len"], c["ctx"].shape[1], c["model_tokens"], c["model_conf_logit"],
                     c["model_point_mass"], c["estimator"], c["lam"], c["budget"],
                     c["target_bf16"].reshape(-1, c["V"]), np.arange(c["BS"]) * 16, c["u_acc"], c["u_smp"],
                     c["temperature"], c["n_min"], c["n_max"], 15, 256)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20:
            break
    return {"value": n / el, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole steps over the full BS-128 batch (single-threaded C oracle, fp64), {el:.1f} s"}


def dense_headline(K, W, hip):
    """The dense verify + draft step at BS 128: bf16 target [128, 8, V] and
    draft [128, 7, V] rows with probabilistic slots at T = 1, the commit of the
    emitted tokens, then the n-gram draft over the updated contexts.  K steps
    captured in one HIP graph (checked against an eager step first)."""
    import numpy as np
    import torch
    import draft_verification_spec_amd as S
    from workloads import synth
    dev = torch.device("cuda:0")
    c = synth.dense_headline(ctx_extra=64)
    BS, V, B = c["BS"], c["V"], c["B"]
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    target = synth.as_torch_bf16(c["target_bf16"]).to(dev).reshape(-1, V)
    draft = synth.as_torch_bf16(c["draft_bf16"]).to(dev).reshape(-1, V)
    rb, drb = g(np.arange(BS, dtype=np.int64) * (B + 1)), g(np.arange(BS, dtype=np.int64) * B)
    tokens, flags = g(c["tokens"]), g(np.zeros((BS, B), np.uint8))
    n_slots = g(np.full(BS, B, np.int32))
    u_acc, u_smp = g(c["u_acc"]), g(c["u_smp"])
    ctx, ctx_len = g(c["ctx"]), g(c["ctx_len"])
    ctx_len_new = torch.empty_like(ctx_len)
    stream = torch.cuda.Stream()
    bufs = {"ws_v": torch.empty(1 << 26, dtype=torch.uint8, device=dev),
            "ws_ng": torch.empty(1 << 20, dtype=torch.uint8, device=dev)}

    def step():
        out = S.spec_verify_chain(target, rb, tokens, n_slots, c["temperature"], u_accept=u_acc, u_sample=u_smp,
                                  slot_flags=flags, draft_logits=draft, draft_row_base=drb, ctx=ctx,
                                  ctx_len=ctx_len, ctx_len_out=ctx_len_new, out=bufs.get("vf"),
                                  out_flags=bufs.get("vfl"), write_flags=True, workspace=bufs["ws_v"])
        d = S.spec_ngram_draft(ctx, ctx_len_new, c["n_min"], c["n_max"], c["max_draft"], c["copy_cap"],
                               out=bufs.get("ng"), workspace=bufs["ws_ng"])
        bufs.setdefault("vf", {k: v for k, v in out.items() if k != "out_flags"})
        bufs.setdefault("vfl", out["out_flags"])
        bufs.setdefault("ng", d)
        return out, d

    with torch.cuda.stream(stream):
        step()
        out, d = step()
        torch.cuda.synchronize()
        ref = [t.cpu().clone() for t in list(out.values()) + list(d)]
        gK = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gK, stream=stream):
            for _ in range(K):
                step()
        gK.replay()
        torch.cuda.synchronize()
        got = [t.cpu() for t in list(out.values()) + list(d)]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), "dense graph replay differs from the eager step"
        for _ in range(max(1, W // K)):
            gK.replay()
        torch.cuda.synchronize()
        t0, t1 = hip.event(), hip.event()
        hip.record(t0, stream.cuda_stream)
        gK.replay()
        hip.record(t1, stream.cuda_stream)
        torch.cuda.synchronize()
    ms = hip.ms(t0, t1)
    rows_bytes = BS * (2 * B + 1) * V * 2
    ctx_bytes = int(c["ctx_len"].sum()) * 4
    step_bytes = rows_bytes + ctx_bytes
    gbps = step_bytes / (ms / K * 1e-3) / 1e9
    return {"workload": "dense verify + commit + n-gram draft: BS=128, V=151936, B=7, bf16 target [128,8,V] and "
                        "draft [128,7,V], probabilistic slots, T=1.0, 8192-token contexts",
            "steps_per_s": K / (ms * 1e-3), "ms_per_step": ms / K, "algorithmic_bytes": step_bytes,
            "GBps": gbps, "frac": gbps / PEAK_HBM_GBPS}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the step shards by request; "
              "see DESIGN.md). Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import draft_verification_spec_amd as S
    from workloads import synth

    dev = torch.device("cuda:0")
    c = synth.config2(ctx_extra=64)
    BS, V, L = c["BS"], c["V"], 15
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ctx = g(c["ctx"])
    ctx_len = g(c["ctx_len"])
    ctx_len_new = torch.empty_like(ctx_len)
    tokens_d, conf_d, pm_d = g(c["model_tokens"]), g(c["model_conf_logit"]), g(c["model_point_mass"])
    target = synth.as_torch_bf16(c["target_bf16"]).to(dev).reshape(-1, V)
    row_base = g(np.arange(BS, dtype=np.int64) * c["target_rows_per_req"])
    u_acc, u_smp = g(c["u_acc"][:, :L]), g(c["u_smp"])
    est = c["estimator"]

    stream = torch.cuda.Stream()
    hip = Hip()
    bufs = {}

    def step(prof=None):
        d, dl, f = S.spec_ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], L, c["copy_cap"],
                                      out=bufs.get("ng"), workspace=bufs.get("ws_ng"))
        al = S.spec_allocate_budget(mode="chain", model_tokens=tokens_d, model_conf=conf_d, ngram_draft=d,
                                    ngram_len=dl, ngram_feat=f, est=est, lam=c["lam"], budget=c["budget"],
                                    policy="proposed", conf_is_logit=True, model_point_mass=pm_d, ld=L,
                                    out=bufs.get("al"), workspace=bufs.get("ws_al"))
        out = S.spec_verify_chain(target, row_base, al["chain_tokens"], al["alloc_len"], c["temperature"],
                                  u_accept=u_acc, u_sample=u_smp, slot_flags=al["slot_flags"],
                                  out_flags=al["out_flags"], ctx=ctx, ctx_len=ctx_len, ctx_len_out=ctx_len_new,
                                  out=bufs.get("vf"), max_slots=c["budget"],
                                  workspace=bufs.get("ws_v"), prof_events=prof)
        bufs.setdefault("ng", (d, dl, f))
        bufs.setdefault("al", al)
        bufs.setdefault("vf", {k: v for k, v in out.items() if k != "out_flags"})
        return d, al, out

    with torch.cuda.stream(stream):
        # preallocate workspaces once (the graph must not allocate)
        bufs["ws_ng"] = torch.empty(1 << 22, dtype=torch.uint8, device=dev)
        bufs["ws_al"] = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        bufs["ws_v"] = torch.empty(1 << 24, dtype=torch.uint8, device=dev)
        step()
        torch.cuda.synchronize()
        d, al, out = step()
        torch.cuda.synchronize()
        ref = {k: v.cpu().clone() for k, v in out.items()}
        ref_ctx = ctx.cpu().clone()
        total_rows = int(al["total_rows"].item())

    K, W = args.steps, args.warmup
    ev_b = [hip.event() for _ in range(K)]
    ev_e = [hip.event() for _ in range(K)]
    t0, t1, t2, t3 = (hip.event() for _ in range(4))
    s = stream.cuda_stream

    # Region 1, eager launches: an event pair attached to every statistics
    # kernel's dispatch gives that kernel's live average duration.
    with torch.cuda.stream(stream):
        for _ in range(W):
            step()
        torch.cuda.synchronize()
        hip.record(t0, s)
        for k in range(K):
            step(prof=(ev_b[k], ev_e[k]))
        hip.record(t1, s)
        torch.cuda.synchronize()
    eager_ms = hip.ms(t0, t1)
    stats_ms = [hip.ms(a, b) for a, b in zip(ev_b, ev_e)]
    for k2, v in out.items():
        assert torch.equal(v.cpu(), ref[k2]), f"eager timed steps differ from the reference step in {k2}"

    # Region 2, the K steps captured in one HIP graph, replayed once.
    mode = "graph"
    total_ms = eager_ms
    if args.eager:
        mode = "eager"
    else:
        try:
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=stream):
                step()
            gK = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gK, stream=stream):
                for k in range(K):
                    step()
            # every replay must equal the eager step (with eager work in between)
            for rep in range(3):
                g1.replay()
                torch.cuda.synchronize()
                for k2, v in out.items():
                    assert torch.equal(v.cpu(), ref[k2]), f"graph replay {rep} differs in {k2}"
                assert torch.equal(ctx.cpu(), ref_ctx)
                with torch.cuda.stream(stream):
                    step()
                torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                for _ in range(W):
                    g1.replay()
                torch.cuda.synchronize()
                hip.record(t2, s)
                gK.replay()
                hip.record(t3, s)
                torch.cuda.synchronize()
            total_ms = hip.ms(t2, t3)
            for k2, v in out.items():
                assert torch.equal(v.cpu(), ref[k2]), f"graph timed steps differ from the reference step in {k2}"
        except Exception as e:  # capture unsupported here: keep the eager region's figure
            print(f"[bench] graph capture failed ({e}); reporting the eager region", file=sys.stderr, flush=True)
            mode = "eager"
            total_ms = eager_ms

    ms_step = total_ms / K
    stats_avg = float(np.mean(stats_ms))
    stats_bytes = total_rows * V * 2                     # one bf16 read of every verified row
    ctx_bytes = int(c["ctx_len"].sum()) * 4               # one read of every context
    step_bytes = stats_bytes + ctx_bytes
    achieved = stats_bytes / (stats_avg * 1e-3) / 1e9
    traffic = traffic_from_profile()
    res = {
        "metric": METRIC,
        "value": K / (total_ms * 1e-3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "batch budget allocation + verify + n-gram draft: BS=128, V=151936, model chain "
                               "B=7 (greedy) + n-gram chain up to 15 (n 5..15), budget 256 draft slots, lambda 0.309, "
                               "bf16 target rows, T=1.0, 8192-token contexts",
                   "global_batch": BS, "seq_len": int(c["ctx"].shape[1] - 64), "timing": mode,
                   "verified_rows_per_step": total_rows},
        "eager": {"steps_per_s": K / (eager_ms * 1e-3), "ms_per_step": eager_ms / K},
        "roofline": {"bound": "hbm", "kernel": STATS_KERNEL, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "bytes_per_launch": stats_bytes, "avg_launch_ms": stats_avg},
        "step_hbm": {"algorithmic_bytes": step_bytes, "GBps": step_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS},
    }
    if not args.no_dense:
        res["dense_headline"] = dense_headline(K, W, hip)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
