#!/usr/bin/env python3
"""Benchmark of the speculative-decoding step on one MI355X.

The reported step (the metric: verify + draft at BS 128, V = 151,936, B = 7)
is the dense one: rejection-sampling verification of every request's 7-token
model chain against bf16 target rows [128, 8, V] and draft rows [128, 7, V]
(probabilistic slots, T = 1.0, uniforms drawn in the kernel with
Philox4x32-10), the commit of the emitted tokens after each 8,192-token
context, then the n-gram draft over the updated contexts, fused into the same
call (synthetic, seeded; see workloads/synth.py).  The commit writes the new
lengths to a separate buffer, so every timed step does the same work.

Further records: the batch-allocation step (n-gram draft -> chain selection
and budget allocation of 256 slots -> verification -> commit) at BS 128; the
tree step (n-gram chains -> tree build with the Eq. (6) scores -> greedy
verification -> commit) at BS 64; the same allocation step on the
large-batch stress workload (BS 256, 32,768-token contexts, budget 512,
T = 0.7); the reported step with fp32 rows; a plain device copy (the
achievable HBM rate in the same run); and the CPU oracle on the reported
step's inputs, on one host core and on all of them.  The secondary records
run first, the reported step last.

Timing, per workload, on one stream: W warm-up steps, K eager steps with an
event pair attached to the dispatch of every statistics kernel (that
kernel's live average duration), then the K steps captured in one HIP graph
(checked against the eager step first), W warm-up replays and one timed
replay of the K-step graph between two events, which gives the throughput;
then K replays of a one-step graph, each between two events, which give the
p10 / p50 / p90 of the step time.  Prints one JSON line.
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
RNG = (20261202, 1)             # the dense step draws its uniforms in the kernel (Philox4x32-10)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E, AMD's published figure
STATS_KERNEL = "k_stats_rows"   # the HBM-bound pass of the dense step
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "stats_rows_dense_bs128_v151936_bf16_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "draft_verification_spec_amd", "csrc", f)
                  for f in ("verify.hip", "common.hpp")]


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    # the step is ~0.1 ms: a few hundred warm-up steps bring the GPU to its steady clocks
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-budget", action="store_true", help="skip the batch-allocation step record")
    p.add_argument("--no-tree", action="store_true", help="skip the tree step record")
    p.add_argument("--no-stress", action="store_true", help="skip the large-batch stress step record")
    p.add_argument("--no-fp32", action="store_true", help="skip the fp32 record of the reported step")
    p.add_argument("--no-ceiling", action="store_true", help="skip the device-copy ceiling record")
    p.add_argument("--no-sizing-loop", action="store_true",
                   help="skip the host sizing loop timing of the batch-allocation step")
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


def cpu_threads():
    """Host cores this process may use (its affinity, capped by OMP_NUM_THREADS when set)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(c, reps=3):
    """The oracle, as it stands, on the whole reported step (BS 128: draw the
    uniforms, verify every request, commit, n-gram draft of the committed
    contexts) on the same inputs as the GPU: single-threaded, and with the
    requests split over every host core this process may use (threads; the
    oracle's C calls release the GIL).  Median of `reps` runs of each."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as O
    O.build()
    BS, V, B = c["BS"], c["V"], c["B"]
    tgt = c["target_bf16"].reshape(-1, V)
    dft = c["draft_bf16"].reshape(-1, V)
    T_ctx = c["ctx"].shape[1]

    def part(lo, hi, u_acc, u_smp):
        n = hi - lo
        o = O.verify_chain(tgt[lo * (B + 1):hi * (B + 1)], np.arange(n) * (B + 1), c["tokens"][lo:hi],
                           np.zeros((n, B), np.uint8), np.full(n, B, np.int32), u_acc[lo:hi], u_smp[lo:hi],
                           c["temperature"], draft_logits=dft[lo * B:hi * B], draft_row_base=np.arange(n) * B)
        ctx, ctx_len = O.commit(c["ctx"][lo:hi].copy(), c["ctx_len"][lo:hi].copy(), T_ctx, o["out_tokens"],
                                o["out_num"], o["flags"])
        O.ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], c["max_draft"], c["copy_cap"])

    def step(threads):
        t0 = time.perf_counter()
        u_acc, u_smp = O.step_uniforms(BS, B, *RNG)
        if threads == 1:
            part(0, BS, u_acc, u_smp)
        else:
            cuts = np.linspace(0, BS, threads + 1).astype(int)
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(lambda i: part(cuts[i], cuts[i + 1], u_acc, u_smp), range(threads)))
        return time.perf_counter() - t0

    n = cpu_threads()
    one = sorted(step(1) for _ in range(reps))[reps // 2]
    alln = sorted(step(n) for _ in range(reps))[reps // 2]
    return {"value": 1.0 / alln, "unit": "steps/s", "cores": n, "kind": "oracle",
            "sample": f"the whole reported step (BS {BS}: uniforms, verify, commit, n-gram draft; C oracle, fp64), "
                      f"requests split over {n} threads; median of {reps} runs",
            "cpu_model": cpu_model(), "ms_per_step": alln * 1e3,
            "single_core": {"value": 1.0 / one, "unit": "steps/s", "cores": 1, "ms_per_step": one * 1e3}}


def copy_ceiling(hip, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of nbytes (torch), timed with events:
    bytes read plus written per second, the achievable HBM rate of a
    streaming kernel on this GPU in this run."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    for _ in range(3):
        dst.copy_(src)
    ms = []
    for _ in range(reps):
        hip.record(e0, stream)
        dst.copy_(src)
        hip.record(e1, stream)
        ms.append(hip.ms(e0, e1))
    ms.sort()
    med = ms[reps // 2]
    return {"kind": "device copy (torch)", "bytes_moved": 2 * nbytes, "ms": med,
            "GBps": 2 * nbytes / (med * 1e-3) / 1e9, "frac": 2 * nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def run_timed(step, outputs, K, W, hip, stream, eager_only=False):
    """Times `step` (already run once, so its buffers exist).  The graphs are
    captured first, so that the timed regions follow each other with no host
    work between them: W eager warm-up steps, K eager steps with the
    statistics kernel's event pair attached to its dispatch, W warm-up
    replays of a one-step graph, one replay of a K-step graph between two
    events (the throughput), and K one-step replays each between two events
    (the step-time distribution).  Afterwards every region's outputs must
    equal the reference step's, and the one-step graph is replayed three more
    times with eager steps in between, each checked."""
    import numpy as np
    import torch
    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        ref = [t.cpu().clone() for t in outputs()]
    ev_b = [hip.event() for _ in range(K)]
    ev_e = [hip.event() for _ in range(K)]
    pb = [hip.event() for _ in range(K)]
    pe = [hip.event() for _ in range(K)]
    t0, t1, t2, t3 = (hip.event() for _ in range(4))
    s = stream.cuda_stream

    def same(tag):
        for i, (a, b) in enumerate(zip(outputs(), ref)):
            assert torch.equal(a.cpu(), b), f"{tag}: output {i} differs from the reference step"

    g1 = gK = None
    if not eager_only:
        try:
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=stream):
                step()
            gK = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gK, stream=stream):
                for _ in range(K):
                    step()
        except Exception as e:  # capture unsupported here: keep the eager region's figure
            print(f"[bench] graph capture failed ({e}); reporting the eager region", file=sys.stderr, flush=True)
            g1 = gK = None
    with torch.cuda.stream(stream):
        for _ in range(W):
            step()
        hip.record(t0, s)
        for k in range(K):
            step(prof=(ev_b[k], ev_e[k]))
        hip.record(t1, s)
        if gK is not None:
            for _ in range(W):
                g1.replay()
            hip.record(t2, s)
            gK.replay()
            hip.record(t3, s)
            for k in range(K):
                hip.record(pb[k], s)
                g1.replay()
                hip.record(pe[k], s)
        torch.cuda.synchronize()
    eager_ms = hip.ms(t0, t1)
    stats_ms = [hip.ms(a, b) for a, b in zip(ev_b, ev_e)]
    out = {"mode": "eager", "ms_per_step": eager_ms / K, "steps_per_s": K / (eager_ms * 1e-3),
           "eager_ms_per_step": eager_ms / K, "stats_ms": float(np.mean(stats_ms))}
    if gK is not None:
        total_ms = hip.ms(t2, t3)
        per_ms = [hip.ms(a, b) for a, b in zip(pb, pe)]
        p10, p50, p90 = (float(np.percentile(per_ms, q)) for q in (10, 50, 90))
        out.update(mode="graph", ms_per_step=total_ms / K, steps_per_s=K / (total_ms * 1e-3),
                   step_ms_percentiles={"p10": p10, "p50": p50, "p90": p90, "steps": len(per_ms),
                                        "of": "single-step graph replays, each between two events"})
    same("timed steps")
    if g1 is not None:
        for rep in range(3):   # every replay equals the eager step, with eager work in between
            g1.replay()
            torch.cuda.synchronize()
            same(f"graph replay {rep}")
            with torch.cuda.stream(stream):
                step()
            torch.cuda.synchronize()
    return out


def headline(K, W, hip, eager_only, fp32=False):
    """The dense verify + commit + n-gram draft step (the reported one); with
    fp32 the same rows stored as fp32 (the bf16 values upcast exactly)."""
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
    if fp32:
        target, draft = target.float(), draft.float()
    rb, drb = g(np.arange(BS, dtype=np.int64) * (B + 1)), g(np.arange(BS, dtype=np.int64) * B)
    tokens, flags = g(c["tokens"]), g(np.zeros((BS, B), np.uint8))
    n_slots = g(np.full(BS, B, np.int32))
    ctx, ctx_len = g(c["ctx"]), g(c["ctx_len"])
    ctx_len_new = torch.empty_like(ctx_len)
    stream = torch.cuda.Stream()
    bufs = {"ws_v": torch.empty(1 << 26, dtype=torch.uint8, device=dev),
            "hist": torch.zeros(B + 1, dtype=torch.int32, device=dev)}

    def step(prof=None):
        # verification, commit and the next n-gram draft over the committed
        # contexts, in one call (the draft runs in the drawing workgroups)
        out = S.spec_verify_chain(target, rb, tokens, n_slots, c["temperature"], rng=RNG,
                                  accept_hist=bufs["hist"] if prof is not None else None,
                                  slot_flags=flags, draft_logits=draft, draft_row_base=drb, ctx=ctx,
                                  ctx_len=ctx_len, ctx_len_out=ctx_len_new, out=bufs.get("vf"),
                                  out_flags=bufs.get("vfl"), write_flags=True, workspace=bufs["ws_v"],
                                  prof_events=prof, ngram=(c["n_min"], c["n_max"], c["max_draft"], c["copy_cap"]),
                                  ngram_out=bufs.get("ng"))
        bufs.setdefault("vf", {k: v for k, v in out.items() if k not in ("out_flags", "ngram_draft", "ngram_len",
                                                                          "ngram_feat")})
        bufs.setdefault("vfl", out["out_flags"])
        bufs.setdefault("ng", (out["ngram_draft"], out["ngram_len"], out["ngram_feat"]))

    with torch.cuda.stream(stream):
        step()
    outputs = lambda: list(bufs["vf"].values()) + [bufs["vfl"], ctx_len_new, ctx] + list(bufs["ng"])

    def measure():
        t = run_timed(step, outputs, K, W, hip, stream, eager_only)
        # acceptance of the timed eager steps (the histogram is fed only there)
        h = bufs["hist"].cpu().numpy().astype(np.float64)
        al = float((h * np.arange(B + 1)).sum() / h.sum())
        t.update(acceptance={"accepted_per_request": al, "tokens_per_request_step": al + 1.0,
                             "histogram": [int(x) for x in h / max(1, K)]})
        rows_bytes = BS * (2 * B + 1) * V * (4 if fp32 else 2)   # every verified target and draft row
        ctx_bytes = int(c["ctx_len"].sum()) * 4
        t.update(c=c, rows_bytes=rows_bytes, ctx_bytes=ctx_bytes, BS=BS, V=V, B=B, T_ctx=int(c["ctx"].shape[1] - 64))
        return t
    return measure


def budget_step(K, W, hip, eager_only, config=2, sizing=True):
    """The batch-allocation step: n-gram draft, selection and allocation of
    the budget's slots, verification of the chosen chains, commit; at BS 128
    with a budget of 256 (config=2: the draft of the committed contexts runs
    inside the verify call), or the large-batch stress workload at BS 256,
    32,768-token contexts, budget 512 and T = 0.7 (config=4: a drafter launch
    first)."""
    import numpy as np
    import torch
    import draft_verification_spec_amd as S
    from workloads import synth
    dev = torch.device("cuda:0")
    c = synth.config2(ctx_extra=64) if config == 2 else synth.config4(ctx_extra=64)
    BS, V, L = c["BS"], c["V"], 15
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ctx, ctx_len = g(c["ctx"]), g(c["ctx_len"])
    ctx_len_new = torch.empty_like(ctx_len)
    tokens_d, conf_d, pm_d = g(c["model_tokens"]), g(c["model_conf_logit"]), g(c["model_point_mass"])
    target = synth.as_torch_bf16(c["target_bf16"]).to(dev).reshape(-1, V)
    row_base = g(np.arange(BS, dtype=np.int64) * c["target_rows_per_req"])
    u_acc, u_smp = g(c["u_acc"][:, :L]), g(c["u_smp"])
    stream = torch.cuda.Stream()
    bufs = {"ws_ng": torch.empty(1 << 22, dtype=torch.uint8, device=dev),
            "ws_al": torch.empty(1 << 20, dtype=torch.uint8, device=dev),
            "ws_v": torch.empty(1 << 24, dtype=torch.uint8, device=dev)}

    # The 8,192-token contexts are drafted inside the verify call (the drawing
    # workgroups scan the committed context, as in the dense step); the
    # 32,768-token ones by the drafter kernel, whose 1,024-thread scan takes
    # such a text in one batch.  Fused drafts go to a buffer of their own, so
    # every timed step repeats the same work on the same inputs.
    fused = config == 2
    if fused:
        with torch.cuda.stream(stream):
            bufs["ng0"] = S.spec_ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], L, c["copy_cap"],
                                             workspace=bufs["ws_ng"])
            bufs["ng"] = tuple(torch.empty_like(x) for x in bufs["ng0"])

    def step(prof=None, lam=c["lam"], budget=c["budget"]):
        if fused:
            d, dl, f = bufs["ng0"]
        else:
            d, dl, f = S.spec_ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], L, c["copy_cap"],
                                          out=bufs.get("ng"), workspace=bufs["ws_ng"])
            bufs.setdefault("ng", (d, dl, f))
        al = S.spec_allocate_budget(mode="chain", model_tokens=tokens_d, model_conf=conf_d, ngram_draft=d,
                                    ngram_len=dl, ngram_feat=f, est=c["estimator"], lam=lam,
                                    budget=budget, policy="proposed", conf_is_logit=True,
                                    model_point_mass=pm_d, ld=L, out=bufs.get("al"), workspace=bufs["ws_al"])
        out = S.spec_verify_chain(target, row_base, al["chain_tokens"], al["alloc_len"], c["temperature"],
                                  u_accept=u_acc, u_sample=u_smp, slot_flags=al["slot_flags"],
                                  out_flags=al["out_flags"], ctx=ctx, ctx_len=ctx_len, ctx_len_out=ctx_len_new,
                                  out=bufs.get("vf"), max_slots=budget, workspace=bufs["ws_v"],
                                  prof_events=prof,
                                  ngram=(c["n_min"], c["n_max"], L, c["copy_cap"]) if fused else None,
                                  ngram_out=bufs["ng"] if fused else None)
        bufs.setdefault("al", al)
        bufs.setdefault("vf", {k: v for k, v in out.items()
                               if k not in ("out_flags", "ngram_draft", "ngram_len", "ngram_feat")})

    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
    total_rows = int(bufs["al"]["total_rows"].item())
    surv = bufs["al"]["survival"].cpu().numpy().ravel()   # the host copy the next step's sizing reads
    outputs = lambda: list(bufs["vf"].values()) + [bufs["al"]["out_flags"], ctx_len_new, ctx] + list(bufs["ng"])

    def measure():
        t = run_timed(step, outputs, K, W, hip, stream, eager_only)
        if config == 2 and sizing:
            t["sizing_loop"] = sizing_loop(step, bufs, surv, BS, K, stream)
        return _budget_result(t, S, surv, BS, V, total_rows, c, config)
    return measure


def sizing_loop(step, bufs, surv, BS, K, stream, c0=None, p=0.3):
    """Eager steps whose budget b* and slot price lambda = G(b*) p the host
    sizes from survivals ([HS] Section 2 "Asynchronous scheduling", Section
    4.4): "async" from the survivals of two steps before, copied to pinned
    host memory after each allocation and waited for by their event only;
    "sync" from the step just run, waiting for it before the next launch;
    "fixed" with the scalars held (no sizing).  Host wall time per step,
    launches included; every step repeats the same inputs, so all three run
    the same work."""
    import torch
    import draft_verification_spec_amd as S
    c0 = float(BS) if c0 is None else c0
    ring = [torch.empty(surv.size, dtype=torch.float32).pin_memory() for _ in range(3)]
    evs = [torch.cuda.Event() for _ in range(3)]
    # the scalars the sizing settles on (the price changes the chains chosen,
    # and so the survivals it is sized from)
    b0, lam0, _ = S.spec_size_budget(surv, BS, c0, p)
    with torch.cuda.stream(stream):
        for _ in range(10):
            step(lam=lam0, budget=b0)
            b1, lam1, _ = S.spec_size_budget(bufs["al"]["survival"].cpu().numpy(), BS, c0, p)
            if (b1, lam1) == (b0, lam0):
                break
            b0, lam0 = b1, lam1
    res = {"b_star": b0, "lambda": lam0, "cost_model": "C(b) = BS + 0.3 b", "steps": K}
    with torch.cuda.stream(stream):
        for _ in range(20):
            step(lam=lam0, budget=b0)
        for mode in ("fixed", "async", "sync"):
            b, lam = b0, lam0
            seen = set()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for t in range(K):
                if mode == "async" and t >= 2:
                    evs[(t - 2) % 3].synchronize()
                    b, lam, _ = S.spec_size_budget(ring[(t - 2) % 3].numpy(), BS, c0, p)
                step(lam=lam, budget=b)
                seen.add(b)
                if mode != "fixed":
                    ring[t % 3].copy_(bufs["al"]["survival"].view(-1), non_blocking=True)
                    evs[t % 3].record(stream)
                if mode == "sync":
                    evs[t % 3].synchronize()
                    b, lam, _ = S.spec_size_budget(ring[t % 3].numpy(), BS, c0, p)
            torch.cuda.synchronize()
            res[mode + "_ms_per_step"] = (time.perf_counter() - t0) / K * 1e3
            res[mode + "_budgets"] = sorted(seen)
    return res


def _budget_result(t, S, surv, BS, V, total_rows, c, config):
    rows_bytes = total_rows * V * 2
    step_bytes = rows_bytes + int(c["ctx_len"].sum()) * 4
    workload = ("batch budget allocation + verify + commit + n-gram draft: BS=128, V=151936, model chain "
                "B=7 (greedy) + n-gram chain up to 15 (n 5..15), budget 256 draft slots, lambda 0.309, "
                "bf16 target rows, T=1.0, 8192-token contexts" if config == 2 else
                "large-batch stress, n-gram draft + allocation + verify + commit: BS=256, V=151936, Zipf(1.1) "
                "32768-token contexts with planted repeats, model chain B=7 (greedy) + n-gram up to 15 with the "
                "Table 5 estimator, budget 512, lambda 0.309, bf16 target rows, T=0.7")
    return {"workload": workload,
            "timing": t["mode"], "steps_per_s": t["steps_per_s"], "ms_per_step": t["ms_per_step"],
            "step_ms_percentiles": t.get("step_ms_percentiles"),
            "sizing_loop": t.get("sizing_loop"),
            "verified_rows_per_step": total_rows, "algorithmic_bytes": step_bytes,
            "GBps": step_bytes / (t["ms_per_step"] * 1e-3) / 1e9,
            "frac": step_bytes / (t["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "stats_kernel": {"kernel": "k_stats_flat", "avg_launch_ms": t["stats_ms"],
                             "GBps": rows_bytes / (t["stats_ms"] * 1e-3) / 1e9},
            # host work, timed after every GPU record (no idle gap between them)
            "host_budget_sizing": lambda: host_sizing(S, surv, BS)}


def tree_step(K, W, hip, eager_only):
    """The tree step (the tree workload: BS 64, V 151,936, fp32 rows, T = 0):
    n-gram chains from the anchor and each of the 8 picks -> tree build with
    the Eq. (6) scores and its S(n) curve -> greedy verification of the 16
    rows -> commit.  The stand-in target rows are made once for the tree the
    step builds (it is the same every step)."""
    import numpy as np
    import torch
    import draft_verification_spec_amd as S
    from workloads import synth
    dev = torch.device("cuda:0")
    c = synth.config3_inputs()
    BS, V, P, Kc, R = c["BS"], c["V"], c["P"], c["Kc"], c["rows_cap"]
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    qr, ex, el = synth.tree_queries(c["ctx"], c["ctx_len"], c["block"])
    f = synth.tree_score_inputs(BS, P, Kc)
    stride = c["ctx"].shape[1] + R
    ctx_h = np.zeros((BS, stride), np.int32)
    ctx_h[:, :c["ctx"].shape[1]] = c["ctx"]
    ctx, ctx_len = g(ctx_h), g(c["ctx_len"])
    ctx_len_new = torch.empty_like(ctx_len)
    qr_d, ex_d, el_d, block = g(qr), g(ex), g(el), g(c["block"])
    stream = torch.cuda.Stream()
    bufs = {"ws_t": torch.empty(1 << 24, dtype=torch.uint8, device=dev),
            "tfl": torch.zeros(BS, dtype=torch.int32, device=dev)}   # OR-ed flags: the same every step

    feats = dict(coef=f["coef"], h=g(f["h"]), sigma=g(f["sigma"]), r_share=g(f["r_share"]), psi_ctx=g(f["psi_ctx"]),
                 b_req=g(f["b_req"]), p_src=g(f["p_src"]))

    def build():
        # the tree's n-gram fill: copies, then the follower fallback on the
        # last three tokens
        d, dl, ft, fol = S.spec_ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], c["L"], c["copy_cap"],
                                            query_req=qr_d, extra=ex_d, extra_len=el_d, out=bufs.get("ng"),
                                            follow_ctx=3)
        sc = dict(feats, ngram_feat=ft)
        t = S.spec_allocate_budget(mode="tree", block=block, ngram_draft=d, ngram_len=dl, ngram_follow=fol, scores=sc,
                                   c_max=c["c_max"], depth_max=c["depth_max"], rows_cap=R, s_curve=True,
                                   out=bufs.get("tr"))
        bufs.setdefault("ng", (d, dl, ft, fol))
        bufs.setdefault("tr", t)
        return t

    with torch.cuda.stream(stream):
        t = build()
        torch.cuda.synchronize()
    rows = synth.tree_target_rows(3, t["node_token"].cpu().numpy(), t["parent_row"].cpu().numpy(),
                                  t["n_rows"].cpu().numpy(), c["truth"], V, R)
    logits = g(rows).reshape(-1, V)
    del rows
    rb = g(np.arange(BS, dtype=np.int64) * R)

    def step(prof=None):
        tr = build()
        out = S.spec_verify_tree(logits, rb, tr["node_token"], tr["parent_row"], tr["n_rows"], out_flags=bufs["tfl"],
                                 ctx=ctx,
                                 ctx_len=ctx_len, ctx_len_out=ctx_len_new, out=bufs.get("vt"), prof_events=prof,
                                 workspace=bufs["ws_t"])
        bufs.setdefault("vt", out)

    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
    outputs = lambda: list(bufs["vt"].values()) + [ctx_len_new, ctx] + list(bufs["tr"].values())
    return lambda: _tree_result(run_timed(step, outputs, K, W, hip, stream, eager_only), bufs, c, V)


def _tree_result(tm, bufs, c, V):
    rows_bytes = int(bufs["tr"]["n_rows"].sum().item()) * V * 4
    step_bytes = rows_bytes + int(c["ctx_len"].sum()) * 4
    return {"workload": "tree: n-gram chains from the anchor and 8 picks (n 3..15, follower fallback on the last "
                        "3 tokens) -> tree build with Eq. (6) "
                        "scores and S(n) -> greedy verification of up to 16 rows -> commit; BS=64, V=151936, "
                        "fp32 rows, 4096-token contexts, drafter block 8 x 4",
            "timing": tm["mode"], "steps_per_s": tm["steps_per_s"], "ms_per_step": tm["ms_per_step"],
            "step_ms_percentiles": tm.get("step_ms_percentiles"),
            "verified_rows_per_step": int(bufs["tr"]["n_rows"].sum().item()), "algorithmic_bytes": step_bytes,
            "GBps": step_bytes / (tm["ms_per_step"] * 1e-3) / 1e9,
            "frac": step_bytes / (tm["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "mean_S16": float(bufs["tr"]["s_curve"][:, -1].mean().item()),
            "mean_committed": float(bufs["vt"]["out_num"].float().mean().item()),
            "stats_kernel": {"kernel": "k_stats_rows (argmax)", "avg_launch_ms": tm["stats_ms"],
                             "GBps": rows_bytes / (tm["stats_ms"] * 1e-3) / 1e9,
                             "frac": rows_bytes / (tm["stats_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS}}


def host_sizing(S, surv, BS, calls=2000):
    """Host time of the next step's budget sizing (spec_size_budget) over the
    step's survivals, with a linear cost model of one unit per request and a
    slot cost of 0.3 units (the scale of the slot price the pages report at
    BS 128)."""
    b, lam, g = S.spec_size_budget(surv, BS, float(BS), 0.3)
    t0 = time.perf_counter()
    for _ in range(calls):
        S.spec_size_budget(surv, BS, float(BS), 0.3)
    us = (time.perf_counter() - t0) / calls * 1e6
    return {"survivals": int(surv.size), "us_per_call": us, "b_star": b, "lambda": lam,
            "cost_model": "C(b) = BS + 0.3 b", "includes": "ctypes marshalling"}


def read_ceiling(hip, nbytes, reps=5):
    """The streaming-read probe (libspec_probe.so: the statistics pass's load
    pattern without its arithmetic) over nbytes, timed with events: the
    achievable HBM read rate of this kernel shape on this GPU in this run."""
    import torch
    from draft_verification_spec_amd import build as hb
    lib = C.CDLL(hb.PROBE_LIB)
    lib.spec_probe_stream_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(3)
    out = torch.zeros((nbytes + 32767) // 32768, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = hip.event(), hip.event()
    call = lambda: lib.spec_probe_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), C.c_void_p(stream))
    for _ in range(20):
        assert call() == 0
    ms = []
    for _ in range(reps):
        hip.record(e0, stream)
        call()
        hip.record(e1, stream)
        ms.append(hip.ms(e0, e1))
    ms.sort()
    med = ms[reps // 2]
    return {"kind": "streaming read probe (non-temporal 16-byte loads, 32 KB per 256-thread workgroup)",
            "bytes": nbytes, "ms": med, "GBps": nbytes / (med * 1e-3) / 1e9,
            "frac": nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBPS}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the step would shard by "
              "request, each GPU running its own requests). Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    K, W = args.steps, args.warmup
    hip = Hip()
    # every record's inputs are made and resident first; the timed regions
    # then follow one another, the reported step last
    plan = []
    if not args.no_budget:
        plan.append(("budget_step", budget_step(K, W, hip, args.eager, sizing=not args.no_sizing_loop)))
    if not args.no_tree:
        plan.append(("tree_step", tree_step(K, W, hip, args.eager)))
    if not args.no_stress:
        plan.append(("stress_step", budget_step(K, W, hip, args.eager, config=4)))
    if not args.no_fp32:
        plan.append(("fp32_step", headline(K, W, hip, args.eager, fp32=True)))
    plan.append(("headline", headline(K, W, hip, args.eager)))
    extra = {}
    for name, measure in plan:
        extra[name] = measure()
    h = extra.pop("headline")
    if "fp32_step" in extra:
        f = extra.pop("fp32_step")
        fb = f["rows_bytes"] + f["ctx_bytes"]
        extra["fp32_step"] = {
            "workload": "the reported step with fp32 rows: target [128,8,V] and draft [128,7,V] fp32",
            "timing": f["mode"], "steps_per_s": f["steps_per_s"], "ms_per_step": f["ms_per_step"],
            "algorithmic_bytes": fb, "GBps": fb / (f["ms_per_step"] * 1e-3) / 1e9,
            "frac": fb / (f["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "step_ms_percentiles": f.get("step_ms_percentiles"),
            "stats_kernel": {"kernel": STATS_KERNEL, "avg_launch_ms": f["stats_ms"],
                             "GBps": f["rows_bytes"] / (f["stats_ms"] * 1e-3) / 1e9,
                             "frac": f["rows_bytes"] / (f["stats_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS}}
        del f
    ms_step = h["ms_per_step"]
    step_bytes = h["rows_bytes"] + h["ctx_bytes"]
    achieved = h["rows_bytes"] / (h["stats_ms"] * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": h["steps_per_s"],
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
        "config": {"workload": "dense verify + commit + n-gram draft: BS=128, V=151936, B=7, bf16 target "
                               "[128,8,V] and draft [128,7,V] rows, probabilistic slots, T=1.0, 8192-token "
                               "contexts, n-gram n 5..15, up to 15 tokens",
                   "global_batch": h["BS"], "seq_len": h["T_ctx"], "draft_len": h["B"], "timing": h["mode"]},
        "eager": {"ms_per_step": h["eager_ms_per_step"]},
        "step_ms_percentiles": h.get("step_ms_percentiles"),
        "roofline": {"bound": "hbm", "kernel": STATS_KERNEL, "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_from_profile(),
                     "bytes_per_launch": h["rows_bytes"], "avg_launch_ms": h["stats_ms"]},
        "step_hbm": {"algorithmic_bytes": step_bytes, "GBps": step_bytes / (ms_step * 1e-3) / 1e9,
                     "frac": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "acceptance": dict(h["acceptance"], us_per_emitted_token=ms_step * 1e3 / (h["BS"] *
                                                                               h["acceptance"]["tokens_per_request_step"])),
    }
    for rec in extra.values():
        if callable(rec.get("host_budget_sizing")):
            rec["host_budget_sizing"] = rec["host_budget_sizing"]()
    res.update(extra)
    if not args.no_ceiling:
        res["hbm_ceiling"] = {"read_probe": read_ceiling(hip, h["rows_bytes"]), "copy": copy_ceiling(hip)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(h["c"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
