#!/usr/bin/env python3
"""Benchmark of the fused FP8 block-quantized MoE forward on one MI355X.

Headline workload (one "step"): a DeepSeek-V3-shaped routed-expert layer,
H=7168, I=2048, E=256, top_k=8 softmax routing with renormalisation and a
seeded +-0.5 per-expert logit bias (load skew), FP8 e4m3fn weights with
128x128 block scales (~11.3 GB, drawn N(0, 0.02)), bf16 activations N(0, 1)
with dynamic per-token 128-group quantisation; one decode batch of T=64
tokens plus one prefill batch of T=8192 tokens through the whole path
(router, sort-and-pad, activation quant, GEMM1 + SiLU*mul + requant, GEMM2,
routing-weighted combine).  Inputs are resident in HBM before timing starts,
and the weights (11.3 GB) exceed the 256 MB last-level cache, so every call
streams them from HBM.

Sections (--sections, default all of them):
  layer    the headline step: plain moe_fp8_forward calls timed over exactly
           --steps steps (value, ms_per_step, per-phase median / p10 / p90),
           then a second pass through moe_fp8_forward_traced, whose HIP events
           on the launch stream give every stage's time, the dominant kernel
           and its roofline;
  configs  every other workload as its own line: tiny T=16, Mixtral-shaped
           T=64 / 512, Qwen3-shaped T=1 / 32 / 4096 (twelve rotating weight
           replicas, so the experts a small batch touches never sit in the
           last-level cache); tokens/s, both roofline fractions, the target;
  quant    the standalone activation quantiser on bf16 [16384, 7168] with 1%
           x100 outliers (three rotating inputs), block and MXFP8 scales;
  linear   the dense block-FP8 and MXFP8 linears on a DeepSeek-V3-shaped down
           projection (7168 x 18432) at M = 64 and 8192;
  batched  the batched (masked) expert format;
  mx       the MXFP8 layer on the headline inputs;
  peaks    what the part sustains: a read-only HBM stream, a device copy and
           register-only MFMA chains of both GEMMs' instruction types.

Prints one JSON line.  value = tokens per second over the headline step.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused FP8 MoE tokens/s + % of HBM/MFMA roofline, decode M=64 & prefill M=8192"
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_FP8_PEAK = 5.0e15     # dense FP8 FLOP/s
MFMA_F16_PEAK = 2.5e15     # dense f16 / bf16 FLOP/s
SECTIONS = ["layer", "configs", "quant", "linear", "batched", "mx", "peaks"]
# targets of the configurations: decode batches >= 60% of the HBM roofline,
# prefill batches >= 50% of the dense-FP8 MFMA peak (a Mixtral-shaped T=512
# batch stays below the ridge even at peak and is held to the HBM target)
TARGETS = {("tiny", 16): None, ("mixtral", 64): ("hbm", 0.6), ("mixtral", 512): ("hbm", 0.6),
           ("dsv3", 64): ("hbm", 0.6), ("dsv3", 8192): ("mfma", 0.5),
           ("qwen3", 1): ("hbm", 0.6), ("qwen3", 32): ("hbm", 0.6), ("qwen3", 4096): ("mfma", 0.5)}

# HBM bytes per launch of the two GEMMs, from rocprofv3 FETCH_SIZE (x2) and
# WRITE_SIZE (x1) passes, each scaled by what the same counter reads for a
# plain 1 GiB copy (profiles/hbm_counters_dsv3_*.md).  Valid only for the
# kernel code they were taken on: the line reports null traffic once the code
# of gemm.hip (kernel_code_digest: the file without its comments and blank
# lines) differs from this digest.
TRAFFIC_CODE_DIGEST = "f355efd5f8a833c1ec06e02486f4c97e5ed28a4025b35fd8c88a4556356b4231"
TRAFFIC = {  # (read bytes, write bytes) per launch, DeepSeek-V3-shaped workload
    "prefill.gemm1": (11285952866, 184021248),
    "prefill.gemm2": (5035629129, 968259253),
    "decode.gemm1": (4795568361, 5713685),
    "decode.gemm2": (2408830357, 7340587),
}


def kernel_code_digest(path):
    """sha256 of a C++ source without its // comments, trailing blanks and
    blank lines: edits to the comments leave it unchanged, any code edit
    changes it."""
    lines = []
    for line in open(path, encoding="utf-8"):
        cut = line.find("//")
        while cut >= 0 and line.count('"', 0, cut) % 2:
            cut = line.find("//", cut + 2)       # inside a string literal
        code = (line[:cut] if cut >= 0 else line).rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dsv3", choices=["dsv3", "mixtral", "qwen3", "tiny"])
    p.add_argument("--cpu-sample-tokens", type=int, default=16)
    p.add_argument("--phase", default="both", choices=["both", "decode", "prefill"],
                   help="headline step with one batch size only (for per-kernel profiles)")
    p.add_argument("--sections", default=",".join(SECTIONS),
                   help="comma-separated subset of " + ",".join(SECTIONS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--layer-only", action="store_true", help="same as --sections layer")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="also run a plain device-to-device copy of this many MiB (three times), "
                        "the reference kernel that scales the HBM byte counters")
    a = p.parse_args(argv)
    a.sections = ["layer"] if a.layer_only else [s for s in a.sections.split(",") if s]
    bad = [s for s in a.sections if s not in SECTIONS]
    if bad:
        p.error(f"unknown sections {bad}")
    return a


def batch_sizes(name):
    from synth import MOE_WORKLOADS
    t = MOE_WORKLOADS[name]["T"]
    return (min(t), max(t)) if len(t) > 1 else (t[0], t[0])


def algorithmic(ids, T, H, I, E, k):
    """Bytes and FLOPs the method must move / compute (no padding, no
    intermediates), per stage and for the layer."""
    import numpy as np
    P = T * k
    active = int(np.unique(ids).size)
    w13_b = active * (2 * I * H + 4 * (2 * I // 128) * (H // 128))
    w2_b = active * (H * I + 4 * (H // 128) * (I // 128))
    a_b = P * I + 4 * P * (I // 128)
    return {
        "active_experts": active,
        "layer_bytes": w13_b + w2_b + 2 * T * H + 2 * T * H + 4 * T * E,
        "layer_flops": 6 * P * H * I,
        "stage": {
            "router": (4 * T * E + 8 * P, 0),
            "align": (8 * P, 0),
            "quant": (2 * T * H + T * H + 4 * T * (H // 128), 0),
            "gemm1": (w13_b + T * H + 4 * T * (H // 128) + a_b, 4 * P * H * I),
            "gemm2": (w2_b + a_b + 2 * P * H, 2 * P * H * I),
            "combine": (2 * P * H + 8 * P + 2 * T * H, 0),
        },
    }


def roofline_of(nbytes, flops, seconds, mfma_peak=MFMA_FP8_PEAK):
    """Whichever of the HBM and MFMA times is longer at the published peaks
    bounds the work; achieved rate and fraction of that peak."""
    t_hbm, t_mfma = nbytes / HBM_PEAK, flops / mfma_peak
    if t_mfma > t_hbm:
        return roofline_at(nbytes, flops, seconds, "mfma", mfma_peak)
    return roofline_at(nbytes, flops, seconds, "hbm")


def roofline_at(nbytes, flops, seconds, bound, mfma_peak=MFMA_FP8_PEAK):
    """The roofline entry against a given bound: "hbm" (bytes over 8 TB/s) or
    "mfma" (flops over the given MFMA peak)."""
    if bound == "mfma":
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": a, "peak": mfma_peak / 1e12, "unit": "TFLOP/s",
                "frac": a / (mfma_peak / 1e12)}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": a / (HBM_PEAK / 1e9)}


def fractions(nbytes, flops, seconds):
    """Both fractions of the published roofline, and their maximum (the
    roofline fraction of the measurement plan: max(B/BW, F/PEAK_FP8) / t)."""
    h = nbytes / seconds / HBM_PEAK
    m = flops / seconds / MFMA_FP8_PEAK
    return {"hbm_frac": h, "mfma_frac": m, "roofline_frac": max(h, m),
            "bound_at_peak": "mfma" if flops / MFMA_FP8_PEAK > nbytes / HBM_PEAK else "hbm"}


def stats(ms):
    """median, p10, p90 and mean of a list of milliseconds"""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "mean_ms": float(a.mean()), "n": int(a.size)}


def cpu_threads():
    """CPU threads the oracle may use: the process's CPU affinity, capped by
    the thread count the environment grants (OMP_NUM_THREADS, when set)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def cpu_baseline(w, x_dec, logits_dec, k, n_tok):
    """The oracle, as it stands, on the first n_tok tokens of the decode batch."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import moe as ref_moe
    from oracle import router as ref_router
    logits = logits_dec[:n_tok].cpu().numpy()
    x = x_dec[:n_tok].float().cpu().numpy()
    ids, _ = ref_router.topk_softmax(logits, k, True)
    experts = np.unique(ids)
    sel = torch.from_numpy(experts).cuda()
    E = w["w13"].shape[0]
    w13 = np.zeros((E,) + tuple(w["w13"].shape[1:]), np.uint8)
    w2 = np.zeros((E,) + tuple(w["w2"].shape[1:]), np.uint8)
    w13[experts] = w["w13"][sel].cpu().numpy()
    w2[experts] = w["w2"][sel].cpu().numpy()
    w13s, w2s = w["w13_scale"].cpu().numpy(), w["w2_scale"].cpu().numpy()
    threads = cpu_threads()
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        ref_moe.moe_forward(x, logits, w13, w13s, w2, w2s, k, True)
        dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n_tok} tokens of the T=64 decode batch ({experts.size} experts, "
                      f"{n_tok * k} token-expert pairs), float64 dequantised GEMMs; {dt:.1f} s"}


def timed_calls(fn, n, warmup=3):
    """fn(i) for i < n after fn(0 .. warmup - 1), each timed call bracketed by
    HIP events on the current stream; returns the per-call milliseconds.

    The timed calls are enqueued right behind the warm-up calls, with no
    synchronisation in between, so the GPU never waits on the host between
    two launches: each pair of events measures the call's GPU time, as a
    back-to-back or graph-replayed loop sees it.  (After an idle GPU the
    first calls of a microsecond-scale layer would also measure the host's
    launch latency.)"""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    for i in range(n):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def run_layer(args, moe, dev, c, w, phases, order):
    """The headline step: plain forwards timed over exactly args.steps steps,
    then a traced pass for the stage times."""
    import numpy as np
    import torch
    H, I, E, k = c["H"], c["I"], c["E"], c["top_k"]

    def run(ph, events=None):
        moe.moe_fp8_forward(ph["x"], ph["logits"], *w, k, True, out=ph["out"], workspace=ph["ws"],
                            events=events)

    for _ in range(args.warmup):
        for n in order:
            run(phases[n])
    # exactly args.steps steps, plain forwards; events between the phases
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        for i, n in enumerate(order):
            run(phases[n])
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [ev[s][0].elapsed_time(ev[s][-1]) for s in range(args.steps)]
    phase_ms = {n: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
                for i, n in enumerate(order)}

    # the same steps through the traced forward: per-stage HIP events on the launch stream
    nst = len(moe.STAGES)
    tev = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
               for _ in range(args.steps)] for n in order}
    for n in order:
        for lst in tev[n]:
            for e in lst:
                e.record()          # creates the HIP events
    torch.cuda.synchronize()
    for s in range(args.steps):
        for n in order:
            run(phases[n], tev[n][s])
    torch.cuda.synchronize()

    result, kernels = {}, {}
    for n in order:
        ph = phases[n]
        T = ph["T"]
        taps = moe.workspace_taps(ph["ws"], T, H, I, E, k)
        alg = algorithmic(taps["topk_ids"].cpu().numpy(), T, H, I, E, k)
        st = np.array([[tev[n][s][i].elapsed_time(tev[n][s][i + 1]) for i in range(nst)]
                       for s in range(args.steps)])
        sm = stats(phase_ms[n])
        lb, lf = alg["layer_bytes"], alg["layer_flops"]
        t = sm["median_ms"] * 1e-3
        tgt = TARGETS.get((args.workload, T))
        fr = fractions(lb, lf, t)
        result[n] = {"T": T, **sm, "tokens_per_s": T / t, "active_experts": alg["active_experts"],
                     "alg_bytes": lb, "alg_flops": lf, **fr,
                     "target": None if tgt is None else
                     {"bound": tgt[0], "frac": tgt[1], "met": fr[tgt[0] + "_frac"] >= tgt[1]},
                     "stage_ms_mean": {s: float(v) for s, v in zip(moe.STAGES, st.mean(axis=0))},
                     "stage_ms_median": {s: float(v) for s, v in zip(moe.STAGES, np.median(st, axis=0))},
                     "traced_ms_mean": float(st.sum(axis=1).mean())}
        for i, s in enumerate(moe.STAGES):
            b, f = alg["stage"][s]
            kernels[f"{n}.{s}"] = {"ms": float(st[:, i].mean()), "bytes": b, "flops": f, "phase": n}
    return {"wall_s": wall, "step_ms": stats(step_ms), "phases": result, "kernels": kernels}


def dominant_roofline(kernels, workload, peaks):
    """Roofline of the kernel with the longest mean launch: a prefill-phase
    kernel against the dense-FP8 MFMA peak (the bar prefill batches are held
    to), a decode-phase kernel against the HBM peak."""
    name = max(kernels, key=lambda s: kernels[s]["ms"])
    k = kernels[name]
    bound = "mfma" if k["phase"] == "prefill" and k["flops"] else "hbm"
    roof = roofline_at(k["bytes"], k["flops"], k["ms"] * 1e-3, bound)
    if bound == "mfma":
        roof["frac_of_f16_peak"] = roof["achieved"] / (MFMA_F16_PEAK / 1e12)
    roof["hbm_frac"] = k["bytes"] / (k["ms"] * 1e-3) / HBM_PEAK
    if peaks:
        key = "mfma_fp8_TFLOP_per_s" if bound == "mfma" else "hbm_read_GB_per_s"
        roof["frac_of_measured_peak"] = roof["achieved"] / peaks[key]
    traffic = None
    src = os.path.join(ROOT, "fp8_block_quantized_amd", "csrc", "gemm.hip")
    same_code = kernel_code_digest(src) == TRAFFIC_CODE_DIGEST
    if workload == "dsv3" and same_code and name in TRAFFIC:
        traffic = float(sum(TRAFFIC[name]))
    roof.update({"kernel": name, "traffic": traffic, "traffic_unit": "bytes per launch",
                 "alg_bytes_per_launch": k["bytes"], "alg_flops_per_launch": k["flops"],
                 "ms_per_launch": k["ms"], "timing": "mean of HIP events on the launch stream "
                                                     "around the kernel, traced pass"})
    return roof


def run_configs(args, moe, dev, skip):
    """Every other workload and batch size, plain forwards, median / p10 / p90."""
    import numpy as np
    import torch
    from synth import MOE_WORKLOADS, make_activations, make_weights
    out = {}
    for name in ("tiny", "mixtral", "qwen3", "dsv3"):
        c = MOE_WORKLOADS[name]
        Ts = [T for T in c["T"] if (name, T) not in skip]
        if not Ts:
            continue
        H, I, E, k = c["H"], c["I"], c["E"], c["top_k"]
        base = 1000 * c["index"]
        w = make_weights(H, I, E, base + 2, dev)
        wbytes = sum(t.numel() * t.element_size() for t in w)
        # replicas so that the weights a call touches are not in the 256 MB
        # last-level cache when it comes round again (a copy of the whole set
        # per replica; small-batch calls touch only a few experts of each)
        nrep = 12 if name == "qwen3" else 1
        reps = [w] + [tuple(t.clone() for t in w) for _ in range(nrep - 1)]
        for T in Ts:
            x, logits = make_activations(H, E, T, base, c["logits"], dev)
            ws = moe.alloc_workspace(T, H, I, E, k, dev)
            o = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            # the warm-up calls go once round the replicas, so that the timed
            # calls see the steady state of the rotation (no first touch of a
            # replica's pages inside the timed region)
            ms = timed_calls(lambda i: moe.moe_fp8_forward(x, logits, *reps[i % nrep], k, True,
                                                           out=o, workspace=ws), args.steps,
                             warmup=max(3, nrep))
            taps = moe.workspace_taps(ws, T, H, I, E, k)
            alg = algorithmic(taps["topk_ids"].cpu().numpy(), T, H, I, E, k)
            sm = stats(ms)
            fr = fractions(alg["layer_bytes"], alg["layer_flops"], sm["median_ms"] * 1e-3)
            tgt = TARGETS.get((name, T))
            out[f"{name}.T{T}"] = {
                "workload": f"{name}-shaped H={H} I={I} E={E} top_k={k}", "T": T,
                "block_m": taps["block_m"], **sm, "tokens_per_s": T / (sm["median_ms"] * 1e-3),
                "active_experts": alg["active_experts"], "alg_bytes": alg["layer_bytes"],
                "alg_flops": alg["layer_flops"], **fr, "weight_replicas": nrep,
                "weight_bytes_per_replica": wbytes,
                "target": None if tgt is None else
                {"bound": tgt[0], "frac": tgt[1], "met": fr[tgt[0] + "_frac"] >= tgt[1]}}
            del x, logits, ws, o
        del w, reps
        torch.cuda.empty_cache()
    return out


def run_quant(args, moe, dev):
    import numpy as np
    import torch
    from synth import QUANT_WORKLOAD, quant_input
    M, K = QUANT_WORKLOAD["M"], QUANT_WORKLOAD["K"]
    xq_in = [quant_input(device=dev, seed_base=4000 + 10 * i) for i in range(3)]
    q_out = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(3)]
    s_out = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _ in range(3)]
    ms = timed_calls(lambda i: moe.per_token_group_quant_fp8(xq_in[i % 3], q=q_out[i % 3],
                                                             scales=s_out[i % 3]), args.steps)
    sm = stats(ms)
    q_bytes = 2 * M * K + M * K + 4 * M * (K // 128)
    res = {"M": M, "K": K, **sm, "alg_bytes": q_bytes,
           "GB_per_s": q_bytes / (sm["median_ms"] * 1e-3) / 1e9,
           "hbm_frac": q_bytes / (sm["median_ms"] * 1e-3) / HBM_PEAK}
    e_out = [torch.empty((M, K // 32), dtype=torch.uint8, device=dev) for _ in range(3)]
    ms = timed_calls(lambda i: moe.per_token_group_quant_fp8_fmt(xq_in[i % 3], 32, "ue8m0",
                                                                 q=q_out[i % 3], scales=e_out[i % 3]),
                     args.steps)
    sm = stats(ms)
    q_bytes = 2 * M * K + M * K + M * (K // 32)
    res["mxfp8_group32_ue8m0"] = {**sm, "alg_bytes": q_bytes,
                                  "GB_per_s": q_bytes / (sm["median_ms"] * 1e-3) / 1e9,
                                  "hbm_frac": q_bytes / (sm["median_ms"] * 1e-3) / HBM_PEAK}
    return res


def run_linear(args, moe, dev):
    import torch
    from synth import LINEAR_WORKLOAD, MX_LINEAR_WORKLOAD, make_linear, make_mx_linear

    def time_linear(fn, ws_bytes, make, wl, scale_bytes):
        LN, LK = wl["N"], wl["K"]
        res = {"workload": f"DeepSeek-V3-shaped dense down projection N={LN} K={LK}"}
        for LM in wl["M"]:
            lx, lw, lws = make(LM, LN, LK, 1000 * wl["index"], device=dev)
            # three weight replicas in rotation (3 x 132 MB > the 256 MB cache),
            # so that every call streams its weights from HBM
            lrep = [(lw, lws)] + [(lw.clone(), lws.clone()) for _ in range(2)]
            lout = torch.empty((LM, LN), dtype=torch.bfloat16, device=dev)
            lwsp = torch.empty(ws_bytes(LM, LN, LK), dtype=torch.uint8, device=dev)
            ms = timed_calls(lambda i: fn(lx, *lrep[i % 3], out=lout, workspace=lwsp), args.steps)
            sm = stats(ms)
            lbytes = LN * LK + scale_bytes(LN, LK) + 2 * LM * LK + 2 * LM * LN
            r = roofline_of(lbytes, 2 * LM * LN * LK, sm["median_ms"] * 1e-3, MFMA_FP8_PEAK)
            r.update({"M": LM, **sm, "alg_bytes": lbytes, "alg_flops": 2 * LM * LN * LK})
            res[f"M{LM}"] = r
            del lx, lw, lws, lrep, lout, lwsp
        return res

    dense = time_linear(moe.fp8_block_linear, moe.fp8_block_linear_workspace_bytes, make_linear,
                        LINEAR_WORKLOAD, lambda n, k: 4 * (n // 128) * (k // 128))
    dense_mx = time_linear(moe.mxfp8_linear, moe.mxfp8_linear_workspace_bytes, make_mx_linear,
                           MX_LINEAR_WORKLOAD, lambda n, k: n * (k // 32))
    return dense, dense_mx


def run_batched(args, moe, dev):
    import torch
    from synth import BATCHED_WORKLOAD as BW
    from synth import make_weights
    bE, bM, bH, bI = BW["E"], BW["M"], BW["H"], BW["I"]
    gb = torch.Generator(device="cpu").manual_seed(1000 * BW["index"] + 1)
    bcounts = torch.randint(BW["min_count"], bM + 1, (bE,), generator=gb, dtype=torch.int32)
    bx = torch.randn((bE, bM, bH), generator=torch.Generator(device=dev).manual_seed(1000 * BW["index"]),
                     device=dev).to(torch.bfloat16)
    bw = make_weights(bH, bI, bE, 1000 * BW["index"] + 2, dev)
    bc_dev = bcounts.to(dev)
    bout = torch.empty_like(bx)
    bws = torch.empty(moe.moe_fp8_batched_workspace_bytes(bE, bM, bH, bI), dtype=torch.uint8, device=dev)
    ms = timed_calls(lambda i: moe.moe_fp8_batched_experts(bx, bc_dev, *bw, out=bout, workspace=bws),
                     args.steps)
    sm = stats(ms)
    rows = int(bcounts.sum())
    active = int((bcounts > 0).sum())
    wbytes = active * (2 * bI * bH + bH * bI + 4 * (2 * bI // 128) * (bH // 128) + 4 * (bH // 128) * (bI // 128))
    bbytes = wbytes + 2 * rows * bH + 2 * bE * bM * bH
    bflops = 6 * rows * bH * bI
    # GEMM1 (4 H I flops per row) runs on f16 MFMAs, GEMM2 (2 H I) on FP8 ones:
    # the peak of the mix is 6 / (4 / f16 peak + 2 / FP8 peak)
    blend = 6.0 / (4.0 / MFMA_F16_PEAK + 2.0 / MFMA_FP8_PEAK)
    batched = roofline_of(bbytes, bflops, sm["median_ms"] * 1e-3, blend)
    batched.update({"workload": f"DeepSeek-V3-shaped experts of one rank of eight: E={bE} max_tokens={bM} "
                                f"H={bH} I={bI}, counts uniform in [{BW['min_count']}, {bM}]",
                    "rows": rows, **sm, "alg_bytes": bbytes, "alg_flops": bflops,
                    "hbm_frac": bbytes / (sm["median_ms"] * 1e-3) / HBM_PEAK})
    return batched


def run_mx(args, moe, dev, c, phases, order):
    import numpy as np
    import torch
    from synth import make_mx_weights
    H, I, E, k = c["H"], c["I"], c["E"], c["top_k"]
    mxw = make_mx_weights(H, I, E, 1000 * c["index"] + 2, dev)
    res = {"workload": f"{args.workload}-shaped MoE layer with MXFP8 weights and activations"}
    for n in order:
        ph = phases[n]
        T = ph["T"]
        mws = torch.empty(moe.moe_fp8_mx_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device=dev)
        ms = timed_calls(lambda i: moe.moe_fp8_mx_forward(ph["x"], ph["logits"], *mxw, k, True,
                                                          out=ph["out"], workspace=mws), args.steps)
        sm = stats(ms)
        ids = moe.workspace_taps(mws, T, H, I, E, k, mx=True)["topk_ids"].cpu().numpy()
        e_act = int(np.unique(ids).size)
        mbytes = e_act * (2 * I * H + H * I) * 33 // 32 + 4 * T * H
        mflops = 6 * T * k * H * I
        r = roofline_of(mbytes, mflops, sm["median_ms"] * 1e-3, MFMA_FP8_PEAK)
        r.update({"T": T, **sm, "tokens_per_s": T / (sm["median_ms"] * 1e-3), "active_experts": e_act,
                  "alg_bytes": mbytes, "alg_flops": mflops,
                  **fractions(mbytes, mflops, sm["median_ms"] * 1e-3)})
        res[n] = r
        del mws
    del mxw
    torch.cuda.empty_cache()
    return res


def run_peaks(args, moe, dev):
    """What the part sustains: a read-only stream of 4 GiB (the weight-streaming
    decode GEMMs' bound), a 1 GiB device copy (read + write) and register-only
    MFMA chains of the two GEMMs' instruction types."""
    import torch
    nb = 4 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    nblk = 2048              # eight 16-byte loads in flight per thread: 7.0 TB/s on the box
    sink = torch.empty(nblk * 256, dtype=torch.int32, device=dev)
    ms = timed_calls(lambda i: moe.moe_hbm_read_probe(src, nblk, sink), 5, warmup=2)
    peaks = {"hbm_read_GB_per_s": nb / (min(ms) * 1e-3) / 1e9}
    del src, sink
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ms = timed_calls(lambda i: dst.copy_(src), 5, warmup=2)
    peaks["hbm_copy_GB_per_s"] = 2 * nb / (min(ms) * 1e-3) / 1e9
    del src, dst
    nblk = 2048
    sink = torch.empty(nblk * 256, dtype=torch.float32, device=dev)
    for kind, iters in (("f16", 5000), ("fp8", 2500)):
        fl = [0]

        def go(i):
            fl[0] = moe.moe_mfma_rate_probe(kind, iters, nblk, sink)
        ms = timed_calls(go, 3, warmup=1)
        peaks[f"mfma_{kind}_TFLOP_per_s"] = fl[0] / (min(ms) * 1e-3) / 1e12
    del sink
    return peaks


def progress(what, t0):
    """one line per finished section on stderr, so a long run shows it is alive"""
    print(f"[bench] {what} done after {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)


def main():
    t_start = time.perf_counter()
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

    import fp8_block_quantized_amd as moe
    from synth import MOE_WORKLOADS, make_activations, make_weights

    moe.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = MOE_WORKLOADS[args.workload]
    H, I, E, k = c["H"], c["I"], c["E"], c["top_k"]
    base = 1000 * c["index"]
    T_dec, T_pre = batch_sizes(args.workload)
    # the headline weights and batches, for the sections that run on them
    need_layer = "layer" in args.sections or "mx" in args.sections
    w = make_weights(H, I, E, base + 2, dev) if "layer" in args.sections else None
    phases = {}
    for name, T in (("decode", T_dec), ("prefill", T_pre)):
        if args.phase not in ("both", name) or not need_layer:
            continue
        x, logits = make_activations(H, E, T, base, c["logits"], dev)
        phases[name] = {"T": T, "x": x, "logits": logits,
                        "ws": moe.alloc_workspace(T, H, I, E, k, dev),
                        "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev)}
    order = ["decode", "prefill"] if T_dec != T_pre else ["decode"]
    if args.phase != "both":
        order = [args.phase]
    order = [n for n in order if n in phases]

    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8e4m3 (GEMM2 FP8 MFMA, f32 acc; GEMM1 exact f16 MFMA, f64 acc at decode, "
                    "f32 at prefill; bf16 in/out)",
           "data": "synthetic",
           "config": {"workload": f"{args.workload}-shaped MoE layer H={H} I={I} E={E} top_k={k}, "
                                  + " + ".join(f"{n} T={phases[n]['T']}" for n in order) + " per step",
                      "H": H, "I": I, "E": E, "top_k": k, "T": {n: phases[n]["T"] for n in order},
                      "block_m": {n: moe.moe_fp8_block_m(phases[n]["T"], H, I, E, k) for n in order},
                      "sections": args.sections}}
    layer = None
    if "layer" in args.sections:
        layer = run_layer(args, moe, dev, c, w, phases, order)
        tokens = sum(phases[n]["T"] for n in order)
        out["value"] = tokens / (layer["wall_s"] / args.steps)
        out["ms_per_step"] = layer["wall_s"] / args.steps * 1e3
        out["step_ms"] = layer["step_ms"]
        out["phases"] = layer["phases"]
        progress("layer", t_start)

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if "configs" in args.sections:
        out["configs"] = run_configs(args, moe, dev, skip={(args.workload, T) for T in (T_dec, T_pre)}
                                     if layer else set())
        progress("configs", t_start)
    if "quant" in args.sections:
        out["quant_standalone"] = run_quant(args, moe, dev)
        progress("quant", t_start)
    if "linear" in args.sections:
        out["dense_linear"], out["dense_linear_mxfp8"] = run_linear(args, moe, dev)
        progress("linear", t_start)
    if "batched" in args.sections:
        out["batched_experts"] = run_batched(args, moe, dev)
        progress("batched", t_start)
    if "mx" in args.sections:
        out["moe_mxfp8"] = run_mx(args, moe, dev, c, phases, order)
        progress("mx", t_start)
    peaks = None
    if "peaks" in args.sections:
        peaks = run_peaks(args, moe, dev)
        progress("peaks", t_start)
    out["measured_peaks"] = peaks
    out["roofline"] = dominant_roofline(layer["kernels"], args.workload, peaks) if layer else None
    out["kernels"] = layer["kernels"] if layer else None

    if layer and not args.no_cpu_baseline and "decode" in phases:
        ph = phases["decode"]
        wd = dict(zip(("w13", "w13_scale", "w2", "w2_scale"), w))
        out["cpu_baseline"] = cpu_baseline(wd, ph["x"], ph["logits"], k, args.cpu_sample_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
