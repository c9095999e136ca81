#!/usr/bin/env python3
"""Benchmark of the fused FP8 block-quantized MoE forward on one MI355X.

Workload (default "dsv3"): a DeepSeek-V3-shaped routed-expert layer, H=7168,
I=2048, E=256, top_k=8 softmax routing with renormalisation and a seeded
+-0.5 per-expert logit bias (load skew), FP8 e4m3fn weights with 128x128
block scales (~11.3 GB, drawn N(0, 0.02)), bf16 activations N(0, 1) with
dynamic per-token 128-group quantisation.  One step = one decode batch of
T=64 tokens plus one prefill batch of T=8192 tokens through the whole path
(router, sort-and-pad, activation quant, GEMM1 + SiLU*mul + requant, GEMM2 +
routing weight, combine).  Inputs are resident in HBM before timing starts.
The standalone activation quantiser is also timed on its own workload, bf16
[16384, 7168] with 1% x100 outliers, and the dense block-FP8 linear on a
DeepSeek-V3-shaped down projection (7168 x 18432) at M = 64 and 8192.

Prints one JSON line.  value = tokens per second over the step.
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
# MFMA type of each contraction: GEMM1 runs on f16 MFMAs of exactly converted
# e4m3 operands, GEMM2 on FP8 MFMAs
STAGE_PEAK = {"gemm1": MFMA_F16_PEAK, "gemm2": MFMA_FP8_PEAK}

# HBM bytes per launch of the two GEMMs, from rocprofv3 FETCH_SIZE (x2) and
# WRITE_SIZE (x1) passes, each scaled by what the same counter reads for a
# plain 1 GiB copy (profiles/hbm_counters_dsv3_*.md).  Valid only for the
# kernel source they were taken on: bench reports null traffic once
# gemm.hip differs from this hash.
TRAFFIC_SOURCE_SHA256 = "c57127a888b3849badba0b4dbc0ef443f82969b6c542f60ea5be158607bd4216"
TRAFFIC = {  # (read bytes, write bytes) per launch, DeepSeek-V3-shaped workload
    "prefill.gemm1": (10748266557, 184470912),
    "prefill.gemm2": (4397065067, 1208267115),
    "decode.gemm1": (4795674564, 5724203),
    "decode.gemm2": (2408673012, 7340288),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dsv3", choices=["dsv3", "mixtral", "qwen3", "tiny"])
    p.add_argument("--cpu-sample-tokens", type=int, default=16)
    p.add_argument("--phase", default="both", choices=["both", "decode", "prefill"],
                   help="time one batch size only (for per-kernel profiles)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--layer-only", action="store_true",
                   help="time only the MoE layer (skip the standalone quantiser, dense linears, "
                        "batched experts and MXFP8 layer)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="also run a plain device-to-device copy of this many MiB (three times), "
                        "the reference kernel that scales the HBM byte counters")
    return p.parse_args()


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
    t_hbm, t_mfma = nbytes / HBM_PEAK, flops / mfma_peak
    if t_mfma > t_hbm:
        a = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": a, "peak": mfma_peak / 1e12, "unit": "TFLOP/s",
                "frac": a / (mfma_peak / 1e12)}
    a = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": a / (HBM_PEAK / 1e9)}


def cpu_baseline(w, x_dec, logits_dec, k, n_tok):
    """The oracle, as it stands, on the first n_tok tokens of the decode batch."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

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
    t0 = time.perf_counter()
    ref_moe.moe_forward(x, logits, w13, w13s, w2, w2s, k, True)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_tok} tokens of the T=64 decode batch ({experts.size} experts, "
                      f"{n_tok * k} token-expert pairs), float64 dequantised GEMMs; {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fp8_block_quantized_amd as moe
    from synth import MOE_WORKLOADS, make_activations, make_weights, quant_input

    moe.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = MOE_WORKLOADS[args.workload]
    H, I, E, k = c["H"], c["I"], c["E"], c["top_k"]
    base = 1000 * c["index"]
    T_dec, T_pre = batch_sizes(args.workload)
    w13, w13s, w2, w2s = make_weights(H, I, E, base + 2, dev)
    wts = {"w13": w13, "w13_scale": w13s, "w2": w2, "w2_scale": w2s}
    phases = {}
    for name, T in (("decode", T_dec), ("prefill", T_pre)):
        if args.phase not in ("both", name):
            continue
        x, logits = make_activations(H, E, T, base, c["logits"], dev)
        phases[name] = {"T": T, "x": x, "logits": logits,
                        "ws": moe.alloc_workspace(T, H, I, E, k, dev),
                        "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev)}
    order = ["decode", "prefill"] if T_dec != T_pre else ["decode"]
    if args.phase != "both":
        order = [args.phase]

    def run(ph, events=None):
        moe.moe_fp8_forward(ph["x"], ph["logits"], w13, w13s, w2, w2s, k, True,
                            out=ph["out"], workspace=ph["ws"], events=events)

    for _ in range(args.warmup):
        for n in order:
            run(phases[n])
    torch.cuda.synchronize()

    nst = len(moe.STAGES)
    evs = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
               for _ in range(args.steps)] for n in order}
    for n in order:
        for lst in evs[n]:
            for e in lst:
                e.record()          # creates the HIP events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for n in order:
            run(phases[n], evs[n][s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    result_phases = {}
    kernels = {}
    for n in order:
        ph = phases[n]
        T = ph["T"]
        taps = moe.workspace_taps(ph["ws"], T, H, I, E, k)
        alg = algorithmic(taps["topk_ids"].cpu().numpy(), T, H, I, E, k)
        st_ms = np.array([[evs[n][s][i].elapsed_time(evs[n][s][i + 1]) for i in range(nst)]
                          for s in range(args.steps)]).mean(axis=0)
        layer_ms = float(st_ms.sum())
        lb, lf = alg["layer_bytes"], alg["layer_flops"]
        result_phases[n] = {
            "T": T, "ms": layer_ms, "tokens_per_s": T / (layer_ms * 1e-3),
            "active_experts": alg["active_experts"],
            "alg_bytes": lb, "alg_flops": lf,
            "hbm_frac": lb / (layer_ms * 1e-3) / HBM_PEAK,
            "mfma_frac": lf / (layer_ms * 1e-3) / MFMA_FP8_PEAK,
            "stage_ms": {s: float(v) for s, v in zip(moe.STAGES, st_ms)},
        }
        for s, v in zip(moe.STAGES, st_ms):
            b, f = alg["stage"][s]
            kernels[f"{n}.{s}"] = {"ms": float(v), "bytes": b, "flops": f,
                                   "peak": STAGE_PEAK.get(s, MFMA_FP8_PEAK)}

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def extras():
        """The timed sections after the layer: standalone quantiser, dense
        linears, batched experts and the MXFP8 layer."""
        # standalone activation quantiser, rotating three input buffers (> MALL)
        from synth import QUANT_WORKLOAD
        M, K = QUANT_WORKLOAD["M"], QUANT_WORKLOAD["K"]
        xq_in = [quant_input(device=dev, seed_base=4000 + 10 * i) for i in range(3)]
        q_out = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(3)]
        s_out = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _ in range(3)]
        for i in range(3):
            moe.per_token_group_quant_fp8(xq_in[i], q=q_out[i], scales=s_out[i])
        qe = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
        torch.cuda.synchronize()
        for s in range(args.steps):
            qe[2 * s].record()
            moe.per_token_group_quant_fp8(xq_in[s % 3], q=q_out[s % 3], scales=s_out[s % 3])
            qe[2 * s + 1].record()
        torch.cuda.synchronize()
        q_ms = float(np.mean([qe[2 * s].elapsed_time(qe[2 * s + 1]) for s in range(args.steps)]))
        q_bytes = 2 * M * K + M * K + 4 * M * (K // 128)
        quant = {"M": M, "K": K, "ms": q_ms, "GB_per_s": q_bytes / (q_ms * 1e-3) / 1e9,
                 "hbm_frac": q_bytes / (q_ms * 1e-3) / HBM_PEAK}

        # the same quantiser with MXFP8 scales: groups of 32, UE8M0 exponent bytes
        e_out = [torch.empty((M, K // 32), dtype=torch.uint8, device=dev) for _ in range(3)]
        for i in range(3):
            moe.per_token_group_quant_fp8_fmt(xq_in[i], 32, "ue8m0", q=q_out[i], scales=e_out[i])
        torch.cuda.synchronize()
        for s in range(args.steps):
            qe[2 * s].record()
            moe.per_token_group_quant_fp8_fmt(xq_in[s % 3], 32, "ue8m0", q=q_out[s % 3], scales=e_out[s % 3])
            qe[2 * s + 1].record()
        torch.cuda.synchronize()
        q_ms = float(np.mean([qe[2 * s].elapsed_time(qe[2 * s + 1]) for s in range(args.steps)]))
        q_bytes = 2 * M * K + M * K + M * (K // 32)
        quant["mxfp8_group32_ue8m0"] = {"ms": q_ms, "GB_per_s": q_bytes / (q_ms * 1e-3) / 1e9,
                                        "hbm_frac": q_bytes / (q_ms * 1e-3) / HBM_PEAK}
        del xq_in, q_out, s_out, e_out

        # dense linears (the layer's E = 1 neighbour), decode and prefill batches:
        # block FP8 (128x128 weight blocks, float32 scales) and MXFP8 ([1, 32], UE8M0)
        from synth import LINEAR_WORKLOAD, MX_LINEAR_WORKLOAD, make_linear, make_mx_linear

        def time_linear(fn, ws_bytes, make, wl, scale_bytes):
            LN, LK = wl["N"], wl["K"]
            res = {"workload": f"DeepSeek-V3-shaped dense down projection N={LN} K={LK}"}
            for LM in wl["M"]:
                lx, lw, lws = make(LM, LN, LK, 1000 * wl["index"], device=dev)
                # three weight replicas in rotation (3 x 132 MB > the 256 MB MALL),
                # so that every call streams its weights from HBM
                lrep = [(lw, lws)] + [(lw.clone(), lws.clone()) for _ in range(2)]
                lout = torch.empty((LM, LN), dtype=torch.bfloat16, device=dev)
                lwsp = torch.empty(ws_bytes(LM, LN, LK), dtype=torch.uint8, device=dev)
                for i in range(3):
                    fn(lx, *lrep[i], out=lout, workspace=lwsp)
                le = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                torch.cuda.synchronize()
                le[0].record()
                for i in range(args.steps):
                    fn(lx, *lrep[i % 3], out=lout, workspace=lwsp)
                le[1].record()
                torch.cuda.synchronize()
                lms = le[0].elapsed_time(le[1]) / args.steps
                lbytes = LN * LK + scale_bytes(LN, LK) + 2 * LM * LK + 2 * LM * LN
                r = roofline_of(lbytes, 2 * LM * LN * LK, lms * 1e-3, MFMA_FP8_PEAK)
                r.update({"M": LM, "ms": lms, "alg_bytes": lbytes, "alg_flops": 2 * LM * LN * LK})
                res[f"M{LM}"] = r
                del lx, lw, lws, lrep, lout, lwsp
            return res

        dense = time_linear(moe.fp8_block_linear, moe.fp8_block_linear_workspace_bytes, make_linear,
                            LINEAR_WORKLOAD, lambda n, k: 4 * (n // 128) * (k // 128))
        dense_mx = time_linear(moe.mxfp8_linear, moe.mxfp8_linear_workspace_bytes, make_mx_linear,
                               MX_LINEAR_WORKLOAD, lambda n, k: n * (k // 32))

        # batched (masked) expert format: one rank's experts, device-side counts
        from synth import BATCHED_WORKLOAD as BW
        bE, bM, bH, bI = BW["E"], BW["M"], BW["H"], BW["I"]
        gb = torch.Generator(device="cpu").manual_seed(1000 * BW["index"] + 1)
        bcounts = torch.randint(BW["min_count"], bM + 1, (bE,), generator=gb, dtype=torch.int32)
        bx = torch.randn((bE, bM, bH), generator=torch.Generator(device=dev).manual_seed(1000 * BW["index"]),
                         device=dev).to(torch.bfloat16)
        bw = make_weights(bH, bI, bE, 1000 * BW["index"] + 2, dev)
        bc_dev = bcounts.to(dev)
        bout = torch.empty_like(bx)
        bws = torch.empty(moe.moe_fp8_batched_workspace_bytes(bE, bM, bH, bI), dtype=torch.uint8, device=dev)
        for _ in range(3):
            moe.moe_fp8_batched_experts(bx, bc_dev, *bw, out=bout, workspace=bws)
        be = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        be[0].record()
        for _ in range(args.steps):
            moe.moe_fp8_batched_experts(bx, bc_dev, *bw, out=bout, workspace=bws)
        be[1].record()
        torch.cuda.synchronize()
        bms = be[0].elapsed_time(be[1]) / args.steps
        rows = int(bcounts.sum())
        active = int((bcounts > 0).sum())
        wbytes = active * (2 * bI * bH + bH * bI + 4 * (2 * bI // 128) * (bH // 128) + 4 * (bH // 128) * (bI // 128))
        bbytes = wbytes + 2 * rows * bH + 2 * bE * bM * bH
        bflops = 6 * rows * bH * bI
        # GEMM1 (4 H I flops per row) runs on f16 MFMAs, GEMM2 (2 H I) on FP8 ones:
        # the peak of the mix is 6 / (4 / f16 peak + 2 / FP8 peak)
        blend = 6.0 / (4.0 / MFMA_F16_PEAK + 2.0 / MFMA_FP8_PEAK)
        batched = roofline_of(bbytes, bflops, bms * 1e-3, blend)
        batched.update({"workload": f"DeepSeek-V3-shaped experts of one rank of eight: E={bE} max_tokens={bM} "
                                    f"H={bH} I={bI}, counts uniform in [{BW['min_count']}, {bM}]",
                        "rows": rows, "ms": bms, "alg_bytes": bbytes, "alg_flops": bflops})
        del bx, bw, bout, bws

        # the MXFP8 layer ([1, 32] blocks, UE8M0 scales, FP8 MFMAs in both GEMMs)
        # on the same inputs, with the same weights cast to MXFP8
        from synth import make_mx_weights
        mxw = make_mx_weights(H, I, E, base + 2, dev)
        mx_layer = {"workload": f"{args.workload}-shaped MoE layer with MXFP8 weights and activations"}
        for n in order:
            ph = phases[n]
            T = ph["T"]
            mws = torch.empty(moe.moe_fp8_mx_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device=dev)
            for _ in range(3):
                moe.moe_fp8_mx_forward(ph["x"], ph["logits"], *mxw, k, True, out=ph["out"], workspace=mws)
            me = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            me[0].record()
            for _ in range(args.steps):
                moe.moe_fp8_mx_forward(ph["x"], ph["logits"], *mxw, k, True, out=ph["out"], workspace=mws)
            me[1].record()
            torch.cuda.synchronize()
            mms = me[0].elapsed_time(me[1]) / args.steps
            ids = moe.workspace_taps(mws, T, H, I, E, k, mx=True)["topk_ids"].cpu().numpy()
            e_act = int(np.unique(ids).size)
            mbytes = e_act * (2 * I * H + H * I) * 33 // 32 + 4 * T * H
            mflops = 6 * T * k * H * I
            r = roofline_of(mbytes, mflops, mms * 1e-3, MFMA_FP8_PEAK)
            r.update({"T": T, "ms": mms, "tokens_per_s": T / (mms * 1e-3), "active_experts": e_act,
                      "alg_bytes": mbytes, "alg_flops": mflops})
            mx_layer[n] = r
            del mws
        del mxw
        # what this part sustains: a plain 1 GiB device copy (read + write) and
        # register-only MFMA chains of the two GEMMs' instruction types
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        copy_ms = []
        for _ in range(5):
            ce[0].record()
            dst.copy_(src)
            ce[1].record()
            torch.cuda.synchronize()
            copy_ms.append(ce[0].elapsed_time(ce[1]))
        del src, dst
        nblk = 2048
        sink = torch.empty(nblk * 256, dtype=torch.float32, device=dev)
        peaks = {"hbm_copy_GB_per_s": 2 * nb / (min(copy_ms) * 1e-3) / 1e9}
        for kind, iters in (("f16", 5000), ("fp8", 2500)):
            moe.moe_mfma_rate_probe(kind, 100, nblk, sink)
            torch.cuda.synchronize()
            ce[0].record()
            fl = moe.moe_mfma_rate_probe(kind, iters, nblk, sink)
            ce[1].record()
            torch.cuda.synchronize()
            peaks[f"mfma_{kind}_TFLOP_per_s"] = fl / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e12
        del sink
        return quant, dense, dense_mx, batched, mx_layer, peaks

    if args.layer_only:
        quant = dense = dense_mx = batched = mx_layer = peaks = None
    else:
        quant, dense, dense_mx, batched, mx_layer, peaks = extras()

    dom_name = max(kernels, key=lambda s: kernels[s]["ms"])
    dom = kernels[dom_name]
    roof = roofline_of(dom["bytes"], dom["flops"], dom["ms"] * 1e-3, dom["peak"])
    traffic = None
    src = os.path.join(ROOT, "fp8_block_quantized_amd", "csrc", "gemm.hip")
    with open(src, "rb") as fh:
        same_source = hashlib.sha256(fh.read()).hexdigest() == TRAFFIC_SOURCE_SHA256
    if args.workload == "dsv3" and same_source and dom_name in TRAFFIC:
        traffic = float(sum(TRAFFIC[dom_name]))
    if peaks:
        key = {"GB/s": "hbm_copy_GB_per_s"}.get(roof["unit"],
                                              "mfma_f16_TFLOP_per_s" if dom["peak"] == MFMA_F16_PEAK
                                              else "mfma_fp8_TFLOP_per_s")
        roof["frac_of_measured_peak"] = roof["achieved"] / peaks[key]
    roof.update({"kernel": dom_name, "traffic": traffic, "traffic_unit": "bytes per launch",
                 "alg_bytes_per_launch": dom["bytes"], "alg_flops_per_launch": dom["flops"],
                 "ms_per_launch": dom["ms"]})

    tokens = sum(phases[n]["T"] for n in order)
    ms_step = wall / args.steps * 1e3
    out = {
        "metric": METRIC, "value": tokens / (wall / args.steps), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 (GEMM2 FP8 MFMA, f32 acc; GEMM1 exact f16 MFMA, f64 acc at decode, "
                 "f32 at prefill; bf16 in/out)",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}-shaped MoE layer H={H} I={I} E={E} top_k={k}, "
                               + " + ".join(f"{n} T={phases[n]['T']}" for n in order) + " per step",
                   "H": H, "I": I, "E": E, "top_k": k, "T": {n: phases[n]["T"] for n in order},
                   "block_m": {n: moe.moe_fp8_block_m(phases[n]["T"], H, I, E, k) for n in order}},
        "roofline": roof,
        "phases": result_phases,
        "quant_standalone": quant,
        "dense_linear": dense,
        "dense_linear_mxfp8": dense_mx,
        "batched_experts": batched,
        "moe_mxfp8": mx_layer,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline and "decode" in phases:
        ph = phases["decode"]
        out["cpu_baseline"] = cpu_baseline(wts, ph["x"], ph["logits"], k, args.cpu_sample_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
