#!/usr/bin/env python3
"""Benchmark of the block-scaled TN GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

One step is one call of the headline path: the W4A4 NVFP4 TN GEMM
C[8192,5376] = A[8192,14336] . W[5376,14336]^T (NVFP4 E2M1 codes, E4M3 scales
per 16, FP32 tensor scales; exact E2M1->E4M3 conversion onto the FP8 MFMA,
per-16 FP32 scale step, BF16 output), inputs resident in HBM.  W warmup steps
run untimed, then exactly K steps are timed between two device
synchronisations with HIP events on the stream the kernel runs on.  `value`
is TFLOP/s = 2*M*N*K / time per step.  The headline's inputs are uploaded
first and its steps are timed after the decode and BF16 legs, on a GPU at
the clock it holds under load; every other leg warms up for WARM_S seconds
of calls before it is timed.

The same JSON line also carries: the roofline of that kernel, the FP64 CPU
oracle timed on the host on a bounded sample of the same workload
(`cpu_baseline`), a sampled parity check of the timed output against the
oracle, the W4A8 swap-AB decode shapes (M = 1, 8, 32, 128; GB/s against the
HBM roofline, weights rotated over 8 copies so the 256 MB Infinity Cache
cannot serve them), the small-M W4A16 shapes (M = 1, 16, 128, likewise), and
the BF16 and MXFP8-MoE configurations.  Decode-sized calls are timed as HIP
graphs of back-to-back calls replayed on the device ("us"; the per-call
launch cost of the Python binding exceeds such a kernel's duration), with
the eager per-call loop beside them ("eager_us").

Only one GPU is supported: --gpus N with N > 1 exits with a message.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, N, K = 8192, 5376, 14336
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "fp32": 157.3, "hbm": 8000.0}  # TFLOP/s, GB/s
# plain FP32 vector FMA without packed instructions: 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz
PEAK_VALU_F32 = 78.6
# seconds of warm-up calls (beyond the warm-up count) before each secondary leg is timed
WARM_S = 0.25


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline kernel only")
    ap.add_argument("--only", default="",
                    help="w4a4|w4a8|w4a16|bf16|bf16_grad|moe|moe_decode|moe_nvfp4 (profiling runs)")
    ap.add_argument("--moe-dec-tokens", default="1,16",
                    help="token counts of the decode-sized MoE calls")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain copy kernel of this many MiB (counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'--only w4a4 --copy-calib-mib N' into profiles/traffic.json")
    return ap.parse_args()


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_scaled_precision_tn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_file, key):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(p))[key]
    except (OSError, KeyError, ValueError):
        return None
    if d.get("src_hash") != src_hash(kernel_file, "common.h"):
        return None
    return d.get("bytes_per_launch")


def _pmc_means(d, counter):
    """Mean counter value per dispatch, by kernel name, from a rocprofv3 --pmc
    CSV directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(fetch_dir, write_dir, calib_mib):
    """HBM traffic of the W4A4 kernel per launch: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by bytes/KiB-read of the plain copy kernel of
    known size from the same run (it reads and writes calib_mib MiB)."""
    fetch, write = _pmc_means(fetch_dir, "FETCH_SIZE"), _pmc_means(write_dir, "WRITE_SIZE")
    pick = lambda d, sub: [v for k, v in d.items() if sub in k]  # noqa: E731
    kf, kw = pick(fetch, "w4a4_fp8route"), pick(write, "w4a4_fp8route")
    cf, cw = pick(fetch, "MulFunctor"), pick(write, "MulFunctor")
    if not (kf and kw and cf and cw):
        raise SystemExit(f"kernels not found: {sorted(fetch)}")
    nbytes = calib_mib * (1 << 20)
    f_fetch, f_write = nbytes / (cf[0] * 1024), nbytes / (cw[0] * 1024)
    t_fetch, t_write = kf[0] * 1024 * f_fetch, kw[0] * 1024 * f_write
    algo = M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + 8 + 2 * M * N
    out = {"w4a4_m8192": {
        "src_hash": src_hash("gemm_w4a4.hip", "common.h"),
        "bytes_per_launch": round(t_fetch + t_write),
        "fetch_bytes": round(t_fetch), "write_bytes": round(t_write),
        "fetch_kib_raw": kf[0], "write_kib_raw": kw[0],
        "copy_calibration": {"mib": calib_mib, "fetch_kib_raw": cf[0], "write_kib_raw": cw[0],
                             "fetch_factor": f_fetch, "write_factor": f_write},
        "algorithmic_bytes": algo,
        "traffic_over_algorithmic": round((t_fetch + t_write) / algo, 3)}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def warm(torch, fn, warmup, warm_s):
    """warmup calls of fn, then more (in batches of 8) until warm_s seconds
    have passed: a secondary leg's calls then start at the clock the GPU holds
    under load, whatever --warmup says."""
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(8):
            fn(0)
        torch.cuda.synchronize()


def timed(torch, fn, steps, warmup, stream, warm_s=WARM_S):
    warm(torch, fn, warmup, warm_s)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per call


def timed_graph(torch, fn, calls, steps, warmup):
    """Device time per call of fn(0) .. fn(calls - 1) captured back to back
    in one HIP graph and replayed `steps` times: the launch cost of the
    Python binding (about 15-20 us per call, more than a decode-sized
    kernel takes) is paid once at capture, as in a graph-replayed decode
    step.  Arguments must not allocate inside the calls (workspaces passed
    in)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(calls):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    warm(torch, lambda i: g.replay(), warmup, WARM_S)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (steps * calls)  # ms per call


def main():
    args = parse()
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.copy_calib_mib or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_scaled_precision_tn_amd as mg
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    mg.load()  # the HIP library must be built: there is no fallback
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    # the secondary legs (everything but the headline) take at least 20 timed
    # calls after at least 10 warm-up calls and WARM_S seconds of further
    # calls, whatever --steps / --warmup say, so a short headline run does not
    # leave them on the clock ramp
    s2, w2 = max(args.steps, 20), max(args.warmup, 10)

    def todev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def f32(v):
        return torch.tensor([float(v)], dtype=torch.float32, device=dev)

    # ------------------------------------------------------ W4A4 (headline)
    run_w4a4 = args.only in ("", "w4a4")
    if run_w4a4:
        t0 = time.time()
        inp = synth.w4a4(M, N, K, seed=0)
        gen_s = time.time() - t0
        d = {k: todev(v) for k, v in inp.items() if isinstance(v, np.ndarray) and v.ndim}
        Sa4, Sw4 = f32(inp["Sa"]), f32(inp["Sw"])
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    # --------------------------------------------------- W4A8 decode shapes
    if args.only in ("", "w4a8") and not args.quick:
        w = synth.w4a8(1, N, K, seed=0)  # the weight tensor is shared by every M
        copies = 8  # 8 x 43.4 MB > 256 MB Infinity Cache
        wq = [todev(w["wq"]) for _ in range(copies)]
        ws = [todev(w["ws"]) for _ in range(copies)]
        Sw = f32(w["Sw"])
        dec = []
        for Mi in (1, 8, 32, 128):
            a = synth.normal((Mi, K), 1.0, Mi, synth.ROLE_A)
            aq, atok = synth.quant_fp8_token(a)
            aq, atok = todev(aq), todev(atok)
            Cd = torch.empty((Mi, N), dtype=torch.bfloat16, device=dev)
            wsp = mg.workspace(mg.mgemm_workspace_bytes(mg.OP_W4A8, Mi, N, K), "w4a8")
            call = lambda i: mg.mgemm_w4a8(aq, atok, wq[i % copies], ws[i % copies], Sw, Cd, ws=wsp)  # noqa: E731
            ms = timed_graph(torch, call, 2 * copies, max(args.steps, 20), w2)
            ms_e = timed(torch, call, max(args.steps, 40), w2, stream)
            nbytes = N * K // 2 + N * K // 16 + Mi * K + 4 * Mi + 2 * Mi * N
            gbps = nbytes / (ms * 1e-3) / 1e9
            dec.append({"M": Mi, "us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                        "frac_hbm": round(gbps / PEAK["hbm"], 4), "bytes": nbytes,
                        "tflops": round(2.0 * Mi * N * K / (ms * 1e-3) / 1e12, 2),
                        "eager_us": round(ms_e * 1e3, 2)})
        out["decode"] = dec
        del wq, ws
        torch.cuda.empty_cache()

    # -------------------------------------------------- W4A16 decode shapes
    if args.only in ("", "w4a16") and not args.quick:
        w = synth.w4a16(1, N, K, seed=0)  # the weight tensor is shared by every M
        copies = 8
        wq = [todev(w["wq"]) for _ in range(copies)]
        ws = [todev(w["ws"]) for _ in range(copies)]
        Sw = f32(w["Sw"])
        dec = []
        for Mi in (1, 16, 128):
            a = todev(synth.to_bf16_bits(synth.normal((Mi, K), 1.0, Mi, synth.ROLE_A)).view(np.int16))
            a = a.view(torch.bfloat16)
            Cd = torch.empty((Mi, N), dtype=torch.bfloat16, device=dev)
            wsp = mg.workspace(mg.mgemm_workspace_bytes(mg.OP_W4A16, Mi, N, K), "w4a16")
            call = lambda i: mg.mgemm_w4a16(a, wq[i % copies], ws[i % copies], Sw, Cd, ws=wsp)  # noqa: E731
            ms = timed_graph(torch, call, 2 * copies, max(args.steps, 20), w2)
            ms_e = timed(torch, call, max(args.steps, 40), w2, stream)
            nbytes = N * K // 2 + N * K // 16 + 2 * Mi * K + 2 * Mi * N
            gbps = nbytes / (ms * 1e-3) / 1e9
            dec.append({"M": Mi, "us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                        "frac_hbm": round(gbps / PEAK["hbm"], 4), "bytes": nbytes,
                        "tflops": round(2.0 * Mi * N * K / (ms * 1e-3) / 1e12, 2),
                        "eager_us": round(ms_e * 1e3, 2)})
        out["w4a16_decode"] = dec
        del wq, ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ BF16
    if args.only in ("", "bf16", "bf16_grad") and not args.quick:
        Mb = 4096
        b = synth.bf16(Mb, N, K, seed=0)
        A = todev(b["a"].view(np.int16)).view(torch.bfloat16)
        W = todev(b["w"].view(np.int16)).view(torch.bfloat16)
        Cb = torch.empty((Mb, N), dtype=torch.bfloat16, device=dev)
        if args.only != "bf16_grad":
            ms = timed(torch, lambda i: mg.mgemm_bf16(A, W, Cb), s2, w2, stream)
            tf = 2.0 * Mb * N * K / (ms * 1e-3) / 1e12
            ms_t = timed(torch, lambda i: torch.matmul(A, W.t()), s2, w2, stream)
            tf_t = 2.0 * Mb * N * K / (ms_t * 1e-3) / 1e12
            out["bf16"] = {"M": Mb, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(tf, 1),
                           "frac_bf16_peak": round(tf / PEAK["bf16"], 4),
                           "torch_matmul_tflops": round(tf_t, 1)}
        # its backward: dX = dY . W (A doubles as dX's shape donor), dW = dY^T . X
        dY = Cb.normal_()
        dX = torch.empty((Mb, K), dtype=torch.bfloat16, device=dev)
        dW = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        ms_d = timed(torch, lambda i: mg.mgemm_bf16_dgrad(dY, W, dX), s2, w2, stream)
        ms_w = timed(torch, lambda i: mg.mgemm_bf16_wgrad(dY, A, dW), s2, w2, stream)
        fl = 2.0 * Mb * N * K
        out["bf16_grad"] = {"M": Mb, "N": N, "K": K, "dgrad_ms": round(ms_d, 4),
                            "dgrad_tflops": round(fl / (ms_d * 1e-3) / 1e12, 1),
                            "wgrad_ms": round(ms_w, 4),
                            "wgrad_tflops": round(fl / (ms_w * 1e-3) / 1e12, 1)}
        del A, W, Cb, dY, dX, dW
        torch.cuda.empty_cache()

    # ------------------------------------------------ W4A4 (headline), timed
    # Timed after the decode and BF16 legs: its inputs were uploaded first,
    # and the GPU now runs at the clock it holds under sustained load, where a
    # cold start would put the first timed steps on the clock ramp (a short
    # run's 5 warm-up steps take 10 ms).
    if run_w4a4:
        call = lambda i: mg.mgemm_w4a4(d["aq"], d["as_"], Sa4, d["wq"], d["ws"], Sw4, C)  # noqa: E731
        ms = timed(torch, call, args.steps, args.warmup, stream, warm_s=0.0)  # exactly W warm-up steps
        flops = 2.0 * M * N * K
        tflops = flops / (ms * 1e-3) / 1e12
        groups = M * N * (K // 16)
        traffic = traffic_for("gemm_w4a4.hip", "w4a4_m8192")
        out["w4a4"] = dict(ms=ms, tflops=tflops, gen_s=gen_s)
        # The exact FP8 route is bound by the vector ALU: one FP32 fused
        # multiply-add per output per 16-element group (the group-scale step),
        # M*N*K/16 per launch, against the MFMA work of 2 FP8 MFMAs per 32x32
        # block and group.  `roofline` is that ALU work against the published
        # FP32 vector peak (which counts packed FP32 instructions; these
        # kernels emit none, so 78.6 TFLOP/s is the attainable half); `mfma_roofline`
        # the GEMM flops against the FP8 MFMA peak (the metric's "% MFMA peak").
        alu = 2.0 * groups / (ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "alu", "achieved": round(alu, 2), "peak": PEAK["fp32"],
                           "unit": "TFLOP/s", "frac": round(alu / PEAK["fp32"], 4),
                           "traffic": traffic,
                           "what": "per-group FP32 scale FMAs, M*N*K/16 per launch, 2 flops each",
                           "frac_of_unpacked_fp32": round(alu / PEAK_VALU_F32, 4)}
        out["mfma_roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK["fp8"],
                                "unit": "TFLOP/s", "frac": round(tflops / PEAK["fp8"], 4)}
        # sampled parity of the timed output against the oracle (bench sanity)
        rng = np.random.default_rng(1)
        pm, pn = rng.integers(0, M, 64), rng.integers(0, N, 64)
        cbits = C.view(torch.int16)[torch.from_numpy(pm).to(dev), torch.from_numpy(pn).to(dev)]
        out["_sample"] = (inp, pm, pn, cbits.cpu().numpy().view(np.uint16))
        del d, C, Sa4, Sw4
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------- MoE
    if args.only in ("", "moe", "moe_decode") and not args.quick:
        T, H, I, E, topk = 4096, 4096, 1536, 64, 8
        m = synth.moe(T, H, I, E, topk, seed=0)
        dm = {k: todev(v) for k, v in m.items()}
        o = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        wsp = mg.workspace(mg.mgemm_workspace_bytes(mg.OP_MOE, T=T, H=H, I=I, E=E, topk=topk), "moe")
        call = lambda i: mg.mgemm_moe_mxfp8_glu(dm["xq"], dm["xs"], dm["ids"], dm["tw"], dm["w13q"],  # noqa: E731
                                                dm["w13s"], dm["w2q"], dm["w2s"], o, ws=wsp)
        if args.only != "moe_decode":
            ms = timed(torch, call, s2, w2, stream)
            fl = 2.0 * T * topk * (H * 2 * I + I * H)
            tf = fl / (ms * 1e-3) / 1e12
            out["moe"] = {"T": T, "H": H, "I": I, "E": E, "topk": topk, "ms": round(ms, 3),
                          "tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK["fp8"], 4)}
            # the same call routed from the router logits inside the call
            lgf = todev(synth.moe_logits(T, E, seed=0))
            fid = torch.empty((T, topk), dtype=torch.int32, device=dev)
            fw = torch.empty((T, topk), dtype=torch.float32, device=dev)
            callf = lambda i: mg.mgemm_moe_mxfp8_glu_logits(  # noqa: E731
                dm["xq"], dm["xs"], lgf, topk, dm["w13q"], dm["w13s"], dm["w2q"], dm["w2s"], o,
                fid, fw, ws=wsp)
            msf = timed(torch, callf, s2, w2, stream)
            # the same routing as two calls: the router, then the MoE on its ids
            callu = lambda i: (mg.mgemm_moe_route_topk(lgf, topk, fid, fw),  # noqa: E731
                               mg.mgemm_moe_mxfp8_glu(dm["xq"], dm["xs"], fid, fw, dm["w13q"],
                                                      dm["w13s"], dm["w2q"], dm["w2s"], o, ws=wsp))
            msu = timed(torch, callu, s2, w2, stream)
            out["moe_fused_route"] = [{"T": T, "ms": round(msf, 3), "tflops": round(fl / (msf * 1e-3) / 1e12, 1),
                                       "router_then_moe_ms": round(msu, 3),
                                       "what": "routing from FP32 logits inside the call"}]
            del fid, fw
        # the router top-k that produces such ids and weights (FP32 logits)
        if args.only != "moe_decode":
            lg = todev(synth.moe_logits(T, E, seed=0))
            rids = torch.empty((T, topk), dtype=torch.int32, device=dev)
            rw = torch.empty((T, topk), dtype=torch.float32, device=dev)
            callr = lambda i: mg.mgemm_moe_route_topk(lg, topk, rids, rw)  # noqa: E731
            us = timed(torch, callr, s2, w2, stream) * 1e3
            rb = T * E * 4 + T * topk * 8
            out["moe_route"] = {"T": T, "E": E, "topk": topk, "us": round(us, 2),
                                "GBps": round(rb / us / 1e3, 1)}
            del lg, rids, rw
        # decode-sized calls (the swap-AB kernels): successive calls take
        # successive groups of Td tokens of the same inputs, so they name
        # different experts and the weights they stream (1.25 GB in all) do
        # not stay in the 256 MB Infinity Cache between calls
        dec = []
        for Td in [int(v) for v in args.moe_dec_tokens.split(",") if v] if args.only != "moe" else []:
            groups = max(1, min(16, T // Td))
            sls = [{k: dm[k][g * Td:(g + 1) * Td].contiguous() for k in ("xq", "xs", "ids", "tw")}
                   for g in range(groups)]
            od = torch.empty((Td, H), dtype=torch.bfloat16, device=dev)
            wsd = mg.workspace(mg.mgemm_workspace_bytes(mg.OP_MOE, T=Td, H=H, I=I, E=E, topk=topk),
                               "moe_dec")
            calld = lambda i, sls=sls, od=od, wsd=wsd: mg.mgemm_moe_mxfp8_glu(  # noqa: E731
                sls[i % len(sls)]["xq"], sls[i % len(sls)]["xs"], sls[i % len(sls)]["ids"],
                sls[i % len(sls)]["tw"], dm["w13q"], dm["w13s"], dm["w2q"], dm["w2s"], od, ws=wsd)
            steps_d = len(sls) * max(1, s2 // len(sls))
            us = timed_graph(torch, calld, len(sls), max(1, s2 // len(sls)), w2) * 1e3
            us_e = timed(torch, calld, steps_d, w2, stream) * 1e3
            ne = np.mean([len(np.unique(m["ids"][g * Td:(g + 1) * Td])) for g in range(groups)])
            nbytes = (ne * 3 * I * H * (1 + 1 / 32)                  # expert weights, codes + scales
                      + Td * H * (1 + 1 / 32) + Td * topk * 8 + 2 * Td * H)   # x, routing, out
            row = {"T": Td, "experts": round(float(ne), 2), "token_groups": groups,
                   "us": round(us, 2), "bytes": int(nbytes), "GBps": round(nbytes / us / 1e3, 1),
                   "frac_hbm": round(nbytes / us / 1e3 / PEAK["hbm"], 4), "eager_us": round(us_e, 2)}
            # the same calls routed from the router logits inside the call
            lgs = [todev(synth.moe_logits(T, E, seed=0)[g * Td:(g + 1) * Td]) for g in range(groups)]
            fid = torch.empty((Td, topk), dtype=torch.int32, device=dev)
            fw = torch.empty((Td, topk), dtype=torch.float32, device=dev)
            callf = lambda i, sls=sls, od=od, wsd=wsd, lgs=lgs: mg.mgemm_moe_mxfp8_glu_logits(  # noqa: E731
                sls[i % len(sls)]["xq"], sls[i % len(sls)]["xs"], lgs[i % len(lgs)], topk,
                dm["w13q"], dm["w13s"], dm["w2q"], dm["w2s"], od, fid, fw, ws=wsd)
            row["fused_route_us"] = round(timed_graph(torch, callf, len(sls), max(1, s2 // len(sls)), w2) * 1e3, 2)
            callu = lambda i, sls=sls, od=od, wsd=wsd, lgs=lgs: (  # noqa: E731
                mg.mgemm_moe_route_topk(lgs[i % len(lgs)], topk, fid, fw),
                mg.mgemm_moe_mxfp8_glu(sls[i % len(sls)]["xq"], sls[i % len(sls)]["xs"], fid, fw,
                                       dm["w13q"], dm["w13s"], dm["w2q"], dm["w2s"], od, ws=wsd))
            row["router_then_moe_us"] = round(timed_graph(torch, callu, len(sls), max(1, s2 // len(sls)), w2) * 1e3, 2)
            dec.append(row)
        out["moe_decode"] = dec
        del dm, o
        torch.cuda.empty_cache()

    # ---------------------------------------------------- NVFP4 MoE (W4A4 route)
    if args.only in ("", "moe_nvfp4") and not args.quick:
        T, H, I, E, topk = 4096, 4096, 1536, 64, 8
        m4 = synth.moe_nvfp4(T, H, I, E, topk, seed=0)
        d4 = {k: todev(v) for k, v in m4.items() if k not in ("Sx", "Sh")}
        o4 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        ws4 = mg.workspace(mg.mgemm_workspace_bytes(mg.OP_MOE_NVFP4, T=T, H=H, I=I, E=E, topk=topk),
                           "moe_nvfp4")
        sx, sh = f32(m4["Sx"]), f32(m4["Sh"])
        call4 = lambda i: mg.mgemm_moe_nvfp4_glu(  # noqa: E731
            d4["xq"], d4["xs"], sx, d4["ids"], d4["tw"], d4["w13q"], d4["w13s"], d4["Sw13"],
            d4["w2q"], d4["w2s"], d4["Sw2"], sh, o4, ws=ws4)
        ms = timed(torch, call4, s2, w2, stream)
        fl = 2.0 * T * topk * (H * 2 * I + I * H)
        tf = fl / (ms * 1e-3) / 1e12
        fmas = T * topk * (H * 2 * I + I * H) / 16          # per-group scale FMAs
        out["moe_nvfp4"] = {"T": T, "H": H, "I": I, "E": E, "topk": topk, "ms": round(ms, 3),
                            "tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK["fp8"], 4),
                            "route_fma_tflops": round(2 * fmas / (ms * 1e-3) / 1e12, 2)}
        del d4, o4, m4
        torch.cuda.empty_cache()

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.mul(x, 1.0, out=y)  # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()

    # ----------------------------------------------------- CPU baseline leg
    cpu = None
    par = None
    if run_w4a4 and not args.no_cpu_baseline:
        import oracle
        from oracle import NVFP4, Operand
        inp, pm, pn, gbits = out.pop("_sample")
        A_op = Operand(NVFP4, inp["aq"], inp["as_"], tscale=float(inp["Sa"]))
        W_op = Operand(NVFP4, inp["wq"], inp["ws"], tscale=float(inp["Sw"]))
        cores = max(1, min(os.cpu_count() or 1, 16))
        c64, b64 = oracle.gemm_points(A_op, W_op, pm, pn, nthreads=cores)
        ref = oracle.bf16_rne(c64)
        o_ord = lambda b: np.where(b & 0x8000, -(b & 0x7FFF).astype(np.int64), (b & 0x7FFF).astype(np.int64))  # noqa: E731
        par = {"points": int(len(pm)), "max_bf16_ulp": int(np.max(np.abs(o_ord(gbits) - o_ord(ref))))}
        # calibrate on scattered outputs, then time the first output rows: those
        # run about 1.7x faster than the calibration predicts, so a 22 s
        # prediction gives 10-15 s of oracle work
        rng = np.random.default_rng(2)
        t0 = time.time()
        oracle.gemm_points(A_op, W_op, rng.integers(0, M, 256), rng.integers(0, N, 256), nthreads=cores)
        per_pt = (time.time() - t0) / 256
        npts = int(max(256, min(2_000_000, 22.0 / max(per_pt, 1e-9))))
        sm, sn = np.divmod(np.arange(npts, dtype=np.int64), N)
        t0 = time.time()
        oracle.gemm_points(A_op, W_op, sm, sn, nthreads=cores)
        dt = time.time() - t0
        cpu = {"value": round(npts * 2.0 * K / dt / 1e12, 8), "unit": "TFLOP/s", "cores": cores,
               "kind": "oracle", "sample": f"{npts} outputs (rows 0..{int(sm[-1])} of C) of the "
               f"W4A4 M={M} K={K} N={N} workload, FP64, {dt:.1f} s"}
    else:
        out.pop("_sample", None)

    w = out.get("w4a4")
    line = {
        "metric": "TFLOP/s + % MFMA peak, W4A4 NVFP4 M=8192 K=14336 N=5376; decode GB/s",
        "value": round(w["tflops"], 2) if w else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(w["ms"], 4) if w else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"W4A4 NVFP4 TN GEMM M={M} K={K} N={N} (FFN down projection shape)",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "roofline": out.get("roofline"),
        "cpu_baseline": cpu,
        "mfma_roofline": out.get("mfma_roofline"),
        "parity_sample": par,
        "decode": out.get("decode"),
        "w4a16_decode": out.get("w4a16_decode"),
        "bf16": out.get("bf16"),
        "bf16_grad": out.get("bf16_grad"),
        "moe": out.get("moe"),
        "moe_decode": out.get("moe_decode"),
        "moe_nvfp4": out.get("moe_nvfp4"),
        "moe_route": out.get("moe_route"),
        "moe_fused_route": out.get("moe_fused_route"),
        "device": torch.cuda.get_device_properties(0).gcnArchName,
        "kernel_src": src_hash("gemm_w4a4.hip", "common.h"),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
