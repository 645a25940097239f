#!/usr/bin/env python3
"""Benchmark of the block-scaled 4-bit quantized-matmul hot path on one MI355X.

One step is one pass over every stage of the path on synthetic input that is
already resident in HBM:

  act_quant   NVFP4 activation quantize X[4096,5120] (tensor amax + codes +
              E4M3 scales + global scale), 1 % outliers at +-20: a burst of
              9 calls over 8 distinct copies of X (cold), per call; each call
              is bsfp_quantize_ws (amax from per-workgroup partial maxima in
              the tensor's workspace, two launches)
  act_quant_warm  the same, 8 calls on one X (warm), per call
  dequant     NVFP4 dequantize of the same tensor (burst of 8 calls, per call)
  w_quant     MXFP4 quantize W[5760,2880] and affine quantize W[1024,512]
              (burst of 8 pairs over 8 distinct copies of W, per pair)
  act_quant_sr  NVFP4 quantize of the same X with stochastic rounding (one
              random word per element, drawn on the device beforehand)
  qmv_sweep   affine g64 decode GEMV over 64 layers x {gate, up, down}
              ([25600,5120], [25600,5120], [5120,25600]): 192 distinct matrices,
              14.17 GB of packed weights (more than the 256 MB Infinity Cache);
              per layer gate and up, which share x, run as one bsfp_qmv_batch
              launch and down as one bsfp_qmv launch (128 launches)
  qmv_sweep_single   the same sweep with one bsfp_qmv launch per matrix (192)
  qmv_mx1 / qmv_mx8   MXFP4 qmv W[5760,2880] at M = 1 and 8: a burst of 32
              calls over 32 distinct weight copies (282 MB, more than the
              Infinity Cache), reported per call (`qmv_fp4_gbs`)
  qmv_nv1     NVFP4 qmv W[25600,5120] at M = 1: a burst of 8 calls over 4
              distinct matrices, reported per call (`qmv_fp4_gbs`)
  qqmm        NVFP4 prefill X[2048,5120] . W[25600,5120]^T (x quantized on the
              fly, alpha = g_x g_w), the headline GEMM
  qqmm_1134 / qqmm_4096   the same GEMM at M = 1134 and 4096
  qq_decode   NVFP4 qq product at M = 1 on W[25600,5120] (x quantized and
              dequantized exactly, then the GEMV; alpha = g_x g_w): a burst of
              8 calls over 4 distinct weight matrices, reported per call
  qmm_mx32 / qmm_mx512   MXFP4 qq GEMM on the scaled MFMA, W[5760,2880]
              (bursts of 8 calls, per call; M = 32 over distinct copies of W)
  qmm_affine  affine weight-only x[2048,5120] . W_up[25600,5120]^T
  qmv_<fmt>    decode GEMV (M = 1) on W[25600,5120] in each format variant:
              mxfp8, affine 4-bit groups 32 / 128, affine 8-bit groups
              32 / 64 / 128 (`qmv_variants_gbs`): a burst of 8 calls over 4
              distinct matrices per format, reported per call
  wonly_M / dense_M   NVFP4 weight-only X[M,5120] . W[25600,5120]^T at
              M = 1134, 2048, 4096: the fused kernel (W decoded in registers)
              and the dense prefill path (W dequantized to bf16 into one
              reused scratch, then a dense bf16 GEMM); `dense_crossover` maps
              their ratio

The JSON line reports the headline metric: `value` is the sustained qmv GB/s
of the 64-layer sweep (algorithmic bytes: packed codes + scales + biases +
x + y per matrix); `qmm_tflops` the NVFP4 qqmm TFLOP/s at M = 2048 per whole
call (activation amax and quantize, then the GEMM).  `roofline` is for the qmv
kernel (HBM), over the mean launch duration of the sweep's back-to-back GEMV
launches (HIP events on their stream); `roofline_qmm` for the qqmm GEMM kernel
alone (fp16 MFMA), over HIP events attached to its first and last launch.
`cpu_baseline` times the CPU oracle on a bounded sample.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFS = 2500.0   # MI355X dense fp16 / bf16 MFMA, vendor figure
FP4_PEAK_TFS = 10100.0       # MI355X dense MXFP4 MFMA, vendor figure

HIDDEN, INTER, LAYERS = 5120, 25600, 64


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="",
                   help="comma-separated stage names (profiling); 'copy' adds a 1 GiB "
                        "streaming kernel used to calibrate HBM byte counters")
    return p.parse_args()


def affine_bytes(N, K, M=1):
    """Algorithmic bytes of one affine qmv: codes + scales + biases + x + y."""
    return N * K // 2 + 2 * 2 * N * (K // 64) + 2 * M * K + 2 * M * N


def fp4_bytes(N, K, G, M=1):
    return N * K // 2 + N * (K // G) + 2 * M * K + 2 * M * N


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards W by output rows, and one GPU's share is the same "
              "kernel at a smaller N)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_bit_fp_amd as b
    import synth_inputs as S

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    log(f"[bench] device {props.name} CUs={props.multi_processor_count} lib={b.version()}")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------- inputs
    t_setup = time.time()
    X_act = to_dev(S.nvfp4_activations())                        # [4096, 5120]
    q_act = b.empty_quantized(b.NVFP4, 4096, HIDDEN, dev)
    dq_act = torch.empty((4096, HIDDEN), dtype=torch.bfloat16, device=dev)
    W_mx_bf = to_dev(S.mxfp4_weights())                          # [5760, 2880]
    q_mx = b.quantize(W_mx_bf, b.MXFP4)
    q_mx_out = b.empty_quantized(b.MXFP4, 5760, 2880, dev)
    _, w_small = S.affine_small()
    W_small = to_dev(w_small)
    q_small_out = b.empty_quantized(b.AFFINE, 1024, 512, dev)

    x_dec = to_dev(S.generic((1, HIDDEN), 1.0, seed=3))
    x_dec_down = to_dev(S.generic((1, INTER), 1.0, seed=3, stream=9))
    sweep = []  # (x, q, y)
    for layer in range(LAYERS):
        for name, (N, K) in (("gate", (INTER, HIDDEN)), ("up", (INTER, HIDDEN)),
                             ("down", (HIDDEN, INTER))):
            seed = 1000 + 3 * layer + {"gate": 0, "up": 1, "down": 2}[name]
            wb = S.torch_normal_bf16((N, K), 0.02, seed, dev)
            q = b.quantize(wb, b.AFFINE)
            del wb
            x = x_dec if K == HIDDEN else x_dec_down
            sweep.append((x, q, torch.empty((1, N), dtype=torch.bfloat16, device=dev)))
    sweep_bytes = sum(affine_bytes(q.rows, q.cols) for _, q, _ in sweep)
    # the same sweep as a decoder runs it: per layer, gate and up (same x) in
    # one bsfp_qmv_batch launch, then down
    sweep_layers = [(sweep[3 * l][0], [sweep[3 * l][1], sweep[3 * l + 1][1]],
                     [sweep[3 * l][2], sweep[3 * l + 1][2]], sweep[3 * l + 2])
                    for l in range(LAYERS)]

    x_mx = {M: to_dev(S.mxfp4_activations(M)) for M in (1, 8, 32, 512)}
    y_mx = {M: torch.empty((M, 5760), dtype=torch.bfloat16, device=dev) for M in (1, 8, 32, 512)}
    ws_mx = {M: torch.empty(b.qmm_workspace_bytes(b.MXFP4, M, 2880, "same"), dtype=torch.uint8,
                            device=dev) for M in (32, 512)}

    Wp = S.torch_normal_bf16((INTER, HIDDEN), 0.02, 55, dev)      # prefill weights
    q_pf = b.quantize(Wp, b.NVFP4)
    del Wp
    x_nv1 = to_dev(S.generic((1, HIDDEN), 1.0, seed=8))
    y_nv1 = torch.empty((1, INTER), dtype=torch.bfloat16, device=dev)
    X_pf = {M: S.torch_normal_bf16((M, HIDDEN), 0.02, 500 + M, dev) for M in (1134, 2048, 4096)}
    Y_pf = {M: torch.empty((M, INTER), dtype=torch.bfloat16, device=dev) for M in X_pf}
    ws_pf = {M: torch.empty(b.qmm_workspace_bytes(b.NVFP4, M, HIDDEN, "same"), dtype=torch.uint8,
                            device=dev) for M in X_pf}
    X_aff = S.torch_normal_bf16((2048, HIDDEN), 1.0, 6, dev)
    Y_aff = torch.empty((2048, INTER), dtype=torch.bfloat16, device=dev)
    q_up0 = sweep[1][1]
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t_setup:.1f}s; sweep {len(sweep)} matrices, "
        f"{sweep_bytes / 1e9:.2f} GB")

    # ------------------------------------------------------------- stages
    stream = torch.cuda.current_stream()  # the library launches on this stream
    # the activation quantize runs as a burst of ACTN calls, per call: over
    # ACTN distinct copies of X (column rotations, 336 MB together, so every
    # call reads X from HBM: cold) and over one X (warm, from the Infinity
    # Cache)
    ACTN = 8
    X_acts = [X_act] + [torch.roll(X_act, shifts=977 * i, dims=1).contiguous()
                        for i in range(1, ACTN)]

    def st_act_quant():
        for Xi in X_acts:
            b.quantize(Xi, b.NVFP4, "compute", out=q_act)
        b.quantize(X_act, b.NVFP4, "compute", out=q_act)  # q_act holds X_act's codes

    def st_act_quant_warm():
        for _ in range(ACTN):
            b.quantize(X_act, b.NVFP4, "compute", out=q_act)

    rbits_act = torch.randint(-(1 << 31), (1 << 31) - 1, (4096 * HIDDEN,), dtype=torch.int32,
                              device=dev)
    q_act_sr = b.empty_quantized(b.NVFP4, 4096, HIDDEN, dev)

    def st_act_quant_sr():
        b.quantize(X_act, b.NVFP4, "compute", out=q_act_sr, rbits=rbits_act)

    # dequantize and weight quantize run as bursts of SHORTN calls, per call;
    # the MXFP4 weight quantize over SHORTN distinct copies of W (265 MB)
    SHORTN = 8
    W_mx_copies = [W_mx_bf] + [torch.roll(W_mx_bf, shifts=32 * i, dims=1).contiguous()
                               for i in range(1, SHORTN)]

    def st_dequant():
        for _ in range(SHORTN):
            b.dequantize(q_act, out=dq_act)

    def st_w_quant():
        for Wi in W_mx_copies[1:] + W_mx_copies[:1]:  # q_mx_out ends with W's own codes
            b.quantize(Wi, b.MXFP4, out=q_mx_out)
            b.quantize(W_small, b.AFFINE, out=q_small_out)

    # The sweep's GEMV launches run back to back on one stream, between one
    # pair of HIP events: the mean launch duration is the sweep's time over
    # its launches (the short gaps between launches included).
    hip = HipEvents(4 * args.steps + 4)
    recording = [False]
    # Attaching the events to the GEMM's launches costs about 5 us per event
    # (each is recorded around its launch), so they ride on every other timed
    # step only, and the whole-call figure comes from the steps without them.
    instrument = [False]
    instrumented_steps = []

    def st_qmv_sweep():
        for x, qs, ys, (xd, qd, yd) in sweep_layers:
            b.qmv_batch(x, qs, outs=ys)
            b.qmv(xd, qd, out=yd)

    def st_qmv_sweep_single():  # one launch per matrix
        for x, q, y in sweep:
            b.qmv(x, q, out=y)


    # The M = 2048 qq stage also times its GEMM launches alone: a pair of HIP
    # events that the library attaches to the first and last GEMM launch of
    # the call (the activation pre-pass runs before it, outside the pair).
    qq_gemm_ev = []

    def qq(M):
        def run():
            if M == 2048 and recording[0] and instrument[0]:
                e0, e1 = hip.take(), hip.take()
                b.time_next_launch(e0, e1)
                qq_gemm_ev.append((e0, e1))
            b.qmm(X_pf[M], q_pf, act="same", workspace=ws_pf[M], out=Y_pf[M])
        return run

    ws_dec = torch.empty(b.qmm_workspace_bytes(b.NVFP4, 1, HIDDEN, "same"), dtype=torch.uint8,
                         device=dev)

    # Short single-kernel stages run as a burst of BURST calls over NDIST
    # distinct weight matrices (together larger than the 256 MB Infinity
    # Cache), so the queue runs ahead of the host and the figure is the
    # kernels' own streaming rate, not one call's host latency; stage times
    # of these stages are per call.
    BURST, NDIST = 8, 4
    per_call = {"qq_decode": BURST,  # stage -> calls per timed burst
                "act_quant": ACTN + 1, "act_quant_warm": ACTN, "dequant": SHORTN,
                "w_quant": SHORTN, "qmm_mx32": SHORTN, "qmm_mx512": SHORTN}
    q_dec = [q_pf] + [b.quantize(S.torch_normal_bf16((INTER, HIDDEN), 0.02, 910 + i, dev),
                                 b.NVFP4) for i in range(NDIST - 1)]

    def st_qq_decode():
        for i in range(BURST):
            b.qmm(x_nv1, q_dec[i % NDIST], act="same", workspace=ws_dec, out=y_nv1)

    # MXFP4 qq GEMM as a burst of SHORTN calls, per call: at M = 32 (a
    # weight-streaming size) over distinct weight copies, at M = 512 on one W
    def mx(M):
        def run():
            for i in range(SHORTN):
                q = q_mx_rot[i] if M <= 32 else q_mx
                b.qmm(x_mx[M], q, act="same", workspace=ws_mx[M], out=y_mx[M])
        return run

    # decode GEMV on 4-bit float weights: MXFP4 W[5760,2880] at M = 1 and 8
    # over MXROT distinct copies, NVFP4 W[25600,5120] at M = 1 over the qq
    # decode stage's NDIST matrices
    MXROT = 32
    q_mx_rot = [q_mx] + [b.quantize(S.torch_normal_bf16((5760, 2880), 0.02, 950 + i, dev),
                                    b.MXFP4) for i in range(MXROT - 1)]

    def qmv_mx(M):
        def run():
            for q in q_mx_rot:
                b.qmv(x_mx[M], q, out=y_mx[M])
        return run

    def st_qmv_nv1():
        for i in range(BURST):
            b.qmv(x_nv1, q_dec[i % NDIST], out=y_nv1)

    per_call.update({"qmv_mx1": MXROT, "qmv_mx8": MXROT, "qmv_nv1": BURST})

    def st_qmm_affine():
        b.qmm(X_aff, q_up0, act="bf16", out=Y_aff)

    # decode GEMV in the format variants (one W[25600,5120] each)
    VARIANTS = {"mxfp8": (b.MXFP8, 8, 32), "aff4g32": (b.AFFINE, 4, 32),
                "aff4g128": (b.AFFINE, 4, 128), "aff8g32": (b.AFFINE, 8, 32),
                "aff8g64": (b.AFFINE, 8, 64), "aff8g128": (b.AFFINE, 8, 128)}
    q_var = {}
    for i, (name, (mode, nb, G)) in enumerate(VARIANTS.items()):
        q_var[name] = []
        for j in range(NDIST):
            wb = S.torch_normal_bf16((INTER, HIDDEN), 0.02, 900 + 16 * i + j, dev)
            q_var[name].append(b.quantize(wb, mode, bits=nb, group=G))
            del wb
        per_call[f"qmv_{name}"] = BURST

    def var_bytes(name):
        mode, nb, G = VARIANTS[name]
        per_group = 4 if mode == b.AFFINE else 1  # bf16 scale + bias, or one E8M0 byte
        return INTER * HIDDEN * nb // 8 + INTER * (HIDDEN // G) * per_group + HIDDEN * 2 + INTER * 2

    def qmv_var(name):
        def run():
            for i in range(BURST):
                b.qmv(x_dec, q_var[name][i % NDIST], out=y_nv1)
        return run

    # dense prefill path vs the fused weight-only kernel on the NVFP4 weights
    dense_scratch = torch.empty(b.qmm_dense_scratch_bytes(INTER, HIDDEN), dtype=torch.uint8,
                                device=dev)

    def wonly(M):
        return lambda: b.qmm(X_pf[M], q_pf, act="bf16", out=Y_pf[M])

    def dense(M):
        return lambda: b.qmm_dense(X_pf[M], q_pf, scratch=dense_scratch, out=Y_pf[M])

    # quantize stages, then every decode GEMV, then the prefill GEMMs
    stages = [("act_quant", st_act_quant), ("act_quant_warm", st_act_quant_warm),
              ("act_quant_sr", st_act_quant_sr),
              ("dequant", st_dequant), ("w_quant", st_w_quant),
              ("qmv_sweep", st_qmv_sweep), ("qmv_sweep_single", st_qmv_sweep_single),
              ("qmv_mx1", qmv_mx(1)), ("qmv_mx8", qmv_mx(8)),
              ("qmv_nv1", st_qmv_nv1), ("qq_decode", st_qq_decode)]
    stages += [(f"qmv_{name}", qmv_var(name)) for name in VARIANTS]
    stages += [("qqmm", qq(2048)), ("qqmm_1134", qq(1134)), ("qqmm_4096", qq(4096)),
               ("qmm_mx32", mx(32)), ("qmm_mx512", mx(512)), ("qmm_affine", st_qmm_affine)]
    for M in (1134, 2048, 4096):
        stages += [(f"wonly_{M}", wonly(M)), (f"dense_{M}", dense(M))]
    if args.only:
        keep = set(args.only.split(","))
        stages = [s for s in stages if s[0] in keep]
        if "copy" in keep:
            # a plain streaming kernel of known size: reads 1 GiB, writes 1 GiB
            c_src = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
            c_dst = torch.empty_like(c_src)
            stages.append(("copy", lambda: torch.bitwise_not(c_src, out=c_dst)))
    names = [n for n, _ in stages]

    ev = {n: [] for n in names}

    def step(record):
        recording[0] = record
        for n, fn in stages:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev[n].append((e0, e1))
            else:
                fn()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    t0 = time.perf_counter()
    for i in range(args.steps):
        instrument[0] = i % 2 == 1 or args.steps == 1
        instrumented_steps.append(instrument[0])
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    def stage_times(n):
        pairs = ev[n]
        if n == "qqmm" and not all(instrumented_steps):  # the steps without the GEMM events
            pairs = [pr for pr, inst in zip(pairs, instrumented_steps) if not inst]
        return [a.elapsed_time(c) for a, c in pairs]

    ms = {n: float(np.median(stage_times(n))) / per_call.get(n, 1) for n in names}
    log("[bench] stage medians (ms): " + ", ".join(f"{n}={ms[n]:.3f}" for n in names))

    out = {"metric": "qmv achieved HBM GB/s (M=1, 4-bit) + qmm TFLOPS at M=2048; % of roofline",
           "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u4 codes, bf16/fp16 MFMA, fp32 acc",
           "data": "synthetic (seeded normal inputs; weights quantized on the GPU)",
           "config": {"workload": "affine 4-bit g64 decode qmv sweep, 64 layers x "
                                  "{gate,up,down} of hidden 5120 / intermediate 25600 "
                                  "(14.17 GB), plus NVFP4 prefill qqmm X[2048,5120] . "
                                  "W[25600,5120]^T and the other hot-path stages",
                      "arch": "gfx950", "device": props.name}}
    out["config"]["gpu"] = device_info(props)
    stage_ms = {n: round(v, 4) for n, v in ms.items()}
    out["stages_ms"] = stage_ms
    if "qmv_sweep" in ms:
        gbs = sweep_bytes / (ms["qmv_sweep"] * 1e-3) / 1e9
        out["value"] = round(gbs, 1)
        out["qmv_sweep_gbs"] = round(gbs, 1)
        launches = 2 * len(sweep_layers)
        per_launch = sweep_bytes / launches
        launch_ms = ms["qmv_sweep"] / launches
        kgbs = per_launch / (launch_ms * 1e-3) / 1e9
        up_bytes = affine_bytes(INTER, HIDDEN)
        out["roofline"] = {"bound": "hbm", "achieved": round(kgbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic("qmv_affine_m1", ["qmv.hip"]),
                           "kernel": "qmv_fast_kernel<affine, M=1>",
                           "bytes_per_launch": int(per_launch),
                           "bytes_per_launch_by_kind": {"gate+up (one qmv_batch launch)":
                                                        2 * up_bytes,
                                                        "down": affine_bytes(HIDDEN, INTER)},
                           "launch_us": round(launch_ms * 1e3, 3),
                           "launches_per_sweep": launches,
                           "note": "per layer, gate and up (which share x) run as one "
                                   "bsfp_qmv_batch launch and down as one bsfp_qmv launch; "
                                   "algorithmic bytes per launch (mean over the two kinds) / "
                                   "mean launch duration: HIP events on the GEMV's stream "
                                   "around the sweep's back-to-back launches (median over "
                                   "the timed steps) divided by their number, so the short "
                                   "gaps between launches count as kernel time"}
    if "qmv_sweep_single" in ms:
        gbs1 = sweep_bytes / (ms["qmv_sweep_single"] * 1e-3) / 1e9
        out["qmv_sweep_single_gbs"] = round(gbs1, 1)
        out["qmv_sweep_single_launch_us"] = round(ms["qmv_sweep_single"] * 1e3 / len(sweep), 3)
    if "qqmm" in ms:
        flop = 2.0 * 2048 * INTER * HIDDEN
        tfs = flop / (ms["qqmm"] * 1e-3) / 1e12
        out["qmm_tflops"] = round(tfs, 1)  # whole call: amax + x quantize + GEMM
        gemm_ms = float(np.mean([hip.elapsed_ms(e0, e1) for e0, e1 in qq_gemm_ev]))
        ktfs = flop / (gemm_ms * 1e-3) / 1e12
        out["roofline_qmm"] = {"bound": "mfma", "achieved": round(ktfs, 1),
                               "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
                               "frac": round(ktfs / MFMA_F16_PEAK_TFS, 4),
                               "traffic": measured_traffic("qqmm_nvfp4_m2048", ["qmm.hip"]),
                               "kernel": "gemm_dq_kernel<NVFP4 qq> (fp16 MFMA), NVFP4 qqmm M=2048",
                               "launch_us": round(gemm_ms * 1e3, 2),
                               "whole_call_tflops": round(tfs, 1),
                               "note": "2*M*N*K over the GEMM's own duration (HIP events on its "
                                       "first and last launch: 256x256 tiles, then the last "
                                       "round's columns on 128x64 tiles), mean of the timed "
                                       "steps that carry them (every other step: each event "
                                       "costs about 5 us around its launch); whole_call_tflops "
                                       "adds the activation amax and quantize pre-pass and is "
                                       "taken on the steps without those events"}
        for M in (1134, 4096):
            key = f"qqmm_{M}"
            if key in ms:
                out[f"qmm_tflops_m{M}"] = round(2.0 * M * INTER * HIDDEN / (ms[key] * 1e-3) / 1e12, 1)
    if "qmm_affine" in ms:
        out["qmm_affine_tflops"] = round(2.0 * 2048 * INTER * HIDDEN / (ms["qmm_affine"] * 1e-3) / 1e12, 1)
    var = {name: round(var_bytes(name) / (ms[f"qmv_{name}"] * 1e-3) / 1e9, 1)
           for name in VARIANTS if f"qmv_{name}" in ms}
    if var:
        out["qmv_variants_gbs"] = var
    cross = {}
    for M in (1134, 2048, 4096):
        if f"dense_{M}" in ms and f"wonly_{M}" in ms:
            flop = 2.0 * M * INTER * HIDDEN
            cross[str(M)] = {"dense_tflops": round(flop / (ms[f"dense_{M}"] * 1e-3) / 1e12, 1),
                             "fused_tflops": round(flop / (ms[f"wonly_{M}"] * 1e-3) / 1e12, 1),
                             "dense_over_fused": round(ms[f"wonly_{M}"] / ms[f"dense_{M}"], 3)}
    if cross:
        out["dense_crossover"] = cross
    fp4 = {}
    for key, stage, nbytes in (("mxfp4_m1", "qmv_mx1", fp4_bytes(5760, 2880, 32, 1)),
                               ("mxfp4_m8", "qmv_mx8", fp4_bytes(5760, 2880, 32, 8)),
                               ("nvfp4_m1", "qmv_nv1", fp4_bytes(INTER, HIDDEN, 16, 1))):
        if stage in ms:
            fp4[key] = round(nbytes / (ms[stage] * 1e-3) / 1e9, 1)
    if fp4:
        out["qmv_fp4_gbs"] = fp4
    if "qq_decode" in ms:
        out["qq_decode_gbs"] = round(fp4_bytes(INTER, HIDDEN, 16) / (ms["qq_decode"] * 1e-3) / 1e9, 1)
    if "qmm_mx32" in ms:  # HBM-bound size: weight + activation bytes per call
        out["qmm_mx32_gbs"] = round((fp4_bytes(5760, 2880, 32, 32) + 32 * 2880 * 2)
                                    / (ms["qmm_mx32"] * 1e-3) / 1e9, 1)
    if "qmm_mx512" in ms:  # against the dense FP4 MFMA peak
        tf = 2.0 * 512 * 5760 * 2880 / (ms["qmm_mx512"] * 1e-3) / 1e12
        out["qmm_mx512_tflops"] = round(tf, 1)
        out["qmm_mx512_frac_fp4"] = round(tf / FP4_PEAK_TFS, 4)
    # amax pass + quantize pass: X read twice, codes and scales written
    nbytes = 4096 * HIDDEN * 2 * 2 + 4096 * HIDDEN // 2 + 4096 * HIDDEN // 16
    if "act_quant" in ms:
        out["act_quant_gbs"] = round(nbytes / (ms["act_quant"] * 1e-3) / 1e9, 1)
    if "act_quant_warm" in ms:
        out["act_quant_warm_gbs"] = round(nbytes / (ms["act_quant_warm"] * 1e-3) / 1e9, 1)
    if "act_quant_sr" in ms:  # + 4 bytes of random word per element
        nbytes = 4096 * HIDDEN * (2 * 2 + 4) + 4096 * HIDDEN // 2 + 4096 * HIDDEN // 16
        out["act_quant_sr_gbs"] = round(nbytes / (ms["act_quant_sr"] * 1e-3) / 1e9, 1)

    # Every hot-path row against the roofline that bounds it: algorithmic bytes
    # (HBM rows) or 2*M*N*K flops (MFMA rows) over the stage's time per call.
    def hbm_row(stage, nbytes):
        if stage in ms:
            a = nbytes / (ms[stage] * 1e-3) / 1e9
            return {"stage": stage, "bound": "hbm", "achieved": round(a, 1), "unit": "GB/s",
                    "peak": HBM_PEAK_GBS, "frac": round(a / HBM_PEAK_GBS, 4)}

    def mfma_row(stage, flop, peak):
        if stage in ms:
            a = flop / (ms[stage] * 1e-3) / 1e12
            return {"stage": stage, "bound": "mfma", "achieved": round(a, 1), "unit": "TFLOP/s",
                    "peak": peak, "frac": round(a / peak, 4)}

    NX = 4096 * HIDDEN
    rows = {
        "a1+a2 NVFP4 activation amax + quantize [4096,5120], cold":
            hbm_row("act_quant", NX * 2 * 2 + NX // 2 + NX // 16),
        "a3+a4 MXFP4 quantize W[5760,2880] + affine quantize W[1024,512]":
            hbm_row("w_quant", 5760 * 2880 * 2 + 5760 * 2880 // 2 + 5760 * 90
                    + 1024 * 512 * 2 + 1024 * 512 // 2 + 2 * 2 * 1024 * 8),
        "a5 NVFP4 dequantize [4096,5120]": hbm_row("dequant", NX // 2 + NX // 16 + NX * 2),
        "a6 affine qmv sweep (gate+up batched)": hbm_row("qmv_sweep", sweep_bytes),
        "a6 affine qmv sweep, one launch per matrix": hbm_row("qmv_sweep_single", sweep_bytes),
        "a7 NVFP4 qmv [25600,5120] M=1": hbm_row("qmv_nv1", fp4_bytes(INTER, HIDDEN, 16, 1)),
        "a7 MXFP4 qmv [5760,2880] M=1": hbm_row("qmv_mx1", fp4_bytes(5760, 2880, 32, 1)),
        "a7 MXFP4 qmv [5760,2880] M=8": hbm_row("qmv_mx8", fp4_bytes(5760, 2880, 32, 8)),
        "a8+a9+a12 NVFP4 qqmm M=2048, whole call":
            mfma_row("qqmm", 2.0 * 2048 * INTER * HIDDEN, MFMA_F16_PEAK_TFS),
        "a10 MXFP4 qq M=512": mfma_row("qmm_mx512", 2.0 * 512 * 5760 * 2880, FP4_PEAK_TFS),
        "a10 MXFP4 qq M=32 (weight-streaming size)":
            hbm_row("qmm_mx32", fp4_bytes(5760, 2880, 32, 32) + 32 * 2880 * 2),
        "a11 affine weight-only qmm M=2048":
            mfma_row("qmm_affine", 2.0 * 2048 * INTER * HIDDEN, MFMA_F16_PEAK_TFS),
        "n1 NVFP4 qq decode M=1": hbm_row("qq_decode", fp4_bytes(INTER, HIDDEN, 16)),
        "n2 dense prefill path M=2048":
            mfma_row("dense_2048", 2.0 * 2048 * INTER * HIDDEN, MFMA_F16_PEAK_TFS),
        "n3 MXFP8 qmv [25600,5120] M=1": hbm_row("qmv_mxfp8", var_bytes("mxfp8")),
        "n4 NVFP4 stochastic-rounding quantize [4096,5120]":
            hbm_row("act_quant_sr", NX * (2 * 2 + 4) + NX // 2 + NX // 16),
    }
    out["row_rooflines"] = {k: v for k, v in rows.items() if v is not None}

    if not args.no_cpu_baseline and out["value"] is not None:
        out["cpu_baseline"] = cpu_baseline(log)
    print(json.dumps(out), flush=True)


class HipEvents:
    """A pool of timing-enabled hipEvent_t handles from the HIP runtime that
    PyTorch already loaded (plain handles for bsfp_time_next_launch)."""

    def __init__(self, n):
        import ctypes as C
        self.C = C
        self.rt = C.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.pool = []
        for _ in range(n):
            e = C.c_void_p()
            if self.rt.hipEventCreate(C.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.pool.append(e.value)
        self.next = 0

    def take(self):
        e = self.pool[self.next]
        self.next += 1
        return e

    def elapsed_ms(self, a, b):
        ms = self.C.c_float()
        if self.rt.hipEventElapsedTime(self.C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def measured_traffic(name, sources):
    """HBM bytes per launch from the committed counter summary profiles/<name>_traffic.txt.

    The summary records FETCH_SIZE + WRITE_SIZE per dispatch (scaled by the
    factor a 1 GiB copy kernel gives) together with the SHA-256 of the
    kernel sources it was taken on; once those sources change the figure no
    longer describes the kernel and None is returned.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in ["bsfp_device.hpp"] + sources:
        with open(os.path.join(ROOT, "block_scaled_bit_fp_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest() or "hbm_bytes_per_launch" not in fields:
        return None
    return int(float(fields["hbm_bytes_per_launch"]))


def host_info():
    """nproc, CPU model and the oracle's OpenMP thread count on this host."""
    import ctypes as C
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    gomp = C.CDLL("libgomp.so.1")  # the OpenMP runtime the oracle links
    return {"nproc": os.cpu_count(), "cpus_usable": len(os.sched_getaffinity(0)),
            "cpu_model": model, "omp_threads": int(gomp.omp_get_max_threads()),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def device_info(props):
    """GPU engine clock, CU count, gfx target and the HIP / ROCm versions."""
    import ctypes as C

    import torch
    rt = C.CDLL("libamdhip64.so")
    clk, rtv, drv = C.c_int(0), C.c_int(0), C.c_int(0)
    rt.hipDeviceGetAttribute(C.byref(clk), 5, 0)  # hipDeviceAttributeClockRate (kHz)
    rt.hipRuntimeGetVersion(C.byref(rtv))
    rt.hipDriverGetVersion(C.byref(drv))
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"device": props.name, "gfx": props.gcnArchName.split(":")[0],
            "cus": props.multi_processor_count, "peak_engine_clock_mhz": clk.value // 1000,
            "hbm_gib": round(props.total_memory / 2 ** 30, 1), "hip_runtime": rtv.value,
            "hip_driver": drv.value, "rocm": rocm, "torch": torch.__version__,
            "torch_hip": torch.version.hip}


def cpu_baseline(log):
    """The oracle (plain C: fp32 quantizer decisions, fp64 dequantize and
    matmul, OpenMP over outputs in the matmul only) timed on a bounded sample
    of every workload, once on one thread and once on all of them.  The
    headline `value` is the affine decode qmv on all threads (the metric's
    unit); `configs` holds the rest."""
    import ctypes as C

    import numpy as np

    import synth_inputs as S
    from oracle import oracle as o

    gomp = C.CDLL("libgomp.so.1")
    all_threads = int(gomp.omp_get_max_threads())

    def timed(fn, min_s=1.0, max_reps=50):
        fn()  # first call outside the clock (page-in)
        reps, t = 0, 0.0
        while (t < min_s and reps < max_reps) or reps == 0:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            reps += 1
        return t / reps

    def both(fn, work, unit_div):
        res = {}
        for label, n in (("single_thread", 1), ("all_threads", all_threads)):
            gomp.omp_set_num_threads(n)
            res[label] = round(work / timed(fn) / unit_div, 4)
        gomp.omp_set_num_threads(all_threads)
        return res

    cfg = {}
    # 1: affine qmv x[1,512] . W[1024,512]^T (whole workload)
    x1, w1 = S.affine_small()
    q1 = o.quantize(o.AFFINE, w1)
    cfg["affine_qmv_1024x512"] = {"unit": "GB/s", "sample": "whole workload", **both(
        lambda: o.matmul_wonly(x1, q1), affine_bytes(1024, 512), 1e9)}
    # 2: NVFP4 activation amax + quantize, the first 256 of the 4096 rows
    xa = np.ascontiguousarray(S.nvfp4_activations()[:256])
    row_bytes = HIDDEN * 2 * 2 + HIDDEN // 2 + HIDDEN // 16
    cfg["nvfp4_quantize_4096x5120"] = {
        "unit": "GB/s", "sample": "rows 0..255 of X (amax over the sample, then quantize); "
        "the quantizer is sequential", **both(lambda: o.quantize(o.NVFP4, xa), 256 * row_bytes,
                                               1e9)}
    # 3: affine decode qmv on W_up, the first 2560 of 25600 rows
    x3, w3 = S.affine_decode("up")
    q3 = o.quantize(o.AFFINE, np.ascontiguousarray(w3[:2560]))
    del w3
    cfg["affine_qmv_25600x5120"] = {"unit": "GB/s", "sample": "rows 0..2559 of W_up",
                                    **both(lambda: o.matmul_wonly(x3, q3),
                                           affine_bytes(2560, HIDDEN), 1e9)}
    # 4: MXFP4 W[5760,2880]: qmv at M = 1 (all rows) and the qq product at
    # M = 512 on the first 576 weight rows
    w4 = S.mxfp4_weights()
    q4 = o.quantize(o.MXFP4, w4)
    q4s = o.quantize(o.MXFP4, np.ascontiguousarray(w4[:576]))
    x41, x4 = S.mxfp4_activations(1), S.mxfp4_activations(512)
    cfg["mxfp4_qmv_m1_5760x2880"] = {"unit": "GB/s", "sample": "whole workload", **both(
        lambda: o.matmul_wonly(x41, q4), fp4_bytes(5760, 2880, 32, 1), 1e9)}
    cfg["mxfp4_qq_m512_5760x2880"] = {
        "unit": "GFLOP/s", "sample": "x[512,2880] against W rows 0..575 (x quantized in the call)",
        **both(lambda: o.matmul_qq(x4, q4s), 2.0 * 512 * 576 * 2880, 1e9)}
    # 5: NVFP4 qq prefill, 64 rows of X[2048,5120] against the first 2560 W rows
    x5, w5 = S.nvfp4_prefill(M=64, N=2560, K=HIDDEN, seed=5)
    q5 = o.quantize(o.NVFP4, w5)
    cfg["nvfp4_qqmm_2048x25600x5120"] = {
        "unit": "GFLOP/s", "sample": "X[64,5120] against W[2560,5120] (x quantized in the call, "
        "g_x from the sample)", **both(lambda: o.matmul_qq(x5, q5), 2.0 * 64 * 2560 * HIDDEN,
                                       1e9)}
    head = cfg["affine_qmv_25600x5120"]
    log("[bench] cpu oracle: " + ", ".join(
        f"{k}={v['single_thread']}/{v['all_threads']} {v['unit']}" for k, v in cfg.items()))
    return {"value": head["all_threads"], "unit": "GB/s", "cores": all_threads, "kind": "oracle",
            "sample": "affine g64 qmv x[1,5120] . W_up[2560 of 25600 rows, 5120]^T: fp64 "
                      "dequantize and dot products, OpenMP over outputs, on all threads; "
                      "`configs` has every workload on one thread and on all",
            "single_thread_value": head["single_thread"], "configs": cfg, "host": host_info()}


if __name__ == "__main__":
    main()
