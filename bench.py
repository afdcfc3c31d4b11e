#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X.

Workload (default): the skewed prefill layer -- T=16384 tokens, d_model=7168,
256 routed experts + 1 shared expert, top-8, SwiGLU width 2048, bf16
activations and weights with fp32 accumulation, fp32 router whose rows carry
a Zipf(1.1) factor, bias starting at 0 -- run as its balancing loop: each
step is one pass of the whole path (route, dispatch, routed expert FFN,
shared expert + combine, sign-step bias update) over the same batch, and the
bias carries from step to step.  Inputs are seeded synthetic data, resident
in HBM before the timed region starts.

Prints ONE JSON line on stdout (progress goes to stderr).
  value          tokens/s over the timed steps (T * steps / wall time)
  roofline       the dominant kernel (the routed gate/up grouped GEMM),
                 average duration from HIP events on the launch stream:
                 MFMA-bound workloads report algorithmic FLOPs per launch
                 (2 * T*k * d * 2I) against the dense MFMA peak of the weight
                 type; HBM-bound ones (FLOP/byte under the ridge, e.g. decode)
                 report algorithmic bytes (touched experts' gate/up weights
                 once, x once, h once) against 8 TB/s
  roofline_down  the same for the routed down GEMM (2 * T*k * I * d FLOPs)
  imbalance_curve  max/mean expert load at every step of the 100-step loop
                 (steps past --steps run untimed, continuing the same loop)
  cpu_baseline   the CPU oracle (fp64, plain loops) timed on a sample of the
                 same workload's tokens through the whole forward
  sub_results    (default workload only) the fp8 prefill, decode, mid-size
                 (T=2048, d=2048, I=512) and EP8-shard (one GPU's 32 experts
                 of an 8-way expert-parallel layer) workloads, 20 timed steps
                 each, with their own roofline entries

--dense-reference instead prints {"dense_reference": [...]}: the routed
gate/up kernel on one dense group (every row on one expert, M = 65536 and
131072 rows) beside the vendor GEMM (torch.matmul / torch._scaled_mm) on the
same product, bf16 and e4m3, for context on the kernel's own efficiency.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA, MI355X
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA, MI355X
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "sparse_expert_routing_amd", "csrc", "ffn_bf16_large.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_gemm_bf16_mi16_gateup_traffic_prefill-zipf-bf16.md")
METRIC = "MoE-layer tokens/s (T=16384,d=7168,256e top-8) + % of MFMA/HBM peak"
TRAFFIC_WORKLOAD = "prefill-zipf-bf16 T16384 d7168 I2048"  # the workload the counter summary covers


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps of the balancing loop")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps (on a scratch copy of the bias)")
    ap.add_argument("--config", type=int, default=4, choices=[2, 3, 4, 5, 6],
                    help="workload (4: the skewed prefill layer the metric is quoted on; 6: one GPU's "
                         "share of an 8-way expert-parallel layer, 32 experts of ~4096 rows)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loop-steps", type=int, default=None,
                    help="length of the balancing loop for the imbalance curve (default: the workload's, 100 for "
                         "the skewed prefill); steps past --steps run untimed; 0: only the timed steps")
    ap.add_argument("--no-sub", action="store_true",
                    help="skewed workload only: skip the fp8 and decode sub-results")
    ap.add_argument("--backward", action="store_true",
                    help="also time the layer backward (moe_backward: bf16 GEMMs, or e4m3 GEMMs with e4m3 weights) after the timed loop and report it")
    ap.add_argument("--fresh-batches", type=int, default=0,
                    help="N > 0: every step takes a new token batch (N batches resident in HBM, cycled); "
                         "default: the same batch every step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (the byte-counter reference)")
    ap.add_argument("--dense-reference", action="store_true",
                    help="only time the routed gate/up kernel on one dense group (every row to one expert) "
                         "beside the vendor GEMM (torch.matmul, torch._scaled_mm) on the same shape; one JSON line")
    ap.add_argument("--dense-reps", type=int, default=100, help="launches per timing in --dense-reference")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the layer on one GPU only (asked for {max(args.gpus, world)}); "
              "the layer has no multi-GPU implementation", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from sparse_expert_routing_amd import _lib

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 3 x 1 GiB")
        return
    _lib.load()  # fails loudly without the HIP library
    if args.dense_reference:
        print(json.dumps({"dense_reference": dense_reference(args.dense_reps)}), flush=True)
        return
    cfg = synth.CONFIGS[args.config]
    K = args.steps
    # the balancing loop of the skewed workload always runs its full length
    # (100 steps) for the imbalance curve; steps past the timed ones are untimed
    curve_steps = max(K, cfg.steps if args.loop_steps is None else args.loop_steps)
    out, inp = measure(cfg, K, args.warmup, curve_steps, args.fresh_batches, backward=args.backward)
    out["metric"] = METRIC
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    del inp
    if args.config == 4 and not args.no_sub:
        # the other full-size workloads, each with its own roofline entry
        sub = {}
        for cid in (5, 3, 2, 6):
            release()
            r, _ = measure(synth.CONFIGS[cid], max(10, min(K, 20)), min(args.warmup, 3), 0, 0)
            sub[r["config"]["workload"]] = r
        out["sub_results"] = sub
    print(json.dumps(out), flush=True)


def dense_reference(reps, rows=(65536, 131072)):
    """The routed gate/up kernel (moe_expert_gate_up) on one dense group of M
    rows (offsets put every row on expert 0), and the vendor GEMM on the same
    [M, d] x [2I, d]^T product: torch.matmul in bf16, torch._scaled_mm in e4m3
    (per-tensor scales; the library applies per-tile E8M0 scales and fuses
    SwiGLU, writing h [M, I] instead of [M, 2I]).  Each timing is the mean of
    the second half of `reps` back-to-back launches (sustained clock), the two
    alternating twice."""
    import torch

    from sparse_expert_routing_amd import _lib
    d, I, E, k = 7168, 2048, 256, 8

    def timed(fn):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
        tail = ms[reps // 2:]
        return sum(tail) / len(tail)

    g = torch.Generator(device="cuda").manual_seed(11)
    res = []
    for M in rows:
        flops = 2.0 * M * 2 * I * d
        for wt in ("bf16", "e4m3"):
            ds = _lib.desc(M // k, d, E, k, I, "bf16", wt)
            offsets = torch.full((E + 1,), M, dtype=torch.int32, device="cuda")
            offsets[0] = 0
            if wt == "bf16":
                xp = torch.randn(M, d, device="cuda", generator=g).mul_(0.5).to(torch.bfloat16)
                gate = torch.empty(E, I, d, device="cuda", dtype=torch.bfloat16)
                up = torch.empty_like(gate)
                gate[0].normal_(0, 0.02, generator=g)
                up[0].normal_(0, 0.02, generator=g)
                down = torch.empty(E, d, I, device="cuda", dtype=torch.bfloat16)
                ew, xs = _lib.ffn_weights(gate, up, down), None
                b = torch.cat([gate[0], up[0]], 0)
                vendor = lambda: torch.matmul(xp, b.t())  # noqa: E731
            else:
                # random e4m3 codes below 0x78 (finite), E8M0 scales 2^-7
                xp = torch.randint(0, 0x78, (M, d), device="cuda", dtype=torch.uint8, generator=g)
                xs = torch.full((M, d // 128), 120, device="cuda", dtype=torch.uint8)
                gate = torch.empty(E, I, d, device="cuda", dtype=torch.uint8)
                up = torch.empty_like(gate)
                gate[0].random_(0, 0x78, generator=g)
                up[0].random_(0, 0x78, generator=g)
                down = torch.empty(E, d, I, device="cuda", dtype=torch.uint8)
                s_gu = torch.full((E, I // 128, d // 128), 120, device="cuda", dtype=torch.uint8)
                s_d = torch.full((E, d // 128, I // 128), 120, device="cuda", dtype=torch.uint8)
                ew = _lib.ffn_weights(gate, up, down, s_gu, s_gu, s_d)
                a8 = xp.view(torch.float8_e4m3fn)
                b8 = torch.cat([gate[0], up[0]], 0).view(torch.float8_e4m3fn)
                one = torch.ones((), device="cuda", dtype=torch.float32)
                vendor = lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one,  # noqa: E731
                                                  out_dtype=torch.bfloat16)
            ws = torch.empty(_lib.workspace_bytes(ds, _lib.MOE_WS_FFN), dtype=torch.uint8, device="cuda")
            ours = lambda: _lib.moe_expert_gate_up(ds, xp, xs, offsets, ew, ws)  # noqa: E731
            t_o, t_v = [], []
            for _ in range(2):
                t_o.append(timed(ours))
                t_v.append(timed(vendor))
            peak = PEAK_BF16_TFLOPS if wt == "bf16" else PEAK_FP8_TFLOPS
            o, v = min(t_o), min(t_v)
            r = {"dtype": wt, "M": M, "N": 2 * I, "K": d, "ours_ms": round(o, 4), "vendor_ms": round(v, 4),
                 "ours_tflops": round(flops / o / 1e9, 1), "vendor_tflops": round(flops / v / 1e9, 1),
                 "ours_frac": round(flops / o / 1e9 / peak, 4), "vendor_frac": round(flops / v / 1e9 / peak, 4)}
            log(f"[bench] dense {wt} {M}x{2 * I}x{d}: ours {o:.3f} ms ({r['ours_frac']:.3f} of peak), "
                f"vendor {v:.3f} ms ({r['vendor_frac']:.3f})")
            res.append(r)
            del xp, xs, gate, up, down, ws, ew
            release()
    return res


def release():
    import gc

    import torch
    gc.collect()
    torch.cuda.empty_cache()


def measure(cfg, K, warmup, curve_steps, fresh_batches, backward=False):
    """Time K steps of the workload's loop (each step the whole path plus the
    bias step, the bias carried from step to step) after `warmup` untimed
    steps on a scratch copy of the bias; then, up to `curve_steps`, more
    untimed steps continuing the same loop, for the imbalance curve.
    Returns (result dict, host inputs)."""
    import numpy as np
    import torch

    import synth
    from sparse_expert_routing_amd import _lib
    from sparse_expert_routing_amd.layer import layer_from_inputs, upload

    T, d, I, E, k = cfg.T, cfg.d, cfg.I, cfg.E, cfg.k
    A = T * k

    t0 = time.time()
    log(f"[bench] generating inputs for {cfg.name} (seed {cfg.seed})")
    inp = synth.make_inputs(cfg)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; uploading")
    layer = layer_from_inputs(inp)
    if fresh_batches > 0:
        xs = [upload(synth.make_x_step(cfg, b)) for b in range(fresh_batches)]
    else:
        xs = [upload(inp["x"])]
    bias0 = upload(inp["bias"])
    D = layer.desc
    stream = torch.cuda.current_stream()

    def step(bias, ev=None, s=0):
        x = xs[s % len(xs)]
        if ev is not None:
            ev[0].record(stream)
        _lib.moe_route(D, x, layer.wr, bias, layer.idx, layer.w, None, layer.ws, stream)
        if ev is not None:
            ev[1].record(stream)
        _lib.moe_dispatch(D, layer.idx, x, layer.counts, layer.offsets, layer.row_src, layer.row_of,
                          None, None, layer.ws, stream)
        if ev is not None:
            ev[2].record(stream)
        _lib.moe_expert_gate_up_rows(D, x, layer.row_src, layer.offsets, layer.ex_w, layer.ws, stream)
        if ev is not None:
            ev[3].record(stream)
        _lib.moe_expert_down(D, layer.offsets, layer.ex_w, layer.y_perm, layer.ws, stream)
        if ev is not None:
            ev[4].record(stream)
        _lib.moe_combine(D, x, layer.sh_w, layer.y_perm, layer.row_of, layer.w, layer.y, layer.ws, stream)
        if ev is not None:
            ev[5].record(stream)
        _lib.moe_bias_update(D, layer.counts, cfg.gamma, bias, stream)
        if ev is not None:
            ev[6].record(stream)

    log(f"[bench] {cfg.name}: warmup {warmup} steps")
    scratch_bias = bias0.clone()
    for w_ in range(warmup):
        step(scratch_bias, None, w_)
    torch.cuda.synchronize()

    n_all = max(K, curve_steps)
    bias = bias0.clone()
    counts_hist = torch.empty((n_all, E), dtype=torch.int32, device="cuda")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K)]
    log(f"[bench] {cfg.name}: timing {K} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(K):
        step(bias, events[s], s)
        counts_hist[s].copy_(layer.counts, non_blocking=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    if n_all > K:
        log(f"[bench] {cfg.name}: {n_all - K} more loop steps (untimed) for the imbalance curve")
        for s in range(K, n_all):
            step(bias, None, s)
            counts_hist[s].copy_(layer.counts, non_blocking=True)
        torch.cuda.synchronize()

    names = ["route", "dispatch", "expert_gate_up", "expert_down", "combine", "bias_update"]
    phase = {n: float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(K)]))
             for i, n in enumerate(names)}
    # per-step device time (first to last event of a step): mean, median, extremes
    step_dev = np.array([events[s][0].elapsed_time(events[s][6]) for s in range(K)])
    ch_all = counts_hist.cpu().numpy().astype(np.float64)
    imb = ch_all.max(axis=1) / ch_all.mean(axis=1)
    ch = ch_all[:K]  # the timed steps
    tiles = np.ceil(ch / 256.0).sum(axis=1)  # launched 256-row tiles of the routed GEMMs
    # the same tiles weighted by their height: live 32-row blocks / 8 (a block
    # with no rows issues no MFMA)
    tiles_h = (np.ceil(ch / 32.0) / 8.0).sum(axis=1)

    touched = float((ch > 0).sum(axis=1).mean())
    s_w = 1 if cfg.wt == "e4m3" else 2
    peak_flops = PEAK_FP8_TFLOPS if cfg.wt == "e4m3" else PEAK_BF16_TFLOPS
    sc = 4.0 * (I // 128) * (d // 128) if cfg.wt == "e4m3" else 0.0  # one expert matrix's block scales
    # gate/up: 2 * A * d * 2I FLOPs; bytes: the touched experts' gate and up
    # weights (+ block scales) read once, x read once, h written once
    gu = roofline_entry(2.0 * A * d * (2 * I), touched * (2.0 * I * d * s_w + 2 * sc) + T * d * 2.0 + A * I * s_w,
                        phase["expert_gate_up"], peak_flops)
    # down: 2 * A * I * d FLOPs; bytes: the touched experts' down weights
    # (+ scales) once, h read once, y_perm (bf16) written once
    dn = roofline_entry(2.0 * A * I * d, touched * (1.0 * I * d * s_w + sc) + A * I * s_w + A * d * 2.0,
                        phase["expert_down"], peak_flops)
    large = A >= 128 * E
    kname = ("k_gemm_fp8_mx" if large and I % 256 == 0 and d % 256 == 0 else "k_gemm_fp8") if cfg.wt == "e4m3" else \
        ("k_gemm_bf16_mi16" if large else "k_gemm_skinny" if A <= 4 * E else "k_gemm_bf16")
    total_flops = 2.0 * T * d * E + 6.0 * (A + T) * d * I
    ms_step = wall / K * 1e3
    log(f"[bench] {cfg.name}: {ms_step:.3f} ms/step, phases (ms): " + ", ".join(f"{n} {v:.3f}" for n, v in phase.items()))
    log(f"[bench] gate/up GEMM {gu['achieved']:.1f} {gu['unit']} ({100 * gu['frac']:.1f}% of peak); down "
        f"{dn['achieved']:.1f} {dn['unit']} ({100 * dn['frac']:.1f}%); layer {total_flops / (ms_step * 1e-3) / 1e12:.1f} "
        f"TFLOP/s; max/mean load {imb[0]:.2f} -> {imb[-1]:.2f} over {len(imb)} steps; 256-row tiles "
        f"{tiles.mean():.0f}, weighted by height {tiles_h.mean():.1f} (ideal {A / 256:.0f})")

    gu.update({"kernel": f"routed gate/up grouped GEMM ({kname}, SwiGLU epilogue"
                         + (" + e4m3 quantisation)" if cfg.wt == "e4m3" else ")"),
               "traffic": measured_traffic() if cfg.name == TRAFFIC_WORKLOAD else None,
               "touched_experts": touched})
    dn.update({"kernel": f"routed down grouped GEMM ({kname}, bf16 store epilogue)", "touched_experts": touched})
    out = {
        "metric": f"MoE-layer tokens/s ({cfg.name}) + % of MFMA/HBM peak",
        "value": T * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "e4m3": "e4m3"}[cfg.wt],
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "d_model": d, "experts": E, "top_k": k, "shared_experts": 1,
                   "expert_intermediate": I, "router": "fp32 sigmoid", "router_row_skew": cfg.skew,
                   "bias_start": cfg.bias, "gamma": cfg.gamma, "loop_steps_timed": K, "seed": cfg.seed,
                   "batches": "fixed" if fresh_batches <= 0 else f"fresh ({fresh_batches} cycled)"},
        "roofline": gu,
        "roofline_down": dn,
        "phases_ms": phase,
        "step_ms_device": {"mean": float(step_dev.mean()), "median": float(np.median(step_dev)),
                           "min": float(step_dev.min()), "max": float(step_dev.max())},
        "phase_roofline": phase_roofline(cfg, phase),
        "layer_tflops": total_flops / (ms_step * 1e-3) / 1e12,
        "imbalance_max_over_mean": {"first": float(imb[0]), "last": float(imb[-1])},
        "imbalance_curve": [round(float(v), 4) for v in imb],
        "imbalance_curve_steps": {"timed": K, "untimed_after": int(n_all - K)},
        "routed_row_tiles_mean": float(tiles.mean()),
        "routed_row_tiles_height_weighted_mean": float(tiles_h.mean()),
        "routed_row_tiles_ideal": A / 256.0,
    }
    if backward:
        out["backward"] = time_backward(cfg, layer, xs[(K - 1) % len(xs)], min(K, 20))
    return out, inp


def roofline_entry(flops, nbytes, ms, peak_flops):
    """Achieved rate of one GEMM launch against its bound: MFMA (algorithmic
    FLOPs) when its FLOPs per algorithmic byte exceed the ridge point
    (peak FLOP/s / 8 TB/s), else HBM (algorithmic bytes)."""
    hbm = flops / nbytes < peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm:
        achieved, peak = nbytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBS
    else:
        achieved, peak = flops / (ms * 1e-3) / 1e12, peak_flops
    return {"bound": "hbm" if hbm else "mfma", "achieved": achieved, "peak": peak,
            "unit": "GB/s" if hbm else "TFLOP/s", "frac": achieved / peak,
            "flops_per_launch": flops, "bytes_per_launch": nbytes, "avg_launch_ms": ms}


def phase_roofline(cfg, phase):
    """Route, dispatch and bias update against the HBM peak over the bytes
    they must move (and the router's FLOPs): route reads x and W_r once and
    writes idx and the weights; dispatch (the GEMM gathers x itself) reads
    idx and writes counts, offsets, row_src and row_of; the bias update reads
    the counts and reads and writes the bias."""
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    xb = 4 if cfg.act == "f32" else 2
    b = {"route": T * d * xb + E * d * 4 + T * k * 8,
         "dispatch": T * k * 4 + E * 4 + (E + 1) * 4 + 2 * T * k * 4,
         "bias_update": E * 4 + 2 * E * 4}
    out = {}
    for n, nb in b.items():
        ms = phase[n]
        out[n] = {"bytes": nb, "gbs": nb / (ms * 1e-3) / 1e9, "frac_of_hbm": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    fl = 2.0 * T * d * E
    out["route"]["flops"] = fl
    out["route"]["tflops"] = fl / (phase["route"] * 1e-3) / 1e12
    return out


def time_backward(cfg, layer, x, n):
    """moe_backward on the last timed step's routing (a seeded dy), n timed calls after
    2 warm-up calls, HIP events on the launch stream.  Algorithmic FLOPs per call: per
    routed row and per shared row 16*d*I (recompute gate/up 4, dh 2, dx 4, dW gate/up 4,
    dW down 2, all x d*I), plus the router's 2 * 2*k*d per token."""
    import torch
    from sparse_expert_routing_amd import _lib
    T, d, I, k, E = cfg.T, cfg.d, cfg.I, cfg.k, cfg.E
    if cfg.act != "bf16" or cfg.wt not in ("bf16", "e4m3"):
        return None
    D = layer.desc
    stream = torch.cuda.current_stream()
    dev = dict(device="cuda", dtype=torch.float32)
    grads = dict(dx=torch.empty((T, d), **dev), dw_router=torch.empty((E, d), **dev),
                 dw_gate=torch.empty((E, I, d), **dev), dw_up=torch.empty((E, I, d), **dev),
                 dw_down=torch.empty((E, d, I), **dev), ds_gate=torch.empty((I, d), **dev),
                 ds_up=torch.empty((I, d), **dev), ds_down=torch.empty((d, I), **dev),
                 dg=torch.empty((T, k), **dev))
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    dy = torch.randn((T, d), generator=gen, **dev)
    ws = torch.empty(_lib.workspace_bytes(D, _lib.MOE_WS_BACKWARD), dtype=torch.uint8, device="cuda")

    def call():
        _lib.moe_backward(D, x, layer.wr, layer.idx, layer.w, layer.offsets, layer.row_src, layer.row_of,
                          layer.ex_w, layer.sh_w, layer.y_perm, dy, grads, ws, stream)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 16.0 * (T * k + T) * d * I + 4.0 * T * k * d
    peak = PEAK_FP8_TFLOPS if cfg.wt == "e4m3" else PEAK_BF16_TFLOPS
    log(f"[bench] backward {ms:.3f} ms, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s algorithmic")
    return {"ms": ms, "calls": n, "gemm_dtype": cfg.wt, "flops_per_call": flops,
            "tflops": flops / (ms * 1e-3) / 1e12, "peak_tflops": peak,
            "frac_of_peak": flops / (ms * 1e-3) / 1e12 / peak}


def measured_traffic():
    """HBM bytes per gate/up launch from the committed FETCH_SIZE / WRITE_SIZE
    summary (counter runs scaled by a plain-copy calibration), or None when
    the kernel source has changed since those counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(line.split(":", 1) for line in f if line.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
        with open(KERNEL_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if kv.get("source_sha256", "").strip() != sha:
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_baseline(cfg, inp, target_s):
    """The oracle (plain fp64 loops, OpenMP over tokens), as it stands, on a
    sample of the workload's tokens through the whole forward."""
    import numpy as np

    import oracle

    sh = oracle.shape_of(cfg)

    def run(n):
        toks = (np.arange(n, dtype=np.int64) * (cfg.T // n)).astype(np.int32)
        t = time.perf_counter()
        oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"], toks)
        return time.perf_counter() - t

    cores = oracle.num_threads()
    n0 = max(cores, 8)
    t0 = run(n0)
    n = int(min(cfg.T, max(n0, round(n0 * target_s / max(t0, 1e-3)))))
    n = max(cores, (n // cores) * cores)
    log(f"[bench] oracle: {n0} tokens in {t0:.2f}s; timing {n} tokens on {cores} threads")
    t = run(n)
    # the same on one core, on a few tokens (about 3 s)
    n1 = max(2, min(n, round(3.0 / max(t0 * cores / n0, 1e-3))))
    oracle.set_threads(1)
    try:
        t1 = run(n1)
    finally:
        oracle.set_threads(cores)
    log(f"[bench] oracle on 1 core: {n1} tokens in {t1:.2f}s")
    return {"value": n / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of the {cfg.T} tokens (every {cfg.T // n}th) through route + 8 routed experts + "
                      f"shared expert + combine in fp64; {t:.1f}s",
            "value_1core": n1 / t1, "sample_1core": f"{n1} tokens (every {cfg.T // n1}th) on 1 thread; {t1:.1f}s"}


if __name__ == "__main__":
    main()
