"""Benchmark of the batch-invariant hot path on one MI355X.

One step = one pass of the whole path over one batch of M = 4096 synthetic rows
at Llama-3-8B projection shapes (K = 4096):
    H  = bi_rmsnorm(X, g)                      X [M, 4096] ~ N(0,1), g ~ N(1, 0.1^2)
    Q  = bi_gemm(H, Wq)     N = 4096            W* ~ N(0, 0.02^2), stored [N, K]
    KV = bi_gemm(H, Wkv)    N = 1024
    U  = bi_gemm(H, Wup)    N = 14336
    D  = bi_gemm(U, Wdown)  K = 14336, N = 4096
    L  = bi_lora_shrink(H, A, split 8)   and the unsplit pass and the atomic
         control (A [16, 4096] ~ N(0, 0.01^2), fp32 out)
    bi_row_bitdiff_batch: probe rows of every output (H, Q, KV, U, D, L, Lu) against
         the same rows computed alone, in one launch, counted on every timed step
Inputs are resident in HBM before timing starts.  ``value`` is the step's
algorithmic TFLOP/s (2*M*N*K per GEMM, 2*M*R*K per shrink) over the timed
steps.  ``roofline`` is for the dominant kernel (the 256x256-tile GEMM, which
runs Q, U and D), timed with HIP events around its launches on the launch
stream.  ``cpu_baseline`` is the fp64 CPU oracle timed on a bounded row sample
of the same step.  ``clock`` is the shader clock and socket power read during
the untimed settle steps, and the dominant kernel's fraction of the MFMA peak
scaled to that clock (the published peak assumes 2.4 GHz).

After the step, the rest of the headline metric is graph-timed on its own:
``gemm_over_m`` (bi_gemm at M = 2048, 4096, 8192 on the four projections, with
geometric means), ``gemm_fill_over_m`` (the same for bi_gemm_fill, whose bits
equal bi_gemm's at every M but whose tile follows M), ``gemm_small_m`` (the
fixed split-K GEMM at M = 1, 16, 64: time and HBM GB/s), ``rmsnorm`` (GB/s over rotated copies, beside a plain device
copy of the same bytes), ``shrink`` (the variants at M = 4096 and the two
latency ratios the LoRA page reports), the shrink's replay variation, and
``stream70b`` (the Llama-3-70B MLP shape over a 200-batch dynamic stream).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--M 4096]
       [--step-only]    skip the metric parts after the step
       [--sweep FILE]   also time each kernel over an M sweep (JSONL to FILE)
       [--replays FILE] also run the 1000-replay shrink protocol at every M
       [--only NAME]    run only one kernel repeatedly (for rocprofv3 runs)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "batch-invariant bf16 GEMM TFLOP/s (% MFMA peak) over M; RMSNorm GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
SPEC_SCLK_MHZ = 2400.0        # the clock the published peaks assume
K_MODEL, N_Q, N_KV, N_UP = 4096, 4096, 1024, 14336
R_LORA = 16


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--M", type=int, default=4096)
    ap.add_argument("--sweep", default=None)
    ap.add_argument("--only", default=None,
                    choices=["gemm", "gemm_kv", "gemm_kv_fill", "gemm_up", "gemm_up_fill", "gemm_down", "rmsnorm", "shrink_det8",
                             "shrink_two_pass", "shrink_atomic8", "shrink_unsplit", "copy",
                             "splitk", "attention", "expand"])
    ap.add_argument("--iters", type=int, default=50, help="launches for --only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="report the step only (skip the metric's GEMM-over-M, RMSNorm, shrink, "
                         "replay and 70B-stream parts)")
    ap.add_argument("--replays", default=None,
                    help="also run the shrink replay protocol over every configured M (JSONL to FILE)")
    ap.add_argument("--settle", type=float, default=2.5,
                    help="seconds of untimed steps before the warm-up steps, so the GPU "
                         "clocks leave their idle state (a few 1 ms steps do not); the "
                         "clock is read during them (the SMI table refreshes about once "
                         "a second)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "this path has no multi-GPU mode; row sharding needs no exchange and is "
              "written up with the design notes", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from invariant_deterministic_amd import binding as bi
    from invariant_deterministic_amd import synth, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M = args.M

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    x = workloads.llama8b_x(K_MODEL, rows=M)
    g = synth.normal_bf16((K_MODEL,), 2002, mean=1.0, std=0.1)
    ws_h = [workloads.llama8b_w(i) for i in range(4)]
    a = workloads.lora_inputs(1)[1]
    X, G, A = to_dev(x), to_dev(g), to_dev(a)
    Wq, Wkv, Wup, Wdown = (to_dev(w) for w in ws_h)
    H = torch.empty((M, K_MODEL), dtype=torch.bfloat16, device=dev)
    Q = torch.empty((M, N_Q), dtype=torch.bfloat16, device=dev)
    KV = torch.empty((M, N_KV), dtype=torch.bfloat16, device=dev)
    U = torch.empty((M, N_UP), dtype=torch.bfloat16, device=dev)
    D = torch.empty((M, K_MODEL), dtype=torch.bfloat16, device=dev)
    L = torch.empty((M, R_LORA), dtype=torch.float32, device=dev)
    Lu = torch.empty_like(L)
    La = torch.empty_like(L)
    WS = torch.empty(bi.bi_lora_shrink_workspace_bytes(M, R_LORA, 8), dtype=torch.uint8, device=dev)
    eps = workloads.EPS
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    if args.only:
        run_only(args, bi, torch, dev, X, G, H, Wq, Wkv, Wup, Wdown, U, A, L, WS, La, Lu, eps)
        return

    # Probe rows: each computed alone through the whole chain, for the in-step
    # bitwise check of every output the step writes.
    probes = sorted({0, 1, 255, 256, M // 2, M - 1} & set(range(M)))
    P = len(probes)
    solo = {"H": torch.empty((P, K_MODEL), dtype=torch.bfloat16, device=dev),
            "Q": torch.empty((P, N_Q), dtype=torch.bfloat16, device=dev),
            "KV": torch.empty((P, N_KV), dtype=torch.bfloat16, device=dev),
            "U": torch.empty((P, N_UP), dtype=torch.bfloat16, device=dev),
            "D": torch.empty((P, K_MODEL), dtype=torch.bfloat16, device=dev),
            "L": torch.empty((P, R_LORA), dtype=torch.float32, device=dev),
            "Lu": torch.empty((P, R_LORA), dtype=torch.float32, device=dev)}
    for i, p in enumerate(probes):
        h1 = solo["H"][i:i + 1]
        bi.bi_rmsnorm(X[p:p + 1], G, y=h1, eps=eps)
        bi.bi_gemm(h1, Wq, y=solo["Q"][i:i + 1])
        bi.bi_gemm(h1, Wkv, y=solo["KV"][i:i + 1])
        bi.bi_gemm(h1, Wup, y=solo["U"][i:i + 1])
        bi.bi_gemm(solo["U"][i:i + 1], Wdown, y=solo["D"][i:i + 1])
        bi.bi_lora_shrink(h1, A, y=solo["L"][i:i + 1], split_k=8)
        bi.bi_lora_shrink(h1, A, y=solo["Lu"][i:i + 1], split_k=1)
    outs = {"H": H, "Q": Q, "KV": KV, "U": U, "D": D, "L": L, "Lu": Lu}
    probe_pos = torch.tensor(probes, dtype=torch.int64, device=dev)
    probe_ids = torch.arange(P, dtype=torch.int64, device=dev)
    # one counts slot per output and per step (the gate step, then each timed
    # step), so that every timed step's comparison is kept, not just the last
    nslots = 1 + args.steps
    counts = torch.zeros((nslots, len(outs), P, 2), dtype=torch.int64, device=dev)
    scratch_counts = torch.zeros((len(outs), P, 2), dtype=torch.int64, device=dev)

    ev_pairs = []

    def step(timed: bool, slot=None):
        bi.bi_rmsnorm(X, G, y=H, eps=eps)
        for w, y, inp in ((Wq, Q, H), (Wkv, KV, H), (Wup, U, H), (Wdown, D, U)):
            big = w.shape[0] >= 4096
            if timed and big:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            bi.bi_gemm(inp, w, y=y)
            if timed and big:
                e1.record()
                ev_pairs.append((e0, e1, 2.0 * M * w.shape[0] * w.shape[1]))
        bi.bi_lora_shrink(H, A, y=L, split_k=8)
        bi.bi_lora_shrink(H, A, y=Lu, split_k=1)
        bi.bi_lora_shrink_atomic(H, A, y=La, split_k=8)
        cs = counts[slot] if slot is not None else scratch_counts
        # every output's probe rows against their solo rows, in one launch
        bi.bi_row_bitdiff_batch([(outs[name], solo[name], probe_pos, probe_ids, cs[j])
                                 for j, name in enumerate(outs)], check_rows=False)

    # Gate before timing: the path must be batch-invariant on this input.
    step(False, slot=0)
    torch.cuda.synchronize()
    gate = {name: int(counts[0, j, :, 0].sum()) for j, name in enumerate(outs)}
    if any(gate.values()):
        print(json.dumps({"error": "batch-invariance gate failed", "diff_bits": gate}))
        sys.exit(1)

    # Untimed: let the clocks ramp from idle (measured: with only a handful of
    # warm-up steps the GEMMs run ~8 % slower than in steady state).
    # The shader clock and socket power are sampled during these steps (a
    # read-only query from a side thread), not during the timed ones.
    t_settle = time.time()
    settle_steps = 0
    with ClockSampler() as clk:
        while time.time() - t_settle < args.settle:
            for _ in range(20):
                step(False)
            settle_steps += 20
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(True, slot=1 + i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps

    flop_gemm = 2.0 * M * (K_MODEL * (N_Q + N_KV + N_UP) + N_UP * K_MODEL)
    flop_shrink = 3 * 2.0 * M * R_LORA * K_MODEL
    value = (flop_gemm + flop_shrink) / (ms_step * 1e-3) / 1e12

    durs = [e0.elapsed_time(e1) for e0, e1, _ in ev_pairs]
    flops = [f for _, _, f in ev_pairs]
    avg_ms = sum(durs) / len(durs)
    avg_flop = sum(flops) / len(flops)
    achieved = avg_flop / (avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(), "traffic_unit": "HBM bytes per launch (rocprofv3)",
                "kernel": "gemm_pp_kernel<256,256> (Q, U, D projections)",
                "avg_launch_us": round(avg_ms * 1e3, 2),
                "flop_per_launch": avg_flop}

    timed_bits = counts[1:, :, :, 0].sum(dim=(0, 2)).tolist()
    invariance = {"probe_rows": P, "outputs": list(outs),
                  "timed_steps_checked": args.steps,
                  "diff_bits_timed_steps": {n: int(b) for n, b in zip(outs, timed_bits)}}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_projections_step", "M": M, "K": K_MODEL,
                   "N": [N_Q, N_KV, N_UP], "down_proj": [N_UP, K_MODEL], "lora_rank": R_LORA,
                   "lora_split_k": 8, "parallelism": "single-gpu"},
        "roofline": roofline,
        "invariance": invariance,
        "settle": {"seconds": args.settle, "untimed_steps": settle_steps},
        "clock": clk.summary(achieved),
    }
    if not args.step_only:
        print("# metric parts: GEMM over M, RMSNorm, shrink, replays, 70B stream",
              file=sys.stderr, flush=True)
        out.update(metric_parts(bi, torch, dev, H, Wq, Wkv, Wup, Wdown, A, G, eps))
        invariance.update(out.pop("replays"))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, g, ws_h, a, eps)
    if args.sweep:
        out["sweep_file"] = args.sweep
        sweep(args.sweep, bi, torch, dev, to_dev)
    if args.replays:
        replay_table(args.replays, bi, torch, dev, to_dev)
    print(json.dumps(out), flush=True)


GiB = 1 << 30


def _copies(nbytes: int) -> int:
    """Copies of a buffer set that together touch at least 1 GiB, so the
    256 MB last-level cache cannot serve a rotated loop."""
    return max(1, min(64, -(-GiB // max(1, nbytes))))


def _geomean(v):
    import math
    return math.exp(sum(math.log(x) for x in v) / len(v))


def metric_parts(bi, torch, dev, H, Wq, Wkv, Wup, Wdown, A, G, eps):
    """The parts of the headline metric beyond the step, each graph-timed:
    the batch-invariant GEMM over M at every projection shape, RMSNorm over
    rotated copies at the configured batch sizes, the three shrink variants at
    M = 4096 with the pages' two latency ratios, the replay variation of the
    atomic control against the deterministic split, and the Llama-3-70B
    dynamic-batch stream."""
    from invariant_deterministic_amd import harness, synth, workloads
    res = {}

    # GEMM over M (compute-bound from M ~ 350: the inputs need no rotation)
    xp = {4096: synth.device_normal_bf16((8192, 4096), 3101),
          14336: synth.device_normal_bf16((8192, 14336), 3102)}
    shapes = (("q", Wq), ("kv", Wkv), ("up", Wup), ("down", Wdown))
    g_out = {"kernel": "bi_gemm (one tile configuration per (N, K))", "peak_tflops": PEAK_BF16_TFLOPS,
             "shapes": {}}
    # bi_gemm_fill: the same bits as bi_gemm at every M (each configuration
    # runs the same matrix-core steps in the same order) with the tile picked
    # from M; reported beside the single-configuration figures, not instead
    f_out = {"kernel": "bi_gemm_fill (bi_gemm's bits; tile chosen per call from M)",
             "peak_tflops": PEAK_BF16_TFLOPS, "shapes": {}}
    fracs, ffracs = [], []
    for name, W in shapes:
        N, K = W.shape
        y = torch.empty((8192, N), dtype=torch.bfloat16, device=dev)
        pts, fpts = {}, {}
        for M in (2048, 4096, 8192):
            xm, ym = xp[K][:M], y[:M]
            ms = _time_loop(torch, lambda i: bi.bi_gemm(xm, W, y=ym), 20)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            pts[str(M)] = {"us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                           "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
            fracs.append(tf / PEAK_BF16_TFLOPS)
            cf = bi.bi_gemm_fill_config_id(M, N, K)
            if cf != bi.bi_gemm_config_id(N, K):
                # gate: bi_gemm_fill is timed only if it reproduces bi_gemm's bits here
                y2 = bi.bi_gemm_fill(xm, W)
                if not torch.equal(y2.view(torch.int16), ym.view(torch.int16)):
                    raise SystemExit(f"bi_gemm_fill differs from bi_gemm at M={M} N={N} K={K}")
                del y2
                ms = _time_loop(torch, lambda i: bi.bi_gemm_fill(xm, W, y=ym), 20)
                tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            fpts[str(M)] = {"config": cf, "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                            "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
            ffracs.append(tf / PEAK_BF16_TFLOPS)
        gm = _geomean([v["frac"] for v in pts.values()])
        g_out["shapes"][name] = {"K": K, "N": N, "config": bi.bi_gemm_config_id(N, K), "M": pts,
                                 "geomean_frac": round(gm, 4)}
        f_out["shapes"][name] = {"K": K, "N": N, "M": fpts,
                                 "geomean_frac": round(_geomean([v["frac"] for v in fpts.values()]), 4)}
        print(f"# gemm over M {name}: " + ", ".join(f"M={m} {v['frac']:.3f}" for m, v in pts.items())
              + "; fill: " + ", ".join(f"M={m} {v['frac']:.3f}" for m, v in fpts.items()),
              file=sys.stderr, flush=True)
        del y
    g_out["geomean_frac_all"] = round(_geomean(fracs), 4)
    f_out["geomean_frac_all"] = round(_geomean(ffracs), 4)
    res["gemm_over_m"] = g_out
    res["gemm_fill_over_m"] = f_out

    # Decode-sized batches: the fixed split-K GEMM (split from (N, K); one
    # launch up to 16 rows) on each projection, the weight rotated over
    # >= 1 GiB of copies so that it streams from HBM.  HBM-bound: bytes =
    # 2(MK + NK + MN).  Gated: the rows of a batch equal those rows computed
    # in a 65-row batch (the two-launch path) bit for bit.
    GiB = 1 << 30
    s_out = {"kernel": "bi_gemm_splitk (split from (N, K))", "bytes": "2*(M*K + N*K + M*N)",
             "peak_gbs": PEAK_HBM_GBS, "shapes": {}}
    for name, W in shapes:
        N, K = W.shape
        S = bi.bi_gemm_splitk_for(N, K)
        cw = max(1, min(64, -(-GiB // (2 * N * K))))
        Ws = [W] + [W.clone() for _ in range(cw - 1)]
        x65 = xp[K][:65]
        ref = bi.bi_gemm_splitk(x65, W, split_k=S)
        pts = {}
        for M in (1, 16, 64):
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(bi.bi_gemm_splitk_workspace_bytes(M, N, S), dtype=torch.uint8, device=dev)
            bi.bi_gemm_splitk(x65[:M], W, y=y, split_k=S, ws=ws)
            if not torch.equal(y.view(torch.int16), ref[:M].view(torch.int16)):
                raise SystemExit(f"bi_gemm_splitk rows differ between batch sizes M={M} N={N} K={K}")
            xm = x65[:M]
            ms = _time_loop(torch, lambda i: bi.bi_gemm_splitk(xm, Ws[i % cw], y=y, split_k=S, ws=ws),
                            4 * cw)
            by = 2.0 * (M * K + N * K + M * N)
            pts[str(M)] = {"us": round(ms * 1e3, 2), "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                           "frac": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        s_out["shapes"][name] = {"K": K, "N": N, "split_k": S, "M": pts}
        print(f"# split-K {name} (S={S}): " + ", ".join(f"M={m} {v['us']} us {v['frac']:.3f}" for m, v in pts.items()),
              file=sys.stderr, flush=True)
        del Ws
    res["gemm_small_m"] = s_out
    del xp

    # RMSNorm, K = 4096, inputs and outputs rotated over >= 1 GiB
    K = 4096
    r_out = {"K": K, "bytes": "4*M*K + 2*K", "peak_gbs": PEAK_HBM_GBS, "M": {}}
    for M in (1, 7, 128, 2048, 8192):
        c = _copies(4 * M * K)
        xs = [synth.device_normal_bf16((M, K), 2100 + i) for i in range(c)]
        ys = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(c)]
        ms = _time_loop(torch, lambda i: bi.bi_rmsnorm(xs[i % c], G, y=ys[i % c], eps=eps), 4 * c)
        gbs = (4.0 * M * K + 2 * K) / (ms * 1e-3) / 1e9
        r_out["M"][str(M)] = {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                              "frac": round(gbs / PEAK_HBM_GBS, 4), "rotating_copies": c}
        del xs, ys
    print(f"# rmsnorm: " + ", ".join(f"M={m} {v['frac']:.3f}" for m, v in r_out["M"].items()),
          file=sys.stderr, flush=True)
    res["rmsnorm"] = r_out

    # The practical ceiling beside the 8 TB/s spec: a plain device copy (torch)
    # of the bytes RMSNorm moves at M = 2048 and 8192 (16 and 64 MiB each
    # way), rotated the same way
    ref = {}
    for mib in (16, 64):
        nb = mib << 20
        c = _copies(2 * nb)
        srcs = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(c)]
        dsts = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(c)]
        ms = _time_loop(torch, lambda i: dsts[i % c].copy_(srcs[i % c]), 4 * c)
        gbs = 2.0 * nb / (ms * 1e-3) / 1e9
        ref[f"{mib}MiB_each_way"] = {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                                     "frac": round(gbs / PEAK_HBM_GBS, 4)}
        del srcs, dsts
    r_out["device_copy_reference"] = ref
    print(f"# device copy: " + ", ".join(f"{k} {v['frac']:.3f}" for k, v in ref.items()),
          file=sys.stderr, flush=True)

    # LoRA shrink at M = 4096, x rotated over >= 1 GiB
    M, K, R = 4096, 4096, R_LORA
    c = _copies(2 * M * K)
    xs = [synth.device_normal_bf16((M, K), 4100 + i) for i in range(c)]
    y = torch.empty((M, R), dtype=torch.float32, device=dev)
    ws = torch.empty(bi.bi_lora_shrink_workspace_bytes(M, R, 8), dtype=torch.uint8, device=dev)
    by = 2.0 * M * K + 2 * R * K + 4 * M * R
    s_out = {"M": M, "K": K, "R": R, "bytes": "2*M*K + 2*R*K + 4*M*R", "peak_gbs": PEAK_HBM_GBS,
             "rotating_copies": c, "variants": {}}
    t = {}
    for name, fn in (("det8", lambda i: bi.bi_lora_shrink(xs[i % c], A, y=y, split_k=8)),
                     ("det8_two_pass", lambda i: bi.bi_lora_shrink_two_pass(xs[i % c], A, y=y,
                                                                          split_k=8, ws=ws)),
                     ("atomic8", lambda i: bi.bi_lora_shrink_atomic(xs[i % c], A, y=y, split_k=8)),
                     ("unsplit", lambda i: bi.bi_lora_shrink(xs[i % c], A, y=y, split_k=1))):
        ms = _time_loop(torch, fn, 4 * c)
        t[name] = ms
        gbs = by / (ms * 1e-3) / 1e9
        s_out["variants"][name] = {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                                   "frac": round(gbs / PEAK_HBM_GBS, 4)}
    s_out["det8_latency_over_atomic8"] = round(t["det8"] / t["atomic8"], 4)
    s_out["det8_speedup_over_unsplit"] = round(t["unsplit"] / t["det8"] - 1.0, 4)
    s_out["pages"] = {"det8_over_atomic8_added_latency": "+1.02..2.62 %",
                      "det8_speedup_over_unsplit": "16.8..21.1 %", "hardware": "not stated"}
    print(f"# shrink M=4096: " + ", ".join(f"{k} {v['us']} us" for k, v in s_out["variants"].items()),
          file=sys.stderr, flush=True)
    res["shrink"] = s_out
    del xs

    # Identical-input replay at M = 4096: the atomic control against the
    # deterministic split (a replay differs when any output bit differs from
    # replay 0)
    Hm = H[:M]
    rep = {}
    for name, fn in (("det8", lambda xb: bi.bi_lora_shrink(xb, A, y=y, split_k=8)),
                     ("atomic8", lambda xb: bi.bi_lora_shrink_atomic(xb, A, y=y, split_k=8))):
        r = harness.replay_variation(fn, Hm, 201)
        rep[name] = {"replays": r["replays"], "differing": r["differing"],
                     "frac_differing": round(r["frac_differing"], 4),
                     "diff_elems": r["diff_elems"], "elems_per_replay": r["elems_per_replay"]}
    res["replays"] = {"shrink_replays_m4096": rep}
    print(f"# replays M=4096: atomic8 {rep['atomic8']['differing']}/200, det8 "
          f"{rep['det8']['differing']}/200", file=sys.stderr, flush=True)

    # Llama-3-70B MLP shape under the dynamic-batch stream: 200 batches,
    # M ~ U{1..4096}, 8 probe rows at random positions, each checked bitwise
    # against its solo output
    cfg = workloads.LLAMA70B
    probes, batches = workloads.llama70b_stream()
    Xp = synth.device_normal_bf16((cfg["pool_rows"], cfg["K"]), 5101)
    W70 = synth.device_normal_bf16((cfg["N"], cfg["K"]), 5102, std=cfg["w_std"])
    solo = torch.cat([bi.bi_gemm(Xp[int(p):int(p) + 1], W70) for p in probes], dim=0)
    ybuf = torch.empty((cfg["m_max"], cfg["N"]), dtype=torch.bfloat16, device=dev)
    xbs, checks = [], []
    for b in batches:
        idx = torch.from_numpy(b["rows"]).to(dev)
        xbs.append(Xp.index_select(0, idx))
        present = [q for q in range(len(probes)) if b["probe_pos"][q] >= 0]
        checks.append((torch.tensor([int(b["probe_pos"][q]) for q in present], dtype=torch.int64,
                                    device=dev),
                       torch.tensor(present, dtype=torch.int64, device=dev)))
    cnt = torch.zeros((len(batches), len(probes), 2), dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i, xb in enumerate(xbs):
        bi.bi_gemm(xb, W70, y=ybuf[:xb.shape[0]])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    for i, xb in enumerate(xbs):  # the comparison, outside the timed loop
        bi.bi_gemm(xb, W70, y=ybuf[:xb.shape[0]])
        pos, pid = checks[i]
        if pos.numel():
            bi.bi_row_bitdiff(ybuf, solo, pos, pid, counts=cnt[i, :pos.numel()], check_rows=False)
    torch.cuda.synchronize()
    ms_all = [xb.shape[0] for xb in xbs]
    fl = sum(2.0 * m * cfg["N"] * cfg["K"] for m in ms_all)
    res["stream70b"] = {"K": cfg["K"], "N": cfg["N"], "batches": len(xbs), "M_min": min(ms_all),
                        "M_max": max(ms_all), "rows": sum(ms_all), "ms": round(ms, 3),
                        "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                        "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "probe_rows_checked": int(sum(c[0].numel() for c in checks)),
                        "probe_diff_bits": int(cnt[:, :, 0].sum())}
    print(f"# 70b stream: {res['stream70b']['tflops']} TFLOP/s, "
          f"{res['stream70b']['probe_diff_bits']} differing bits", file=sys.stderr, flush=True)
    return res


def replay_table(path, bi, torch, dev, to_dev):
    """The replay protocol of the LoRA shrink over every configured M: each
    variant replayed 1000 times on the same buffers; one JSON line per
    (variant, M) into ``path``."""
    from invariant_deterministic_amd import harness, workloads
    c = workloads.LORA
    x, a = workloads.lora_inputs()
    X, A = to_dev(x), to_dev(a)
    recs = []
    for M in c["Ms"]:
        Xm = X[:M]
        y = torch.empty((M, 16), dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, bi.bi_lora_shrink_workspace_bytes(M, 16, 8)), dtype=torch.uint8,
                         device=dev)
        for v, fn in (("det8", lambda xb: bi.bi_lora_shrink(xb, A, y=y, split_k=8)),
                      ("det8_two_pass", lambda xb: bi.bi_lora_shrink_two_pass(xb, A, y=y, split_k=8,
                                                                              ws=ws)),
                      ("unsplit", lambda xb: bi.bi_lora_shrink(xb, A, y=y, split_k=1)),
                      ("atomic8", lambda xb: bi.bi_lora_shrink_atomic(xb, A, y=y, split_k=8))):
            r = harness.replay_variation(fn, Xm, c["replays"])
            r.update(variant=v, M=M)
            recs.append(r)
            print(f"# replays {v} M={M}: {r['differing']}/{r['comparisons']} differ, "
                  f"{r['diff_elems']} elements", file=sys.stderr, flush=True)
    with open(path, "w") as f:
        for r in recs:
            f.write(json.dumps(r) + "\n")


class ClockSampler:
    """Samples the card's shader clock (mean over its XCDs) and socket power
    every ``period`` seconds from a background thread through the ROCm SMI
    library's metrics table; read-only.  The firmware refreshes that table
    about once a second (measured), so readings from the first ``skip``
    seconds may still describe the time before the sampled work and are
    dropped, and a reading repeated unchanged counts once.  Records nothing,
    and says why, when the library cannot read exactly one card."""

    def __init__(self, period: float = 0.05, skip: float = 1.0):
        self.period = period
        self.skip = skip
        self.samples = []
        self.err = None
        self._thread = None
        self._smi = None
        import threading
        self._stop = threading.Event()

    def __enter__(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) != 1:
                raise RuntimeError(f"{len(handles)} GPUs visible to amdsmi")
            self._handle = handles[0]
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        except Exception as e:  # no SMI access: the bench runs without clocks
            self.err = repr(e)[:200]
        return self

    @staticmethod
    def _num(v):
        return float(v) if isinstance(v, (int, float)) and not isinstance(v, bool) and v > 0 else None

    def _run(self):
        t0 = time.time()
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
            except Exception as e:
                self.err = repr(e)[:200]
                return
            clks = [c for c in map(self._num, m.get("current_gfxclks") or []) if c]
            if not clks and self._num(m.get("current_gfxclk")):
                clks = [self._num(m.get("current_gfxclk"))]
            power = self._num(m.get("current_socket_power")) or self._num(m.get("average_socket_power"))
            # memory (UMC) clock, where the metrics table reports one
            uclk = self._num(m.get("current_uclk")) or self._num(m.get("average_uclk_frequency"))
            if clks and time.time() - t0 >= self.skip:
                r = (sum(clks) / len(clks), power, uclk)
                if not self.samples or self.samples[-1] != r:
                    self.samples.append(r)
            self._stop.wait(self.period)

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        return False

    def summary(self, achieved_tflops: float):
        if not self.samples:
            return {"source": "amdsmi gpu_metrics", "readings": 0,
                    "error": self.err or f"no reading after the first {self.skip} s"}
        mhz = [c for c, _, _ in self.samples]
        watts = [w for _, w, _ in self.samples if w]
        uclk = [u for _, _, u in self.samples if u]
        mean = sum(mhz) / len(mhz)
        peak_at_clock = PEAK_BF16_TFLOPS * mean / SPEC_SCLK_MHZ
        return {"source": "amdsmi gpu_metrics, sampled during the untimed settle steps",
                "readings": len(mhz), "sclk_mhz_mean": round(mean, 1),
                "sclk_mhz_min": round(min(mhz), 1), "sclk_mhz_max": round(max(mhz), 1),
                "spec_sclk_mhz": SPEC_SCLK_MHZ,
                "socket_power_w_mean": round(sum(watts) / len(watts), 1) if watts else None,
                "mclk_mhz_mean": round(sum(uclk) / len(uclk), 1) if uclk else None,
                "mfma_peak_at_mean_clock": round(peak_at_clock, 1),
                "roofline_frac_at_mean_clock": round(achieved_tflops / peak_at_clock, 4)}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_256x256_llama8b_m4096_hbm.txt")
GEMM_SOURCE = os.path.join(ROOT, "invariant_deterministic_amd", "csrc", "gemm.hip")


def code_sha256(path: str) -> str:
    """sha256 of a C/HIP source with its comments and whitespace removed, so
    that it changes with the code and not with the commentary."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the dominant GEMM from the committed rocprofv3
    counter summary, or None when the kernel code changed since the counters
    were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.split()[0] if v.split() else ""
    if fields.get("code_sha256") != code_sha256(GEMM_SOURCE) or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def cpu_baseline(x, g, ws_h, a, eps):
    """The oracle as it stands, on a bounded sample of one step: 80 rows through
    RMSNorm, the four projections and the shrink (about 31 GFLOP of fp64,
    10-20 s on the host cores)."""
    import numpy as np

    import oracle
    rows = 80
    xs = x[:rows]
    t = time.perf_counter()
    h = oracle.rmsnorm(xs, g, eps)
    hb = oracle.bf16_round(h)
    flop = 0.0
    for i, w in enumerate(ws_h[:3]):
        oracle.gemm(hb, w)
        flop += 2.0 * rows * w.shape[0] * w.shape[1]
    u = oracle.bf16_round(oracle.gemm(hb, ws_h[2]))
    flop += 2.0 * rows * ws_h[2].shape[0] * ws_h[2].shape[1]
    oracle.gemm(u, ws_h[3])
    flop += 2.0 * rows * ws_h[3].shape[0] * ws_h[3].shape[1]
    oracle.lora_shrink(hb, a)
    flop += 2.0 * rows * a.shape[0] * a.shape[1]
    sec = time.perf_counter() - t
    return {"value": round(flop / sec / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(sec, 2),
            "sample": f"{rows} rows of the step (RMSNorm, Q/KV/Up/Down projections, LoRA shrink), "
                      f"fp64, {flop / 1e9:.1f} GFLOP; Up computed twice (timed as in the step "
                      "and again to feed Down)"}


def _time_loop(torch, fn, n, reps=7, warm_s=0.03):
    """Median over reps of (n launches) / n, in ms.  The n launches are
    captured once in a HIP graph and the graph is replayed between HIP events,
    so the figure is device time, not the host's launch rate (the kernels here
    issue no memset, which keeps them safe to capture).  Untimed replays fill
    the first ``warm_s`` seconds: the card's clock follows its load with a
    delay of milliseconds, so a point timed right after a different load
    (full-chip GEMMs before a half-chip one, say) would otherwise measure the
    previous load's clock."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_s
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / n)
    del g
    ts.sort()
    return ts[len(ts) // 2]


def sweep(path, bi, torch, dev, to_dev):
    """Per-kernel throughput over M, each kernel alone; inputs rotate through
    >= 1 GiB of copies so the 256 MB last-level cache cannot serve them."""
    import numpy as np

    from invariant_deterministic_amd import synth, workloads
    recs = []
    GiB = 1 << 30

    def copies(nbytes):
        return max(1, min(64, -(-GiB // max(1, nbytes))))

    # GEMM over M for each projection shape
    for si, (K, N) in enumerate(workloads.LLAMA8B["shapes"]):
        W = to_dev(workloads.llama8b_w(si))
        xpool = to_dev(workloads.llama8b_x(K))
        # below M ~ 1000 the weight read dominates: rotate weight copies past the cache
        cw = copies(2 * N * K)
        Ws = [W] + [W.clone() for _ in range(cw - 1)]
        for M in (1, 5, 33, 127, 512, 1000, 2048, 4096, 8192):
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            n = 20 if M >= 2048 else 4 * cw
            if M >= 2048:
                ms = _time_loop(torch, lambda i: bi.bi_gemm(xpool[:M], W, y=y), n)
            else:
                ms = _time_loop(torch, lambda i: bi.bi_gemm(xpool[:M], Ws[i % cw], y=y), n)
            fl = 2.0 * M * N * K
            by = 2.0 * (M * K + N * K + M * N)
            t_roof = max(fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
            recs.append({"kernel": "bi_gemm", "K": K, "N": N, "M": M, "us": ms * 1e3,
                         "tflops": fl / (ms * 1e-3) / 1e12, "gbs": by / (ms * 1e-3) / 1e9,
                         "frac_mfma": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "frac_roofline": t_roof / (ms * 1e-3),
                         "config": bi.bi_gemm_config_id(N, K)})
            print(f"# sweep gemm K={K} N={N} M={M}: {recs[-1]['tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            cf = bi.bi_gemm_fill_config_id(M, N, K)
            if cf != bi.bi_gemm_config_id(N, K):
                # the same bits with the tile picked from M (bi_gemm_fill)
                if M >= 2048:
                    msf = _time_loop(torch, lambda i: bi.bi_gemm_fill(xpool[:M], W, y=y), n)
                else:
                    msf = _time_loop(torch, lambda i: bi.bi_gemm_fill(xpool[:M], Ws[i % cw], y=y), n)
                recs.append({"kernel": "bi_gemm_fill", "K": K, "N": N, "M": M, "us": msf * 1e3,
                             "tflops": fl / (msf * 1e-3) / 1e12,
                             "frac_mfma": fl / (msf * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                             "config": cf})
                print(f"# sweep gemm_fill K={K} N={N} M={M} cfg={cf}: "
                      f"{recs[-1]['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
            if M <= 64:
                S = bi.bi_gemm_splitk_for(N, K)
                ws = torch.empty(bi.bi_gemm_splitk_workspace_bytes(M, N, S), dtype=torch.uint8,
                                 device=dev)
                ms2 = _time_loop(torch, lambda i: bi.bi_gemm_splitk(xpool[:M], Ws[i % cw], y=y,
                                                                     split_k=S, ws=ws), n)
                recs.append({"kernel": "bi_gemm_splitk", "K": K, "N": N, "M": M, "split_k": S,
                             "us": ms2 * 1e3, "tflops": fl / (ms2 * 1e-3) / 1e12,
                             "gbs": by / (ms2 * 1e-3) / 1e9,
                             "frac_hbm": by / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBS})
                print(f"# sweep gemm_splitk K={K} N={N} M={M} S={S}: {ms2*1e3:.1f} us "
                      f"({recs[-1]['gbs']:.0f} GB/s) vs bi_gemm {ms*1e3:.1f} us",
                      file=sys.stderr, flush=True)
        del W, Ws, xpool
    # The 70B MLP shape of the dynamic-batch stream (K = 8192, N = 28672, W 448 MiB)
    c70 = workloads.LLAMA70B
    W = to_dev(workloads.llama70b_w())
    xpool = to_dev(workloads.llama70b_x_pool())
    K, N = c70["K"], c70["N"]
    for M in (1, 64, 1024, 2048, 4096):
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ms = _time_loop(torch, lambda i: bi.bi_gemm(xpool[:M], W, y=y), 10)
        fl = 2.0 * M * N * K
        by = 2.0 * (M * K + N * K + M * N)
        t_roof = max(fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
        recs.append({"kernel": "bi_gemm", "K": K, "N": N, "M": M, "us": ms * 1e3,
                     "tflops": fl / (ms * 1e-3) / 1e12, "gbs": by / (ms * 1e-3) / 1e9,
                     "frac_mfma": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "frac_roofline": t_roof / (ms * 1e-3),
                     "config": bi.bi_gemm_config_id(N, K)})
        print(f"# sweep gemm K={K} N={N} M={M}: {recs[-1]['tflops']:.1f} TFLOP/s "
              f"({ms*1e3:.1f} us)", file=sys.stderr, flush=True)
    del W, xpool
    # Reference: a plain device copy (torch) of the same bytes as RMSNorm at
    # M = 2048 / 8192 and of 512 MiB -- the practical read+write rate of HBM
    # on this part, beside the 8 TB/s spec.
    for nbytes in (16 << 20, 64 << 20, 512 << 20):
        c = copies(2 * nbytes)
        srcs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(c)]
        dsts = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(c)]
        ms = _time_loop(torch, lambda i: dsts[i % c].copy_(srcs[i % c]), 4 * c)
        recs.append({"kernel": "device_copy_reference", "bytes_each_way": nbytes, "us": ms * 1e3,
                     "gbs": 2.0 * nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": 2.0 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "rotating_copies": c})
        print(f"# sweep copy {nbytes >> 20} MiB: {recs[-1]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
        del srcs, dsts
    # RMSNorm over M (K = 4096), rotating buffers
    K = 4096
    wv = to_dev(synth.normal_bf16((K,), 2002, mean=1.0, std=0.1))
    for M in (1, 7, 128, 2048, 8192, 65536):
        per = 4 * M * K
        c = copies(per)
        xs = [torch.randn((M, K), device=dev).to(torch.bfloat16) for _ in range(c)]
        ys = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(c)]
        ms = _time_loop(torch, lambda i: bi.bi_rmsnorm(xs[i % c], wv, y=ys[i % c]), 4 * c)
        by = 4.0 * M * K + 2 * K
        recs.append({"kernel": "bi_rmsnorm", "K": K, "M": M, "us": ms * 1e3,
                     "gbs": by / (ms * 1e-3) / 1e9, "frac_hbm": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "rotating_copies": c})
        print(f"# sweep rmsnorm M={M}: {recs[-1]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
        del xs, ys
    # LoRA shrink over M, three variants, rotating buffers
    a = to_dev(workloads.lora_inputs(1)[1])
    for M in (1, 8, 64, 512, 4096, 16384, 65536):
        per = 2 * M * 4096
        c = copies(per)
        xs = [torch.randn((M, 4096), device=dev).to(torch.bfloat16) for _ in range(c)]
        y = torch.empty((M, 16), dtype=torch.float32, device=dev)
        ws = torch.empty(bi.bi_lora_shrink_workspace_bytes(M, 16, 8), dtype=torch.uint8, device=dev)
        by = 2.0 * M * 4096 + 2 * 16 * 4096 + 4 * M * 16
        res = {}
        for name, fn in (("det8", lambda i: bi.bi_lora_shrink(xs[i % c], a, y=y, split_k=8)),
                         ("det8_two_pass", lambda i: bi.bi_lora_shrink_two_pass(xs[i % c], a, y=y, split_k=8, ws=ws)),
                         ("unsplit", lambda i: bi.bi_lora_shrink(xs[i % c], a, y=y, split_k=1)),
                         ("atomic8", lambda i: bi.bi_lora_shrink_atomic(xs[i % c], a, y=y, split_k=8))):
            ms = _time_loop(torch, fn, 4 * c)
            res[name] = ms
            recs.append({"kernel": f"bi_lora_shrink_{name}", "M": M, "us": ms * 1e3,
                         "gbs": by / (ms * 1e-3) / 1e9, "frac_hbm": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "rotating_copies": c})
        recs.append({"kernel": "lora_ratios", "M": M,
                     "det8_over_atomic8": res["det8"] / res["atomic8"],
                     "unsplit_over_det8": res["unsplit"] / res["det8"]})
        print(f"# sweep shrink M={M}: det8 {res['det8']*1e3:.1f}us two-pass {res['det8_two_pass']*1e3:.1f}us "
              f"atomic {res['atomic8']*1e3:.1f}us "
              f"unsplit {res['unsplit']*1e3:.1f}us", file=sys.stderr, flush=True)
        del xs
    # Decode attention (Llama-3-8B heads: H = 32, Hkv = 8, D = 128; split 256),
    # every sequence at T tokens; bytes = the K and V caches read once.
    H, Hkv, D, T = 32, 8, 128, 4096
    for B in (1, 8, 32, 64):
        per = 2 * B * T * Hkv * D * 2
        c = copies(per)
        ks = [torch.randn((B, T, Hkv, D), device=dev).to(torch.bfloat16) for _ in range(c)]
        vs = [torch.randn((B, T, Hkv, D), device=dev).to(torch.bfloat16) for _ in range(c)]
        q = torch.randn((B, H, D), device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        ws = torch.empty(bi.bi_decode_attention_workspace_bytes(B, H, T, D, 256), dtype=torch.uint8,
                         device=dev)
        ms = _time_loop(torch, lambda i: bi.bi_decode_attention(q, ks[i % c], vs[i % c], lens, o=o,
                                                                 split_size=256, ws=ws), 4 * c)
        by = float(per + 2 * 2 * B * H * D)
        recs.append({"kernel": "bi_decode_attention", "B": B, "T": T, "H": H, "Hkv": Hkv, "D": D,
                     "us": ms * 1e3, "gbs": by / (ms * 1e-3) / 1e9,
                     "frac_hbm": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "rotating_copies": c})
        print(f"# sweep attention B={B} T={T}: {ms*1e3:.1f} us {recs[-1]['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
        del ks, vs
    # LoRA expand y = bf16(base + l . b^T) at d_model = 4096, rank 16
    N, R = 4096, 16
    b = torch.randn((N, R), device=dev).to(torch.bfloat16)
    for M in (512, 4096, 16384):
        per = 4 * M * N
        c = copies(per)
        ls = [torch.randn((M, R), device=dev) for _ in range(c)]
        bases = [torch.randn((M, N), device=dev).to(torch.bfloat16) for _ in range(c)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(c)]
        ms = _time_loop(torch, lambda i: bi.bi_lora_expand(ls[i % c], b, base=bases[i % c],
                                                            y=ys[i % c]), 4 * c)
        by = 4.0 * M * N + 4 * M * R + 2 * N * R
        recs.append({"kernel": "bi_lora_expand", "M": M, "N": N, "R": R, "us": ms * 1e3,
                     "gbs": by / (ms * 1e-3) / 1e9, "frac_hbm": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "rotating_copies": c})
        print(f"# sweep expand M={M}: {ms*1e3:.1f} us {recs[-1]['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
        del ls, bases, ys
    with open(path, "w") as f:
        for r in recs:
            f.write(json.dumps(r) + "\n")


def run_only(args, bi, torch, dev, X, G, H, Wq, Wkv, Wup, Wdown, U, A, L, WS, La, Lu, eps):
    """Launch one kernel ``--iters`` times (for rocprofv3 traces and counters).
    The HBM-bound kernels (RMSNorm, the shrinks, the expand, attention) cycle
    through copies of their inputs and outputs that touch >= 1 GiB together,
    so the 256 MB last-level cache cannot serve them; the GEMMs reuse the
    step's buffers (they are compute-bound)."""
    from invariant_deterministic_amd import synth
    n = args.iters
    M = H.shape[0]
    if args.only == "copy":
        # a plain device copy of known size (256 MiB), to calibrate the HBM
        # byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(n):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "iters": n, "bytes_each_way": 256 << 20}), flush=True)
        return
    bi.bi_rmsnorm(X, G, y=H, eps=eps)
    U.copy_(torch.randn(U.shape, device=dev).to(torch.bfloat16))
    Q = torch.empty((M, Wq.shape[0]), dtype=torch.bfloat16, device=dev)
    KV = torch.empty((M, Wkv.shape[0]), dtype=torch.bfloat16, device=dev)
    U2 = torch.empty_like(U)
    D = torch.empty((M, Wdown.shape[0]), dtype=torch.bfloat16, device=dev)
    K = K_MODEL
    c = 1
    launch = None
    if args.only == "rmsnorm":
        c = _copies(4 * M * K)
        xs = [synth.device_normal_bf16((M, K), 2200 + i) for i in range(c)]
        ys = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(c)]
        launch = lambda i: bi.bi_rmsnorm(xs[i % c], G, y=ys[i % c], eps=eps)
    elif args.only.startswith("shrink"):
        c = _copies(2 * M * K)
        xs = [synth.device_normal_bf16((M, K), 4200 + i) for i in range(c)]
        y = torch.empty((M, R_LORA), dtype=torch.float32, device=dev)
        fn = {"shrink_det8": lambda xb: bi.bi_lora_shrink(xb, A, y=y, split_k=8),
              "shrink_two_pass": lambda xb: bi.bi_lora_shrink_two_pass(xb, A, y=y, split_k=8, ws=WS),
              "shrink_atomic8": lambda xb: bi.bi_lora_shrink_atomic(xb, A, y=y, split_k=8),
              "shrink_unsplit": lambda xb: bi.bi_lora_shrink(xb, A, y=y, split_k=1)}[args.only]
        launch = lambda i: fn(xs[i % c])
    elif args.only == "expand":
        # LoRA expand at d_model 4096, rank 16, from shrink outputs
        N = Wq.shape[0]
        bexp = synth.device_normal_bf16((N, R_LORA), 4300)
        c = _copies(4 * M * N)
        ls = [synth.device_normal_bf16((M, R_LORA), 4400 + i, dtype=torch.float32) for i in range(c)]
        bases = [synth.device_normal_bf16((M, N), 4500 + i) for i in range(c)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(c)]
        launch = lambda i: bi.bi_lora_expand(ls[i % c], bexp, base=bases[i % c], y=ys[i % c])
    elif args.only == "attention":
        # decode attention at Llama-3-8B heads, 64 sequences of 4096 tokens
        # (1 GiB of K and V, more than the last-level cache), split 256
        B, T, Hh, Hkv, Dh = 64, 4096, 32, 8, 128
        q = synth.device_normal_bf16((B, Hh, Dh), 4600)
        c = 2
        kcs = [synth.device_normal_bf16((B, T, Hkv, Dh), 4700 + i) for i in range(c)]
        vcs = [synth.device_normal_bf16((B, T, Hkv, Dh), 4800 + i) for i in range(c)]
        lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        o = torch.empty((B, Hh, Dh), dtype=torch.bfloat16, device=dev)
        aws = torch.empty(bi.bi_decode_attention_workspace_bytes(B, Hh, T, Dh, 256),
                          dtype=torch.uint8, device=dev)
        launch = lambda i: bi.bi_decode_attention(q, kcs[i % c], vcs[i % c], lens, o=o, split_size=256,
                                                  ws=aws)
    elif args.only == "splitk":
        # skinny GEMMs: the fixed split-K path on the four projections at
        # M <= 64 (the weight read dominates), each with its split from (N, K)
        ms = min(M, 64)
        sk = []
        for w, inp, y in ((Wq, H, Q), (Wkv, H, KV), (Wup, H, U2), (Wdown, U, D)):
            S = bi.bi_gemm_splitk_for(w.shape[0], w.shape[1])
            ws = torch.empty(bi.bi_gemm_splitk_workspace_bytes(ms, w.shape[0], S),
                             dtype=torch.uint8, device=dev)
            sk.append((inp[:ms], w, y[:ms], S, ws))

        def launch(i):
            for inp, w, y, S, ws in sk:
                bi.bi_gemm_splitk(inp, w, y=y, split_k=S, ws=ws)
    else:
        launch = {"gemm": lambda i: bi.bi_gemm(H, Wq, y=Q),
                  "gemm_kv": lambda i: bi.bi_gemm(H, Wkv, y=KV),
                  "gemm_kv_fill": lambda i: bi.bi_gemm_fill(H, Wkv, y=KV),
                  "gemm_up": lambda i: bi.bi_gemm(H, Wup, y=U2),
                  "gemm_up_fill": lambda i: bi.bi_gemm_fill(H, Wup, y=U2),
                  "gemm_down": lambda i: bi.bi_gemm(U, Wdown, y=D)}[args.only]
    torch.cuda.synchronize()
    for i in range(n):
        launch(i)
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "iters": n, "M": M, "rotating_copies": c}), flush=True)


if __name__ == "__main__":
    main()
