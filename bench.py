#!/usr/bin/env python3
"""Throughput of the FlashAttention forward and Flash-Decoding hot path on
one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  1. fa_fwd on prefill_8k  (B=1, H=32, N=8192, d=128, bf16 N(0,1), non-causal)
  2. fa_decode on decode_32k (B=1, H=32, L=32768, d=128, bf16 N(0,1), split-KV
     + combine), reading one of four rotating KV caches so that the 512 MiB
     cache is not served from the 256 MB last-level cache.
Inputs are resident in HBM before timing starts.  W untimed warm-up steps,
then exactly K timed steps between device synchronisations; each kernel is
bracketed by HIP events on the stream it is launched on.  After an idle
period the GPU's clock ramps up over its first few tens of launches (about
35 ms of work: prefill_8k runs 1.15 ms per launch in the first ten, 0.87 ms
from the fortieth on), so the default W = 60 steps times the steady state.

Printed: one JSON line.  `value` is fa_fwd TFLOP/s on prefill_8k (algorithmic
4*B*H*N^2*d FLOPs over the measured kernel time); decode GB/s (algorithmic
K+V bytes over split+combine time) is reported beside it, together with the
roofline fractions against the published peaks and against the ceilings two
measurement kernels reach in the same run (a bf16 MFMA loop, a read-only HBM
stream), the extra workloads (fp32_small, causal_4k, decode_varlen, and the
backward fa_bwd on prefill_8k and causal_4k) and the float64 oracle timed on
a bounded sample on the host cores (which also checks sampled outputs of the
timed launches).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_prefill_8k_traffic.json")
# sources of the prefill_8k kernel (non-causal d = 128): its HIP file and the
# generator of its tile loop
KERNEL_SRC = [os.path.join(ROOT, "exact_io_aware_02_amd", "csrc", "fa_fwd_bf16_asm.hip"),
              os.path.join(ROOT, "exact_io_aware_02_amd", "gen_fwd_asm.py")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _timed(fn, steps, warmup, torch):
    """Run fn(i) warmup+steps times; returns the mean event time (ms) of the
    timed calls, recorded on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = []
    for i in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def _interleaved(variants, rounds, per, torch):
    """Mean ms per launch of each variant {name: (setup, fn)}, the variants
    taking turns within each round (so that clock drift hits all alike);
    setup() runs before a variant's turn, and its first launch is not
    timed."""
    tot = {k: 0.0 for k in variants}
    for _ in range(rounds):
        for k, (setup, fn) in variants.items():
            setup()
            fn(0)
            evs = []
            for i in range(per):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn(i + 1)
                b.record()
                evs.append((a, b))
            torch.cuda.synchronize()
            tot[k] += sum(a.elapsed_time(b) for a, b in evs)
    return {k: v / (rounds * per) for k, v in tot.items()}


def _traffic(n_launch_bytes_alg):
    """Measured HBM bytes per fa_fwd launch from committed rocprofv3 counters,
    valid only while the kernel source is unchanged."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        h.update(open(path, "rb").read())
    src = h.hexdigest()
    if t.get("kernel_sha256") != src:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(Q, K, V, seconds, torch):
    """The float64 oracle, as it stands, on whole heads of prefill_8k until
    about `seconds` of host time is spent (at least one head)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    B, H, N, d = Q.shape
    flops = 0.0
    spent = 0.0
    heads = 0
    for h in range(H):
        q, k, v = (t[0, h].float().cpu().numpy().astype(np.float64) for t in (Q, K, V))
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, 1 / math.sqrt(d), causal=False)
        spent += time.perf_counter() - t0
        flops += 4.0 * N * N * d
        heads += 1
        if spent >= seconds:
            break
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "cpu_count": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "kind": "oracle",
        "sample": f"{heads} of {H} heads of prefill_8k (all {N} query rows each), float64 numpy",
        "seconds": round(spent, 3),
    }


def oracle_fp32_small(Q, K, V):
    """Host seconds of the oracle on the whole fp32_small workload (the
    device inputs copied to the host; median of five runs)."""
    import numpy as np

    import oracle

    q, k, v = (t[0, 0].double().cpu().numpy() for t in (Q, K, V))
    ts = []
    for _ in range(5):
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, 1 / math.sqrt(q.shape[1]), causal=False)
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def parity_sample(Q, K, V, O, L, q, Kc, Vc, o, lengths, torch):
    import numpy as np

    import oracle

    N, d = Q.shape[2], Q.shape[3]
    rows = np.array([0, 1, 127, 128, 4095, 8190, 8191])
    dO = dL = 0.0
    for h in (0, 31):
        f = lambda t: t.float().cpu().numpy().astype(np.float64)
        o_ref, l_ref = oracle.attention_rows(f(Q[0, h, rows]), f(K[0, h]), f(V[0, h]), 1 / math.sqrt(d), q_pos=rows)
        dO = max(dO, float(np.abs(f(O[0, h, rows]) - o_ref).max()))
        dL = max(dL, float(np.abs(f(L[0, h, rows]) - l_ref).max()))
    Ld = int(lengths[0])
    dd = 0.0
    for h in (0, 31):
        k = Kc[0, h].float().cpu().numpy().astype(np.float64)
        v = Vc[0, h].float().cpu().numpy().astype(np.float64)
        o_ref, _ = oracle.decode_ref(q[0, h].float().cpu().numpy().astype(np.float64), k[:Ld], v[:Ld], 1 / math.sqrt(d))
        dd = max(dd, float(np.abs(o[0, h].float().cpu().numpy() - o_ref).max()))
    return {"prefill_8k_max_abs_dO": dO, "prefill_8k_max_abs_dL": dL, "decode_32k_max_abs_do": dd,
            "rows_checked": "prefill: 7 rows x 2 heads; decode: 2 heads"}


def measured_ceilings(torch, fa, cus):
    """Ceilings that the two measurement kernels of the library reach on this
    GPU, timed with HIP events on the stream they run on:
      * fa_probe_mfma_bf16: 2 workgroups of 4 wavefronts per compute unit,
        each wavefront 16384 rounds of 4 independent 32x32x16 bf16 MFMAs;
        also the shader clock its wavefronts ran at (s_memtime cycles over
        s_memrealtime ticks); and fa_probe_mfma_bf16_mixed, the same loop on
        pseudo-random operands that differ between consecutive products;
      * fa_probe_hbm_read: one read of a 4 GiB buffer (16 times the last
        level cache), 64 workgroups of 256 threads per compute unit."""
    out = {}
    wg, iters = 2 * cus, 16384
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(wg, 2, dtype=torch.int64, device="cuda")
    ms = _timed(lambda i: fa.fa_probe_mfma_bf16(wg, iters, sink, stamps), 5, 3, torch)
    flop = wg * 4.0 * iters * 4 * 2 * 32 * 32 * 16
    st = stamps.cpu().double()
    clk = (st[:, 0] / (st[:, 1] / 1e8)).median().item() / 1e9
    out["mfma_bf16"] = {"value": round(flop / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                        "kernel": "fa_probe_mfma_bf16", "ms_per_launch": round(ms, 4),
                        "clock_ghz": round(clk, 3), "workgroups": wg, "iters": iters}
    # the same loop on random operands that change from product to product
    ms = _timed(lambda i: fa.fa_probe_mfma_bf16_mixed(wg, iters, sink, stamps, seed=i + 1), 5, 3, torch)
    st = stamps.cpu().double()
    clk = (st[:, 0] / (st[:, 1] / 1e8)).median().item() / 1e9
    out["mfma_bf16_mixed"] = {"value": round(flop / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                              "kernel": "fa_probe_mfma_bf16_mixed", "ms_per_launch": round(ms, 4),
                              "clock_ghz": round(clk, 3), "workgroups": wg, "iters": iters}
    del sink, stamps
    nbytes = 4 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    wg = 64 * cus
    sink = torch.zeros(wg, dtype=torch.int32, device="cuda")
    ms = _timed(lambda i: fa.fa_probe_hbm_read(buf, sink), 5, 2, torch)
    out["hbm_read"] = {"value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                       "kernel": "fa_probe_hbm_read", "ms_per_launch": round(ms, 4), "bytes": nbytes,
                       "workgroups": wg}
    del buf, sink
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps first (the clock ramps over the first ~40 launches after idle)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="host time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip causal_4k and decode_varlen")
    ap.add_argument("--num-splits", type=int, default=0, help="decode splits (0 = automatic)")
    ap.add_argument("--exp2-poly", type=int, default=0, choices=(0, 4, 8, 16),
                    help="exponentials per 64 that the d = 128 forward evaluates by polynomial in the "
                         "timed steps (0: hardware exponential only, the library default)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (calibrates "
                         "HBM byte counters under rocprofv3)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            "bench.py measures one GPU: the FlashAttention forward and Flash-Decoding kernels "
            "run on a single MI355X here; multi-GPU runs are not part of this library "
            "(see DESIGN.md for how the path would shard).",
            file=sys.stderr,
        )
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_02_amd as fa
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda"
    K_, W_ = args.steps, args.warmup

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")

    fa.fa_set_fwd_exp2_poly(args.exp2_poly)

    # ---------------- inputs (resident in HBM before timing)
    cfg = synth.WORKLOADS["prefill_8k"]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    Q, K, V = synth.prefill_inputs("prefill_8k", dev)
    O = torch.empty_like(Q)
    L = torch.empty(B, H, N, device=dev)
    scale = 1 / math.sqrt(d)

    dcfg = synth.WORKLOADS["decode_32k"]
    n_rot = 4
    caches = [synth.decode_inputs("decode_32k", dev, seed_offset=r) for r in range(n_rot)]
    lengths = caches[0][3]
    Lkv = torch.tensor(lengths, dtype=torch.int32, device=dev)
    Bd, Hd, dd = dcfg["B"], dcfg["H"], dcfg["d"]
    od = torch.empty(Bd, Hd, dd, dtype=torch.bfloat16, device=dev)
    splits = args.num_splits
    torch.cuda.synchronize()
    log("inputs ready")

    def run_fwd(i):
        fa.fa_fwd(Q, K, V, O, L, causal=False, scale=scale)

    def run_dec(i):
        q, Kc, Vc, _ = caches[i % n_rot]
        fa.fa_decode(q, Kc, Vc, od, Lkv, num_splits=splits)

    # ---------------- the timed steps
    for i in range(W_):
        run_fwd(i)
        run_dec(i)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for i in range(K_):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        run_fwd(i)
        e[1].record()
        run_dec(i)
        e[2].record()
        evs.append(e)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / K_
    fwd_t = sorted(e[0].elapsed_time(e[1]) for e in evs)
    dec_t = sorted(e[1].elapsed_time(e[2]) for e in evs)
    fwd_ms = sum(fwd_t) / K_
    dec_ms = sum(dec_t) / K_
    log(f"fa_fwd {fwd_ms:.4f} ms, fa_decode {dec_ms * 1e3:.2f} us, wall/step {wall_ms:.4f} ms")

    flops = 4.0 * B * H * N * N * d
    tflops = flops / (fwd_ms * 1e-3) / 1e12
    dec_bytes = 2.0 * Bd * Hd * int(lengths[0]) * dd * 2
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    plan = fa.fa_fwd_plan(B, H, N, d, 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    result = {
        "metric": "fa_fwd TFLOP/s (% MFMA peak) at N=8192,d=128; decode GB/s (% HBM peak) L=32k",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": W_,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 tensors of the workload shapes",
        "config": {
            "workload": "prefill_8k (B=1,H=32,N=8192,d=128, non-causal) + decode_32k (B=1,H=32,L=32768,d=128)",
            "prefill": {"B": B, "H": H, "N": N, "d": d, "causal": False,
                        "block_rows": plan["block_rows"], "block_cols": plan["block_cols"],
                        "workgroups": plan["workgroups"], "exp2_poly_per64": args.exp2_poly},
            "decode": {"B": Bd, "H": Hd, "L": int(lengths[0]), "d": dd,
                       "num_splits": splits if splits else f"auto ({cus} CUs)", "rotating_caches": n_rot},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic(None),
            "kernel": "fwd_bf16_asm_kernel<false>",
            "ms_per_launch": round(fwd_ms, 5),
            "ms_per_launch_median": round(fwd_t[K_ // 2], 5),
            "ms_per_launch_min": round(fwd_t[0], 5),
        },
        "decode": {
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "us_per_step": round(dec_ms * 1e3, 2),
            "us_per_step_median": round(dec_t[K_ // 2] * 1e3, 2),
            "us_per_step_min": round(dec_t[0] * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                         "bytes_per_step": dec_bytes},
        },
    }

    # ---------------- measured ceilings beside the published peaks
    ceil = measured_ceilings(torch, fa, cus)
    log(f"ceilings {ceil}")
    result["roofline"]["measured_ceiling"] = ceil["mfma_bf16"]
    result["roofline"]["frac_of_measured"] = round(tflops / ceil["mfma_bf16"]["value"], 4)
    result["roofline"]["measured_ceiling_mixed_operands"] = ceil["mfma_bf16_mixed"]
    result["roofline"]["frac_of_measured_mixed"] = round(tflops / ceil["mfma_bf16_mixed"]["value"], 4)
    result["decode"]["roofline"]["measured_ceiling"] = ceil["hbm_read"]
    result["decode"]["roofline"]["frac_of_measured"] = round(dec_gbs / ceil["hbm_read"]["value"], 4)

    # ---------------- extra workloads (the small fp32 case, the causal
    # target and varlen decode)
    if not args.no_extra:
        Qs, Ks, Vs = synth.prefill_inputs("fp32_small", dev)
        Os = torch.empty_like(Qs)
        Ls = torch.empty(Qs.shape[:3], device=dev)
        ms_s = _timed(lambda i: fa.fa_fwd_f32(Qs, Ks, Vs, Os, Ls), K_, W_, torch)
        c1 = synth.WORKLOADS["fp32_small"]
        fl_s = 4.0 * c1["B"] * c1["H"] * c1["N"] ** 2 * c1["d"]
        result["fp32_small"] = {"us_per_launch": round(ms_s * 1e3, 2), "unit": "us",
                                "tflops": round(fl_s / (ms_s * 1e-3) / 1e12, 4),
                                "shape": "B=1 H=1 N=256 d=64 fp32, non-causal"}
        log(f"fp32_small {ms_s * 1e3:.2f} us")
        c3 = synth.WORKLOADS["causal_4k"]
        Qc, Kc3, Vc3 = synth.prefill_inputs("causal_4k", dev)
        Oc = torch.empty_like(Qc)
        Lc = torch.empty(Qc.shape[:3], device=dev)
        ms_c = _timed(lambda i: fa.fa_fwd(Qc, Kc3, Vc3, Oc, Lc, causal=True), K_, W_, torch)
        Bc, Hc, Nc, dc = c3["B"], c3["H"], c3["N"], c3["d"]
        alg = 4.0 * dc * Bc * Hc * Nc * (Nc + 1) / 2
        pc = fa.fa_fwd_plan(Bc, Hc, Nc, dc, 1)
        executed = 4.0 * pc["tiles_visited"] * pc["block_rows"] * pc["block_cols"] * dc
        tf_c = alg / (ms_c * 1e-3) / 1e12
        result["causal_4k"] = {
            "value": round(tf_c, 2), "unit": "TFLOP/s", "ms_per_launch": round(ms_c, 5),
            "frac_of_peak": round(tf_c / PEAK_BF16_TFLOPS, 4),
            "frac_of_measured": round(tf_c / ceil["mfma_bf16"]["value"], 4),
            "flops_algorithmic": alg, "flops_executed_tiles": executed,
        }
        log(f"causal_4k {ms_c:.4f} ms -> {tf_c:.1f} TFLOP/s")

        # exponentials by polynomial: every share against the hardware
        # exponential, interleaved launch by launch on both prefill workloads
        shares = (0, 4, 8, 16)
        runs = {"prefill_8k": (lambda i: fa.fa_fwd(Q, K, V, O, L, causal=False, scale=scale), flops),
                "causal_4k": (lambda i: fa.fa_fwd(Qc, Kc3, Vc3, Oc, Lc, causal=True), alg)}
        result["exp2_poly"] = {"unit": "TFLOP/s", "note": "exponentials per 64 by polynomial on the "
                               "multiply-add units; shares timed in turn, 8 rounds of 5 launches each"}
        for wname, (fn, fl) in runs.items():
            ms = _interleaved({k: (lambda k=k: fa.fa_set_fwd_exp2_poly(k), fn) for k in shares}, 8, 5, torch)
            result["exp2_poly"][wname] = {str(k): round(fl / (v * 1e-3) / 1e12, 1) for k, v in ms.items()}
            log(f"exp2 poly {wname} {result['exp2_poly'][wname]}")
        fa.fa_set_fwd_exp2_poly(args.exp2_poly)
        del Qc, Kc3, Vc3, Oc, Lc

        # decode_32k in one launch (the last split workgroup merges) against
        # split + combine, interleaved, both with caller workspaces
        S_d = fa.fa_decode_plan(Bd, Hd, dd, splits)["num_splits"] if splits else 0
        ws_ex = torch.empty(fa.fa_decode_workspace_bytes(Bd, Hd, dd, S_d), dtype=torch.uint8, device=dev)
        ws_fu = torch.zeros(fa.fa_decode_fused_workspace_bytes(Bd, Hd, dd, S_d), dtype=torch.uint8, device=dev)

        def dec_ex(i):
            q, Kc, Vc, _ = caches[i % n_rot]
            fa.fa_decode_ex(q, Kc, Vc, od, Lkv, ws_ex, num_splits=S_d)

        def dec_fused(i):
            q, Kc, Vc, _ = caches[i % n_rot]
            fa.fa_decode_fused(q, Kc, Vc, od, Lkv, ws_fu, num_splits=S_d)

        ms_d = _interleaved({"split_combine": (lambda: None, dec_ex), "fused": (lambda: None, dec_fused)},
                            8, 8, torch)
        result["decode"]["one_launch"] = {
            "us_per_step": round(ms_d["fused"] * 1e3, 2), "two_launch_us_per_step": round(ms_d["split_combine"] * 1e3, 2),
            "value": round(dec_bytes / (ms_d["fused"] * 1e-3) / 1e9, 1), "unit": "GB/s",
            "note": "fa_decode_fused against fa_decode_ex, timed in turn, 8 rounds of 8 launches each"}
        log(f"decode_32k one launch {ms_d['fused'] * 1e3:.2f} us against two {ms_d['split_combine'] * 1e3:.2f} us")
        del ws_ex, ws_fu

        qv, Kv, Vv, lv = synth.decode_inputs("decode_varlen", dev)
        Lv = torch.tensor(lv, dtype=torch.int32, device=dev)
        ov = torch.empty_like(qv)
        ms_v = _timed(lambda i: fa.fa_decode(qv, Kv, Vv, ov, Lv, num_splits=splits), K_, W_, torch)
        vbytes = 2.0 * qv.shape[1] * qv.shape[2] * 2 * int(lv.sum())
        gbs_v = vbytes / (ms_v * 1e-3) / 1e9
        result["decode_varlen"] = {
            "value": round(gbs_v, 1), "unit": "GB/s", "us_per_launch": round(ms_v * 1e3, 2),
            "frac_of_peak": round(gbs_v / PEAK_HBM_GBS, 4), "bytes": vbytes,
            "lengths": [int(x) for x in lv],
        }
        del qv, Kv, Vv, ov
        log(f"decode_varlen {ms_v * 1e3:.1f} us -> {gbs_v:.1f} GB/s")

    # ---------------- the backward (gradients by recomputation from O and L)
    if not args.no_extra:
        result["backward"] = {}
        for name in ("prefill_8k", "causal_4k"):
            bc = synth.WORKLOADS[name]
            Bb, Hb, Nb, db_ = bc["B"], bc["H"], bc["N"], bc["d"]
            Qb, Kb, Vb = (Q, K, V) if name == "prefill_8k" else synth.prefill_inputs(name, dev)
            dOb = synth.torch_normal(850, (Bb, Hb, Nb, db_), dev, "bf16")
            Ob = torch.empty_like(Qb)
            Lb = torch.empty(Bb, Hb, Nb, device=dev)
            fa.fa_fwd(Qb, Kb, Vb, Ob, Lb, causal=bc["causal"])
            gq, gk, gv = (torch.empty_like(Qb) for _ in range(3))
            ms_b = _timed(lambda i: fa.fa_bwd(Qb, Kb, Vb, Ob, dOb, Lb, gq, gk, gv, causal=bc["causal"]), K_, W_, torch)
            pairs = Nb * (Nb + 1) / 2 if bc["causal"] else Nb * Nb
            alg = 10.0 * db_ * Bb * Hb * pairs
            result["backward"][name] = {
                "value": round(alg / (ms_b * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_launch": round(ms_b, 4),
                "frac_of_peak": round(alg / (ms_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "flops_algorithmic": alg, "flops_executed": 1.4 * alg,
                "note": "10 N^2 d per head (the lecture notes' count with recomputation; causal: unmasked pairs); "
                        "the kernels execute 14 N^2 d (dQ recomputes S and dP)",
            }
            log(f"backward {name} {ms_b:.3f} ms -> {result['backward'][name]['value']} TFLOP/s")
            del Ob, Lb, gq, gk, gv, dOb
            if name != "prefill_8k":
                del Qb, Kb, Vb

    # ---------------- float64 oracle on the host cores: the baseline, its
    # time on fp32_small, and a sampled check of the timed outputs
    if not args.no_cpu_baseline:
        cb = cpu_baseline(Q, K, V, args.cpu_seconds, torch)
        if "fp32_small" in result:
            cb["fp32_small_seconds"] = round(oracle_fp32_small(Qs, Ks, Vs), 5)
            result["fp32_small"]["oracle_seconds"] = cb["fp32_small_seconds"]
        q0, Kc0, Vc0, _ = caches[(K_ - 1) % n_rot]
        fa.fa_decode(q0, Kc0, Vc0, od, Lkv, num_splits=splits)
        torch.cuda.synchronize()
        cb["check"] = parity_sample(
            Q, K, V, O, L, q0, Kc0.view(Bd, Hd, -1, dd), Vc0.view(Bd, Hd, -1, dd), od, lengths, torch)
        result["cpu_baseline"] = cb
        log(f"cpu baseline {result['cpu_baseline']}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
