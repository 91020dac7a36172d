#!/usr/bin/env python3
"""Benchmark of the multi-user BitDelta decode apply on one MI355X.

Workload (default): the Llama-3.1-8B-shaped q_proj, W_base 4096x4096 bf16,
16 users' packed 1-bit deltas with one fp32 scale per matrix, a decode batch
of 16 tokens (one per user, in a seeded shuffled order), fp32 output.  A step
is one bd_apply of that layer: a single kernel (k_decode_unit) that groups the
batch by user, encodes the tokens for the delta products, and computes the
shared base product and every user's delta product in one pass over W_base and
the packed banks.  The K timed steps are captured in a HIP graph and replayed,
as a serving loop would issue them, so host launch overhead is not part of the
GPU time.  Steps rotate over R independent input sets (weights, banks,
activations) so consecutive steps do not hit the 256 MB last-level cache; all
inputs are resident in HBM before the timed region starts.  The two-launch
decode calls (bd_decode_prepare + bd_decode_apply) are timed beside it.

Printed: one JSON line with the apply throughput in algorithmic HBM GB/s
(value), tokens/s, per-kernel HIP-event timings, the roofline of the dominant
kernel, the compress leg (bd_compress on the same matrix shape), and the CPU
oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
METRIC = ("multi-user BitDelta decode apply: achieved HBM GB/s (% peak) and tokens/s per GPU")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--sets", type=int, default=16, help="rotating input sets")
    ap.add_argument("--compress-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="output rows of the oracle's sampled apply")
    ap.add_argument("--workloads", action="store_true",
                    help="also time one layer step of workloads 3-5 (stderr, one JSON line each)")
    ap.add_argument("--merge", action="store_true",
                    help="also time the dense merge path for one hot user against the fused "
                         "delta apply, per token count (stderr, one JSON line per shape)")
    ap.add_argument("--load", action="store_true",
                    help="also time loading one user's packed deltas of the Llama-3.1-8B linear "
                         "stack from pinned host memory, against the dense bf16 weights (stderr)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device 3 times (a plain "
                         "copy kernel of known size, to calibrate HBM byte counters)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("bd_apply.hip", "bd_compress.hip", "bd_decode.hip", "bd_internal.h"):
        with open(os.path.join(ROOT, "tenant_serving_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(workload, {}).get(kernel)
    if not e or e.get("source_digest") != kernel_source_digest():
        return None
    return e.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tenant_serving_amd import bitdelta as B
    from tenant_serving_amd import synth as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = max(1, args.sets)
    w0 = S.workload(2)
    mat = w0.matrices[0]
    d_out, d_in, U, T = mat.d_out, mat.d_in, w0.n_users, w0.T
    w = dataclasses.replace(w0, matrices=[mat] * R, xgroups=[d_in] * R)
    p = B.params("matrix")

    # ---------------------------------------------------------- resident inputs
    ids_np = S.user_ids(w0)
    ids = torch.from_numpy(ids_np).to(dev)
    sets = []
    wf = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)
    cws = B.workspace(B.bd_compress_workspace_bytes(p, d_out, d_in), dev)
    for s in range(R):
        wb = S.dev_wbase(w, s)
        signs = torch.empty((U, d_out, d_in // 64), dtype=torch.int64, device=dev)
        scales = torch.empty((U, 1), dtype=torch.float32, device=dev)
        for u in range(U):
            S.dev_wfine(w, s, u, wb, out=wf)
            B.compress(wf, wb, p, signs_out=signs[u], scales_out=scales[u], ws=cws)
        x = S.dev_x(w, s)
        y = torch.empty((T, d_out), dtype=torch.float32, device=dev)
        sets.append((wb, signs, scales, x, y))
    ws_bytes = B.bd_apply_workspace_bytes(p, T, U, d_out, d_in, B.BD_BF16, B.BD_F32)
    wss = [B.workspace(ws_bytes, dev) for _ in range(R)]  # one prepared batch per input set
    torch.cuda.synchronize()
    assert B.bd_device_status(cws) == B.BD_OK

    def step(k):
        wb, signs, scales, x, y = sets[k % R]
        return B.bd_apply(x, wb, signs, scales, p, U, ids, y, wss[k % R])

    def prep(k):  # the two-launch decode path, timed beside the step
        wb, signs, scales, x, y = sets[k % R]
        return B.bd_decode_prepare(x, ids, U, scales, p, wss[k % R])

    def main_pass(k):
        wb, signs, scales, x, y = sets[k % R]
        return B.bd_decode_apply(x, wb, signs, scales, p, U, y, wss[k % R])

    # eager warmup, and the eager result of every set (the graph replays must match it)
    for k in range(max(args.warmup, R)):
        assert step(k) == B.BD_OK
    torch.cuda.synchronize()
    y_eager = [sets[r][4].clone() for r in range(R)]

    # The K timed steps are captured once into a HIP graph and replayed, so host launch
    # overhead (Python, ctypes) is not part of the measured GPU time.
    K = args.steps

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(min(K, R)):  # warm the side stream before capture
                assert fn(k) == B.BD_OK
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for k in range(K):
                fn(k)
        return g

    def timed_replay(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e6 / K, e0.elapsed_time(e1) * 1e3 / K

    # ------------------------------------------------------------- timed steps
    g_step = capture(step)
    g_step.replay()
    torch.cuda.synchronize()
    wall_us, gpu_step_us = timed_replay(g_step)
    assert B.bd_device_status(wss[0]) == B.BD_OK
    for r in range(R):  # every replayed step reproduces the eager result bit for bit
        assert torch.equal(sets[r][4], y_eager[r]), f"graph replay differs from eager (set {r})"
    ms_per_step = wall_us * 1e-3

    # the two-launch decode path on the same inputs (not the step; for comparison)
    g_prep, g_main = capture(prep), capture(main_pass)
    g_prep.replay()
    g_main.replay()
    torch.cuda.synchronize()
    _, prep_us = timed_replay(g_prep)
    _, main_us = timed_replay(g_main)

    # the same steps on an INT8 base (bd_quantize_base once per set, then bd_apply_q8):
    # one byte per base weight instead of two
    q8 = [B.quantize_base(sets[r][0]) for r in range(R)]
    y8 = [torch.empty((T, d_out), dtype=torch.float32, device=dev) for _ in range(R)]

    def step_q8(k):
        wb, signs, scales, x, y = sets[k % R]
        q, qs = q8[k % R]
        return B.bd_apply_q8(x, q, qs, signs, scales, p, U, ids, y8[k % R], wss[k % R])

    for k in range(R):
        assert step_q8(k) == B.BD_OK
    g_q8 = capture(step_q8)
    g_q8.replay()
    torch.cuda.synchronize()
    _, q8_us = timed_replay(g_q8)
    assert B.bd_device_status(wss[0]) == B.BD_OK

    # algorithmic bytes (each byte the math must touch once)
    n_active = len(set(int(u) for u in ids_np if 0 <= u < U))
    bytes_w = d_out * d_in * 2
    bytes_bits = n_active * (d_out * d_in // 8 + 4)
    bytes_x, bytes_y = T * d_in * 2, T * d_out * 4
    bytes_step = bytes_w + bytes_bits + bytes_x + bytes_y + 4 * T
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    # the step is one launch of k_decode_unit: it reads the ids, X, W, the active users'
    # bits and scales once from HBM and writes y once
    dom, dom_us, dom_bytes = "k_decode_unit", gpu_step_us, bytes_step
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom, w0.name),
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3)}

    # ------------------------------------------------------------ compress leg
    n_c = min(8, U)
    wfs = []
    for u in range(n_c):
        t = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)
        S.dev_wfine(w, u % R, u, sets[u % R][0], out=t)
        wfs.append((t, sets[u % R][0]))
    c_signs = torch.empty((d_out, d_in // 64), dtype=torch.int64, device=dev)
    c_scales = torch.empty(1, dtype=torch.float32, device=dev)
    KC = max(1, args.compress_steps)

    def comp(k):
        return B.bd_compress(wfs[k % n_c][0], wfs[k % n_c][1], p, c_signs, c_scales, cws)

    for k in range(4):
        assert comp(k) == B.BD_OK
    torch.cuda.synchronize()
    g_comp = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        comp(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g_comp):
        for k in range(KC):
            comp(k)
    g_comp.replay()
    torch.cuda.synchronize()
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    g_comp.replay()
    ce1.record()
    torch.cuda.synchronize()
    assert B.bd_device_status(cws) == B.BD_OK
    comp_us = ce0.elapsed_time(ce1) * 1e3 / KC
    comp_bytes = 2 * d_out * d_in * 2 + d_out * d_in // 8 + 4
    comp_gbs = comp_bytes / (comp_us * 1e-6) / 1e9
    compress = {"call_us": round(comp_us, 3), "algorithmic_bytes": comp_bytes,
                "achieved": round(comp_gbs, 1), "unit": "GB/s",
                "frac": round(comp_gbs / HBM_PEAK_GBS, 4)}

    # per-layer axis choice on the same matrices (no clipping): one statistics pass
    # over W_fine and W_base, then two small reductions
    a_ws = B.workspace(B.bd_select_axis_workspace_bytes(d_out, d_in, 0.0), dev)
    a_err = torch.empty(2, dtype=torch.float64, device=dev)
    a_axis = torch.empty(1, dtype=torch.int32, device=dev)

    def axis_sel(k):
        return B.bd_select_axis(wfs[k % n_c][0], wfs[k % n_c][1], 0.0, a_err, a_axis, a_ws)

    for k in range(4):
        assert axis_sel(k) == B.BD_OK
    torch.cuda.synchronize()
    g_ax = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        axis_sel(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g_ax):
        for k in range(KC):
            axis_sel(k)
    g_ax.replay()
    torch.cuda.synchronize()
    ce0.record()
    g_ax.replay()
    ce1.record()
    torch.cuda.synchronize()
    assert B.bd_device_status(a_ws) == B.BD_OK
    ax_us = ce0.elapsed_time(ce1) * 1e3 / KC
    ax_bytes = 2 * d_out * d_in * 2
    ax_gbs = ax_bytes / (ax_us * 1e-6) / 1e9
    axis_select = {"call_us": round(ax_us, 3), "algorithmic_bytes": ax_bytes,
                   "achieved": round(ax_gbs, 1), "unit": "GB/s",
                   "frac": round(ax_gbs / HBM_PEAK_GBS, 4)}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w0.name, "d_out": d_out, "d_in": d_in, "n_users": U,
                   "active_users": n_active, "tokens": T, "scale": "matrix fp32",
                   "y_dtype": "fp32", "rotating_sets": R, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": bytes_step,
        "gpu_step_us_events": round(gpu_step_us, 3),
        "timing": "the K steps (one k_decode_unit launch each) captured in one HIP graph, "
                  "replayed once between device synchronisations (wall clock -> ms_per_step; "
                  "HIP events on the same stream -> gpu_step_us_events = the kernel's average "
                  "launch time); the two-launch path timed the same way from graphs of its K "
                  "prepare and K apply launches",
        "kernels_us": {"k_decode_unit": round(gpu_step_us, 3)},
        "two_launch_path_us": {"k_decode_prep": round(prep_us, 3), "k_decode": round(main_us, 3)},
        "roofline": roofline,
        "compress": compress,
        "axis_select": axis_select,
        "int8_base_step": {"kernel": "k_decode_unit (INT8 base)", "us": round(q8_us, 3),
                           "algorithmic_bytes": bytes_step - d_out * d_in + 4 * d_out,
                           "achieved": round((bytes_step - d_out * d_in + 4 * d_out) / (q8_us * 1e-6) / 1e9, 1),
                           "unit": "GB/s",
                           "frac": round((bytes_step - d_out * d_in + 4 * d_out) / (q8_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernel_source_digest": kernel_source_digest(),
    }

    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = nb

    # --------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, ids_np, args.cpu_rows, bytes_step, R)
    print(json.dumps(out), flush=True)
    if args.load:
        print(json.dumps(load_leg()), file=sys.stderr, flush=True)
    if args.merge:
        for line in merge_leg():
            print(json.dumps(line), file=sys.stderr, flush=True)
    if args.workloads:
        for line in workloads_leg():
            print(json.dumps(line), file=sys.stderr, flush=True)


def workloads_leg(reps=10):
    """One layer step of workloads 3, 4 and 5 through the prepared-batch calls: per
    distinct input width one bd_batch_prepare (the grouping and tile packing of the
    batch), then per matrix bd_base_gemm and bd_delta_apply.  Random banks (the time
    does not depend on the bit values; parity at these sizes is tested separately).
    The step is captured `reps` times in a HIP graph and replayed."""
    import torch

    from tenant_serving_amd import bitdelta as B
    from tenant_serving_amd import synth as S

    dev = torch.device("cuda:0")
    out = []
    for wid in (3, 4, 5):
        w = S.workload(wid)
        ids_np = S.user_ids(w)
        ids = torch.from_numpy(ids_np).to(dev)
        T, U = w.T, w.n_users
        nact = len(set(int(u) for u in ids_np if 0 <= u < U))
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + wid)
        xs, batches, mats = {}, {}, []
        tot_bytes = tot_flops = 0
        for m in w.matrices:
            p = B.params(m.mode, w.group_size, w.clip_k,
                         B.BD_F16 if m.scale_dtype == S.S_F16 else B.BD_F32)
            wb = (torch.randn(m.d_out, m.d_in, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
            signs = torch.randint(-2**62, 2**62, (U, m.d_out, m.d_in // 64), dtype=torch.int64,
                                  device=dev, generator=gen)
            n_sc = B.bd_scales_count(p, m.d_out, m.d_in)
            scales = (torch.rand(U, n_sc, device=dev, generator=gen) * 1e-3).to(B.scales_dtype(p))
            if m.xgroup not in xs:
                xs[m.xgroup] = torch.randn(T, m.d_in, device=dev, generator=gen).to(torch.bfloat16)
            if m.d_in not in batches:
                batches[m.d_in] = (xs[m.xgroup], B.workspace(
                    B.bd_batch_workspace_bytes(T, U, m.d_in, B.BD_BF16), dev))
            y = torch.empty(T, m.d_out, device=dev)
            mats.append((xs[m.xgroup], p, wb, signs, scales, y, batches[m.d_in][1]))
            tot_bytes += (m.d_out * m.d_in * 2 + nact * (m.d_out * m.d_in // 8 + scales.element_size() * n_sc)
                          + T * m.d_in * 2 + T * m.d_out * 4 + 4 * T)
            tot_flops += 2 * T * m.d_out * m.d_in

        def step():
            for x, bt in batches.values():
                assert B.bd_batch_prepare(x, ids, U, bt) == B.BD_OK
            for x, p, wb, signs, scales, y, bt in mats:
                assert B.bd_base_gemm(x, wb, y) == B.BD_OK
                assert B.bd_delta_apply(bt, x, U, signs, scales, p, y) == B.BD_OK

        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(reps):
                step()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out.append({"workload": w.name, "matrices": len(w.matrices), "tokens": T, "n_users": U,
                    "active_users": nact, "us_per_step": round(us, 1),
                    "algorithmic_bytes": tot_bytes, "achieved_GBs": round(tot_bytes / us / 1e3, 1),
                    "frac_of_hbm_peak": round(tot_bytes / us / 1e3 / HBM_PEAK_GBS, 4),
                    "base_TFLOPs": round(tot_flops / us / 1e6, 1)})
        del mats, xs, batches, g
        torch.cuda.empty_cache()
    return out


LLAMA8B_LINEARS = ((4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),  # q k v o
                   (14336, 4096), (14336, 4096), (4096, 14336))            # gate up down


def load_leg(layers=32, reps=3):
    """Cold load of one user's deltas for the Llama-3.1-8B linear stack ([P5] "Key
    Contributions" 4: the packed delta moved in one transfer per module; [P1] "How
    BitDelta Works": the base stays resident and only deltas move).  Pinned host
    buffers, device-resident destination, graph-free timed copies on one stream:
    (a) one transfer per layer (all its matrices packed), (b) one per matrix, and
    (c) the dense bf16 weights of the same matrices, one transfer per layer."""
    import torch

    from tenant_serving_amd.banks import module_layout

    dev = torch.device("cuda:0")
    offs, layer_bytes = module_layout(LLAMA8B_LINEARS, [1] * len(LLAMA8B_LINEARS))
    dense_layer = sum(o * i * 2 for o, i in LLAMA8B_LINEARS)
    hb = torch.empty(layers * layer_bytes, dtype=torch.uint8, pin_memory=True)
    db = torch.empty(layers * layer_bytes, dtype=torch.uint8, device=dev)

    def timed(fn):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            t = time.perf_counter() - t0
            best = t if best is None or t < best else best
        return best

    def per_layer():
        for l in range(layers):
            a = l * layer_bytes
            db[a:a + layer_bytes].copy_(hb[a:a + layer_bytes], non_blocking=True)

    def per_matrix():
        for l in range(layers):
            a = l * layer_bytes
            for (s_off, c_off), (o, i) in zip(offs, LLAMA8B_LINEARS):
                n = o * i // 8
                db[a + s_off:a + s_off + n].copy_(hb[a + s_off:a + s_off + n], non_blocking=True)
                db[a + c_off:a + c_off + 4].copy_(hb[a + c_off:a + c_off + 4], non_blocking=True)

    t_layer, t_matrix = timed(per_layer), timed(per_matrix)
    del db
    hd = torch.empty(layers * dense_layer, dtype=torch.uint8, pin_memory=True)
    dd = torch.empty(layers * dense_layer, dtype=torch.uint8, device=dev)

    def dense():
        for l in range(layers):
            a = l * dense_layer
            dd[a:a + dense_layer].copy_(hd[a:a + dense_layer], non_blocking=True)

    t_dense = timed(dense)
    del hd, dd, hb
    torch.cuda.empty_cache()
    return {"leg": "load", "model": "Llama-3.1-8B linear stack (32 x q,k,v,o,gate,up,down)",
            "delta_bytes": layers * layer_bytes, "dense_bf16_bytes": layers * dense_layer,
            "delta_one_transfer_per_layer_s": round(t_layer, 4),
            "delta_one_transfer_per_matrix_s": round(t_matrix, 4),
            "dense_one_transfer_per_layer_s": round(t_dense, 4),
            "delta_GBs": round(layers * layer_bytes / t_layer / 1e9, 1),
            "dense_GBs": round(layers * dense_layer / t_dense / 1e9, 1),
            "speedup_vs_dense": round(t_dense / t_layer, 2)}


def merge_leg(reps=20, token_counts=(16, 32, 64, 128, 256, 512, 1024)):
    """The dense merge path for a hot user ([P2] "Systems Mechanics": the per-user weight
    W_u = W_base + scale (.) sign materialised, then one plain GEMM for the user's tokens)
    against the fused path (the shared base GEMM over the user's tokens plus its delta
    apply), on the Llama-3.1-8B q_proj and gate shapes with MATRIX fp32 scales, n tokens
    of one user.  Per shape: bd_reconstruct (W_base + delta into bf16) once; per n:
    bd_base_gemm on W_base, bd_delta_apply on a prepared batch of the n tokens, and
    bd_base_gemm on W_u.  Each call is captured `reps` times in a HIP graph and replayed.
    fused = base + delta; merged with W_u kept = the GEMM on W_u; merged afresh = that
    plus the reconstruct."""
    import torch

    from tenant_serving_amd import bitdelta as B

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    out = []

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    for name, d_out, d_in in (("q_proj", 4096, 4096), ("gate_proj", 14336, 4096)):
        p = B.params("matrix")
        wb = (torch.randn(d_out, d_in, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        signs = torch.randint(-2**62, 2**62, (1, d_out, d_in // 64), dtype=torch.int64,
                              device=dev, generator=gen)
        scales = torch.full((1, 1), 5e-4, device=dev)
        wu = torch.empty(d_out, d_in, dtype=torch.bfloat16, device=dev)
        recon_us = timed(lambda: B.bd_reconstruct(signs[0], scales[0], p, d_out, d_in, wb, wu))
        rows = []
        for n in token_counts:
            x = torch.randn(n, d_in, device=dev, generator=gen).to(torch.bfloat16)
            ids = torch.zeros(n, dtype=torch.int32, device=dev)
            bt = B.workspace(B.bd_batch_workspace_bytes(n, 1, d_in, B.BD_BF16), dev)
            assert B.bd_batch_prepare(x, ids, 1, bt) == B.BD_OK
            y = torch.empty(n, d_out, device=dev)
            base_us = timed(lambda: B.bd_base_gemm(x, wb, y))
            delta_us = timed(lambda: B.bd_delta_apply(bt, x, 1, signs, scales, p, y))
            gemm_u_us = timed(lambda: B.bd_base_gemm(x, wu, y))
            rows.append({"tokens": n, "base_gemm_us": round(base_us, 2),
                         "delta_apply_us": round(delta_us, 2), "fused_us": round(base_us + delta_us, 2),
                         "merged_gemm_us": round(gemm_u_us, 2),
                         "merged_afresh_us": round(recon_us + gemm_u_us, 2)})
            del x, ids, bt, y
        cross = next((r["tokens"] for r in rows if r["merged_afresh_us"] <= r["fused_us"]), None)
        out.append({"leg": "merge", "matrix": name, "d_out": d_out, "d_in": d_in,
                    "reconstruct_us": round(recon_us, 2), "merged_weight_bytes": 2 * d_out * d_in,
                    "crossover_tokens_afresh": cross, "rows": rows})
        del wb, signs, wu
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, ids_np, rows, bytes_step, n_sets, seconds=12.0, max_calls=2048):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    applies of all tokens on `rows` output rows of input set 0's bank (compressed
    by the oracle first, not timed in the rate), one per token set, cycling over
    the token sets until about `seconds` of apply time (at most `max_calls`)."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle as O

    from tenant_serving_amd import synth as S

    mat = w.matrices[0]
    d_out, d_in, U = mat.d_out, mat.d_in, w.n_users
    rows = max(1, min(rows, d_out))
    t0 = time.perf_counter()
    wb = S.host_wbase(w, 0)
    words, scs = [], []
    for u in range(U):
        wf = S.host_wfine(w, 0, u, wbase=wb)
        ww, ss, _, _ = O.compress(wf, wb, O.MATRIX, dtype=O.BF16)
        words.append(ww[:rows])
        scs.append(ss)
    t1 = time.perf_counter()
    xs = [S.host_x(w, g) for g in range(max(1, n_sets))]
    wrows, wst, sst = wb[:rows], np.stack(words), np.stack(scs)
    calls, spent = 0, 0.0
    while calls < max_calls and (calls == 0 or spent < seconds):
        x = xs[calls % len(xs)]
        t2 = time.perf_counter()
        O.apply(x, wrows, wst, sst, O.MATRIX, ids_np)
        spent += time.perf_counter() - t2
        calls += 1
    sample_bytes = bytes_step * rows / d_out
    return {"value": round(calls * sample_bytes / spent / 1e9, 4), "unit": "GB/s",
            "cores": min(O.num_threads(), w.T), "kind": "oracle",
            "sample": f"{calls} applies of all {w.T} tokens on {rows} of {d_out} output rows "
                      f"of one bank, cycling over {len(xs)} token sets (fp64 plain loops, "
                      f"OpenMP over tokens); rate = calls x that share of the step's "
                      f"algorithmic bytes / total oracle apply time",
            "apply_calls": calls, "apply_s": round(spent, 3),
            "compress_16_users_s": round(t1 - t0, 3), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
