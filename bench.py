#!/usr/bin/env python3
"""Benchmark of the multi-user BitDelta decode apply on one MI355X.

Workload (the headline): the Llama-3.1-8B-shaped stack, 32 layers x {q, k, v,
o, gate, up, down} bf16 base weights (13.96 GB) with 128 users' packed 1-bit
deltas and one fp32 scale per matrix resident in HBM (111.7 GB, built by
bd_compress from seeded synthetic fine-tunes), and one decode step of 512
tokens whose users are Zipf(1.1) draws.  A step applies every matrix to the
batch: per distinct input width one bd_batch_prepare (tokens grouped by user),
per distinct activation tensor one bd_batch_encode (q/k/v and gate/up share
theirs), per matrix bd_base_gemm (y = X W_base^T) and bd_delta_apply_encoded
(y += scale_u (.) X S_u^T).  Each matrix reads its own activation tensor; no
attention, norms or activations (not on the path).  The K timed steps are
captured in one HIP graph and replayed between device synchronisations.

Printed: one JSON line with the step's throughput in algorithmic HBM GB/s
(value), tokens/s, the per-phase kernel times (HIP events around graphs of one
phase's launches), the roofline of the dominant kernel, the base GEMM's
TFLOP/s, the q_proj decode step and the compress legs, and the CPU oracle
timed on a bounded sample of the same workload on the host.
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
    ap.add_argument("--steps", type=int, default=10, help="timed steps of the stack")
    ap.add_argument("--warmup", type=int, default=3, help="eager steps of the stack before timing")
    ap.add_argument("--decode-steps", type=int, default=400,
                    help="timed steps of the q_proj decode leg")
    ap.add_argument("--sets", type=int, default=16, help="rotating input sets of the decode leg")
    ap.add_argument("--compress-steps", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="output rows per matrix of the oracle's sampled apply")
    ap.add_argument("--no-legs", action="store_true",
                    help="time the stack only (no decode, compress, axis or INT8 legs)")
    ap.add_argument("--workloads", action="store_true",
                    help="also time one layer step of workloads 3 and 4 (stderr)")
    ap.add_argument("--merge", action="store_true",
                    help="also time the dense merge path for one hot user against the fused "
                         "delta apply, per token count (stderr, one JSON line per shape)")
    ap.add_argument("--load", action="store_true",
                    help="also time loading one user's packed deltas of the Llama-3.1-8B linear "
                         "stack from pinned host memory, against the dense bf16 weights (stderr)")
    ap.add_argument("--layers", type=int, default=0,
                    help="stack: first N layers only (0: all 32); for counter runs, not the headline")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy this many MiB device-to-device 3 times (a plain "
                         "copy kernel of known size, to calibrate HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "tenant_serving_amd", "csrc"))):
        if f.endswith((".hip", ".h")) and f.startswith("bd_"):
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


# ---------------------------------------------------------------- HIP-graph timing
def capture(fn, reps):
    """fn() captured `reps` times into one HIP graph (after one eager call on the
    capture stream)."""
    import torch
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
    return g


def replay_timed(g, reps):
    """(wall us, HIP-event us) per repetition of one replay of g."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e6 / reps, e0.elapsed_time(e1) * 1e3 / reps


# ---------------------------------------------------------------- the stack
class Stack:
    """Resident inputs of the 32-layer workload: base weights, 128 users' banks from
    bd_compress, activations, outputs, prepared batches."""

    # matrices of a layer that read one activation tensor: (first, count)
    GROUPS = ((0, 3), (3, 1), (4, 2), (6, 1))

    def __init__(self, dev, layers=0):
        import numpy as np
        import torch

        from tenant_serving_amd import bitdelta as B
        from tenant_serving_amd import synth as S

        self.B = B
        w = self.w = S.workload(5)
        self.U, self.T = w.n_users, w.T
        self.ids_np = S.user_ids(w)
        self.ids = torch.from_numpy(self.ids_np).to(dev)
        self.p = B.params("matrix")
        self.active = sorted(set(int(u) for u in self.ids_np if 0 <= u < self.U))
        # (layers > 0: the first `layers` layers only, for counter runs; every layer has the
        # same launches, so per-launch figures do not change)
        mats = w.matrices[:7 * layers] if layers > 0 else w.matrices
        big = max(m.d_out * m.d_in for m in mats)
        wf = torch.empty(big, dtype=torch.bfloat16, device=dev)
        cws = B.workspace(max(B.bd_compress_workspace_bytes(self.p, m.d_out, m.d_in)
                              for m in mats), dev)
        self.wb, self.signs, self.scales, self.y = [], [], [], []
        t0 = time.perf_counter()
        for mi, m in enumerate(mats):
            wb = S.dev_wbase(w, mi)
            signs = torch.empty((self.U, m.d_out, m.d_in // 64), dtype=torch.int64, device=dev)
            scales = torch.empty((self.U, 1), dtype=torch.float32, device=dev)
            wfv = wf[:m.d_out * m.d_in].view(m.d_out, m.d_in)
            for u in range(self.U):
                S.dev_wfine(w, mi, u, wb, out=wfv)
                st = B.bd_compress(wfv, wb, self.p, signs[u], scales[u], cws)
                assert st == B.BD_OK, st
            self.wb.append(wb)
            self.signs.append(signs)
            self.scales.append(scales)
            self.y.append(torch.empty((self.T, m.d_out), dtype=torch.float32, device=dev))
            if mi % 28 == 27:
                torch.cuda.synchronize()
                log(f"stack: {mi + 1}/{len(mats)} matrices compressed for {self.U} users "
                    f"({time.perf_counter() - t0:.1f} s)")
        torch.cuda.synchronize()
        assert B.bd_device_status(cws) == B.BD_OK
        del wf, cws
        self.xs = [S.dev_x(w, g) for g in range(4 * (len(mats) // 7))]
        self.batches = {}
        for d_in in sorted(set(w.xgroups)):
            self.batches[d_in] = B.workspace(
                B.bd_batch_workspace_bytes(self.T, self.U, d_in, B.BD_BF16), dev)
        self.first_x = {d: next(x for x in self.xs if x.shape[1] == d) for d in self.batches}
        # the grouped base GEMMs' K-split partial products (one workspace for every group)
        need = max(B.bd_base_gemm_n_workspace_bytes(
            B.BD_BF16, self.T, mats[7 * l + f].d_in, [mats[7 * l + f + i].d_out for i in range(c)])
            for l in range(len(mats) // 7) for f, c in self.GROUPS) if len(mats) >= 7 else 0
        self.gemm_ws = B.workspace(need, dev) if need > 0 else None
        torch.cuda.synchronize()
        self.setup_s = time.perf_counter() - t0

        self.mats = mats
        self._account()
        self.n_mats = len(mats)
        self.n_layers = len(mats) // 7

    def _account(self):
        """Algorithmic bytes (each byte the math must touch once, summed per matrix
        apply) and base GEMM flops of one step on the current batch."""
        na, T = len(self.active), self.T
        self.bytes_step = self.bytes_delta = self.flops_gemm = 0
        for m in self.mats:
            self.bytes_step += (m.d_out * m.d_in * 2 + na * (m.d_out * m.d_in // 8 + 4)
                                + T * m.d_in * 2 + T * m.d_out * 4 + 4 * T)
            self.bytes_delta += na * (m.d_out * m.d_in // 8 + 4) + T * m.d_out * 4
            self.flops_gemm += 2 * T * m.d_out * m.d_in

    def set_ids(self, ids_np):
        """Another batch of the same size over the same resident banks."""
        import torch
        self.ids_np = ids_np
        self.ids = torch.from_numpy(ids_np).to(self.ids.device)
        self.active = sorted(set(int(u) for u in ids_np if 0 <= u < self.U))
        self._account()

    # one phase at a time (graphs of one kind of launch, for per-kernel timing)
    def prepare(self):
        B = self.B
        for d_in, bt in self.batches.items():
            assert B.bd_batch_prepare(self.first_x[d_in], self.ids, self.U, bt) == B.BD_OK

    def _groups(self):
        for l in range(self.n_layers):
            for gi, (first, cnt) in enumerate(self.GROUPS):
                x = self.xs[4 * l + gi]
                yield x, self.batches[x.shape[1]], range(7 * l + first, 7 * l + first + cnt)

    def encode_all(self):
        B = self.B
        for x, bt, _ in self._groups():
            assert B.bd_batch_encode(bt, x, self.U, None, self.p) == B.BD_OK

    def _gemm(self, x, ms):
        B = self.B
        assert B.bd_base_gemm_n(x, [self.wb[m] for m in ms], [self.y[m] for m in ms],
                                workspace=self.gemm_ws) == B.BD_OK

    def _delta(self, x, bt, ms):
        B = self.B
        assert B.bd_delta_apply_encoded_n(bt, self.T, x.shape[1], self.U,
                                          [self.signs[m] for m in ms],
                                          [self.scales[m] for m in ms], self.p,
                                          [self.y[m] for m in ms]) == B.BD_OK

    def gemm_all(self):
        for x, _, ms in self._groups():
            self._gemm(x, ms)

    def delta_all(self):
        """The delta products of every matrix on the batch's current encoding (the
        products' time does not depend on which activations are encoded)."""
        for x, bt, ms in self._groups():
            self._delta(x, bt, ms)

    def step(self):
        B = self.B
        self.prepare()
        for x, bt, ms in self._groups():
            assert B.bd_batch_encode(bt, x, self.U, None, self.p) == B.BD_OK
            self._gemm(x, ms)
            self._delta(x, bt, ms)


def stack_leg(args, dev):
    import torch

    S = Stack(dev, args.layers)
    B = S.B
    log(f"stack ready: {S.n_mats} matrices, {S.U} users' banks, {len(S.active)} active "
        f"({S.setup_s:.1f} s)")
    K = max(1, args.steps)
    for _ in range(max(1, args.warmup)):
        S.step()
    torch.cuda.synchronize()
    for bt in S.batches.values():
        assert B.bd_device_status(bt) == B.BD_OK
    check = [0, 4, 6, S.n_mats - 1]
    y_eager = {m: S.y[m].clone() for m in check}

    g = capture(S.step, K)
    g.replay()
    torch.cuda.synchronize()
    wall_us, ev_us = replay_timed(g, K)
    for m in check:  # every replayed step reproduces the eager result bit for bit
        assert torch.equal(S.y[m], y_eager[m]), f"graph replay differs from eager (matrix {m})"
    del g
    log(f"stack step: {wall_us / 1e3:.3f} ms (events {ev_us / 1e3:.3f} ms)")

    phases = {}
    for name, fn in (("prepare", S.prepare), ("encode", S.encode_all), ("gemm", S.gemm_all),
                     ("delta", S.delta_all)):
        gp = capture(fn, K)
        gp.replay()
        _, phases[name] = replay_timed(gp, K)
        del gp
    torch.cuda.synchronize()
    log("phases (us per step): " + ", ".join(f"{k} {v:.1f}" for k, v in phases.items()))

    ms_per_step = wall_us * 1e-3
    value = S.bytes_step / (ms_per_step * 1e-3) / 1e9
    n_gemm = 4 * S.n_layers  # grouped launches: q|k|v, o, gate|up, down
    # delta launches: one per group of matrices (down's 28 units of 512 columns are taken
    # 7 at a time inside its launch)
    n_delta = 4 * S.n_layers
    delta_gbs = S.bytes_delta / (phases["delta"] * 1e-6) / 1e9
    gemm_tfs = S.flops_gemm / (phases["gemm"] * 1e-6) / 1e12
    rl_delta = {"bound": "hbm", "kernel": "k_delta8", "achieved": round(delta_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(delta_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("k_delta8", S.w.name),
                "algorithmic_bytes_per_launch": S.bytes_delta // n_delta,
                "avg_launch_us": round(phases["delta"] / n_delta, 3)}
    rl_gemm = {"bound": "mfma", "kernel": "k_gemm", "achieved": round(gemm_tfs, 1),
               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": round(gemm_tfs / BF16_PEAK_TFLOPS, 4),
               "traffic": measured_traffic("k_gemm", S.w.name),
               "flops_per_launch": S.flops_gemm // n_gemm,
               "avg_launch_us": round(phases["gemm"] / n_gemm, 3)}
    dominant, other = (rl_delta, rl_gemm) if phases["delta"] >= phases["gemm"] else (rl_gemm, rl_delta)

    # the same step on a batch with the mean number of distinct users: Zipf seed 0 draws
    # 83 distinct users of 128, the lightest of seeds 0..39 (mean 91.9); seed 3 draws 92
    from tenant_serving_amd import synth as SY
    ids0 = S.ids_np
    S.set_ids(SY.user_ids(SY.workload(5, seed=3)))
    g3 = capture(S.step, K)
    g3.replay()
    wall3, _ = replay_timed(g3, K)
    del g3
    mean_batch = {"user_ids": "Zipf(1.1), seed 3", "active_users": len(S.active),
                  "ms_per_step": round(wall3 * 1e-3, 4),
                  "achieved_GBs": round(S.bytes_step / (wall3 * 1e-6) / 1e9, 1),
                  "tokens_per_s": round(S.T / (wall3 * 1e-6), 1)}
    S.set_ids(ids0)
    log(f"stack step, seed-3 batch ({mean_batch['active_users']} users): {wall3 / 1e3:.3f} ms")
    out = {
        "value": round(value, 1), "ms_per_step": round(ms_per_step, 4),
        "config": {"workload": S.w.name, "layers": S.n_layers, "matrices": S.n_mats,
                   "n_users": S.U, "active_users": len(S.active), "tokens": S.T,
                   "scale": "matrix fp32", "y_dtype": "fp32",
                   "user_ids": "Zipf(1.1), seed 0 (83 distinct users: the lightest of seeds "
                               "0..39, whose mean is 91.9; step_mean_batch: seed 3, 92 users)",
                   "banks": "bd_compress of seeded synthetic fine-tunes (Laplace b=5e-4)",
                   "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(S.T / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": S.bytes_step,
        "gpu_step_us_events": round(ev_us, 1),
        "phases_us_per_step": {k: round(v, 1) for k, v in phases.items()},
        "phase_launches_per_step": {"prepare": len(S.batches), "encode": 4 * S.n_layers,
                                    "gemm": n_gemm, "delta": n_delta},
        "delta_launches_per_layer": "q|k|v 1, o 1, gate|up 1, down 1 (28 units, 7 at a time)",
        "matrices_per_launch": "q|k|v, o, gate|up, down (grouped calls on one encoding)",
        "roofline": dominant,
        "roofline_secondary": other,
        "base_gemm": {"TFLOPs": round(gemm_tfs, 1), "frac_of_bf16_peak": round(gemm_tfs / BF16_PEAK_TFLOPS, 4),
                      "flops_per_step": S.flops_gemm},
        "setup_s": round(S.setup_s, 1),
        "step_mean_batch": mean_batch,
    }
    return out, S


# ---------------------------------------------------------------- INT8 base and paging legs
def int8_leg(S, dev, K):
    """The same step with the base weights as INT8 rows (bd_quantize_base), grouped as
    the bf16 step is: prepare once per width, then per group of matrices that read the
    same activations one encode, one bd_base_gemm_q8_n (the codes widened on chip, K
    split where the bf16 GEMM splits) and one bd_delta_apply_encoded_n; K steps in one
    HIP graph.  Algorithmic bytes as the bf16 step's with one byte per base weight and
    a scale per row."""
    import torch
    B = S.B
    qs = [B.quantize_base(wb) for wb in S.wb]
    torch.cuda.synchronize()

    def gemm_q8(x, ms):
        assert B.bd_base_gemm_q8_n(x, [qs[m][0] for m in ms], [qs[m][1] for m in ms],
                                   [S.y[m] for m in ms], workspace=S.gemm_ws) == B.BD_OK

    def step():
        S.prepare()
        for x, bt, ms in S._groups():
            assert B.bd_batch_encode(bt, x, S.U, None, S.p) == B.BD_OK
            gemm_q8(x, ms)
            S._delta(x, bt, ms)

    step()
    torch.cuda.synchronize()
    for bt in S.batches.values():
        assert B.bd_device_status(bt) == B.BD_OK
    g = capture(step, K)
    g.replay()
    wall_us, ev_us = replay_timed(g, K)
    del g

    def gemm_all():
        for x, _, ms in S._groups():
            assert B.bd_base_gemm_q8_n(x, [qs[m][0] for m in ms], [qs[m][1] for m in ms],
                                       [S.y[m] for m in ms], workspace=S.gemm_ws) == B.BD_OK

    gp = capture(gemm_all, K)
    gp.replay()
    _, gemm_us = replay_timed(gp, K)
    del gp
    del qs
    nbytes = 0
    for m in range(S.n_mats):
        d_out, d_in = S.wb[m].shape
        nbytes += (d_out * d_in + 4 * d_out + len(S.active) * (d_out * d_in // 8 + 4)
                   + S.T * d_in * 2 + S.T * d_out * 4 + 4 * S.T)
    gbs = nbytes / (wall_us * 1e-6) / 1e9
    return {"ms_per_step": round(wall_us * 1e-3, 4), "gpu_step_us_events": round(ev_us, 1),
            "gemm_phase_us": round(gemm_us, 1),
            "gemm_TFLOPs": round(S.flops_gemm / (gemm_us * 1e-6) / 1e12, 1),
            "algorithmic_bytes_per_step": nbytes, "achieved_GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "calls": "per width one bd_batch_prepare; per group bd_batch_encode, "
                     "bd_base_gemm_q8_n, bd_delta_apply_encoded_n",
            "base": "per-row symmetric INT8 codes + fp32 row scales (bd_quantize_base)"}


def paged_leg(S, dev, n_slots=96, reps=5):
    """Layer 0's seven matrices served from a pool of n_slots device slots (BankPager):
    every one of the 128 users' packed layer-0 module in pinned host memory, the pool
    warmed with this step's users; then a step of another Zipf batch (seed 1), whose
    users not resident are loaded first (one host-to-device copy per module, least
    recently used slots evicted).  Times the cold step (loads + 7 bd_apply_paged) and
    the same batch again (all resident), wall clock around each."""
    import torch

    from tenant_serving_amd import synth as SY
    from tenant_serving_amd.pager import BankPager
    B = S.B
    shapes = [tuple(S.wb[m].shape) for m in range(7)]
    pager = BankPager(shapes, [1] * 7, torch.float32, n_slots, S.U, dev)
    t0 = time.perf_counter()
    for u in range(S.U):
        pager.pack(u, [S.signs[m][u] for m in range(7)], [S.scales[m][u] for m in range(7)])
    pack_s = time.perf_counter() - t0
    ids_b = SY.user_ids(SY.workload(5, seed=1))
    ids_b_dev = torch.from_numpy(ids_b).to(dev)
    ws = {}
    for m in range(7):
        d_out, d_in = shapes[m]
        ws[m] = B.workspace(B.bd_apply_paged_workspace_bytes(S.p, S.T, n_slots, d_out, d_in,
                                                             B.BD_BF16, B.BD_F32), dev)
    xs = [S.xs[0]] * 3 + [S.xs[1]] + [S.xs[2]] * 2 + [S.xs[3]]

    def layer(ids_dev):
        for m in range(7):
            pager.apply(m, xs[m], S.wb[m], S.p, ids_dev, y=S.y[m], ws=ws[m])

    cold, warm, misses = [], [], []
    for r in range(reps):
        pager.ensure(S.ids_np)  # this step's users resident (batch A)
        layer(S.ids)
        torch.cuda.synchronize()
        before = pager.loads
        t1 = time.perf_counter()
        pager.ensure(ids_b)
        layer(ids_b_dev)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        layer(ids_b_dev)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        cold.append(t2 - t1)
        warm.append(t3 - t2)
        misses.append(pager.loads - before)
    for m in range(7):
        assert B.bd_device_status(ws[m]) == B.BD_OK
    users_b = len(set(int(u) for u in ids_b if u >= 0))
    loaded = misses[-1] * pager.slot_bytes
    cold_ms, warm_ms = 1e3 * min(cold), 1e3 * min(warm)
    return {"module": "layer 0: q, k, v, o, gate, up, down", "slot_bytes": pager.slot_bytes,
            "slots": n_slots, "users_in_host_store": S.U, "host_store_pack_s": round(pack_s, 2),
            "cold_batch_users": users_b, "misses_per_cold_step": misses[-1],
            "cold_step_ms": round(cold_ms, 3), "warm_step_ms": round(warm_ms, 3),
            "load_GBs_effective": round(loaded / max(1e-9, (cold_ms - warm_ms) * 1e-3) / 1e9, 1),
            "timing": "wall clock, min over reps; cold = ensure (misses copied from pinned "
                      "host memory) + 7 applies; warm = the 7 applies again"}


# ---------------------------------------------------------------- q_proj decode leg
def decode_leg(args, dev):
    """The Llama-3.1-8B q_proj decode step: 16 users x 1 token on 4096 x 4096, one
    bd_apply (one k_decode_unit launch), rotating over R input sets so consecutive
    steps do not hit the last-level cache; the two-launch path and the INT8 base
    timed beside it."""
    import torch

    from tenant_serving_amd import bitdelta as B
    from tenant_serving_amd import synth as S

    R = max(1, args.sets)
    w0 = S.workload(2)
    mat = w0.matrices[0]
    d_out, d_in, U, T = mat.d_out, mat.d_in, w0.n_users, w0.T
    w = dataclasses.replace(w0, matrices=[mat] * R, xgroups=[d_in] * R)
    p = B.params("matrix")
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
    wss = [B.workspace(ws_bytes, dev) for _ in range(R)]
    torch.cuda.synchronize()
    assert B.bd_device_status(cws) == B.BD_OK
    K = max(R, args.decode_steps)
    ctr = [0]

    def rot(fn):
        def f():
            k = ctr[0]
            ctr[0] += 1
            return fn(k)
        return f

    def step(k):
        wb, signs, scales, x, y = sets[k % R]
        assert B.bd_apply(x, wb, signs, scales, p, U, ids, y, wss[k % R]) == B.BD_OK

    def prep(k):
        wb, signs, scales, x, y = sets[k % R]
        assert B.bd_decode_prepare(x, ids, U, scales, p, wss[k % R]) == B.BD_OK

    def main_pass(k):
        wb, signs, scales, x, y = sets[k % R]
        assert B.bd_decode_apply(x, wb, signs, scales, p, U, y, wss[k % R]) == B.BD_OK

    for k in range(2 * R):
        step(k)
    torch.cuda.synchronize()
    y_eager = [sets[r][4].clone() for r in range(R)]
    g = capture(rot(step), K)
    g.replay()
    torch.cuda.synchronize()
    wall_us, ev_us = replay_timed(g, K)
    assert B.bd_device_status(wss[0]) == B.BD_OK
    for r in range(R):
        assert torch.equal(sets[r][4], y_eager[r]), f"graph replay differs from eager (set {r})"
    ctr[0] = 0
    gp = capture(rot(prep), K)
    ctr[0] = 0
    gm = capture(rot(main_pass), K)
    gp.replay()
    gm.replay()
    _, prep_us = replay_timed(gp, K)
    _, main_us = replay_timed(gm, K)

    q8 = [B.quantize_base(sets[r][0]) for r in range(R)]
    y8 = [torch.empty((T, d_out), dtype=torch.float32, device=dev) for _ in range(R)]

    def step_q8(k):
        wb, signs, scales, x, y = sets[k % R]
        q, qs = q8[k % R]
        assert B.bd_apply_q8(x, q, qs, signs, scales, p, U, ids, y8[k % R], wss[k % R]) == B.BD_OK

    ctr[0] = 0
    g8 = capture(rot(step_q8), K)
    g8.replay()
    _, q8_us = replay_timed(g8, K)
    assert B.bd_device_status(wss[0]) == B.BD_OK

    n_active = len(set(int(u) for u in ids_np if 0 <= u < U))
    bytes_step = (d_out * d_in * 2 + n_active * (d_out * d_in // 8 + 4) + T * d_in * 2
                  + T * d_out * 4 + 4 * T)
    bytes_q8 = bytes_step - d_out * d_in + 4 * d_out
    gbs = bytes_step / (ev_us * 1e-6) / 1e9
    out = {"workload": w0.name, "kernel": "k_decode_unit", "d_out": d_out, "d_in": d_in,
           "n_users": U, "tokens": T, "rotating_sets": R, "steps": K,
           "us_per_step_wall": round(wall_us, 3), "us_per_step_events": round(ev_us, 3),
           "algorithmic_bytes": bytes_step, "achieved": round(gbs, 1), "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4),
           "traffic": measured_traffic("k_decode_unit", w0.name),
           "tokens_per_s": round(T / (wall_us * 1e-6), 1),
           "two_launch_path_us": {"k_decode_prep": round(prep_us, 3), "k_decode": round(main_us, 3)},
           "int8_base_step": {"kernel": "k_decode_unit (INT8 base)", "us": round(q8_us, 3),
                              "algorithmic_bytes": bytes_q8,
                              "achieved": round(bytes_q8 / (q8_us * 1e-6) / 1e9, 1),
                              "frac": round(bytes_q8 / (q8_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
    del g, gp, gm, g8
    return out, (w, sets, cws)


def compress_legs(args, dev, decode_state):
    """bd_compress per call: (a) one user's q_proj, MATRIX scale, no clipping (one
    streaming pass); (b) one user's MLP gate_proj 14336 x 4096 of the clipped MLP
    workload, GROUP 128 fp32 scales, 3-sigma clipping (three passes: mean, squared
    deviations, pack); (c) bd_select_axis on (a)'s matrices."""
    import torch

    from tenant_serving_amd import bitdelta as B
    from tenant_serving_amd import synth as S

    w, sets, cws = decode_state
    R = len(sets)
    mat = w.matrices[0]
    d_out, d_in = mat.d_out, mat.d_in
    p = B.params("matrix")
    KC = max(1, args.compress_steps)
    n_c = min(8, w.n_users)
    wfs = []
    for u in range(n_c):
        t = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)
        S.dev_wfine(w, u % R, u, sets[u % R][0], out=t)
        wfs.append((t, sets[u % R][0]))
    c_signs = torch.empty((d_out, d_in // 64), dtype=torch.int64, device=dev)
    c_scales = torch.empty(1, dtype=torch.float32, device=dev)
    ctr = [0]

    def comp():
        k = ctr[0]
        ctr[0] += 1
        assert B.bd_compress(wfs[k % n_c][0], wfs[k % n_c][1], p, c_signs, c_scales, cws) == B.BD_OK

    g = capture(comp, KC)
    g.replay()
    _, comp_us = replay_timed(g, KC)
    assert B.bd_device_status(cws) == B.BD_OK
    comp_bytes = 2 * d_out * d_in * 2 + d_out * d_in // 8 + 4
    comp_gbs = comp_bytes / (comp_us * 1e-6) / 1e9
    out = {"compress": {"matrix": "q_proj 4096 x 4096 bf16, MATRIX fp32, no clip",
                        "call_us": round(comp_us, 3), "algorithmic_bytes": comp_bytes,
                        "achieved": round(comp_gbs, 1), "unit": "GB/s",
                        "frac": round(comp_gbs / HBM_PEAK_GBS, 4)}}

    # (b) the clipped GROUP compress of the MLP workload
    w3 = S.workload(3)
    m3 = w3.matrices[0]
    p3 = B.params("group", w3.group_size, w3.clip_k, B.BD_F32)
    wb3 = S.dev_wbase(w3, 0)
    wf3 = [S.dev_wfine(w3, 0, u, wb3) for u in range(2)]
    s3 = torch.empty((m3.d_out, m3.d_in // 64), dtype=torch.int64, device=dev)
    n_sc3 = B.bd_scales_count(p3, m3.d_out, m3.d_in)
    c3 = torch.empty(n_sc3, dtype=torch.float32, device=dev)
    ws3 = B.workspace(B.bd_compress_workspace_bytes(p3, m3.d_out, m3.d_in), dev)
    ctr[0] = 0

    def comp3():
        k = ctr[0]
        ctr[0] += 1
        assert B.bd_compress(wf3[k % 2], wb3, p3, s3, c3, ws3) == B.BD_OK

    KC3 = max(1, KC // 4)
    g3 = capture(comp3, KC3)
    g3.replay()
    _, c3_us = replay_timed(g3, KC3)
    assert B.bd_device_status(ws3) == B.BD_OK
    N3 = m3.d_out * m3.d_in
    c3_bytes = 3 * (2 * N3 * 2) + N3 // 8 + 4 * n_sc3
    c3_gbs = c3_bytes / (c3_us * 1e-6) / 1e9
    out["compress_clip3_group128"] = {
        "matrix": f"{w3.name} gate_proj {m3.d_out} x {m3.d_in} bf16, GROUP 128 fp32, clip 3 sigma "
                  "(0.1% injected +-50 sigma outliers)",
        "passes": 3, "call_us": round(c3_us, 3), "algorithmic_bytes": c3_bytes,
        "achieved": round(c3_gbs, 1), "unit": "GB/s", "frac": round(c3_gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_one_pass_statistics": 2 * (2 * N3 * 2) + N3 // 8 + 4 * n_sc3}
    del g, g3, wf3, wb3

    # (c) the per-layer axis choice on (a)'s matrices
    a_ws = B.workspace(B.bd_select_axis_workspace_bytes(d_out, d_in, 0.0), dev)
    a_err = torch.empty(2, dtype=torch.float64, device=dev)
    a_axis = torch.empty(1, dtype=torch.int32, device=dev)
    ctr[0] = 0

    def axis_sel():
        k = ctr[0]
        ctr[0] += 1
        assert B.bd_select_axis(wfs[k % n_c][0], wfs[k % n_c][1], 0.0, a_err, a_axis, a_ws) == B.BD_OK

    ga = capture(axis_sel, KC)
    ga.replay()
    _, ax_us = replay_timed(ga, KC)
    assert B.bd_device_status(a_ws) == B.BD_OK
    ax_bytes = 2 * d_out * d_in * 2
    ax_gbs = ax_bytes / (ax_us * 1e-6) / 1e9
    out["axis_select"] = {"call_us": round(ax_us, 3), "algorithmic_bytes": ax_bytes,
                          "achieved": round(ax_gbs, 1), "unit": "GB/s",
                          "frac": round(ax_gbs / HBM_PEAK_GBS, 4)}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("building the 32-layer stack (128 users' banks through bd_compress)")
    st, S = stack_leg(args, dev)
    out = {"metric": METRIC, "value": st.pop("value"), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": st.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    out.update(st)
    out["timing"] = ("the K steps captured in one HIP graph, replayed once between device "
                     "synchronisations (wall clock -> ms_per_step; HIP events on the replay "
                     "stream -> gpu_step_us_events); each phase's launches of K steps captured "
                     "and replayed alone the same way (HIP events -> phases_us_per_step; the "
                     "roofline's avg_launch_us is the phase time over its launches)")
    out["kernel_source_digest"] = kernel_source_digest()
    cpu_sample = None
    if not args.no_cpu_baseline:
        cpu_sample = (S.ids_np, S.active, S.bytes_step)
    if not args.no_legs:
        log("INT8 base step")
        out["int8_base_step"] = int8_leg(S, dev, max(1, args.steps // 2))
        torch.cuda.empty_cache()
        log("paged banks (layer 0)")
        out["paged_layer0"] = paged_leg(S, dev)
    del S
    torch.cuda.empty_cache()

    if not args.no_legs:
        log("q_proj decode leg")
        dec, state = decode_leg(args, dev)
        out["decode_q_proj_16users"] = dec
        log("compress legs")
        out.update(compress_legs(args, dev, state))
        del state
        torch.cuda.empty_cache()

    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = nb
        del src, dst

    if cpu_sample is not None:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(*cpu_sample, rows=args.cpu_rows)
    print(json.dumps(out), flush=True)
    if args.load:
        print(json.dumps(load_leg()), file=sys.stderr, flush=True)
    if args.merge:
        for line in merge_leg():
            print(json.dumps(line), file=sys.stderr, flush=True)
    if args.workloads:
        for line in workloads_leg():
            print(json.dumps(line), file=sys.stderr, flush=True)


def cpu_baseline(ids_np, active, bytes_step, rows=64, seconds=12.0, max_calls=200):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: the 7
    matrices of layer 0 of the stack, `rows` seeded output rows of each, all 512
    tokens and every active user.  The oracle compresses those rows of each active
    user's fine-tune itself (not timed; the scale is the absmean of the sampled rows),
    then applies the batch to them repeatedly until about `seconds` of apply time."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle as O

    from tenant_serving_amd import synth as S

    w = S.workload(5)
    rng = np.random.default_rng(5)
    remap = {u: i for i, u in enumerate(active)}
    sub_ids = np.array([remap.get(int(u), -1) for u in ids_np], dtype=np.int32)
    t0 = time.perf_counter()
    layer = []
    sample_bytes = 0
    for m in range(7):
        mat = w.matrices[m]
        r = sorted(rng.choice(mat.d_out, size=min(rows, mat.d_out), replace=False).tolist())
        wb = S.host_wbase(w, m, rows=r)
        words, scs = [], []
        for u in active:
            wf = S.host_wfine(w, m, u, rows=r, wbase=wb)
            ww, ss, _, _ = O.compress(wf, wb, O.MATRIX, dtype=O.BF16)
            words.append(ww)
            scs.append(ss)
        x = S.host_x(w, mat.xgroup)
        layer.append((x, wb, np.stack(words), np.stack(scs)))
        na, T = len(active), w.T
        full = (mat.d_out * mat.d_in * 2 + na * (mat.d_out * mat.d_in // 8 + 4)
                + T * mat.d_in * 2 + T * mat.d_out * 4 + 4 * T)
        sample_bytes += full * len(r) / mat.d_out  # the sampled rows' share of the apply
    t1 = time.perf_counter()
    calls, spent = 0, 0.0
    while calls < max_calls and (calls == 0 or spent < seconds):
        t2 = time.perf_counter()
        for x, wb, words, scs in layer:
            O.apply(x, wb, words, scs, O.MATRIX, sub_ids)
        spent += time.perf_counter() - t2
        calls += 1
    return {"value": round(calls * sample_bytes / spent / 1e9, 4), "unit": "GB/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{calls} passes over layer 0's 7 matrices of the stack, {rows} seeded "
                      f"output rows each, all {w.T} tokens, {len(active)} active users (the "
                      f"oracle's own compress of those rows, untimed); fp64 plain loops, "
                      f"OpenMP over tokens; rate = passes x the sampled rows' share of those "
                      f"matrices' algorithmic bytes / total oracle apply time",
            "passes": calls, "apply_s": round(spent, 3), "sample_bytes": int(sample_bytes),
            "oracle_compress_s": round(t1 - t0, 3), "host_cpus": os.cpu_count()}


def workloads_leg(reps=10):
    """One layer step of workloads 3 and 4 through the prepared-batch calls, grouped as
    the stack's step is: per distinct input width one bd_batch_prepare (the grouping and
    tile packing of the batch), then per activation tensor one bd_batch_encode, one
    bd_base_gemm_n and one bd_delta_apply_encoded_n over the matrices that read it
    (gate|up; down alone).  Random banks (the time does not depend on the bit values;
    parity at these sizes is tested separately).  The step is captured `reps` times in a
    HIP graph and replayed."""
    import torch

    from tenant_serving_amd import bitdelta as B
    from tenant_serving_amd import synth as S

    dev = torch.device("cuda:0")
    out = []
    for wid in (3, 4):
        w = S.workload(wid)
        ids_np = S.user_ids(w)
        ids = torch.from_numpy(ids_np).to(dev)
        T, U = w.T, w.n_users
        nact = len(set(int(u) for u in ids_np if 0 <= u < U))
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + wid)
        xs, batches, groups = {}, {}, {}
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
            # matrices that read one activation tensor share its encoding (COL scales are
            # folded into the encoded tokens: a COL matrix keeps an encoding of its own)
            key = (m.xgroup, len(groups)) if m.mode == S.COL else (m.xgroup, -1)
            groups.setdefault(key, (xs[m.xgroup], p, batches[m.d_in][1], []))[3].append(
                (wb, signs, scales, y))
            tot_bytes += (m.d_out * m.d_in * 2 + nact * (m.d_out * m.d_in // 8 + scales.element_size() * n_sc)
                          + T * m.d_in * 2 + T * m.d_out * 4 + 4 * T)
            tot_flops += 2 * T * m.d_out * m.d_in
        need = max(B.bd_base_gemm_n_workspace_bytes(B.BD_BF16, T, x.shape[1],
                                                    [wb.shape[0] for wb, _, _, _ in ms])
                   for x, _, _, ms in groups.values())
        gws = B.workspace(need, dev) if need > 0 else None

        def step():
            for x, bt in batches.values():
                assert B.bd_batch_prepare(x, ids, U, bt) == B.BD_OK
            for x, p, bt, ms in groups.values():
                col = ms[0][2] if p.mode == B.BD_SCALE_COL else None
                assert B.bd_batch_encode(bt, x, U, col, p) == B.BD_OK
                assert B.bd_base_gemm_n(x, [m[0] for m in ms], [m[3] for m in ms],
                                        workspace=gws) == B.BD_OK
                assert B.bd_delta_apply_encoded_n(bt, T, x.shape[1], U, [m[1] for m in ms],
                                                  [m[2] for m in ms], p,
                                                  [m[3] for m in ms]) == B.BD_OK

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
                    "base_TFLOPs": round(tot_flops / us / 1e6, 1),
                    "calls": "per width bd_batch_prepare; per activation tensor bd_batch_encode, "
                             "bd_base_gemm_n, bd_delta_apply_encoded_n"})
        del groups, xs, batches, g, gws
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




if __name__ == "__main__":
    main()
