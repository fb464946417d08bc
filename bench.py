"""Benchmark: one sparse MoE layer forward on one MI355X.

A step is one whole-layer forward (router -> softmax/top-k -> capacity-limited
dispatch -> SwiGLU expert GEMMs (+ shared expert) -> weighted combine -> load
statistics) over one batch of synthetic input already resident in HBM.

Prints one JSON line: tokens/s of the Mixtral-shaped layer (T=4096, d=4096,
m=14336, E=8, k=2, bf16 activations and weights, fp32 router and accumulation),
a per-phase time split measured with HIP events on the launch stream, the
roofline fraction of the dominant kernel (expert GEMM1: gate/up + SwiGLU), and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from sparse_mixture_experts_23_amd import _lib as L  # noqa: E402
from sparse_mixture_experts_23_amd import api  # noqa: E402
from sparse_mixture_experts_23_amd.workloads import CONFIGS, make_inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MoE-layer tokens/sec on 1 MI355X (Mixtral shape); expert-GEMM % of MFMA peak"

# HBM bytes of one expert GEMM1 launch on the Mixtral-shaped layer: the rocprofv3
# FETCH_SIZE + WRITE_SIZE counters of the kernel (KiB per dispatch), each scaled by
# the bytes-per-KiB that the same counter reports for a plain device copy of known
# size (`bench.py --copy-calibration`).  Valid only for the GEMM source it was
# taken on: reported as null once expert_gemm.hip differs from that hash.
GEMM1_TRAFFIC = {"bytes": 6340091130, "source_sha256": "6c65a95c5971346d7e2a08453f9d4ed1eaa6ca5b244b15606034a24a01a5beab"}
GEMM_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_23_amd", "csrc", "expert_gemm.hip")


def gemm1_traffic_bytes():
    if not GEMM1_TRAFFIC:
        return None
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    return GEMM1_TRAFFIC["bytes"] if sha == GEMM1_TRAFFIC["source_sha256"] else None


SHORT_PHASE_BATCH = 10   # launches per timed batch of a short phase
SHORT_PHASE_MS = 0.2     # phases whose single launch takes less are timed in batches


def copy_calibration(nbytes: int, reps: int):
    """A plain device-to-device copy of nbytes, `reps` times: the reference whose
    FETCH_SIZE / WRITE_SIZE counters calibrate the GEMM's."""
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def _spread(v):
    """Median, 10th and 90th percentile (nearest rank) of sorted step times in ms."""
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]  # noqa: E731
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4), "n": len(v)}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Stages:
    """Pre-allocated buffers so that each C-ABI stage can be timed on its own."""

    def __init__(self, shape, inp):
        dev = inp.x.device
        T, k, E, d, m = shape.T, api.paths(shape), shape.E, shape.d, shape.m
        R = L.moe_max_rows(shape)
        self.shape, self.inp, self.R = shape, inp, R
        z = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        self.ids, self.w, self.status = z(T, k), z(T, k, dt=torch.float32), z(1)
        self.load, self.offsets, self.slot, self.row_of = z(E), z(E + 1), z(T, k), z(T, k)
        self.src, self.stats = z(max(R, 1)), z(L.MOE_STAT_COUNT)
        self.x_perm = z(max(R, 1), d, dt=inp.x.dtype)
        self.h = z(max(R, 1), m, dt=inp.x.dtype)
        self.H = z(max(R, 1), d, dt=torch.float32)
        self.y = z(T, d, dt=torch.float32)
        self.s = z(T, d, dt=torch.float32) if shape.m_shared else None
        self.ws_r = api.workspace(shape, L.MOE_WS_ROUTE, dev)
        self.ws_d = api.workspace(shape, L.MOE_WS_DISPATCH, dev)
        self.ws_f = api.workspace(shape, L.MOE_WS_FFN, dev)
        self.ws_s = api.workspace(shape, L.MOE_WS_SHARED, dev) if shape.m_shared else None
        # load-balance statistics (opt-in diagnostics, timed beside the layer)
        self.prob_sum = z(E, dt=torch.float32)
        self.bal = z(2 * E + L.MOE_BAL_COUNT, dt=torch.float32)
        self.ws_rs = api.workspace(shape, L.MOE_WS_ROUTE_STATS, dev)

    def run(self, phase, st):
        s, i, p = self.shape, self.inp, lambda t: None if t is None else t.data_ptr()  # noqa: E731
        if phase == "route":
            rc = L.moe_route(s, p(i.x), p(i.w_r), p(i.b_r), p(self.ids), p(self.w), p(self.status), p(self.ws_r),
                             self.ws_r.numel(), st)
        elif phase == "dispatch":
            rc = L.moe_dispatch(s, p(i.x), p(self.ids), p(self.w), p(self.load), p(self.offsets), p(self.slot),
                                p(self.row_of),
                                p(self.src), p(self.x_perm), p(self.stats), p(self.ws_d), self.ws_d.numel(), st)
        elif phase == "gemm1":
            rc = L.moe_expert_gemm1(s, p(self.x_perm), p(self.offsets), p(i.w_gate), p(i.w_up), p(self.h),
                                    p(self.ws_f), self.ws_f.numel(), st)
        elif phase == "gemm2":
            rc = L.moe_expert_gemm2(s, p(self.h), p(self.offsets), p(i.w_down), p(self.H), p(self.ws_f),
                                    self.ws_f.numel(), st)
        elif phase == "shared":
            rc = L.moe_shared_ffn(s, p(i.x), p(i.s_gate), p(i.s_up), p(i.s_down), p(self.s), p(self.ws_s),
                                  self.ws_s.numel(), st)
        elif phase == "combine":
            rc = L.moe_combine(s, p(self.H), p(self.row_of), p(self.w), p(self.s), p(self.y), st)
        elif phase == "route_stats":
            rc = L.moe_route_stats(s, p(i.x), p(i.w_r), p(i.b_r), p(self.ids), p(self.w), p(self.status),
                                   p(self.prob_sum), p(self.ws_rs), self.ws_rs.numel(), st)
        elif phase == "balance":
            rc = L.moe_balance(s, p(self.load), p(self.stats), p(self.prob_sum), p(self.bal), st)
        else:
            raise ValueError(phase)
        L.check(rc, phase)


def cpu_baseline(cfg, inp, budget_tokens, layer=None):
    """Time the oracle, as it stands, on a bounded sample of the same workload:
    the first `budget_tokens` tokens form the routing group (same d, m, E, k).
    With `layer` (the timed GPU forward's outputs) and a sample that is the whole
    routing group, the oracle's result also checks this run: the largest
    |y_gpu - y_ref| / (1 + |y_ref|) over every element, the tokens whose score
    margin at the top-k boundary is below 1e-5 (fp64 scores), and the tokens
    whose selected set differs from the GPU's (their rows are left out of the
    error, which then compares two different routings)."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
    except Exception:  # pragma: no cover
        threadpool_info = None
    Ts = min(budget_tokens, cfg.T)
    x = inp.x[:Ts].float().cpu().numpy().astype(np.float64)
    wr = inp.w_r.cpu().numpy()
    b = None if inp.b_r is None else inp.b_r.cpu().numpy()
    experts = (inp.w_gate.float().cpu().numpy(), inp.w_up.float().cpu().numpy(), inp.w_down.float().cpu().numpy())
    shared = None
    if cfg.m_shared:
        shared = (inp.s_gate.float().cpu().numpy(), inp.s_up.float().cpu().numpy(), inp.s_down.float().cpu().numpy())
    C = None if cfg.cf is None else O.capacity(Ts, cfg.k, cfg.E, *cfg.cf)
    # the routing and slot-assignment steps on their own, for the phase split
    t0 = time.perf_counter()
    rt = O.route(x, wr, b, cfg.k, cfg.gate_mode, cfg.renorm_form)
    t1 = time.perf_counter()
    cap = Ts if C is None else C
    if cfg.accept_by_gate:
        O.assign_slots_by_gate(rt.ids, O.round_to_f32(rt.w), cfg.E, cap)
    elif cfg.reroute:
        n = min(2 * cfg.k, cfg.E)
        ids2 = np.full((Ts, 2 * cfg.k), -1, dtype=np.int64)
        ids2[:, :n] = O.select_topk(rt.g32, n)
        O.assign_slots_reroute(ids2, cfg.k, cfg.E, cap)
    else:
        O.assign_slots(rt.ids, cfg.E, cap)
    t2 = time.perf_counter()
    res = O.forward(x, wr, b, experts, cfg.k, cfg.gate_mode, C=C, shared=shared, round_h_bf16=cfg.dtype == "bf16",
                    renorm_form=cfg.renorm_form, accept_by_gate=cfg.accept_by_gate,
                    renorm_survivors=cfg.renorm_survivors, reroute=cfg.reroute)
    dt = time.perf_counter() - t2
    parity = None
    if layer is not None and Ts == cfg.T:
        boundary, _ = O.route_margins(res.route.g64, cfg.k)
        ids_gpu = layer.topk_ids.cpu().numpy()
        same = (np.sort(ids_gpu, axis=1) == np.sort(res.route.ids, axis=1)).all(axis=1)   # every record
        y_gpu = layer.y.cpu().numpy().astype(np.float64)
        err = (np.abs(y_gpu - res.y) / (1.0 + np.abs(res.y)))[same]
        tol = 2e-2 if cfg.dtype == "bf16" else 1e-5
        parity = {"tokens": int(Ts), "elements": int(err.size), "max_rel_err": float(err.max()) if err.size else 0.0,
                  "tol": tol, "within_tol": bool(err.size == 0 or err.max() <= tol),
                  "near_ties": int((boundary < 1e-5).sum()), "set_flips": int((~same).sum()),
                  "slots_equal": bool((layer.slot.cpu().numpy() == res.dispatch.slot).all()) if same.all() else None}
    t_route, t_disp = t1 - t0, t2 - t1
    threads = 1
    if threadpool_info is not None:
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            threads = max(p.get("num_threads", 1) for p in info)
    return {"value": Ts / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{Ts}-token routing group of the {cfg.name} layer (d={cfg.d}, m={cfg.m}, E={cfg.E}, "
                      f"k={cfg.k}), fp64 numpy oracle, {dt:.1f} s",
            "phase_s": {"route": round(t_route, 3), "dispatch": round(t_disp, 3),
                        "experts_and_combine": round(max(dt - t_route - t_disp, 0.0), 3)},
            "cpu": _cpu_model(), "parity_vs_gpu": parity}


def _cpu_model():
    """Host CPU model and socket count from /proc/cpuinfo (Linux)."""
    try:
        txt = open("/proc/cpuinfo").read()
    except OSError:
        return None
    def field(name):
        vals = {ln.split(":", 1)[1].strip() for ln in txt.splitlines() if ln.split(":", 1)[0].strip() == name}
        return sorted(vals)[0] if vals else None

    sockets = {ln.split(":", 1)[1].strip() for ln in txt.splitlines() if ln.startswith("physical id")}
    return {"model": field("model name"), "family": field("cpu family"), "model_id": field("model"),
            "stepping": field("stepping"), "sockets": len(sockets) or None,
            "logical_cpus": txt.count("\nprocessor") + txt.startswith("processor"),
            "threads_visible": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral", choices=sorted(CONFIGS))
    ap.add_argument("--accept-by-gate", action="store_true",
                    help="overflow variant: experts over capacity keep their highest-weight requests")
    ap.add_argument("--renorm-survivors", action="store_true",
                    help="overflow variant: weights renormalised over each token's accepted paths")
    ap.add_argument("--reroute", action="store_true",
                    help="overflow variant: a rejected path goes to the token's next-choice expert")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count T (e.g. 1..64 for decode-sized batches)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra forwards each timed after a 512 MiB cache-flushing write (0: none)")
    ap.add_argument("--phases", default="1", help="0 disables the per-phase timing loop")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer forward is built and timed on a single MI355X; "
              "runs on more than one GPU are not supported.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return

    cfg = CONFIGS[args.workload]
    if args.tokens:
        cfg = cfg.with_tokens(args.tokens)
    if args.accept_by_gate or args.renorm_survivors or args.reroute:
        cfg = cfg.scaled(accept_by_gate=args.accept_by_gate, renorm_survivors=args.renorm_survivors,
                         reroute=args.reroute)
    log(f"[bench] workload {cfg.name}: generating inputs on the GPU")
    inp = make_inputs(cfg, seed=0, device="cuda")
    C = 0 if cfg.cf is None else api.capacity(cfg.T, cfg.k, cfg.E, *cfg.cf)
    shape = api.make_shape(cfg.T, cfg.d, cfg.m, cfg.E, cfg.k, C, cfg.gate_mode, cfg.torch_dtype, cfg.m_shared,
                           accept_by_gate=cfg.accept_by_gate, renorm_survivors=cfg.renorm_survivors,
                           reroute=cfg.reroute)
    layer = api.MoELayer(shape, "cuda")
    fwd = lambda: layer.forward(inp.x, inp.w_r, inp.b_r, inp.w_gate, inp.w_up, inp.w_down,  # noqa: E731
                                inp.s_gate, inp.s_up, inp.s_down)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    layer.check_status()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    # per-step HIP events on the launch stream (for the spread of step times)
    st_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    launch_stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    for a, b in st_ev:
        a.record(launch_stream)
        fwd()
        b.record(launch_stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(a.elapsed_time(b) for a, b in st_ev)
    ms = elapsed * 1e3 / max(args.steps, 1)
    tokens_per_s = cfg.T / (ms / 1e3)
    stats = layer.stats.cpu().tolist()
    load = layer.load.cpu().tolist()
    A = stats[L.MOE_STAT_ACCEPTED]
    log(f"[bench] {ms:.3f} ms/step, {tokens_per_s:,.0f} tokens/s, accepted paths {A}")

    # cold caches: before each step, a 512 MiB write evicts the 256 MB last-level
    # cache and the L2s, so the step reads its inputs from HBM
    cold_ms = []
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.cold_steps)]
        for i, (a, b) in enumerate(cold_ev):
            flush.fill_(i & 0xFF)
            a.record(launch_stream)
            fwd()
            b.record(launch_stream)
        torch.cuda.synchronize()
        cold_ms = sorted(a.elapsed_time(b) for a, b in cold_ev)
        del flush

    # per-phase split with HIP events on the launch stream
    phases = {}
    if args.phases != "0":
        stg = Stages(shape, inp)
        st = torch.cuda.current_stream()
        names = (["route", "dispatch", "gemm1", "gemm2"] + (["shared"] if cfg.m_shared else []) + ["combine"]
                 + ["route_stats", "balance"])
        single = {}
        for n in names:   # warm each stage once, with a rough single-launch time
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            stg.run(n, st.cuda_stream)
            b.record(st)
            single[n] = (a, b)
        torch.cuda.synchronize()
        single = {n: a.elapsed_time(b) for n, (a, b) in single.items()}
        reps = max(args.steps, 1)
        ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
              for n in names}
        # The phases run interleaved, as in a forward, and the whole batch is
        # queued behind a few full forwards: the short phases then run back to back
        # (their events time the GPU, not the host's launch latency), and the GPU
        # never idles, so the heavy GEMMs run at the clock the timed forwards saw
        # (an idle gap lets the power controller overshoot: after one, the first
        # GEMMs run ~20 % slower for several milliseconds).
        # A short phase (under SHORT_PHASE_MS for one launch) is timed over a batch
        # of back-to-back launches (per-launch time = the batch's time / its size):
        # a pair of events around a single launch of a few microseconds adds
        # several microseconds of its own.
        batch = {n: (SHORT_PHASE_BATCH if single[n] < SHORT_PHASE_MS else 1) for n in names}
        for _ in range(4):
            fwd()
        for r in range(reps):
            for n in names:
                a, b = ev[n][r]
                a.record(st)
                for _ in range(batch[n]):
                    stg.run(n, st.cuda_stream)
                b.record(st)
        torch.cuda.synchronize()
        for n in names:
            phases[n] = sum(a.elapsed_time(b) for a, b in ev[n]) / reps / batch[n]
        log("[bench] phases (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in phases.items()))

    d, m, k, T = cfg.d, cfg.m, cfg.k, cfg.T
    es = 2 if cfg.dtype == "bf16" else 4
    gemm1_flop = 4.0 * A * d * m           # gate and up: 2 * A * d * m each
    gemm2_flop = 2.0 * A * d * m
    active = sum(1 for v in load if v > 0)
    roofline = None
    extra = {}
    if phases:
        t1 = phases["gemm1"] * 1e-3
        t2 = phases["gemm2"] * 1e-3
        # counters were taken on the Mixtral-shaped layer at T=4096 only
        traffic = gemm1_traffic_bytes() if (cfg.name == "mixtral" and T == 4096) else None
        rows_per_expert = A / max(active, 1)
        if rows_per_expert >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            # M_e flop per weight byte above the bf16 ridge: MFMA-bound
            ach = gemm1_flop / t1 / 1e12
            roofline = {"bound": "mfma", "kernel": "expert GEMM1 (gate/up + SwiGLU, bf16 MFMA)",
                        "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
        else:
            # few rows per expert: GEMM1 streams the touched gate/up weights
            g1_bytes = active * 2 * d * m * es + A * d * es + A * m * es
            ach = g1_bytes / t1 / 1e9
            roofline = {"bound": "hbm", "kernel": "expert GEMM1 (gate/up + SwiGLU, weight streaming)",
                        "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}
        # algorithmic bytes of the memory-bound phases
        route_bytes = T * d * es + 4 * cfg.E * d + 8 * T * k
        disp_bytes = T * d * es + A * d * es + 12 * T * k + 4 * A
        comb_bytes = A * d * 4 + T * d * 4 + 8 * T * k + (T * d * 4 if cfg.m_shared else 0)
        hbm = lambda b, ms_: round(b / (ms_ * 1e-3) / 1e9, 1)  # noqa: E731
        extra = {
            "phase_ms": {n: round(v, 4) for n, v in phases.items()},
            "expert_gemm_tflops": round((gemm1_flop + gemm2_flop) / (t1 + t2) / 1e12, 2),
            "expert_gemm_mfma_frac": round((gemm1_flop + gemm2_flop) / (t1 + t2) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gemm2_tflops": round(gemm2_flop / t2 / 1e12, 2),
            "hbm_gbs": {"route": hbm(route_bytes, phases["route"]), "dispatch": hbm(disp_bytes, phases["dispatch"]),
                        "combine": hbm(comb_bytes, phases["combine"])},
            "hbm_frac": {"route": round(route_bytes / (phases["route"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "dispatch": round(disp_bytes / (phases["dispatch"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "combine": round(comb_bytes / (phases["combine"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "hbm_algorithmic_bytes": {"route": route_bytes, "dispatch": disp_bytes, "combine": comb_bytes},
            "hbm_peak_gbs": PEAK_HBM_GBS,
        }
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": f"{cfg.name} MoE layer", "T": T, "d": d, "m": m, "E": cfg.E, "k": k,
                   "capacity": C or "unlimited", "gate": "switch" if cfg.gate_mode else "renorm",
                   "shared_expert_m": cfg.m_shared, "router": "fp32", "accumulate": "fp32",
                   "acceptance": "gate weight" if cfg.accept_by_gate else "token order",
                   "rejected_paths": ("reroute to the next choice" if cfg.reroute else "drop")
                   + (", renormalise survivors" if cfg.renorm_survivors else "")},
        "stats": {"accepted_paths": A, "overflow": stats[L.MOE_STAT_OVERFLOW],
                  "max_load": stats[L.MOE_STAT_MAX_LOAD], "rho_max": round(stats[L.MOE_STAT_MAX_LOAD] / (T * k / cfg.E), 4),
                  "tokens_dropped": stats[L.MOE_STAT_TOKENS_DROPPED], "rerouted": stats[L.MOE_STAT_REROUTED],
                  "active_experts": active},
        "roofline": roofline,
        "step_ms": _spread(step_ms),
        "cold_step_ms": _spread(cold_ms) if cold_ms else None,
        **extra,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on a {args.cpu_sample_tokens}-token sample")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens, layer)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
