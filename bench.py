#!/usr/bin/env python3
"""Benchmark: Q4_0 block-quantized mat-vec throughput on MI355X.

Workload (one "step"): the dense decode-layer projection set at M = 1 in
Q4_0 with hidden size 4096 -- Q 4096->4096, K 4096->1024, V 4096->1024,
O 4096->4096, FFN gate and up 4096->14336, down 14336->4096 -- on seeded
synthetic weights (scales ~U[0.001, 0.02] as binary16, codes ~U{0..15}) and
N(0, 1) activations. A step runs the projections as a decode layer can: Q, K
and V together (one input), then O, then gate and up together (one input),
then down: four batched launches (qmv_batch).

The weights of R distinct copies of the layer set are resident in HBM
(10 copies = 1.23 GB, several times the 256 MB Infinity Cache) and steps
rotate through them, so every step streams its weights from HBM.

Consecutive steps (one per copy, in turn) are captured together into one
HIP graph of 10 steps (40 kernel nodes) and the timed region replays it, so
the figure is the GPU's time, not the host's launch or replay rate.

Output: one JSON line with the effective weight bandwidth (algorithmic
weight bytes / wall time per step), the roofline of the qmv kernel (its
algorithmic bytes per launch / its average launch duration over the timed
region, which holds nothing but its launches) and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
CLOCK_HZ = 2.4e9       # MI355X peak engine clock (counter rates are taken against it)
# rocprofv3's derived metrics collected by the per-kernel profile, passed through
DERIVED = ("VALUBusy", "VALUUtilization", "VmemLatency", "LdsLatency", "LDSBankConflict", "LdsUtil",
           "MemUnitStalled", "OccupancyPercent", "MfmaUtil")
WARMUP_S = 0.3  # minimum untimed warm-up per measurement, seconds
METRIC = "effective weight GB/s and % of HBM peak, Q4_0 qmatmul at M=1 and M=16"
KERNEL_SRCS = [os.path.join(ROOT, "block_quantized_weight_qmatmul_amd", "csrc", f)
               for f in ("qmv.hip", "qmv_mq.hip", "qmv_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qmv_decode_layer_h4096.json")


def kernel_hash() -> str:
    """Hash of the kernel source's code: comments and blank space are left
    out, so that the committed counter figures stay attached to the code they
    were taken on and a comment edit does not orphan them."""
    import re
    src = ""
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def build_layer_sets(R, dev):
    """R copies of the layer set on the device: list of dicts name -> (W, x, y)."""
    import torch

    from block_quantized_weight_qmatmul_amd import synth
    probs = synth.CONFIGS[1]["problems"]
    sets = []
    for r in range(R):
        xin = {  # one input per dependency group
            "qkv": synth.make_x(1, 4096, cfg=1, copy=r, part=0),
            "o": synth.make_x(1, 4096, cfg=1, copy=r, part=3),
            "ffn": synth.make_x(1, 4096, cfg=1, copy=r, part=4),
            "down": synth.make_x(1, 14336, cfg=1, copy=r, part=6),
        }
        xdev = {k: torch.from_numpy(v[0]).to(dev) for k, v in xin.items()}
        group = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "ffn", "up": "ffn", "down": "down"}
        s = {}
        for part, p in enumerate(probs):
            W = torch.from_numpy(synth.make_weights("q4_0", p.N, p.K, cfg=1, copy=r, part=part)).to(dev)
            s[p.name] = (W, xdev[group[p.name]], torch.empty(p.N, dtype=torch.float32, device=dev))
        sets.append(s)
    return sets


GROUPS = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def step_bytes():
    from block_quantized_weight_qmatmul_amd import synth
    return sum(p.weight_bytes for p in synth.CONFIGS[1]["problems"])


def group_bytes(g):
    """Weight bytes of one launch group of the layer set."""
    from block_quantized_weight_qmatmul_amd import synth
    return sum(p.weight_bytes for p in synth.CONFIGS[1]["problems"] if p.name in g)


def fused_layer_set_throughput(sets, args):
    """The layer-set step with Q/K/V stored as one [6144, 4096] matrix and
    gate/up as one [28672, 4096] matrix (a loader may concatenate weights that
    share an input): four single-matrix calls per step. Returns GB/s."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv
    fused = []
    for s in sets:
        qkv = torch.cat([s["q"][0], s["k"][0], s["v"][0]])
        gu = torch.cat([s["gate"][0], s["up"][0]])
        fused.append({"qkv": (qkv, s["q"][1][None, :], torch.empty((1, qkv.shape[0]), device=qkv.device)),
                      "o": (s["o"][0], s["o"][1][None, :], s["o"][2][None, :]),
                      "gu": (gu, s["gate"][1][None, :], torch.empty((1, gu.shape[0]), device=gu.device)),
                      "down": (s["down"][0], s["down"][1][None, :], s["down"][2][None, :])})
    t = time_steps(lambda f: [qmv.qmv_q4_0(*f[n]) for n in ("qkv", "o", "gu", "down")], fused, args.steps,
                   args.warmup)
    del fused
    torch.cuda.empty_cache()
    return step_bytes() * args.steps / t / 1e9


def warm_eager(fn):
    """Call fn (which queues GPU work) until WARMUP_S seconds have passed,
    synchronizing every few calls, so the GPU runs at its working clocks when
    an eager timed region starts."""
    import torch
    t_end = time.perf_counter() + WARMUP_S
    n = 0
    while time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_steps(fn, sets, steps, warmup):
    """Wall time (s) of exactly `steps` steps after at least `warmup` untimed
    ones, bracketed by synchronizations and HIP events. Step i runs on
    sets[i % len(sets)]. Consecutive steps are captured together into HIP
    graphs of at least 8 steps, so each replay keeps the GPU busy long enough
    that the host's replay cost stays out of the timed region (one small graph
    per step measures the host, not the kernels)."""
    import torch
    R = len(sets)
    chunk = R * ((8 + R - 1) // R)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:  # eager pass first: library set-up stays out of the graphs
            fn(s)
    torch.cuda.synchronize()

    def build(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                fn(sets[i % R])
        return g
    full = build(chunk)
    part = build(steps % chunk) if steps % chunk else None
    torch.cuda.synchronize()
    # At least `warmup` steps, and at least WARMUP_S seconds of them: a GPU
    # that has been idle runs the first ~0.1 s of work at lower clocks (the
    # same 200 timed steps measured 6-8% slower after 20 warm-up steps than
    # after 2000).
    t_end = time.perf_counter() + WARMUP_S
    n = 0
    while n < (warmup + chunk - 1) // chunk or time.perf_counter() < t_end:
        full.replay()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps // chunk):
        full.replay()
    if part is not None:
        part.replay()
    e1.record()
    torch.cuda.synchronize()
    del full, part
    return e0.elapsed_time(e1) / 1e3


def stream_read_reference(dev, steps=200):
    """The streaming-read reference (qmv_stream_read: every byte once with
    16-byte non-temporal loads) at the sizes of the layer set's four launches
    and at 1 GiB, graph-timed over windows of a 1.25 GiB buffer (several
    sweeps beyond the Infinity Cache). The sum of the four launches' times is
    the floor of a step made of four dependent streaming launches."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv
    total = 5 * 2**28
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sizes = {}
    for g in GROUPS:
        sizes["+".join(g)] = group_bytes(g)
    sizes["1GiB"] = 2**30
    out = {"kernel": "k_stream_read (qmv_stream_read)", "buffer_bytes": total}
    floor_t = 0.0
    for name, nb in sizes.items():
        n = max(1, min(64, total // nb))
        wins = [buf[i * nb:(i + 1) * nb] for i in range(n)]
        st = steps if nb < 2**29 else 20
        t = time_steps(lambda w: qmv.stream_read(w, sink), wins, st, max(n, 8)) / st
        out[name] = {"bytes": nb, "windows": n, "us_per_call": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1),
                     "pct_hbm_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 2)}
        if name != "1GiB":
            floor_t += t
    nbytes = step_bytes()
    out["layer_set_floor"] = {"us_per_step": round(floor_t * 1e6, 2), "GBps": round(nbytes / floor_t / 1e9, 1),
                              "pct_hbm_peak": round(100 * nbytes / floor_t / 1e9 / HBM_PEAK_GBS, 2)}
    del buf
    torch.cuda.empty_cache()
    return out


def cold_single(dev, sets, reps=5):
    """Cold-single timing: before each launch a 1 GiB streaming read evicts
    the caches, then one launch of each of the layer set's four groups is
    timed alone between HIP events (launch overhead included; median of
    reps). Reported for transparency next to the steady-state sweep."""
    import statistics

    import torch

    from block_quantized_weight_qmatmul_amd import qmv
    flush = torch.empty(2**30, dtype=torch.uint8, device=dev)
    flush.fill_(0)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s0 = sets[0]
    out = {"flush_bytes": 2**30, "reps": reps, "stat": "median"}
    tot = 0.0
    for g in GROUPS:
        nb = group_bytes(g)
        ts = []
        for _ in range(reps):
            qmv.stream_read(flush, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            qmv.qmv_batch("q4_0", [s0[n] for n in g])
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        t = statistics.median(ts)
        tot += t
        out["+".join(g)] = {"bytes": nb, "us": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1)}
    out["layer_set"] = {"us": round(tot * 1e6, 2), "GBps": round(step_bytes() / tot / 1e9, 1)}
    del flush
    torch.cuda.empty_cache()
    return out


def m16_throughput(dev, qtype="q4_0", steps=40, workspace=True):
    """Config 3 (M = 16, K = 5120, N in {5120, 1024, 27648}; Q4_0, or the same
    shapes in Q8_0): each matrix timed on its own, graph-timed over enough
    rotated device copies to stream at least 1.07 GB per sweep (R = 73, 365
    and 14 copies in Q4_0), several calls per graph replay. With `workspace`
    the calls go through qmv_ws with a workspace of qmv_ws_bytes() bytes
    allocated once beforehand (the matrices with few rows then split K over
    workgroups); without, through qmv_q4_0 / qmv_q8_0. The set figure is the
    three matrices' bytes over the sum of their times."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    fn = {"q4_0": qmv.qmv_q4_0, "q8_0": qmv.qmv_q8_0}[qtype]
    out = {"workload": f"{qtype}_m16_k5120_n5120_1024_27648", "timing": "graph",
           "entry": "qmv_ws" if workspace else f"qmv_{qtype}"}
    tot_b, tot_t = 0, 0.0
    for part, p in enumerate(synth.CONFIGS[3]["problems"]):
        W = synth.make_weights(qtype, p.N, p.K, cfg=3, part=part)
        X = synth.make_x(p.M, p.K, cfg=3, part=part)
        nb = W.nbytes
        R = max(4, -(-int(1.07e9) // nb))
        Wd, Xd = torch.from_numpy(W).to(dev), torch.from_numpy(X).to(dev)
        sets = [(Wd if r == 0 else Wd.clone(), Xd, torch.empty((p.M, p.N), device=dev)) for r in range(R)]
        wsb = qmv.ws_bytes(qtype, p.M, p.N, p.K)
        ws = torch.empty(max(256, wsb), dtype=torch.uint8, device=dev) if workspace else None
        n = max(steps, R)
        if workspace:
            t = time_steps(lambda s: qmv.qmv_ws(qtype, s[0], s[1], s[2], ws), sets, n, R) / n
        else:
            t = time_steps(lambda s: fn(s[0], s[1], s[2]), sets, n, R) / n
        out[f"n{p.N}"] = {"weight_bytes": nb, "rotated_copies": R, "workspace_bytes": wsb if workspace else 0,
                          "us_per_call": round(t * 1e6, 2), "GBps": round(nb / t / 1e9, 1),
                          "pct_hbm_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 2),
                          "TFLOPs": round(2.0 * p.M * p.N * p.K / t / 1e12, 2)}
        tot_b += nb
        tot_t += t
        del sets, Wd, Xd, ws
        torch.cuda.empty_cache()
    out.update({"weight_bytes": tot_b, "us_per_set": round(tot_t * 1e6, 2), "GBps": round(tot_b / tot_t / 1e9, 1),
                "pct_hbm_peak": round(100 * tot_b / tot_t / 1e9 / HBM_PEAK_GBS, 2)})
    return out


def dense_m1_throughput(dev, cfg, steps=400):
    """One-problem M = 1 calls of a dense config (0: Q4_0 2048 -> 2048; 2:
    Q8_0 4096 -> 14336 and 14336 -> 4096), each timed on its own: a step is
    one call, steps rotate over enough device copies of the weights to fill
    >= 1.1 GB (beyond the Infinity Cache), several steps per graph replay.
    The copies hold one seeded weight tensor each (the data does not change
    the time; distinct buffers keep every call streaming from HBM)."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    fn = {"q4_0": qmv.qmv_q4_0, "q8_0": qmv.qmv_q8_0}
    out = {"workload": synth.CONFIGS[cfg]["name"]}
    for part, p in enumerate(synth.CONFIGS[cfg]["problems"]):
        W, X = synth.dense_inputs(cfg, p, part)
        R = max(4, -(-int(1.1e9) // p.weight_bytes))
        Wd = torch.from_numpy(W).to(dev)
        Xd = torch.from_numpy(X).to(dev)
        sets = [(Wd if r == 0 else Wd.clone(), Xd if r == 0 else Xd.clone(), torch.empty((1, p.N), device=dev))
                for r in range(R)]
        t = time_steps(lambda s: fn[p.qtype](s[0], s[1], s[2]), sets, steps, 2 * R)
        us = t / steps * 1e6
        out[p.name] = {"N": p.N, "K": p.K, "weight_bytes": p.weight_bytes, "rotated_copies": R,
                       "us_per_call": round(us, 2), "GBps": round(p.weight_bytes / us / 1e3, 1),
                       "pct_hbm_peak": round(100 * p.weight_bytes / us / 1e3 / HBM_PEAK_GBS, 2)}
        del sets, Wd, Xd
        torch.cuda.empty_cache()
    return out


def moe_throughput(dev, T, steps=40, mode="id"):
    """Config 4 (Q4_0 MoE, 128 experts, top-8, hidden 2816, expert
    intermediate 704) for T tokens over rotated stacks (16 for T = 1, 4 for
    T = 32), several steps per graph replay. GB/s counts the weights of the
    distinct selected experts (the bytes a call must read at least).

    mode "id": the gate_up and down id calls alone (down fed a synthetic x).
    mode "ffn_fused": the MoE FFN of the tokens: gate_up id, then the
    one-launch down half (SwiGLU + down + weighted sum), 2 launches.
    mode "ffn_two_call": gate_up id, SwiGLU-fed down id, weighted sum,
    3 launches."""
    import numpy as np
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    R = 16 if T == 1 else 4
    gu, dn = synth.moe_calls(T)
    sets, nbytes = [], 0
    for r in range(R):
        d = synth.moe_inputs(T, copy=r)
        dd = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in d.items()}
        dd["ids"] = dd["ids"].to(torch.int32).contiguous()
        dd["Y_gu"] = torch.empty(T * gu.top_k, gu.N, device=dev)
        dd["Y_dn"] = torch.empty(T * gu.top_k, dn.N, device=dev)
        dd["out"] = torch.empty(T, dn.N, device=dev)
        nexp = synth.distinct(d["ids"])
        nbytes += nexp * (gu.N * (gu.K // 32) + dn.N * (dn.K // 32)) * 18
        sets.append(dd)
    nbytes /= R

    def step(dd):
        qmv.qmv_id("q4_0", dd["W_gate_up"], dd["X_gate_up"], dd["ids"], dd["Y_gu"], gu.N, gu.K,
                   expert_scale=None if mode != "id" else dd["expert_scale"])
        if mode == "id":
            qmv.qmv_id("q4_0", dd["W_down"], dd["X_down"], dd["ids"].view(-1, 1), dd["Y_dn"], dn.N, dn.K,
                       expert_scale=dd["expert_scale"])
        elif mode == "ffn_fused":
            qmv.qmv_moe_down("q4_0", dd["W_down"], dd["Y_gu"], dd["ids"], dd["weights"], dd["out"], dn.N, dn.K,
                             expert_scale=dd["expert_scale"])
        else:
            qmv.qmv_id_swiglu("q4_0", dd["W_down"], dd["Y_gu"], dd["ids"].view(-1, 1), dd["Y_dn"], dn.N, dn.K,
                              expert_scale=dd["expert_scale"])
            qmv.qmv_moe_wsum(dd["Y_dn"], dd["weights"], dd["out"], gu.top_k)
    t = time_steps(step, sets, steps, 4) / steps
    launches = {"id": 2, "ffn_fused": 2, "ffn_two_call": 3}[mode]
    return {"workload": f"q4_0_moe_e128_top8_h2816_i704_t{T}", "mode": mode, "launches": launches,
            "weight_bytes_per_step": round(nbytes), "us_per_step": round(t * 1e6, 2),
            "GBps": round(nbytes / t / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2)}


def lm_head_q6k_throughput(dev, steps=20):
    """The pages' lm_head as Q6_K: [2816 -> 262144] (605.6 MB), one token
    (M = 1), replays of a graph of 8 calls on one copy (it is larger than the chip's last-level
    cache, so every replay streams it from HBM)."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    N, K = 262144, 2816
    W = torch.from_numpy(synth.make_weights("q6_k", N, K, cfg=5)).to(dev)
    X = torch.from_numpy(synth.make_x(1, K, cfg=5)[0]).to(dev)
    Y = torch.empty(N, device=dev)
    nbytes = N * synth.row_bytes("q6_k", K)
    t = time_steps(lambda s: qmv.qmv_q6_k(s[0], s[1], s[2]), [(W, X, Y)], steps, 3) / steps
    del W
    return {"workload": "q6_k_m1_lm_head_2816x262144", "weight_bytes": nbytes, "us_per_call": round(t * 1e6, 2),
            "GBps": round(nbytes / t / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2)}


def lm_head_q8_throughput(dev, steps=20):
    """The pages' lm_head re-quantized to Q8_0: [2816 -> 262144] (784.3 MB),
    one token, replays of a graph of 8 calls on one copy (larger than the
    chip's last-level cache, so every call streams it from HBM)."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    N, K = 262144, 2816
    W = torch.from_numpy(synth.make_weights("q8_0", N, K, cfg=5)).to(dev)
    X = torch.from_numpy(synth.make_x(1, K, cfg=5)).to(dev)
    Y = torch.empty((1, N), device=dev)
    nbytes = N * synth.row_bytes("q8_0", K)
    t = time_steps(lambda s: qmv.qmv_q8_0(s[0], s[1], s[2]), [(W, X, Y)], steps, 3) / steps
    del W
    return {"workload": "q8_0_m1_lm_head_2816x262144", "weight_bytes": nbytes, "us_per_call": round(t * 1e6, 2),
            "GBps": round(nbytes / t / 1e9, 1), "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2)}


def moe_q6k_gate_up_throughput(dev, steps=40):
    """The gate_up id call of one token over Q6_K experts (the pages' production
    MoE stores gate_up experts as Q6_K): 128 experts [1408, 2816], top-8. One
    stack (416 MB, larger than the last-level cache) and 16 routing sets
    replayed in turn; GB/s counts the 8 selected experts' bytes."""
    import numpy as np
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    E, N, K, k = 128, 1408, 2816, 8
    W = torch.from_numpy(synth.make_weights("q6_k", E * N, K, cfg=4, part=7).reshape(E, N, -1)).to(dev)
    X = torch.from_numpy(synth.make_x(1, K, cfg=4, part=7)).to(dev)
    sets = []
    for r in range(16):
        ids = torch.from_numpy(synth.router_topk(1, E, k, cfg=4, copy=r, part=7).astype(np.int32)).to(dev)
        sets.append((ids, torch.empty(k, N, device=dev)))
    nbytes = k * N * synth.row_bytes("q6_k", K)
    t = time_steps(lambda s: qmv.qmv_id("q6_k", W, X, s[0], s[1], N, K), sets, steps, 4) / steps
    del W
    return {"workload": "q6_k_moe_gate_up_e128_top8_h2816_n1408_t1", "weight_bytes_per_call": nbytes,
            "us_per_call": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2)}


def q5k_b9_throughput(dev, steps=48):
    """The pages' B9 group in Q5_K at M = 1: FFN gate and up 2816 -> 5760 and
    the router 2816 -> 128 (one input), one qmv_batch launch per step, and
    for comparison the same as three calls; 16 rotated copies (361 MB,
    larger than the last-level cache)."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    shapes = [("gate", 5760), ("up", 5760), ("router", 128)]
    K = 2816
    sets = []
    for r in range(16):
        x = torch.from_numpy(synth.make_x(1, K, cfg=6, copy=r)[0]).to(dev)
        sets.append([(torch.from_numpy(synth.make_weights("q5_k", n, K, cfg=6, copy=r, part=i)).to(dev), x,
                      torch.empty(n, device=dev)) for i, (_, n) in enumerate(shapes)])
    nbytes = sum(n for _, n in shapes) * synth.row_bytes("q5_k", K)
    t = time_steps(lambda s: qmv.qmv_batch("q5_k", s), sets, steps, 4) / steps
    t3 = time_steps(lambda s: [qmv.qmv_q5_k(W, x, y) for W, x, y in s], sets, steps, 4) / steps
    del sets
    return {"workload": "q5_k_m1_b9_gate_up_2816x5760_router_2816x128", "weight_bytes_per_step": nbytes,
            "entry": "qmv_batch", "launches": 1, "us_per_step": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2),
            "three_calls_us_per_step": round(t3 * 1e6, 2)}


def prefill_throughput(dev, M=512, steps=10):
    """Prefill-sized product (qmv_gemm): M = 512 activation rows through the
    Q4_0 FFN gate matrix 4096 -> 14336 (33 MB), eager raw calls (a call runs
    ~150 us, so the host's launch cost does not show). Beside it, the pages'
    F16-shadow route timed on the same shape: an fp16 GEMM of dequantized weights through
    torch.matmul (hipBLASLt) -- timing only, its fp16 activations do not meet
    the parity tolerance."""
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    N, K = 14336, 4096
    W = torch.from_numpy(synth.make_weights("q4_0", N, K, cfg=8)).to(dev)
    X = torch.from_numpy(synth.make_x(M, K, cfg=8)).to(dev)
    Y = torch.empty((M, N), device=dev)
    st = torch.cuda.current_stream().cuda_stream
    args = (qmv.QMV_Q4_0, W.data_ptr(), W.stride(0), X.data_ptr(), X.stride(0), Y.data_ptr(), Y.stride(0), M, N, K, st)

    def run():
        if qmv.raw_qmv_gemm(*args) != 0:
            raise RuntimeError(qmv.last_error())
    run()
    torch.cuda.synchronize()
    warm_eager(run)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    Wt = torch.randn((K, N), device=dev, dtype=torch.float16)  # the shadow's shape and dtype
    Xh = X.to(torch.float16)
    Yh = torch.matmul(Xh, Wt)
    torch.cuda.synchronize()
    warm_eager(lambda: torch.matmul(Xh, Wt, out=Yh))
    e0.record()
    for _ in range(steps):
        torch.matmul(Xh, Wt, out=Yh)
    e1.record()
    torch.cuda.synchronize()
    t16 = e0.elapsed_time(e1) / 1e3 / steps
    flops = 2.0 * M * N * K
    del W, X, Y, Wt, Xh, Yh
    return {"workload": f"q4_0_prefill_m{M}_4096x14336", "timing": "eager", "us_per_call": round(t * 1e6, 1),
            "TFLOPs": round(flops / t / 1e12, 1), "pct_fp16_mfma_peak": round(100 * flops / t / 2.5e15, 2),
            "f16_shadow_us": round(t16 * 1e6, 1), "f16_shadow_TFLOPs": round(flops / t16 / 1e12, 1)}


def moe_affine4_throughput(dev, steps=48):
    """MoE decode over MLX affine 4-bit expert stacks (the pages' DWQ stacks:
    groups of 32, bf16 scale and bias): 128 experts, gate_up [1408, 2816] and
    down [2816, 704], one token, top-8 -- the gate_up id call and the down id
    call (8 activation rows, one slot each). One stack pair (about 475 MB,
    larger than the last-level cache) and 16 routing sets in turn; GB/s counts
    the 8 selected experts' bytes (codes, scales and biases)."""
    import numpy as np
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    E, H, I, k = 128, 2816, 704, 8

    def stack(N, K, part):
        wq, sc, bi = synth.make_affine4(E * N, K, cfg=4, part=part)
        return tuple(torch.from_numpy(a.reshape(E, N, -1).view(dt)).to(dev)
                     for a, dt in ((wq, np.int32), (sc, np.int16), (bi, np.int16)))
    gu, dn = stack(2 * I, H, 8), stack(H, I, 9)
    X = torch.from_numpy(synth.make_x(1, H, cfg=4, part=8)).to(dev)
    Xd = torch.from_numpy(synth.make_x(k, I, cfg=4, part=9)).to(dev)
    sets = []
    for r in range(16):
        ids = torch.from_numpy(synth.router_topk(1, E, k, cfg=4, copy=r, part=8).astype(np.int32)).to(dev)
        sets.append((ids, torch.empty(k, 2 * I, device=dev), torch.empty(k, H, device=dev)))

    def step(s):
        qmv.qmv_affine4_id(*gu, X, s[0], s[1], 2 * I, H)
        qmv.qmv_affine4_id(*dn, Xd, s[0].view(-1, 1), s[2], H, I)
    per_expert = (2 * I * H // 2 + 2 * I * (H // 32) * 4) + (H * I // 2 + H * (I // 32) * 4)
    nbytes = k * per_expert
    t = time_steps(step, sets, steps, 4) / steps
    del gu, dn
    return {"workload": "affine4_g32_moe_e128_top8_h2816_i704_t1", "launches": 2, "weight_bytes_per_step": nbytes,
            "us_per_step": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
            "pct_hbm_peak": round(100 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2)}


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s: float):
    """The CPU oracle (fp64, OpenMP over rows) timed on a bounded sample of
    the layer set: the first rows of every projection, one thread and all
    the threads this process may use, each the median of 5 passes, the
    sample sized so that all passes together take about target_s seconds.
    Returns the JSON object of the cpu_baseline field."""
    import statistics

    import oracle
    from block_quantized_weight_qmatmul_amd import synth
    probs = synth.CONFIGS[1]["problems"]
    full = {}
    for part, p in enumerate(probs):
        W = synth.make_weights("q4_0", p.N, p.K, cfg=1, part=part)
        X = synth.make_x(1, p.K, cfg=1, part=part)
        full[p.name] = (W, X)
    # all cores of the affinity mask, within the thread budget the
    # environment sets for OpenMP (the host's share when it is shared)
    ncpu = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    cores = min(ncpu, int(env)) if env.isdigit() and int(env) > 0 else ncpu

    def run(frac, threads):
        nbytes, t0 = 0, time.perf_counter()
        for p in probs:
            W, X = full[p.name]
            rows = max(1, int(W.shape[0] * frac))
            oracle.qmv("q4_0", W[:rows], X, nthreads=threads)
            nbytes += rows * W.shape[1]
        return nbytes, time.perf_counter() - t0

    def leg(threads, budget):
        nb, t = run(1 / 64, threads)  # calibration
        frac = min(1.0, (1 / 64) * budget / 5 / max(t, 1e-4))
        res = [run(frac, threads) for _ in range(5)]
        gbs = statistics.median(b / t / 1e9 for b, t in res)
        return gbs, frac, res[0][0]

    one, f1, b1 = leg(1, target_s * 0.5)
    allc, fa, ba = leg(cores, target_s * 0.5)

    def desc(frac, nb):
        return (f"first {frac * 100:.2f}% of the rows of each of the 7 projections of the layer set "
                f"({nb / 1e6:.1f} MB of Q4_0 weights), median of 5 passes")
    return {"value": round(allc, 4), "unit": "GB/s", "cores": cores, "kind": "oracle", "sample": desc(fa, ba),
            "one_thread": {"value": round(one, 4), "unit": "GB/s", "sample": desc(f1, b1)},
            "cpu_model": cpu_model(), "affinity_cpus": ncpu}


def read_traffic(launch_bytes):
    """HBM traffic of the qmv kernel from committed rocprofv3 --pmc summaries,
    when they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return d.get("bytes_per_launch")


def summarize(stats_dir, fetch_dir, write_dir, cmd_note):
    """Turn rocprofv3 CSV output (kernel stats, FETCH_SIZE pass, WRITE_SIZE
    pass of `bench.py --probe-copy-mb`) into the committed summary under
    profiles/: the qmv kernel's average duration and its HBM traffic per
    launch, scaled by what the counters read for a plain copy of known size."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        fs = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        return [r for f in fs for r in csv.DictReader(open(f))]

    out = []
    stats = rows(stats_dir, "*kernel_stats.csv")
    for r in stats:
        if "k_m1" in r["Name"] or "copy" in r["Name"].lower() or "k_generic" in r["Name"]:
            out.append(f"{r['Name'][:90]:90s} calls={r['Calls']:>6s} avg_ns={float(r['AverageNs']):10.1f} "
                       f"min_ns={float(r['MinNs']):10.1f} max_ns={float(r['MaxNs']):10.1f}")

    def counter(d, name):
        per = {"qmv": [], "copy": []}
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != name:
                continue
            k = r["Kernel_Name"]
            if "k_m1" in k:
                per["qmv"].append(float(r["Counter_Value"]))
            elif "MulFunctor" in k or "copyBuffer" in k:
                per["copy"].append(float(r["Counter_Value"]))
        # the calibration copies are the 5 largest of those dispatches
        per["copy"] = sorted(per["copy"])[-5:]
        return per
    fetch, write = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    copy_bytes = 256 * 2**20
    res = {"kernel_source_sha256_16": kernel_hash()}
    if fetch["qmv"] and fetch["copy"] and write["qmv"] and write["copy"]:
        f_scale = copy_bytes / (1024 * statistics.median(fetch["copy"]))
        w_scale = copy_bytes / (1024 * statistics.median(write["copy"]))
        rd = statistics.mean(fetch["qmv"]) * 1024 * f_scale
        wr = statistics.mean(write["qmv"]) * 1024 * w_scale
        res.update({"bytes_per_launch": round(rd + wr), "read_bytes_per_launch": round(rd),
                    "write_bytes_per_launch": round(wr), "fetch_scale": round(f_scale, 4),
                    "write_scale": round(w_scale, 4), "algorithmic_bytes_per_launch": round(step_bytes() / len(GROUPS)),
                    "qmv_dispatches": len(fetch["qmv"])})
        out.append(f"FETCH_SIZE: qmv mean {statistics.mean(fetch['qmv']):.1f} KiB/dispatch over "
                   f"{len(fetch['qmv'])} dispatches; 256 MiB copy median {statistics.median(fetch['copy']):.1f} KiB "
                   f"-> scale {f_scale:.4f}")
        out.append(f"WRITE_SIZE: qmv mean {statistics.mean(write['qmv']):.1f} KiB/dispatch; copy median "
                   f"{statistics.median(write['copy']):.1f} KiB -> scale {w_scale:.4f}")
        out.append(f"traffic per launch: read {rd:.0f} B + write {wr:.0f} B = {rd + wr:.0f} B vs algorithmic "
                   f"{step_bytes() / len(GROUPS):.0f} B (weights only)")
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(res, f, indent=1)
    text = "\n".join([f"# qmv decode-layer set (Q4_0, M=1, hidden 4096), kernel source {kernel_hash()}",
                      f"# command: {cmd_note}", *out]) + "\n"
    with open(os.path.join(ROOT, "profiles", "k_m1c_decode_layer_h4096.txt"), "w") as f:
        f.write(text)
    print(text)


def summarize_trace(trace_csv, out_name, title, kernels, cmd_note):
    """Per-kernel median durations from a rocprofv3 kernel-trace CSV for the
    kernels whose names contain one of `kernels` (comma-separated), grouped
    by launch shape, written to profiles/<out_name>."""
    import csv
    import statistics
    if os.path.basename(out_name) != out_name:
        raise ValueError("out_name must be a file name inside profiles/")
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"].replace("void (anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        short = name.split("(")[0]
        if not any(k in short for k in kernels.split(",")):
            continue
        key = (short, int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# {title}", f"# command: {cmd_note}", "# per-kernel durations from the kernel trace (median over calls)",
             f"#   {'kernel':34s} {'grid_x(threads)':>15s} {'grid_y':>6s} {'wg':>4s} {'calls':>6s} {'median_us':>10s}"]
    for (k, gx, gy, wg), v in sorted(groups.items()):
        lines.append(f"  {k:34s} {gx:15d} {gy:6d} {wg:4d} {len(v):6d} {statistics.median(v):10.2f}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write(text)
    print(text)


# ---------------------------------------------------------------------------
# Per-kernel evidence: one representative call set per kernel, run eagerly a
# few times between separator kernels, for rocprofv3 kernel traces and
# counter passes; and the summarizer that writes profiles/counters_<kernel>.txt
# ---------------------------------------------------------------------------
def kernel_workloads(dev, reps=3):
    """Returns [(name, {kernel-name substring: algorithmic bytes per dispatch},
    call)] for the kernels of the library."""
    import numpy as np
    import torch

    from block_quantized_weight_qmatmul_amd import qmv, synth
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    out = []
    probs = {p.name: p for p in synth.CONFIGS[1]["problems"]}

    def w(qtype, N, K, part=0, cfg=9):
        return T(synth.make_weights(qtype, N, K, cfg=cfg, part=part))

    def x(M, K, part=0, cfg=9):
        return T(synth.make_x(M, K, cfg=cfg, part=part))
    # decode layer set (config 1): grouped Q/K/V and gate/up (k_m1c), single O and down (k_m1)
    qkv = [(w("q4_0", probs[n].N, 4096, i), probs[n].N) for i, n in enumerate(("q", "k", "v"))]
    xq = x(1, 4096)[0]
    ys = [torch.empty(n, device=dev) for _, n in qkv]
    out.append(("layer_qkv_q4_0_4096", {"k_m1c": sum(probs[n].weight_bytes for n in ("q", "k", "v"))},
                lambda: qmv.qmv_batch("q4_0", [(W_, xq, y_) for (W_, _), y_ in zip(qkv, ys)])))
    Wo, xo, yo = w("q4_0", 4096, 4096, 3), x(1, 4096, 3), torch.empty((1, 4096), device=dev)
    out.append(("layer_o_q4_0_4096x4096", {"k_m1": probs["o"].weight_bytes}, lambda: qmv.qmv_q4_0(Wo, xo, yo)))
    gu = [w("q4_0", 14336, 4096, 4 + i) for i in range(2)]
    xg = x(1, 4096, 4)[0]
    yg = [torch.empty(14336, device=dev) for _ in range(2)]
    out.append(("layer_gate_up_q4_0_4096x14336x2", {"k_m1c": 2 * probs["gate"].weight_bytes},
                lambda: qmv.qmv_batch("q4_0", [(gu[i], xg, yg[i]) for i in range(2)])))
    Wd, xd, yd = w("q4_0", 4096, 14336, 6), x(1, 14336, 6), torch.empty((1, 4096), device=dev)
    out.append(("layer_down_q4_0_14336x4096", {"k_m1": probs["down"].weight_bytes}, lambda: qmv.qmv_q4_0(Wd, xd, yd)))
    # config 2, Q8_0
    W8a, x8a, y8a = w("q8_0", 14336, 4096, 7), x(1, 4096, 7), torch.empty((1, 14336), device=dev)
    W8b, x8b, y8b = w("q8_0", 4096, 14336, 8), x(1, 14336, 8), torch.empty((1, 4096), device=dev)
    out.append(("q8_0_m1_4096x14336", {"k_m1": 14336 * 128 * 34}, lambda: qmv.qmv_q8_0(W8a, x8a, y8a)))
    out.append(("q8_0_m1_14336x4096", {"k_m1": 4096 * 448 * 34}, lambda: qmv.qmv_q8_0(W8b, x8b, y8b)))
    # config 3 (M = 16, K = 5120): the matrix cores, without and with a workspace
    for N in (27648, 5120, 1024):
        Wm, Xm, Ym = w("q4_0", N, 5120, N), x(16, 5120, N), torch.empty((16, N), device=dev)
        wsb = qmv.ws_bytes("q4_0", 16, N, 5120)
        ws = torch.empty(max(256, wsb), dtype=torch.uint8, device=dev)
        kb = {"k_mq<": N * 160 * 18}
        if wsb:
            kb["k_mqred"] = wsb + 16 * N * 4
            out.append((f"m16_q4_0_5120x{N}_ws", kb, lambda Wm=Wm, Xm=Xm, Ym=Ym, ws=ws: qmv.qmv_ws("q4_0", Wm, Xm, Ym, ws)))
        else:
            out.append((f"m16_q4_0_5120x{N}", kb, lambda Wm=Wm, Xm=Xm, Ym=Ym: qmv.qmv_q4_0(Wm, Xm, Ym)))
    Wq8, Xq8, Yq8 = w("q8_0", 27648, 5120, 9), x(16, 5120, 9), torch.empty((16, 27648), device=dev)
    out.append(("m16_q8_0_5120x27648", {"k_mq<": 27648 * 160 * 34}, lambda: qmv.qmv_q8_0(Wq8, Xq8, Yq8)))
    # config 4 MoE (T = 1 and 32; and 128 tokens) and the FFN epilogue
    for Tn in (1, 32, 128):
        d = synth.moe_inputs(Tn)
        dd = {k: T(v) for k, v in d.items()}
        dd["ids"] = dd["ids"].to(torch.int32).contiguous()
        g, dn = synth.moe_calls(Tn)
        ne = synth.distinct(d["ids"])
        Ygu = torch.empty(Tn * g.top_k, g.N, device=dev)
        Ydn = torch.empty(Tn * g.top_k, dn.N, device=dev)
        o = torch.empty(Tn, dn.N, device=dev)
        # few pairs: all rows as one matrix; many: grouped by expert, on the
        # matrix cores when experts serve several pairs each
        kid = {1: "k_idv", 32: "k_idp", 128: "k_idq"}[Tn]
        out.append((f"moe_t{Tn}_gate_up_id", {kid: ne * g.N * (g.K // 32) * 18},
                    lambda dd=dd, g=g, Ygu=Ygu: qmv.qmv_id("q4_0", dd["W_gate_up"], dd["X_gate_up"], dd["ids"], Ygu,
                                                            g.N, g.K, expert_scale=dd["expert_scale"])))
        out.append((f"moe_t{Tn}_down_id", {kid: ne * dn.N * (dn.K // 32) * 18},
                    lambda dd=dd, dn=dn, Ydn=Ydn: qmv.qmv_id("q4_0", dd["W_down"], dd["X_down"], dd["ids"].view(-1, 1),
                                                              Ydn, dn.N, dn.K, expert_scale=dd["expert_scale"])))
        if Tn == 1:
            out.append(("moe_t1_down_fused", {"k_moe_down": ne * dn.N * (dn.K // 32) * 18},
                        lambda dd=dd, dn=dn, o=o: qmv.qmv_moe_down("q4_0", dd["W_down"], dd["G_down"], dd["ids"],
                                                                   dd["weights"], o, dn.N, dn.K,
                                                                   expert_scale=dd["expert_scale"])))
            out.append(("moe_t1_wsum", {"k_wsum": 8 * dn.N * 4 + dn.N * 4},
                        lambda dd=dd, Ydn=Ydn, o=o: qmv.qmv_moe_wsum(Ydn, dd["weights"], o, 8)))
    # super-block formats
    N6, K6 = 262144, 2816
    W6, x6, y6 = w("q6_k", N6, K6, 10), x(1, K6, 10)[0], torch.empty(N6, device=dev)
    out.append(("q6_k_lm_head_2816x262144", {"k_q6k": N6 * synth.row_bytes("q6_k", K6)}, lambda: qmv.qmv_q6_k(W6, x6, y6)))
    W5 = [w("q5_k", n, 2816, 11 + i) for i, n in enumerate((5760, 5760, 128))]
    x5 = x(1, 2816, 11)[0]
    y5 = [torch.empty(n, device=dev) for n in (5760, 5760, 128)]
    out.append(("q5_k_b9_2816x5760x2_128", {"k_q6kc": (5760 * 2 + 128) * synth.row_bytes("q5_k", 2816)},
                lambda: qmv.qmv_batch("q5_k", [(W_, x5, y_) for W_, y_ in zip(W5, y5)])))
    E6 = torch.from_numpy(synth.make_weights("q6_k", 128 * 1408, 2816, cfg=9, part=12).reshape(128, 1408, -1)).to(dev)
    x6e = x(1, 2816, 12)
    ids6 = T(synth.router_topk(1, 128, 8, cfg=9, part=12).astype(np.int32))
    y6e = torch.empty(8, 1408, device=dev)
    out.append(("q6_k_moe_gate_up_t1", {"k_id_q6": 8 * 1408 * synth.row_bytes("q6_k", 2816)},
                lambda: qmv.qmv_id("q6_k", E6, x6e, ids6, y6e, 1408, 2816)))
    # the streaming-read reference on 66 MB (the gate+up launch's bytes)
    # (no fill: a fill kernel would read as a workload separator; the data
    # does not matter to the read)
    sbuf = torch.empty(66060288, dtype=torch.uint8, device=dev)
    ssink = torch.empty(1, dtype=torch.int32, device=dev)
    out.append(("stream_read_66MB", {"k_stream_read": 66060288}, lambda: qmv.stream_read(sbuf, ssink)))
    # the generic kernel (K % 64 != 0) and a prefill block set
    Wg, Xg, Yg = w("q4_0", 4096, 4064, 13), x(1, 4064, 13), torch.empty((1, 4096), device=dev)
    out.append(("generic_q4_0_4064x4096", {"k_generic": 4096 * 127 * 18}, lambda: qmv.qmv_q4_0(Wg, Xg, Yg, K=4064)))
    Wp, Xp, Yp = w("q4_0", 14336, 4096, 14), x(512, 4096, 14), torch.empty((512, 14336), device=dev)
    # prefill (the tiled kernel): weights once + X + Y
    out.append(("prefill_q4_0_m512_4096x14336", {"k_gemm": 14336 * 128 * 18 + 512 * 4096 * 4 + 512 * 14336 * 4},
                lambda: qmv.qmv_gemm("q4_0", Wp, Xp, Yp)))
    return out


def run_kernel_workloads(dev, reps, manifest_path):
    """Calibration copies, then each workload `reps` times after a separator
    kernel (a 1-element fill), synchronized; writes the manifest."""
    import torch
    wl = kernel_workloads(dev)
    sep = torch.empty(1, device=dev)
    src = torch.empty(256 * 2**20 // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    for fn in [c for _, _, c in wl]:  # one untimed pass: library set-up stays out
        fn()
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)  # calibration: reads and writes 256 MiB
    torch.cuda.synchronize()
    del src, dst
    for i, (_, _, fn) in enumerate(wl):
        sep.fill_(float(i))
        torch.cuda.synchronize()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
    man = {"reps": reps, "workloads": [{"name": n, "kernels": kb} for n, kb, _ in wl]}
    with open(manifest_path, "w") as f:
        json.dump(man, f, indent=1)
    print(f"kernel workloads done: {len(wl)} x {reps}", flush=True)


def summarize_kernels(trace_dir, pmc_dirs, manifest_path, cmd_note):
    """rocprofv3 CSV output of run_kernel_workloads (a kernel trace and
    counter passes) -> profiles/counters_<kernel>.txt, one per library
    kernel: duration, HBM traffic against algorithmic bytes (scaled by a
    256 MiB copy), L2 hit rate, VALU busy and instructions, occupancy."""
    import csv
    import glob
    import statistics
    man = json.load(open(manifest_path))
    wls = man["workloads"]

    def rows(d, pat):
        return [r for f in glob.glob(os.path.join(d, "**", pat), recursive=True) for r in csv.DictReader(open(f))]

    def segment(disp):
        """dispatches (dict id -> name) in id order split at the fill separators"""
        seg, cur, calib = {}, None, []
        for i in sorted(disp):
            n = disp[i]
            if "FillFunctor" in n or "fill" in n.lower():
                cur = 0 if cur is None else cur + 1
                continue
            if cur is None:
                if "MulFunctor" in n:
                    calib.append(i)
                continue
            seg[i] = cur
        return seg, calib
    tr = rows(trace_dir, "*kernel_trace.csv")
    tdisp = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in tr}
    tdur = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr}
    tseg, _ = segment(tdisp)
    # counters: value per (dispatch, counter), summed over instances
    # the CSV holds each counter summed over its instances; GRBM_GUI_ACTIVE
    # (elapsed GPU cycles) is counted once per XCD, so it is divided by
    # their number (the vendor's derived metrics take its maximum)
    agents = [a for a in rows(pmc_dirs[0], "*agent_info.csv") if a.get("Name", "").startswith("gfx")]
    xcc = int(agents[0].get("Num_Xcc", 1)) if agents else 1
    ncu = int(agents[0].get("Cu_Count", 256)) if agents else 256
    cnt, cdisp = {}, {}
    for pi, d in enumerate(pmc_dirs):
        for r in rows(d, "*counter_collection.csv"):
            key = (d, int(r["Dispatch_Id"]))
            cdisp[key] = r["Kernel_Name"]
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            if pi > 0 and c in ("GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_INSTS_VMEM_RD"):
                c = f"{c}@{pi}"  # counters taken in several passes: each pass's own
            if c == "GRBM_GUI_ACTIVE":
                v /= xcc
            cnt.setdefault(key, {})[c] = cnt.setdefault(key, {}).get(c, 0.0) + v
    per = {}  # (workload index, kernel key) -> counter name -> [values]
    calib = {}
    for d in pmc_dirs:
        disp = {i: n for (dd, i), n in cdisp.items() if dd == d}
        seg, cal = segment(disp)
        for i in cal:
            for c, v in cnt[(d, i)].items():
                calib.setdefault(c, []).append(v)
        for i, wi in seg.items():
            name = disp[i]
            for kk in wls[wi]["kernels"]:
                if kk in name:
                    for c, v in cnt[(d, i)].items():
                        per.setdefault((wi, kk), {}).setdefault(c, []).append(v)
    reps = man["reps"]
    copy = 256 * 2**20
    f_scale = copy / (1024 * statistics.median(calib["FETCH_SIZE"])) if calib.get("FETCH_SIZE") else None
    w_scale = copy / (1024 * statistics.median(calib["WRITE_SIZE"])) if calib.get("WRITE_SIZE") else None
    by_kernel = {}
    for wi, wl in enumerate(wls):
        for kk, alg in wl["kernels"].items():
            # per call of the workload (a call may launch the kernel several
            # times, e.g. the three projections of a group): sums over its
            # dispatches / calls; rates are cycle-weighted over them
            durs = [tdur[i] for i, s in tseg.items() if s == wi and kk in tdisp[i]]
            pv = per.get((wi, kk), {})
            c = {k: sum(v) / reps for k, v in pv.items()}
            # the vendor's derived metrics (rocprofv3 computes them per
            # dispatch): averaged over the workload's dispatches
            for k in DERIVED:
                if k in pv:
                    c[k] = sum(pv[k]) / len(pv[k])
            line = {"workload": wl["name"], "dispatches_per_call": round(len(durs) / reps, 2),
                    "us_per_call": round(sum(durs) / reps, 2) if durs else None, "alg_bytes": alg}
            if durs:
                line["alg_GBps"] = round(alg / (sum(durs) / reps) / 1e3, 1)
            if "FETCH_SIZE" in c and f_scale:
                line["fetch_bytes"] = round(c["FETCH_SIZE"] * 1024 * f_scale)
                line["fetch_over_alg"] = round(line["fetch_bytes"] / alg, 3)
            if "WRITE_SIZE" in c and w_scale:
                line["write_bytes"] = round(c["WRITE_SIZE"] * 1024 * w_scale)
            if "TCC_HIT" in c and "TCC_MISS" in c and c["TCC_HIT"] + c["TCC_MISS"] > 0:
                line["l2_hit_pct"] = round(100 * c["TCC_HIT"] / (c["TCC_HIT"] + c["TCC_MISS"]), 1)
            g = c.get("GRBM_GUI_ACTIVE")
            # cycles of the kernel's time at the nominal 2.4 GHz clock, on
            # every SIMD (4 per CU) or CU of the chip
            cyc = sum(durs) / reps * 1e-6 * CLOCK_HZ if durs else None
            if cyc and "SQ_INSTS_VALU" in c:
                # a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles
                line["valu_busy_pct"] = round(100 * 4 * c["SQ_INSTS_VALU"] / (4 * ncu * cyc), 1)
            if g and "SQ_WAVE_CYCLES" in c:
                line["occupancy_pct"] = round(400 * c["SQ_WAVE_CYCLES"] / g / ncu / 32, 1)
            if "SQ_INST_LEVEL_VMEM" in c and c.get("SQ_INSTS_VMEM_RD@2"):
                # Little's law: vector memory instructions in flight summed per
                # cycle over completed ones = mean latency in cycles
                line["vmem_latency_cycles"] = round(c["SQ_INST_LEVEL_VMEM"] / c["SQ_INSTS_VMEM_RD@2"])
            if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_ACTIVE_INST_LDS"):
                line["lds_bank_conflict_pct"] = round(100 * c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"], 1)
            if cyc and "SQ_ACTIVE_INST_LDS" in c:
                line["lds_active_pct"] = round(100 * c["SQ_ACTIVE_INST_LDS"] / (ncu * cyc), 1)
            if "SQ_WAIT_INST_LDS" in c and c.get("SQ_WAVE_CYCLES@2"):
                line["wave_wait_lds_pct"] = round(100 * c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES@2"], 1)
            if cyc and "TA_BUSY" in c:
                line["ta_busy_pct"] = round(100 * c["TA_BUSY"] / (ncu * cyc), 1)
            for k in DERIVED:
                if k in c:
                    line[k] = round(c[k], 2)
            if "SQ_INSTS_VALU" in c and "SQ_WAVES" in c:
                line["valu_insts_per_wave"] = round(c["SQ_INSTS_VALU"] / max(1, c["SQ_WAVES"]))
                wts = alg / (0.5625 if "q4_0" in wl["name"] else 34 / 32 if "q8_0" in wl["name"] else 1)
                line["valu_lane_insts_per_weight"] = round(c["SQ_INSTS_VALU"] * 64 / wts, 2)
            if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                line["mfma_util_pct"] = round(100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * ncu * 4), 1)
            if cyc and "TCP_TCP_TA_DATA_STALL_CYCLES" in c:
                line["ta_data_stall_pct"] = round(100 * c["TCP_TCP_TA_DATA_STALL_CYCLES"] / cyc / ncu, 1)
            if g and "SQ_WAIT_INST_ANY" in c and "SQ_WAVE_CYCLES" in c and c["SQ_WAVE_CYCLES"] > 0:
                line["wave_wait_inst_pct"] = round(100 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], 1)
            by_kernel.setdefault(kk.strip("<"), []).append(line)
    for k, lines in by_kernel.items():
        text = [f"# {k}: figures per call of each workload (over {reps} calls), kernel sources {kernel_hash()}",
                f"# command: {cmd_note}",
                f"# traffic = FETCH_SIZE / WRITE_SIZE x the scale that makes a 256 MiB copy read 256 MiB "
                f"(fetch scale {f_scale and round(f_scale, 4)}, write scale {w_scale and round(w_scale, 4)}); "
                "valu_busy = 4 cycles x SQ_INSTS_VALU / (SIMDs x kernel cycles at 2.4 GHz); occupancy = "
                "SQ_WAVE_CYCLES share of 32 wave slots per CU; VALU lane instructions per weight = SQ_INSTS_VALU "
                "x 64 / weights; vmem_latency = SQ_INST_LEVEL_VMEM / SQ_INSTS_VMEM_RD (cycles); lds_active = "
                "SQ_ACTIVE_INST_LDS / (CUs x kernel cycles); lds_bank_conflict = SQ_LDS_BANK_CONFLICT / "
                "SQ_ACTIVE_INST_LDS; wave_wait_lds = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; ta_busy = TA_BUSY / (CUs x "
                "kernel cycles); mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x kernel cycles); wave_wait_inst = "
                "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (two passes)"]
        text += [json.dumps(ln) for ln in lines]
        with open(os.path.join(ROOT, "profiles", f"counters_{k}.txt"), "w") as f:
            f.write("\n".join(text) + "\n")
        print("\n".join(text))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        summarize(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-kernels":
        summarize_kernels(sys.argv[2], sys.argv[3].split(","), sys.argv[4], " ".join(sys.argv[5:]))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--kernel-workloads":
        import torch
        from block_quantized_weight_qmatmul_amd import qmv
        qmv.lib()
        run_kernel_workloads(torch.device("cuda:0"), int(sys.argv[2]), sys.argv[3])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        summarize_trace(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], " ".join(sys.argv[6:]))
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=10, help="rotated copies of the layer set")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample size (0 = skip)")
    ap.add_argument("--no-extra", action="store_true", help="skip the M=16 and launch-grouping extras")
    ap.add_argument("--probe-copy-mb", type=int, default=0,
                    help="after the steps, copy a buffer of this many MiB 5 times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of the path is described, not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_quantized_weight_qmatmul_amd import qmv
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    qmv.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    sets = build_layer_sets(args.copies, dev)
    nbytes = step_bytes()

    def grouped(s):
        for g in GROUPS:
            qmv.qmv_batch("q4_0", [s[n] for n in g])

    t = time_steps(grouped, sets, args.steps, args.warmup)
    ms_per_step = t / args.steps * 1e3
    value = nbytes * args.steps / t / 1e9

    # Every launch in the timed region is the batched M = 1 kernel, so its
    # average launch duration is the region's time over its launch count (the
    # short gaps between dependent launches are included).
    launches = args.steps * len(GROUPS)
    per_launch = nbytes / len(GROUPS)
    avg_launch = t / launches
    achieved = per_launch / avg_launch / 1e9
    traffic = read_traffic(per_launch)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_m1c (qmv_batch, M=1)", "launches_per_step": len(GROUPS),
                "avg_launch_us": round(avg_launch * 1e6, 3),
                "algorithmic_bytes_per_launch": round(per_launch)}

    if args.probe_copy_mb:
        src = torch.empty(args.probe_copy_mb * 2**20 // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # a plain streaming copy: reads and writes probe_copy_mb MiB
        torch.cuda.synchronize()
        del src, dst

    extra = {}
    # the streaming-read reference and the cold-single timing (a few seconds)
    ref = stream_read_reference(dev)
    extra["stream_read"] = ref
    floor = ref["layer_set_floor"]
    roofline["reference"] = {"stream_read_1GiB_GBps": ref["1GiB"]["GBps"],
                             "layer_set_floor_GBps": floor["GBps"],
                             "frac_of_floor": round(value / floor["GBps"], 4)}
    extra["cold_single"] = cold_single(dev, sets)
    if not args.no_extra:
        names = ("q", "k", "v", "o", "gate", "up", "down")
        t1 = time_steps(lambda s: qmv.qmv_batch("q4_0", [s[n] for n in names]), sets, args.steps, args.warmup)
        t7 = time_steps(lambda s: [qmv.qmv_q4_0(s[n][0], s[n][1], s[n][2]) for n in names], sets, args.steps,
                        args.warmup)
        extra["layer_set_one_launch_GBps"] = round(nbytes * args.steps / t1 / 1e9, 1)
        extra["layer_set_fused_qkv_gate_up_GBps"] = round(fused_layer_set_throughput(sets, args), 1)
        extra["layer_set_seven_launches_GBps"] = round(nbytes * args.steps / t7 / 1e9, 1)
        extra["q4_0_m1_2048x2048"] = dense_m1_throughput(dev, 0)
        extra["q8_0_m1"] = dense_m1_throughput(dev, 2)
        extra["m16"] = m16_throughput(dev)
        extra["m16_no_workspace"] = m16_throughput(dev, workspace=False)
        extra["m16_q8_0"] = m16_throughput(dev, "q8_0")
        extra["moe_t1"] = moe_throughput(dev, 1)
        extra["moe_t32"] = moe_throughput(dev, 32)
        # 1024 pairs, about 8 per expert: the matrix-core grouped kernel
        extra["moe_t128"] = moe_throughput(dev, 128)
        extra["moe_ffn_t1_fused"] = moe_throughput(dev, 1, mode="ffn_fused")
        extra["moe_ffn_t1_two_call"] = moe_throughput(dev, 1, mode="ffn_two_call")
        extra["moe_ffn_t32_two_call"] = moe_throughput(dev, 32, mode="ffn_two_call")
        extra["moe_ffn_t32_fused"] = moe_throughput(dev, 32, mode="ffn_fused")
        extra["lm_head_q6_k"] = lm_head_q6k_throughput(dev)
        extra["lm_head_q8_0"] = lm_head_q8_throughput(dev)
        extra["moe_q6_k_gate_up_t1"] = moe_q6k_gate_up_throughput(dev)
        extra["q5_k_b9_group"] = q5k_b9_throughput(dev)
        extra["prefill_m512"] = prefill_throughput(dev)
        extra["moe_affine4_t1"] = moe_affine4_throughput(dev)
    del sets
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "q4_0_m1_decode_layer_h4096", "M": 1, "hidden": 4096,
                   "projections": "q,k,v 4096->4096,1024,1024; o 4096->4096; gate,up 4096->14336; down 14336->4096",
                   "launches_per_step": "4 (qkv | o | gate+up | down)", "weight_bytes_per_step": nbytes,
                   "rotated_copies": args.copies, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
