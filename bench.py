#!/usr/bin/env python3
"""Benchmark of the routed int4 MoE FFN hot path on one MI355X.

Workload: one MoE layer decoding one token at page scale -- d_model 6144,
d_ff 2048, 256 routed experts + 1 shared, top-8 sigmoid routing, the whole
4.86 GB int4 table resident in HBM.  One step = the whole hot path for one
token: Q8_0 quantisation of x, sigmoid top-k routing, batch-union dispatch,
gate/up int4 x int8 GEMV with fused SwiGLU + Q8(h), down GEMV, weighted
combine, through one coli_moe_layer call (4 kernels: fused front, gate/up,
down, combine).  Steps cycle through a pool of 64 distinct seeded tokens
(their expert union is 2.2 GB), so the weights stream from HBM rather than
from the 256 MB Infinity Cache.  Steps are captured in HIP graphs (launch
overhead is then the device's, not Python's).

Prints one JSON line with the decode rate (tokens/s per MoE layer), the
roofline of the dominant kernel (gate/up GEMV) against 8 TB/s, and the
oracle timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# HBM bytes per launch of the decode gate/up kernel, from rocprofv3 FETCH_SIZE (x2.0) and
# WRITE_SIZE (x1.0) runs, each scale taken from a copy of known size
# (profiles/decode_gate_up_hbm_traffic.md); valid for the kernel as measured there.
GATE_UP_TRAFFIC_BYTES = 113_782_374
INT8_PEAK_TOPS = 5000.0   # dense int8 matrix-core peak of MI355X
F16_PEAK_TFLOPS = 2500.0  # dense f16 matrix-core peak of MI355X
# fp32 FMAs per second of the vector ALUs without packed instructions: 256 CUs x
# 64 lanes x 2.4 GHz (the 157.3 TFLOP/s vector peak counts packed FMAs, 128 per CU
# per clock, at 2 flops each)
VALU_FMA_PEAK_T = 256 * 64 * 2.4e9 / 1e12
METRIC = "MoE-layer decode tok/s + achieved HBM GB/s (int4 experts); prefill int8 TOPS"


HEAD_LAYER = 78   # the int8 speculative head sits after the 78 main layers


def build_table(w, coli, synth, torch, layer=0, bits=4):
    """Device table from device-generated seeded weights, quantised by the library
    (int4, or int8 for the speculative head)."""
    table = coli.ExpertTable(w.E, w.S, w.D, w.F, weight_bits=bits)
    F, D = w.F, w.D
    scratch = torch.empty(F * D, dtype=torch.float32, device="cuda")
    quant, qdt, per = {4: (coli.coli_quant_weight_q4, torch.uint8, 2),
                       8: (coli.coli_quant_weight_q8, torch.int8, 1),
                       2: (coli.coli_quant_weight_q2, torch.uint8, 4)}[bits]
    q = [torch.empty((F, D // per), dtype=qdt, device="cuda") for _ in range(2)]
    q.append(torch.empty((D, F // per), dtype=qdt, device="cuda"))
    s = [torch.empty(F, dtype=torch.float32, device="cuda") for _ in range(2)]
    s.append(torch.empty(D, dtype=torch.float32, device="cuda"))
    sp = torch.cuda.current_stream().cuda_stream
    for e in range(w.E + w.S):
        for m in range(3):
            rows, cols = synth.weight_shape(w, m)
            synth.weight_device(w, layer, e, m, scratch.data_ptr(), sp)
            quant(scratch[: rows * cols].view(rows, cols), q[m], s[m])
        coli.coli_table_set_expert(table, e, q[0], s[0], q[1], s[1], q[2], s[2])
    torch.cuda.synchronize()
    return table


class HipEvents:
    """hipEvent_t handles for the library's stage events (created and read here,
    since events recorded by the library are invisible to torch.cuda.Event)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


def expert_bytes(w, bits=4):
    gate_up = 2 * (w.F * w.D * bits // 8 + 4 * w.F)
    down = w.D * w.F * bits // 8 + 4 * w.D
    return gate_up, down


def cpu_baseline(w, synth, seconds):
    """The oracle (plain C, OpenMP over rows) on a bounded sample of the workload."""
    import oracle
    sample = list(range(4))
    x = synth.activations(w, len(sample))
    lg = synth.logits(w, len(sample))
    b = synth.router_bias(w)
    xq, xd = oracle.q8_quant(x)
    idx, wt = oracle.route(lg, b, w.k)
    experts = {}
    for e in sorted(set(idx.reshape(-1).tolist()) | {w.E}):   # setup, not timed
        experts[e] = oracle.Expert.quantize(*[synth.weight_host(w, 0, e, m) for m in range(3)])
    tokens = 0
    t0 = time.perf_counter()
    while True:
        for t in range(len(sample)):
            oracle.moe_layer(experts, w.E, w.S, xq[t:t + 1], xd[t:t + 1], idx[t:t + 1],
                             wt[t:t + 1])
            tokens += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": tokens / el, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(sample)} decode tokens of the same layer (their {len(experts)} "
                      f"experts generated and quantised untimed), cycled for {el:.1f} s "
                      f"({tokens} token-layers); quantise+route+MoE per token",
            "host": host_description(),
            "context": PAGES_CPU_CONTEXT}


# The pages' own CPU figures (context only; other machines, whole-model decode
# for the tok/s figures): jeff.news kernel section (int8 matmul on AVX2),
# discuss.pytorch.kr "colibri의 성능" table (cold decode on the 25 GB WSL2
# laptop), and the Apple M5 Max decode figure quoted there.
PAGES_CPU_CONTEXT = {
    "int8_matmul_avx2_gflops": 119,
    "cold_decode_tok_s_wsl2_laptop": [0.05, 0.1],
    "decode_tok_s_m5_max": 1.06,
}


def host_description():
    """nproc, the CPU model and the RAM of the host the oracle runs on."""
    model, ram_kb = "unknown", 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    ram_kb = int(line.split()[1])
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model, "ram_gib": round(ram_kb / 2**20, 1)}


def cpu_full(synth, seconds=5.0):
    """The oracle on every workload at all threads and at one thread (a
    reported baseline; expert generation and quantisation untimed).  Decode
    and verify tokens are cycled for `seconds`; the 2048-token prefill runs in
    full at all threads and on its first 64 tokens at one thread; the 40-layer
    stack runs 8 tokens (all threads) or 1 token (one thread) through all 40
    layers.  Sampled rates are extrapolated to the whole workload and say so."""
    import oracle
    res = {"host": host_description(), "context": PAGES_CPU_CONTEXT, "runs": []}
    all_threads = oracle.num_threads()

    def experts_for(w, layer, idx):
        need = sorted(set(int(e) for e in idx.reshape(-1)) | {w.E})
        return {e: oracle.Expert.quantize(*[synth.weight_host(w, layer, e, m) for m in range(3)])
                for e in need}

    def layer_tokens(w, T, seed=0):
        x, lg, b = synth.activations(w, T, seed), synth.logits(w, T, seed), synth.router_bias(w)
        xq, xd = oracle.q8_quant(x)
        idx, wt = oracle.route(lg, b, w.k)
        return xq, xd, idx, wt

    def note(r):
        res["runs"].append(r)
        print(f"cpu_full: {r['workload']}, {r['threads']} threads: {r['seconds']} s", file=sys.stderr,
              flush=True)

    expert_bytes_w = sum(expert_bytes(synth.WORKLOADS[1]))
    macs_per_pair = 3 * synth.WORKLOADS[1].D * synth.WORKLOADS[1].F
    for threads in (all_threads, 1):
        oracle.set_threads(threads)
        # decode (1 token per layer call) and verify (4 tokens in one call)
        for wl, T in ((1, 1), (2, 4)):
            w = synth.WORKLOADS[wl]
            xq, xd, idx, wt = layer_tokens(w, 4)
            ex = experts_for(w, 0, idx)
            n, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < seconds:
                for t0k in range(0, 4, T):
                    oracle.moe_layer(ex, w.E, w.S, xq[t0k:t0k + T], xd[t0k:t0k + T],
                                     idx[t0k:t0k + T], wt[t0k:t0k + T])
                    n += T
            el = time.perf_counter() - t0
            note({"workload": w.name, "threads": threads, "tokens": n,
                                "seconds": round(el, 2), "tok_s": round(n / el, 2),
                                "int_ops_per_s": round(n * (w.k + w.S) * 2 * macs_per_pair / el, 1),
                                "weight_gb_s": round(n * (w.k + w.S) * expert_bytes_w / el / 1e9, 3)})
        # prefill: 2048 tokens (first 64 at one thread)
        w = synth.WORKLOADS[3]
        xq, xd, idx, wt = layer_tokens(w, w.T)
        Tn = w.T if threads > 1 else 64
        ex = experts_for(w, 0, idx[:Tn])
        t0 = time.perf_counter()
        oracle.moe_layer(ex, w.E, w.S, xq[:Tn], xd[:Tn], idx[:Tn], wt[:Tn])
        el = time.perf_counter() - t0
        del ex
        r = {"workload": w.name, "threads": threads, "tokens": Tn, "seconds": round(el, 2),
             "tok_s": round(Tn / el, 2),
             "int_ops_per_s": round(Tn * (w.k + w.S) * 2 * macs_per_pair / el, 1)}
        if Tn < w.T:
            r["extrapolated_ms_per_pass"] = round(el / Tn * w.T * 1000, 1)
            r["note"] = f"first {Tn} of {w.T} tokens timed; the pass time is extrapolated"
        else:
            r["ms_per_pass"] = round(el * 1000, 1)
        note(r)
        # deep stack: 8 tokens (1 at one thread) through all 40 layers
        w = synth.WORKLOADS[4]
        n = 8 if threads > 1 else 1
        h = synth.hidden0(w, n)
        el = 0.0
        for layer in range(w.layers):
            idx, wt = oracle.route(synth.logits(w, n, 0, layer), synth.router_bias(w, layer), w.k)
            ex = experts_for(w, layer, idx)   # untimed
            t0 = time.perf_counter()
            xh, _ = oracle.rmsnorm(h, 1e-6)
            xq, xd = oracle.q8_quant(xh)
            h, _ = oracle.moe_layer(ex, w.E, w.S, xq, xd, idx, wt, out=h, accumulate=True)
            el += time.perf_counter() - t0
            del ex
            if layer % 8 == 7:
                print(f"cpu_full: deep stack, {threads} threads, layer {layer + 1}", file=sys.stderr,
                      flush=True)
        note({"workload": w.name, "threads": threads, "tokens": n,
                            "seconds": round(el, 2), "ms_per_token": round(el / n * 1000, 1),
                            "tok_s": round(n / el, 3),
                            "extrapolated_s_for_256_tokens": round(el / n * w.steps, 1),
                            "note": f"{n} of {w.steps} tokens through all {w.layers} layers "
                                    f"timed; the 256-token time is extrapolated"})
    oracle.set_threads(all_threads)
    return res


def prefill_leg(table, coli, synth, torch, hev, steps, warmup, bias_free=False, T=None):
    """2048 tokens (or T) through the same layer in one coli_moe_layer call (the
    grouped matrix-core path): pass time, int8-equivalent TOPS of the expert
    matmuls, the per-stage split measured with HIP events, and the roofline of
    the two matrix kernels against the VALU roof of the exact Q8_0 rescale."""
    w = synth.WORKLOADS[3]
    T = T or w.T
    x = torch.from_numpy(synth.activations(w, T)).cuda()
    lg = torch.from_numpy(synth.logits(w, T)).cuda()
    b = torch.from_numpy(synth.router_bias(w)).cuda()
    if bias_free:
        b.zero_()
    y = torch.empty((T, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                     device="cuda")
    tr = {"counts": torch.empty(w.E + w.S, dtype=torch.int32, device="cuda")}

    def once(events=None, trace=None):
        coli.coli_moe_layer(table, x, lg, b, w.k, y, ws, events=events, trace=trace)

    once(trace=tr)
    torch.cuda.synchronize()
    if coli.coli_moe_status(ws) != coli.COLI_OK:
        raise RuntimeError("device-side index check failed (prefill)")
    counts = tr["counts"].cpu().numpy()[: w.E]
    for _ in range(warmup):
        once()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        once()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    names = ("begin", "gate_up", "down", "combine", "end")
    evs = [{k: hev.create() for k in names} for _ in range(3)]
    for e in evs:
        once(events=e)
    torch.cuda.synchronize()

    def avg(a, c):
        return sum(hev.elapsed_ms(e[a], e[c]) for e in evs) / len(evs)

    gu_ms, dn_ms = avg("gate_up", "down"), avg("down", "combine")
    fr_ms, cb_ms = avg("begin", "gate_up"), avg("combine", "end")
    pairs = T * (w.k + w.S)
    ops_gu = 2.0 * pairs * 2 * w.F * w.D
    ops_dn = 2.0 * pairs * w.D * w.F
    tops = (ops_gu + ops_dn) / (ms * 1e-3) / 1e12
    used = int((counts > 0).sum())
    # the exact Q8_0 path costs one fp32 fmaf per (row, pair, 32-column block)
    rescale = pairs * (2 * w.F * (w.D // 32) + w.D * (w.F // 32))
    mm_ms = gu_ms + dn_ms
    fma_rate = rescale / (mm_ms * 1e-3) / 1e12
    mm_tops = (ops_gu + ops_dn) / (mm_ms * 1e-3) / 1e12
    name = w.name if T == w.T else w.name.replace(f"t{w.T}", f"t{T}")
    return {
        "workload": name + (" (router bias 0)" if bias_free else ""),
        "tokens": T, "experts_used": used + w.S, "max_tokens_per_expert": int(counts.max()),
        "ms_per_pass": round(ms, 4), "tok_s": round(T / (ms * 1e-3), 1),
        "int8_tops": round(tops, 1), "int8_peak_tops": INT8_PEAK_TOPS,
        "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
        "kernels_ms": {"front": round(fr_ms, 4), "gate_up": round(gu_ms, 4),
                       "down": round(dn_ms, 4), "combine": round(cb_ms, 4)},
        "gate_up_tops": round(ops_gu / (gu_ms * 1e-3) / 1e12, 1),
        "down_tops": round(ops_dn / (dn_ms * 1e-3) / 1e12, 1),
        "weight_gbps": round((used + w.S) * sum(expert_bytes(w)) / (ms * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "mfma_ffn_kernel (gate/up + down)", "bound": "alu",
                     "achieved": round(fma_rate, 2), "peak": VALU_FMA_PEAK_T,
                     "unit": "T fp32 fmaf/s (exact Q8_0 rescale, unpacked)",
                     "frac": round(fma_rate / VALU_FMA_PEAK_T, 4),
                     "matrix_tops": round(mm_tops, 1),
                     "frac_of_f16_mfma_peak": round(mm_tops / F16_PEAK_TFLOPS, 4),
                     "frac_of_int8_mfma_peak": round(mm_tops / INT8_PEAK_TOPS, 4),
                     "rescale_fmas": rescale},
    }


def decode_cold_leg(step, pool, torch, layer_bytes, tokens=32, reps=4, flush_bytes=512 << 20):
    """Decode steps with a cold Infinity Cache.  Before each step a 512 MiB
    buffer is written, so no expert's rows are left in the 256 MB Infinity
    Cache (the shared expert, which every warm step re-reads 170 MB after its
    last use, included).  Three HIP graphs of `tokens` steps are replayed back
    to back, as the headline steps are: writes + steps, the writes alone, and
    the steps alone; the cold step time is (writes + steps - writes) / tokens,
    so the writes stay outside it."""
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")

    def graph(with_flush, with_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(tokens):
                if with_flush:
                    flush.fill_(float(j + 1))   # a fill kernel (nonzero value)
                if with_steps:
                    step(j % pool)
        return g

    gs = {"cold": graph(True, True), "flush": graph(True, False), "warm": graph(False, True)}

    def timed(g):
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t = {k: timed(g) for k, g in gs.items()}
    cold = (t["cold"] - t["flush"]) / tokens
    warm = t["warm"] / tokens
    del gs, flush
    return {"tokens": tokens, "flush_bytes": flush_bytes,
            "cold_ms_per_step": round(cold, 5), "cold_tok_s": round(1000.0 / cold, 1),
            "cold_weight_gbps": round(layer_bytes / (cold * 1e-3) / 1e9, 1),
            "warm_ms_per_step": round(warm, 5), "flush_ms": round(t["flush"] / tokens, 4)}


def head_leg(coli, synth, torch, hev):
    """The int8 speculative head: its own 6144 x 2048, 256 + 1 expert layer with
    int8 weights (9.7 GB), at decode (1 token per pass) and in the batched
    verify pass (4 tokens per pass)."""
    table = build_table(synth.WORKLOADS[2], coli, synth, torch, layer=HEAD_LAYER, bits=8)
    res = {"workload": "int8 head d6144 f2048 e256+1 top8", "table_bytes": table.bytes}
    res.update(batch_leg(table, 8, (1, 2), coli, synth, torch, hev))
    del table
    torch.cuda.empty_cache()
    return res


def int2_leg(coli, synth, torch, hev):
    """An int2 layer (2-bit weights, 2.43 GB table) at decode (1 token per
    pass) and in the verify pass (4 tokens)."""
    table = build_table(synth.WORKLOADS[2], coli, synth, torch, layer=2, bits=2)
    res = {"workload": "int2 layer d6144 f2048 e256+1 top8", "table_bytes": table.bytes}
    res.update(batch_leg(table, 2, (1, 2), coli, synth, torch, hev))
    del table
    torch.cuda.empty_cache()
    return res


def batch_leg(table, bits, wids, coli, synth, torch, hev, replays=4, pool=64):
    """Passes of T tokens (T of each workload in wids) through coli_moe_layer
    over a pool of 64 seeded passes, graph-captured; weight GB/s counts each
    pass's expert union once; gate/up and down are timed with HIP events."""
    gu_bytes, dn_bytes = expert_bytes(synth.WORKLOADS[wids[0]], bits=bits)
    res = {}
    for wid in wids:
        w = synth.WORKLOADS[wid]
        T, P = w.T, pool
        x = torch.from_numpy(synth.activations(w, P * T, 3000)).cuda()
        lg = torch.from_numpy(synth.logits(w, P * T, 3000)).cuda()
        b = torch.from_numpy(synth.router_bias(w)).cuda()
        y = torch.empty((P * T, w.D), dtype=torch.float32, device="cuda")
        ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                         device="cuda")
        idx = torch.empty((P * T, w.k), dtype=torch.int32, device="cuda")
        wt = torch.empty((P * T, w.k), dtype=torch.float32, device="cuda")
        coli.coli_route_topk(lg, b, w.k, idx, wt)
        ih = idx.cpu().numpy()
        union = [len(set(ih[j * T:(j + 1) * T].reshape(-1).tolist())) + w.S for j in range(P)]

        def step(j, events=None):
            sl = slice(j * T, (j + 1) * T)
            coli.coli_moe_layer(table, x[sl], lg[sl], b, w.k, y[sl], ws, events=events)

        for j in range(P):
            step(j)
        torch.cuda.synchronize()
        if coli.coli_moe_status(ws) != coli.COLI_OK:
            raise RuntimeError("device-side index check failed (int8 head)")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(P):
                step(j)
        g.replay()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(replays):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / (replays * P)
        evs = [{k: hev.create() for k in ("begin", "gate_up", "down", "combine", "end")}
               for _ in range(P)]
        for _ in range(2):
            g.replay()
        for j in range(P):
            step(j, evs[j])
        torch.cuda.synchronize()
        gu_ms = sum(hev.elapsed_ms(e["gate_up"], e["down"]) for e in evs) / P
        dn_ms = sum(hev.elapsed_ms(e["down"], e["combine"]) for e in evs) / P
        u = sum(union) / P
        res[f"t{T}"] = {
            "tokens_per_pass": T, "passes": replays * P, "ms_per_pass": round(ms, 5),
            "tok_s": round(T / (ms * 1e-3), 1), "experts_per_pass": round(u, 2),
            "weight_gbps": round(u * (gu_bytes + dn_bytes) / (ms * 1e-3) / 1e9, 1),
            "gate_up_ms": round(gu_ms, 5), "down_ms": round(dn_ms, 5),
            "gate_up_gbps": round(u * gu_bytes / (gu_ms * 1e-3) / 1e9, 1),
            "down_gbps": round(u * dn_bytes / (dn_ms * 1e-3) / 1e9, 1),
        }
    return res


def tier_leg(coli, synth, torch, layers=4, slots=64, warm=32, timed=32):
    """Decode through `layers` page-shape layers whose experts live only in
    pinned host memory (4.86 GB per layer), each with an HBM tier of `slots`
    experts: Zipf(1.1) routing, the pre-norm residual stack of the deep-decode
    workload.  Per layer and token: RMSNorm+Q8, routing, tier plan, fetch of
    the misses over the host link, forward through the tier.  Three runs of
    `warm` + `timed` tokens: LRU from empty tiers; tiers re-initialised with
    each layer's most used experts of the first run pinned (half the slots);
    the same plus next-layer prefetch on a copy stream (prediction = the next
    layer's actual routing: an upper bound of what readahead can hide)."""
    from dataclasses import replace
    w = replace(synth.WORKLOADS[4], layers=layers)
    stores, tiers = [], []
    for l in range(layers):
        t = build_table(w, coli, synth, torch, layer=l)
        stores.append(t.to_host_store())
        del t
        torch.cuda.empty_cache()
        tiers.append(coli.ExpertTier(w.E, w.S, w.D, w.F, slots))
    N = warm + timed
    lg = [torch.from_numpy(synth.logits(w, N, 0, l)).cuda() for l in range(layers)]
    zero = torch.zeros(w.E, dtype=torch.float32, device="cuda")
    h0 = torch.from_numpy(synth.hidden0(w, N)).cuda()
    xq = torch.empty((1, w.D), dtype=torch.int8, device="cuda")
    xd = torch.empty((1, w.D // 32), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((1, w.k), dtype=torch.float32, device="cuda")
    pidx = torch.empty((1, w.k), dtype=torch.int32, device="cuda")
    pwt = torch.empty((1, w.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(coli.coli_moe_workspace_bytes(tiers[0], 1, w.k), dtype=torch.uint8,
                     device="cuda")
    main = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    expert_bytes_all = sum(expert_bytes(w))

    def run(prefetch):
        h = h0.clone()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        for i in range(N):
            if i == warm:
                torch.cuda.synchronize()
                c0 = [t.st["counters"].cpu().numpy().copy() for t in tiers]
                t0.record()
            hi = h[i:i + 1]
            for l in range(layers):
                if prefetch and l + 1 < layers:
                    started = torch.cuda.Event()
                    started.record(main)
                    copy.wait_event(started)     # layer l+1 of the last token is done
                    with torch.cuda.stream(copy):
                        coli.coli_route_topk(lg[l + 1][i:i + 1], zero, w.k, pidx, pwt)
                        tiers[l + 1].plan(pidx, count_usage=False)
                        tiers[l + 1].fetch(stores[l + 1])
                    ready = torch.cuda.Event()
                    ready.record(copy)
                coli.coli_rmsnorm_q8(hi, 1e-6, xq, xd)
                coli.coli_route_topk(lg[l][i:i + 1], zero, w.k, idx, wt)
                if prefetch and l > 0:
                    main.wait_event(ready_prev)
                tiers[l].plan(idx)
                tiers[l].fetch(stores[l])
                coli.coli_moe_forward(tiers[l], xq, xd, idx, wt, hi, ws, accumulate=True)
                if prefetch and l + 1 < layers:
                    ready_prev = ready
        t1.record()
        torch.cuda.synchronize()
        if coli.coli_moe_status(ws) != coli.COLI_OK or any(t.status() for t in tiers):
            raise RuntimeError("tier leg: device-side check failed")
        c1 = [t.st["counters"].cpu().numpy() for t in tiers]
        hits = sum(int(b[1] - a[1]) for a, b in zip(c0, c1))
        loads = sum(int(b[2] - a[2]) for a, b in zip(c0, c1))
        ms = t0.elapsed_time(t1) / timed
        return {"ms_per_token": round(ms, 3), "tok_s": round(1000.0 / ms, 1),
                "hit_rate": round(hits / max(1, hits + loads), 4),
                "loads_per_token_layer": round(loads / (timed * layers), 3),
                "host_read_gbps": round(loads * expert_bytes_all / (timed * ms * 1e-3) / 1e9, 1)}

    res = {"workload": f"Zipf(1.1) decode, {layers} layers d6144 f2048 e256+1 top8, experts in "
                       f"pinned host memory, {slots} HBM slots per layer",
           "tier_bytes_per_layer": tiers[0].bytes, "store_bytes_per_layer": stores[0].bytes}
    for t, st in zip(tiers, stores):
        t.init(st)
    res["lru"] = run(False)
    pins = [coli.coli_tier_rank(t.st["usage"].cpu().numpy()[: w.E], slots // 2) for t in tiers]
    for t, st, p in zip(tiers, stores, pins):
        t.init(st, p)
    res["learned_pins"] = run(False)
    for t, st, p in zip(tiers, stores, pins):
        t.init(st, p)
    res["learned_pins_prefetch"] = run(True)
    # host-link read rate of the fetch kernel: re-initialising a tier with
    # slots - 1 pins fetches `slots` experts in one launch
    many = list(range(slots - 1))
    for _ in range(2):
        tiers[0].init(stores[0], many)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    tiers[0].init(stores[0], many)
    e1.record()
    torch.cuda.synchronize()
    fms = e0.elapsed_time(e1)
    res["fetch_gbps"] = round(slots * expert_bytes_all / (fms * 1e-3) / 1e9, 1)
    res["fetch_ms_per_expert"] = round(fms / slots, 4)
    del tiers, stores
    torch.cuda.empty_cache()
    return res


def deep_leg(coli, synth, torch, tokens=48, warm=16):
    """The deep decode stack: 40 page-shape layers (194 GB of int4 tables, all
    resident in HBM), Zipf(1.1)-skewed routing per layer, each layer a pre-norm
    residual block h <- h + MoE(RMSNorm(h)) through coli_moe_block (4 kernels:
    RMSNorm+Q8, routing and dispatch fused; gate/up; down; combine into h).
    Tokens run one after another, each through all 40 layers, captured in HIP
    graphs.  A token streams 40 x 9 experts = 6.81 GB of weights, so nothing
    is reused from the 256 MB Infinity Cache between a layer's visits."""
    w = synth.WORKLOADS[4]
    L = w.layers
    tables = [build_table(w, coli, synth, torch, layer=l) for l in range(L)]
    N = warm + tokens
    lg = [torch.from_numpy(synth.logits(w, N, 0, l)).cuda() for l in range(L)]
    bias = [torch.from_numpy(synth.router_bias(w, l)).cuda() for l in range(L)]
    h = torch.from_numpy(synth.hidden0(w, N)).cuda()
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(tables[0], 1, w.k), dtype=torch.uint8,
                     device="cuda")

    def run(t0, t1):
        for i in range(t0, t1):
            for l in range(L):
                coli.coli_moe_block(tables[l], h[i:i + 1], lg[l][i:i + 1], bias[l], w.k, ws)

    g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        run(0, warm)
    with torch.cuda.graph(g_timed):
        run(warm, N)
    g_warm.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    if coli.coli_moe_status(ws) != coli.COLI_OK or not torch.isfinite(h).all():
        raise RuntimeError("deep leg: device-side check failed")
    ms = e0.elapsed_time(e1) / tokens
    per_token = L * (w.k + w.S) * sum(expert_bytes(w))
    res = {"workload": w.name + ", 40 x 4.86 GB tables in HBM, coli_moe_block per layer",
           "tokens_timed": tokens, "ms_per_token": round(ms, 4),
           "us_per_layer": round(1000 * ms / L, 2), "tok_s": round(1000.0 / ms, 1),
           "weight_bytes_per_token": per_token,
           "weight_gbps": round(per_token / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(per_token / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del g_warm, g_timed, tables
    torch.cuda.empty_cache()
    return res


def paths_leg(table, coli, synth, torch, reps=8):
    """The per-shape path choice, measured: the forward of T tokens (page
    shape, router bias N(0, 0.1)) on the GEMV and on the grouped path; the
    automatic choice switches to the grouped path at COLI_GROUPED_MIN_TOKENS."""
    w = synth.WORKLOADS[3]
    b = torch.from_numpy(synth.router_bias(w)).cuda()
    rows = []
    for T in (4, 5, 6, 7, 8, 9, 10, 12, 14, 16, 24, 32, 64, 128, 512):
        x = torch.from_numpy(synth.activations(w, T, 4000)).cuda()
        lg = torch.from_numpy(synth.logits(w, T, 4000)).cuda()
        xq = torch.empty((T, w.D), dtype=torch.int8, device="cuda")
        xd = torch.empty((T, w.D // 32), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
        coli.coli_quant_act_q8(x, xq, xd)
        coli.coli_route_topk(lg, b, w.k, idx, wt)
        y = torch.empty((T, w.D), dtype=torch.float32, device="cuda")
        ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                         device="cuda")
        row = {"tokens": T, "auto": "grouped" if coli.coli_moe_path(table, T, w.k) ==
               coli.COLI_PATH_GROUPED else "gemv"}
        for name, p in (("gemv", coli.COLI_PATH_GEMV), ("grouped", coli.COLI_PATH_GROUPED)):
            for _ in range(2):
                coli.coli_moe_forward_path(table, xq, xd, idx, wt, y, ws, p)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                coli.coli_moe_forward_path(table, xq, xd, idx, wt, y, ws, p)
            e1.record()
            torch.cuda.synchronize()
            row[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
        rows.append(row)
    return rows


def router_leg(coli, synth, torch, steps=50):
    """The router projection (F32 weights [256][6144], fp64 sum) for 1 and 2048
    tokens: `steps` calls captured in a HIP graph, one replay timed (so the
    one-token figure is the kernel and its dispatch, not the host's launch)."""
    w = synth.WORKLOADS[1]
    wr = torch.from_numpy(synth.router_weights(w)).cuda()
    res = {}
    for T in (1, 2048):
        x = torch.from_numpy(synth.activations(w, T, 900)).cuda()
        out = torch.empty((T, w.E), dtype=torch.float32, device="cuda")
        for _ in range(3):
            coli.coli_router_logits(x, wr, out)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                coli.coli_router_logits(x, wr, out)
        g.replay()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        del g
        us = t0.elapsed_time(t1) / steps * 1e3
        nbytes = 4 * (w.E * w.D + T * w.D + T * w.E)
        res[f"t{T}_us"] = round(us, 2)
        res[f"t{T}_gbps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        res[f"t{T}_fp64_tflops"] = round(2.0 * T * w.E * w.D / (us * 1e-6) / 1e12, 2)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--pool", type=int, default=64, help="distinct tokens cycled by the steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle on every workload at all threads and one thread "
                         "(several minutes; reported under cpu_full)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache decode leg")
    ap.add_argument("--eager", action="store_true", help="launch steps directly, no HIP graph")
    ap.add_argument("--prefill-steps", type=int, default=20,
                    help="timed 2048-token passes of the prefill leg (0: skip it)")
    ap.add_argument("--no-head", action="store_true", help="skip the int8 head and int2 legs")
    ap.add_argument("--no-tier", action="store_true", help="skip the expert-tier leg")
    ap.add_argument("--no-paths", action="store_true", help="skip the path-choice leg")
    ap.add_argument("--no-deep", action="store_true",
                    help="skip the 40-layer deep decode stack leg (194 GB of tables)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 8 device-to-device copies of this many bytes (the known-size "
                         "kernel that scales the HBM byte counters under rocprofv3 --pmc)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the hot path runs on one GPU's share and the "
              "library has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.rand(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "copies": 8}), flush=True)
        return
    import synth
    import int4_routed_expert_sigmoid_amd as coli

    w = synth.WORKLOADS[1]
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    table = build_table(w, coli, synth, torch)
    P = args.pool
    x_pool = torch.from_numpy(synth.activations(w, P)).cuda()
    lg_pool = torch.from_numpy(synth.logits(w, P)).cuda()
    bias = torch.from_numpy(synth.router_bias(w)).cuda()
    y_pool = torch.zeros((P, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, 1, w.k), dtype=torch.uint8,
                     device="cuda")

    def step(j, events=None):
        """One token through the layer: f32 x and router logits in, f32 y out."""
        coli.coli_moe_layer(table, x_pool[j:j + 1], lg_pool[j:j + 1], bias, w.k,
                            y_pool[j:j + 1], ws, events=events)

    for j in range(P):                               # setup: one eager pass over the pool
        step(j)
    torch.cuda.synchronize()
    if coli.coli_moe_status(ws) != coli.COLI_OK:
        raise RuntimeError("device-side index check failed")

    def capture(nsteps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(nsteps):
                step(j % P)
        return g

    def run(n, graphs):
        """n steps: full-pool graph replays plus one remainder graph."""
        full, rem = divmod(n, P)
        for _ in range(full):
            graphs[P].replay()
        if rem:
            graphs[rem].replay()

    K, W = args.steps, args.warmup
    graphs = None
    if not args.eager:
        graphs = {n: capture(n) for n in {P, K % P, W % P} - {0}}
    setup_s = time.perf_counter() - t_setup

    # warm-up: W untimed steps
    if graphs:
        run(W, graphs)
    else:
        for i in range(W):
            step(i % P)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    if graphs:
        run(K, graphs)
    else:
        for i in range(K):
            step(i % P)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / K

    # Dominant-kernel timing with HIP events on the forward's stream: one pass
    # of the pool through the profiled forward, enqueued behind a few graph
    # replays so that every event and kernel is already queued when the GPU
    # reaches it.  The library attaches the gate_up / down events to the
    # gate/up kernel's own dispatch (start and end of its execution) and the
    # combine event to the end of the down kernel, so gate_up is the kernel's
    # duration; front, down and combine each include one dispatch gap.
    hev = HipEvents()
    ev_names = ("begin", "gate_up", "down", "combine", "end")
    prof = [{k: hev.create() for k in ev_names} for _ in range(P)]
    if graphs:
        for _ in range(4):
            graphs[P].replay()
    for j in range(P):
        step(j, prof[j])
    torch.cuda.synchronize()
    gu = [hev.elapsed_ms(e["gate_up"], e["down"]) for e in prof]
    dn = [hev.elapsed_ms(e["down"], e["combine"]) for e in prof]
    fr = [hev.elapsed_ms(e["begin"], e["gate_up"]) for e in prof]
    cb = [hev.elapsed_ms(e["combine"], e["end"]) for e in prof]
    gu_ms, dn_ms = sum(gu) / len(gu), sum(dn) / len(dn)
    fr_ms, cb_ms = sum(fr) / len(fr), sum(cb) / len(cb)
    gu_bytes, dn_bytes = expert_bytes(w)
    active = w.k + w.S
    # algorithmic bytes of one gate/up launch: 9 experts' gate+up nibbles and row scales,
    # the token's Q8 block (x, scales, block sums) and the Q8(h) it writes
    gu_alg = active * gu_bytes + (w.D + 4 * w.D // 32 * 2) + active * (w.F + 8 * w.F // 32)
    achieved = gu_alg / (gu_ms * 1e-3) / 1e9
    layer_bytes = active * (gu_bytes + dn_bytes)
    tok_s = 1000.0 / ms_per_step

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xint8 (int32 dot, fp32 rescale)",
        "data": "synthetic (seeded N(0,0.02) weights quantised on device, N(0,1) tokens/logits, "
                "N(0,0.1) bias)",
        "config": {"workload": w.name, "d_model": w.D, "d_ff": w.F, "experts": w.E,
                   "shared": w.S, "top_k": w.k, "tokens_per_step": 1, "token_pool": P,
                   "table_bytes": table.bytes,
                   "launch": "eager" if args.eager else "hipgraph"},
        "weight_gbps_per_step": round(layer_bytes * tok_s / 1e9, 1),
        "kernels_ms": {"front": round(fr_ms, 5), "gate_up": round(gu_ms, 5),
                       "down": round(dn_ms, 5), "combine": round(cb_ms, 5)},
        "down_gbps": round(active * dn_bytes / (dn_ms * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "gate_up_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": GATE_UP_TRAFFIC_BYTES,
                     "algorithmic_bytes": gu_alg},
        "wall_s": round(wall, 3),
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cold:
        out["decode_cold"] = decode_cold_leg(step, P, torch, layer_bytes)
    if args.prefill_steps > 0:
        out["prefill"] = [prefill_leg(table, coli, synth, torch, hev, args.prefill_steps, 3),
                          prefill_leg(table, coli, synth, torch, hev, args.prefill_steps, 3,
                                      bias_free=True)]
        # a larger pass (about 288 tokens per used expert), labelled: the
        # kernels' matrix-core ceiling with fewer partial work items
        big = prefill_leg(table, coli, synth, torch, hev, max(2, args.prefill_steps // 4), 2,
                          T=8192)
        big["label"] = "8192-token sweep point (not a configured workload)"
        out["prefill"].append(big)
    if not args.no_paths:
        out["paths"] = paths_leg(table, coli, synth, torch)
    verify = synth.WORKLOADS[2]
    out["verify"] = {"workload": verify.name, **batch_leg(table, 4, (2,), coli, synth, torch, hev)}
    out["router_logits"] = router_leg(coli, synth, torch)
    if not args.no_head:
        out["int8_head"] = head_leg(coli, synth, torch, hev)
    if not args.no_head:
        out["int2"] = int2_leg(coli, synth, torch, hev)
    if not args.no_tier:
        out["tier"] = tier_leg(coli, synth, torch)
    if not args.no_deep:
        out["deep"] = deep_leg(coli, synth, torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, synth, args.cpu_seconds)
    if args.cpu_full:
        out["cpu_full"] = cpu_full(synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
