#!/usr/bin/env python3
"""Decode-step benchmark of hash-scored top-k sparse attention on one MI355X.

One step = one decode step of one attention layer for the whole batch and
all heads: query soft assignment (or query codes), the score scan over every
cached key, exact top-k per kv head, and exact attention over the gathered
rows.  The prefill hashing is timed separately.

Inputs are resident in HBM before timing.  Each timed step reads a different
copy of the key metadata and K/V (``--rotate`` copies, enough to exceed twice
the 256 MB Infinity Cache), so repeated steps cannot be served from cache.
Exactly ``--steps`` steps are timed back to back: replays of captured graphs
of up to 1024 consecutive steps between two events (``--no-graph`` times
eager launches instead).  The per-step latency percentiles come from a
separate pass that launches each step alone (one-step graph replays with an
event between steps).

Prints one JSON line: decode tokens/s (= batch / step time), the roofline of
the dominant kernel (the step's own filtering scan: the metadata bytes of
every key / its event-timed duration in the step's filter stage), the whole
step's fraction of the HBM roofline, and the CPU oracle's rate on the host
(the whole step over every slab, in single-threaded processes over the
host's CPUs).
Beside them: the prefill hashing, the decode-time append, the step with a
cumulative-mass budget instead of a fixed k, the step with two-level chunk
routing, and dense attention over every cached key (for the sparse/dense
ratio).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak (prefill projection)
MALL_BYTES = 256 * 2 ** 20
METRIC = "decode tokens/s and % of HBM roofline for hash score+top-k+sparse attn"
MASS_P = 0.9  # target of the cumulative-mass variant of the step
ROUTE_OVERSAMPLE = 4  # chunks kept by the routed step, per 64 selected keys


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="longctx_softlsh_b1_n128k")
    ap.add_argument("--rotate", type=int, default=0, help="input copies (0 = auto)")
    ap.add_argument("--kernel-iters", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-prefix leg")
    ap.add_argument("--core-only", action="store_true",
                    help="time the step and the roofline kernel only (no variant legs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replays of a captured graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (HBM counter scale)")
    return ap.parse_args()


def capture(fn):
    """Captures the launches fn makes on the current stream into a graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager pass on a side stream before capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def spin_cycles_per_ms(stream):
    """Cycles of torch's spin kernel per millisecond on this GPU."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cyc = 2_000_000
    torch.cuda._sleep(1000)
    e0.record(stream)
    torch.cuda._sleep(cyc)
    e1.record(stream)
    torch.cuda.synchronize()
    return cyc / max(e0.elapsed_time(e1), 1e-3)


def scan_span_of(w, dev):
    """Keys per chunk of the step's filtering scan (as the library picks it:
    chunks are lengthened when the threshold workgroups would add a round of
    resident workgroups, two per compute unit)."""
    import torch
    chunk, cap = 2048, 2560
    BH, N = w.B * w.Hkv, w.N
    R0 = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    nch0 = -(-N // chunk)
    r_chunks, r_all = -(-BH * nch0 // R0), -(-BH * (nch0 + 1) // R0)
    if r_all == r_chunks:
        return chunk
    nch = r_chunks * R0 // BH - 1
    if nch < 1:
        return chunk
    span = (-(-N // nch) + 63) // 64 * 64
    return span if span <= cap else chunk


def alg_bytes(w, lens, ks):
    """Algorithmic HBM bytes of one step: metadata of every key, the k gathered
    K/V rows per kv head, q in and out/lse out."""
    e = 4 if w.kv_dtype == "f32" else 2
    if w.scheme == "softlsh":
        m = w.L + (2 if w.norm_dtype == "f16" else 4)
    else:
        m = w.code_bits // 8
    meta = sum(int(n) for n in lens) * w.Hkv * m
    gathered = sum(int(k) for k in ks) * w.Hkv * 2 * w.d * e
    qo = w.B * w.Hq * w.d * (e + 4) + w.B * w.Hq * 4
    return meta, gathered, qo


def traffic_record(kernel: str, workload: str, src: str):
    """Measured HBM bytes per launch from a committed counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != sha:
        return None
    try:
        return float(vals["fetch_bytes_per_launch"]) + float(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


CPU_WORKERS_MAX = 16  # the host share one GPU machine gives a run


def _cpu_worker(wname, slabs, conn):
    """One process of the CPU baseline: the float64 oracle's decode step on
    its (b, kv head) slabs, one BLAS thread.  Started before the parent
    touches the GPU; it generates its slabs and their prefill metadata when
    told to (untimed), then times its share of each step on request."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    sys.path.insert(0, ROOT)
    import numpy as np
    import oracle as O
    import workloads as WL
    w = WL.WORKLOADS[wname]
    lens, ks = w.seq_lens(), w.k_per_seq()
    prepared = []
    while True:
        msg = conn.recv()
        if msg == "prepare":
            for (b, h) in slabs:
                n = int(lens[b])
                sl = WL.make_slab(w, b, h, n)
                q64 = WL.storage_to_f64(sl["q"], w.kv_dtype)
                K64 = WL.storage_to_f64(sl["K"], w.kv_dtype)
                V64 = WL.storage_to_f64(sl["V"], w.kv_dtype)
                if w.scheme == "softlsh":
                    W64 = WL.storage_to_f64(WL.make_planes(w, h), w.kv_dtype)
                    meta = (O.hash_keys_softlsh(K64, W64, w.L, w.P),
                            O.value_norms(V64, w.norm_dtype), W64)
                else:
                    R64 = WL.storage_to_f64(WL.make_projection(w, h), w.kv_dtype)
                    meta = (O.binary_codes(K64, R64), None, R64)
                prepared.append((int(ks[b]), q64, K64, V64, meta))
            conn.send("ready")
        elif msg == "go":
            t0 = time.perf_counter()
            for (kb, q64, K64, V64, meta) in prepared:
                if w.scheme == "softlsh":
                    O.decode_slab_softlsh(q64, K64, V64, meta[2], w.L, w.P, w.tau, kb,
                                          w.norm_dtype, ids=meta[0], vnorm=meta[1])
                else:
                    O.decode_slab_hamming(q64, K64, V64, meta[2], kb, kcodes=meta[0])
            conn.send(time.perf_counter() - t0)
        else:
            conn.close()
            return


class CpuBaseline:
    """The oracle's whole decode step (every (b, kv head) slab of the
    workload) on the host, in a pool of single-threaded processes over the
    CPUs this process may run on (at most CPU_WORKERS_MAX).  When the step
    has fewer slabs than there are CPUs, several independent steps run at
    once (every CPU busy), and the rate counts all of them.  The processes
    are spawned before the GPU is initialised; the step time is the wall
    time of one round with every worker running its slabs at once (the
    slowest worker), median of `reps` rounds."""

    def __init__(self, w):
        import multiprocessing as mp
        self.w = w
        self.affinity = len(os.sched_getaffinity(0))
        target = max(1, min(self.affinity, CPU_WORKERS_MAX))
        slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
        self.inflight = max(1, -(-target // len(slabs)))  # steps at once
        slabs = slabs * self.inflight
        nw = max(1, min(target, len(slabs)))
        # longest slabs first, dealt round robin
        lens = w.seq_lens()
        slabs.sort(key=lambda bh: -int(lens[bh[0]]))
        parts = [slabs[i::nw] for i in range(nw)]
        ctx = mp.get_context("spawn")
        self.conns, self.procs = [], []
        for part in parts:
            a, b = ctx.Pipe()
            p = ctx.Process(target=_cpu_worker, args=(w.name, part, b), daemon=True)
            p.start()
            self.conns.append(a)
            self.procs.append(p)
        self.nslabs = len(slabs) // self.inflight

    def run(self, reps=3):
        t0 = time.perf_counter()
        for c in self.conns:
            c.send("prepare")
        for c in self.conns:
            assert c.recv() == "ready"
        prep_s = time.perf_counter() - t0
        steps = []
        for _ in range(reps):
            for c in self.conns:
                c.send("go")
            steps.append(max(c.recv() for c in self.conns))
        self.close()
        steps.sort()
        t_step = steps[len(steps) // 2]
        model = ""
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        return {"value": self.inflight * self.w.B / t_step, "unit": "tokens/s",
                "cores": len(self.procs), "kind": "oracle",
                "sample": (f"{self.inflight} whole decode step(s) at once (query tables or codes, "
                           f"scores, top-k, attention; {self.nslabs} (batch, kv head) slabs each), "
                           f"float64 numpy oracle, {len(self.procs)} single-threaded processes; "
                           f"median of {reps} rounds"),
                "step_s": t_step, "steps_s": steps, "steps_in_flight": self.inflight,
                "affinity_cpus": self.affinity,
                "cpu_model": model, "prepare_s": round(prep_s, 1)}

    def close(self):
        for c in self.conns:
            try:
                c.send("stop")
            except (BrokenPipeError, OSError):
                pass
        for p in self.procs:
            p.join(timeout=10)


SHARED_B, SHARED_NP, SHARED_NS = 8, 32768, 2048


def shared_leg(hst, w, Wp, dev, stream, capture, copies=3, reps=10):
    """Shared-prefix step against the plain step on the same data laid out
    whole, each timed over `copies` rotated input copies by graph replay.
    Data: seeded normal keys, values and queries in the KV dtype; suffix
    lengths uniform in [SHARED_NS / 4, SHARED_NS]; k_b = ceil(N_b / 33)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(20260101)
    B, Hkv, Hq, d, Np, Ns = SHARED_B, w.Hkv, w.Hq, w.d, SHARED_NP, SHARED_NS
    dt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    nd = torch.float16 if w.norm_dtype == "f16" else torch.float32
    slens = torch.randint(Ns // 4, Ns + 1, (B,), generator=g, device=dev, dtype=torch.int32)
    ctx = (Np + slens).to(torch.int64)
    kps = ((ctx + 32) // 33).to(torch.int32)
    kmax = int(kps.max())
    q = torch.randn((B, Hq, d), generator=g, device=dev).to(dt)
    sets, whole = [], []
    for _ in range(copies):
        Kp = torch.randn((1, Hkv, Np, d), generator=g, device=dev).to(dt)
        Vp = torch.randn((1, Hkv, Np, d), generator=g, device=dev).to(dt)
        Ks = torch.randn((B, Hkv, Ns, d), generator=g, device=dev).to(dt)
        Vs = torch.randn((B, Hkv, Ns, d), generator=g, device=dev).to(dt)
        ip, vp = hst.hst_hash_keys_softlsh(Kp, Vp, Wp, w.L, w.P, nd)
        is_, vs_ = hst.hst_hash_keys_softlsh(Ks, Vs, Wp, w.L, w.P, nd, seq_lens=slens)
        sets.append((Kp, Vp, ip, vp, Ks, Vs, is_, vs_))
        Kc = torch.cat([Kp.expand(B, -1, -1, -1), Ks], dim=2).contiguous()
        Vc = torch.cat([Vp.expand(B, -1, -1, -1), Vs], dim=2).contiguous()
        clen = (Np + slens).to(torch.int32)
        ic, vc = hst.hst_hash_keys_softlsh(Kc, Vc, Wp, w.L, w.P, nd, seq_lens=clen)
        whole.append((Kc, Vc, ic, vc))
    clen = (Np + slens).to(torch.int32)
    sstep = hst.DecodeSoftLSHShared(sets[0][4], Np, Hq, w.L, w.P, w.tau, kmax, nd, seq_lens=slens,
                                    k_per_seq=kps)
    pstep = hst.DecodeSoftLSH(whole[0][0], Hq, w.L, w.P, w.tau, kmax, nd, seq_lens=clen,
                              k_per_seq=kps)
    srun = lambda i: sstep(q, *sets[i % copies][:4], *sets[i % copies][4:], Wp)
    prun = lambda i: pstep(q, whole[i % copies][0], whole[i % copies][1], Wp, whole[i % copies][2],
                           whole[i % copies][3])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        gr = capture(lambda: [fn(i) for i in range(copies)])
        gr.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record(stream)
            gr.replay()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3 / copies)
        return sorted(ts)[len(ts) // 2]

    sus, pus = timed(srun), timed(prun)
    e = torch.tensor([], dtype=dt).element_size()
    m = w.L + torch.tensor([], dtype=nd).element_size()
    ktot = int(kps.sum()) * Hkv
    gath = ktot * 2 * d * e
    qo = B * Hq * d * (e + 4)
    sbytes = Hkv * Np * m + int(slens.sum()) * Hkv * m + gath + qo
    pbytes = int(ctx.sum()) * Hkv * m + gath + qo
    return {"B": B, "prefix": Np, "suffix_max": Ns, "us": sus, "plain_us": pus,
            "speedup": pus / sus, "alg_bytes": sbytes, "plain_alg_bytes": pbytes,
            "hbm_frac": sbytes / (sus * 1e-6) / (HBM_PEAK_GBS * 1e9)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU: the decode path has no multi-GPU mode "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    w = None
    import workloads as WL
    w = WL.WORKLOADS[args.workload]
    # the CPU baseline's processes start before anything touches the GPU
    cpu = None if args.no_cpu_baseline else CpuBaseline(w)

    import numpy as np
    import torch

    import hash_scored_top_amd as hst
    from workloads.device import norm_torch_dtype, to_dev

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: generating inputs")
    t0 = time.time()
    x = WL.make_full(w)
    lens, ks = x["seq_lens"], x["k_per_seq"]
    kmax = int(ks.max())
    log(f"generated in {time.time() - t0:.1f}s")

    if args.copy_calibration:
        a = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    K = to_dev(x["K"], w.kv_dtype, dev)
    V = to_dev(x["V"], w.kv_dtype, dev)
    q = to_dev(x["q"], w.kv_dtype, dev)
    ragged = w.ragged is not None
    sl = torch.from_numpy(lens).to(dev) if ragged else None
    kp = torch.from_numpy(ks).to(dev) if ragged else None
    stream = torch.cuda.current_stream(dev)

    # prefill metadata (once per key), timed separately: outputs allocated
    # once, the library call alone inside the events
    tot_keys = sum(int(n) for n in lens) * w.Hkv
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pre_reps = 10
    if w.scheme == "softlsh":
        Wp = to_dev(x["W"], w.kv_dtype, dev)
        nd = norm_torch_dtype(w.norm_dtype)
        ids, vn = hst.hst_hash_keys_softlsh(K, V, Wp, w.L, w.P, nd, seq_lens=sl)
        pre = lambda: hst.hst_hash_keys_softlsh(K, V, Wp, w.L, w.P, nd, seq_lens=sl, ids=ids,
                                                vnorm=vn)
        planes = w.L * w.P
        pre_bytes = tot_keys * (2 * w.d * K.element_size() + w.L + vn.element_size())
    else:
        Rp = to_dev(x["R"], w.kv_dtype, dev)
        codes = hst.hst_hash_keys_binary(K, Rp, seq_lens=sl)
        pre = lambda: hst.hst_hash_keys_binary(K, Rp, seq_lens=sl, codes=codes)
        planes = w.code_bits
        pre_bytes = tot_keys * (w.d * K.element_size() + w.code_bits // 8)
    pre()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(pre_reps):
        pre()
    ev[1].record(stream)
    torch.cuda.synchronize()
    prefill_us = ev[0].elapsed_time(ev[1]) * 1e3 / pre_reps
    pre_flops = 2.0 * tot_keys * planes * w.d
    prefill = {"us": prefill_us, "keys": tot_keys, "planes": planes,
               "tflops": pre_flops / (prefill_us * 1e-6) / 1e12,
               "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
               "mfma_frac": pre_flops / (prefill_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
               "hbm_bytes": pre_bytes,
               "hbm_frac": pre_bytes / (prefill_us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
    log(f"prefill hash {prefill_us:.1f} us ({prefill['tflops']:.0f} TFLOP/s, "
        f"{pre_bytes / (prefill_us * 1e-6) / 1e9:.0f} GB/s)")

    # decode-time append of one token per sequence (rows, metadata, lengths),
    # timed on a cache of the same batch and heads with room for every call
    app_reps = 20
    Ka = torch.zeros((w.B, w.Hkv, app_reps + 1, w.d), dtype=K.dtype, device=dev)
    Va = torch.zeros_like(Ka)
    la = torch.zeros((w.B,), dtype=torch.int32, device=dev)
    kn, vnw = K[:, :, 0].contiguous(), V[:, :, 0].contiguous()
    if w.scheme == "softlsh":
        ida = torch.zeros((w.B, w.Hkv, app_reps + 1, w.L), dtype=torch.uint8, device=dev)
        vna = torch.zeros((w.B, w.Hkv, app_reps + 1), dtype=vn.dtype, device=dev)
        app = lambda: hst.hst_append_kv_softlsh(kn, vnw, Wp, w.L, w.P, Ka, Va, ida, vna, la)
    else:
        ca = torch.zeros((w.B, w.Hkv, app_reps + 1, w.code_bits // 32), dtype=torch.int32,
                         device=dev)
        app = lambda: hst.hst_append_kv_binary(kn, vnw, Rp, Ka, Va, ca, la)
    def app_all():
        for _ in range(app_reps):
            app()

    # eager calls (host marshalling included), then replays of a captured
    # graph of app_reps calls (device time); the lengths restart before each
    app()  # first launches load the kernels
    la.zero_()
    torch.cuda.synchronize()
    ev[0].record(stream)
    app_all()
    ev[1].record(stream)
    torch.cuda.synchronize()
    append_eager_us = ev[0].elapsed_time(ev[1]) * 1e3 / app_reps
    la.zero_()
    app_graph = capture(app_all)
    app_times = []
    for _ in range(5):
        la.zero_()
        ev[0].record(stream)
        app_graph.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        app_times.append(ev[0].elapsed_time(ev[1]) * 1e3 / app_reps)
    append_us = sorted(app_times)[len(app_times) // 2]
    append = {"us": append_us, "eager_us": append_eager_us, "tokens": w.B, "planes": planes}
    log(f"append {append_us:.1f} us for {w.B} tokens ({append_eager_us:.1f} us eager)")
    del Ka, Va, app_graph

    meta_b, gath_b, qo_b = alg_bytes(w, lens, ks)
    step_bytes = meta_b + gath_b + qo_b
    R = args.rotate or max(2, min(16, math.ceil(2 * MALL_BYTES / step_bytes) + 1))
    log(f"step algorithmic bytes {step_bytes / 1e6:.1f} MB; rotating over {R} input copies")
    if w.scheme == "softlsh":
        sets = [(K, V, ids, vn)] + [(K.clone(), V.clone(), ids.clone(), vn.clone())
                                    for _ in range(R - 1)]
        step = hst.DecodeSoftLSH(K, w.Hq, w.L, w.P, w.tau, kmax, vn.dtype, seq_lens=sl,
                                 k_per_seq=kp)
        run = lambda i: step(q, sets[i % R][0], sets[i % R][1], Wp, sets[i % R][2], sets[i % R][3])
    else:
        sets = [(K, V, codes)] + [(K.clone(), V.clone(), codes.clone()) for _ in range(R - 1)]
        step = hst.DecodeHamming(K, w.Hq, kmax, seq_lens=sl, k_per_seq=kp)
        run = lambda i: step(q, sets[i % R][0], sets[i % R][1], Rp, sets[i % R][2])
    torch.cuda.synchronize()

    # exactly args.steps steps (input copy t % R) back to back: replays of
    # captured graphs of up to 1024 consecutive steps (--no-graph: eager
    # launches), between two events.  A spin kernel first keeps the GPU busy
    # while the host enqueues, so no step waits for the host.
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    spin = spin_cycles_per_ms(stream)
    GSTEPS = 1024
    spans = [(s0, min(s0 + GSTEPS, args.steps)) for s0 in range(0, args.steps, GSTEPS)]
    graphs = [] if args.no_graph else [capture(lambda s0=s0, s1=s1: [run(t) for t in range(s0, s1)])
                                       for s0, s1 in spans]
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    log(f"warmup {args.warmup} done; timing {args.steps} steps "
        f"({'eager' if args.no_graph else f'{len(graphs)} graph replay(s)'}, {R} input copies)")
    torch.cuda._sleep(int(spin * min(500.0, 5.0 + 0.2 * args.steps)))
    ev[0].record(stream)
    if args.no_graph:
        for t in range(args.steps):
            run(t)
    else:
        for g in graphs:
            g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    timed = args.steps
    total_ms = ev[0].elapsed_time(ev[1])
    ms_per_step = total_ms / timed
    del graphs
    # per-step latency: each step launched alone (one replay of a captured
    # one-step graph), an event between consecutive steps
    g1 = [capture(lambda i=i: run(i)) for i in range(R)]
    nlat = min(args.steps, 200)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nlat + 1)]
    torch.cuda._sleep(int(spin * min(500.0, 5.0 + 0.2 * nlat)))
    evs[0].record(stream)
    for t in range(nlat):
        g1[t % R].replay()
        evs[t + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[t].elapsed_time(evs[t + 1]) for t in range(nlat)]) * 1e3  # us
    del g1
    log(f"step {ms_per_step * 1e3:.2f} us back to back; alone p50 {np.percentile(per, 50):.2f} us")

    # the step's stages, each between events (the spin kernel first again):
    # prepare (query tables, key sample), filter (the score scan with the
    # threshold and the candidates: the dominant kernel), finish (selection,
    # attention and the split merge)
    iters = args.kernel_iters
    if w.scheme == "softlsh":
        stages = (lambda i: step.prepare(q, Wp, sets[i % R][2], sets[i % R][3]),
                  lambda i: step.filter(sets[i % R][2], sets[i % R][3]),
                  lambda i: step.finish(q, sets[i % R][0], sets[i % R][1], sets[i % R][2],
                                        sets[i % R][3]))
    else:
        stages = (lambda i: step.prepare(q, Rp, sets[i % R][2]),
                  lambda i: step.filter(sets[i % R][2]),
                  lambda i: step.finish(q, sets[i % R][0], sets[i % R][1], sets[i % R][2]))
    for i in range(3):
        for f in stages:
            f(i)
    torch.cuda.synchronize()
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(iters)]
    torch.cuda._sleep(int(spin * min(500.0, 5.0 + 0.3 * iters)))
    for i in range(iters):
        sev[i][0].record(stream)
        for j, f in enumerate(stages):
            f(i)
            sev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    stage_us = [float(np.median([sev[i][j].elapsed_time(sev[i][j + 1]) * 1e3 for i in range(iters)]))
                for j in range(3)]
    log("stages (median us): prepare {:.2f}, filter {:.2f}, finish {:.2f}".format(*stage_us))

    # dominant kernel: the step's own filtering scan (the filter stage is that
    # one launch), with its algorithmic bytes: the metadata of every key
    # (ids + value norm, or the code), read once
    kbytes = meta_b
    if w.scheme == "softlsh":
        f16 = "true" if w.norm_dtype == "f16" else "false"
        span = scan_span_of(w, dev)
        full = "true" if (w.L == 64 and w.P == 8) else "false"  # the full-table variant
        kname = (f"scan_softlsh_kernel<{w.L // 16}, 2, true, {f16}, "
                 f"{'true' if span > 2048 else 'false'}, {full}>")
        ktag = "scan_softlsh_filter"
    else:
        kname = "scan_lane_kernel<2>"
        ktag = "scan_hamming_filter"
    ksrc = os.path.join(ROOT, "hash_scored_top_amd", "csrc", "scan.hip")
    # its average launch duration: a captured graph of 8R filter launches
    # (input copies 0..R-1 in turn, after one prepare) replayed back to back
    # between two events, three times; the threshold the first launch
    # publishes stays set for the others (it holds the same value), so they
    # do not wait for it
    per_graph = 8 * R  # launches per replay: few replays, so replay gaps barely count
    reps = max(2, iters // per_graph)
    stages[0](0)
    gf = capture(lambda: [stages[1](i % R) for i in range(per_graph)])
    gf.replay()
    torch.cuda.synchronize()
    tf = []
    for _ in range(3):
        torch.cuda._sleep(int(spin * 2.0))
        ev[0].record(stream)
        for _ in range(reps):
            gf.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        tf.append(ev[0].elapsed_time(ev[1]) * 1e3 / (reps * per_graph))
    del gf
    kus = float(np.median(tf))
    klaunches = 3 * reps * per_graph
    log(f"filter kernel {kus:.2f} us per launch ({klaunches} back-to-back launches)")
    achieved = kbytes / (kus * 1e-6) / 1e9
    traffic = traffic_record(ktag, w.name, ksrc)

    def time_graph(fn, reps=10):
        """Median per-call time (us) of fn over replays of a captured graph of R calls."""
        g = capture(lambda: [fn(i) for i in range(R)])
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record(stream)
            g.replay()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3 / R)
        return float(np.median(ts))

    # cumulative-mass variant of the step (soft-LSH): the kmax candidates of
    # highest hash score, then the smallest set holding MASS_P of their
    # softmax mass
    mass = None
    if w.scheme == "softlsh" and not args.core_only:
        mstep = hst.DecodeSoftLSHMass(K, w.Hq, w.L, w.P, w.tau, kmax, MASS_P, vn.dtype,
                                      seq_lens=sl, k_per_seq=kp)
        mrun = lambda i: mstep(q, sets[i % R][0], sets[i % R][1], Wp, sets[i % R][2],
                               sets[i % R][3])
        mass_us = time_graph(mrun)
        kept = mstep.counts.cpu().numpy().astype(np.int64)
        cand_rows = sum(min(int(ks[b]), int(lens[b])) for b in range(w.B)) * w.Hkv
        e = K.element_size()
        mbytes = meta_b + qo_b + cand_rows * w.d * e + int(kept.sum()) * 2 * w.d * e
        mass = {"p": MASS_P, "us": mass_us, "tokens_per_s": w.B / (mass_us * 1e-6),
                "kept_mean": float(kept.mean()), "kept_max": int(kept.max()),
                "candidates_per_head": kmax, "alg_bytes": mbytes,
                "hbm_frac": mbytes / (mass_us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
        log(f"mass step (p={MASS_P}) {mass_us:.2f} us, kept {kept.mean():.1f} of {kmax} keys "
            "per head on average")
        del mstep

    # two-level routed variant of the step (soft-LSH): cards of 64-token
    # chunks first, ROUTE_OVERSAMPLE * ceil(k / 64) chunks kept, then the k
    # best keys inside them
    routed = None
    if w.scheme == "softlsh" and w.L in (16, 32, 64, 128) and not args.core_only:
        C = min(256, ROUTE_OVERSAMPLE * math.ceil(kmax / 64))
        cards = [hst.hst_build_cards_softlsh(st_[0], st_[3], Wp, w.L, w.P, seq_lens=sl)
                 for st_ in sets]
        rstep = hst.DecodeSoftLSHRouted(K, w.Hq, w.L, w.P, w.tau, kmax, C, vn.dtype, seq_lens=sl,
                                        k_per_seq=kp)
        rrun = lambda i: rstep(q, sets[i % R][0], sets[i % R][1], Wp, sets[i % R][2],
                               sets[i % R][3], cards[i % R][1], cards[i % R][2])
        routed_us = time_graph(rrun)
        e = K.element_size()
        m = w.L + vn.element_size()
        ncards = sum((int(n) + 63) // 64 for n in lens) * w.Hkv
        kept_keys = sum(min(C * 64, int(n)) for n in lens) * w.Hkv
        rbytes = ncards * m + kept_keys * m + gath_b + qo_b
        routed = {"chunks_kept": C, "us": routed_us, "tokens_per_s": w.B / (routed_us * 1e-6),
                  "alg_bytes": rbytes,
                  "hbm_frac": rbytes / (routed_us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
        log(f"routed step (C={C}) {routed_us:.2f} us, {rbytes / 1e6:.1f} MB")
        del rstep, cards

    # code-length sweep (binary codes): the same step with 64- and 256-bit
    # codes from seeded projections of the same keys (128 bits: the step)
    codes_sweep = None
    if w.scheme == "hamming" and not args.core_only:
        codes_sweep = {"128": {"us": ms_per_step * 1e3, "meta_bytes_per_key": 16}}
        gen = torch.Generator(device=dev)
        gen.manual_seed(20260202)
        for bits in (64, 256):
            Rb = torch.randn((w.Hkv, bits, w.d), generator=gen, device=dev).to(K.dtype)
            cb = [hst.hst_hash_keys_binary(st_[0], Rb, code_bits=bits, seq_lens=sl) for st_ in sets]
            bstep = hst.DecodeHamming(K, w.Hq, kmax, code_bits=bits, seq_lens=sl, k_per_seq=kp)
            brun = lambda i, bstep=bstep, Rb=Rb, cb=cb: bstep(q, sets[i % R][0], sets[i % R][1], Rb,
                                                              cb[i % R])
            codes_sweep[str(bits)] = {"us": time_graph(brun), "meta_bytes_per_key": bits // 8}
            del cb, bstep
        log("code lengths: " + ", ".join(f"{b} bits {v['us']:.1f} us" for b, v in codes_sweep.items()))

    # shared-prefix variant (soft-LSH): a batch of SHARED_B sequences with a
    # common SHARED_NP-key prefix and ragged own suffixes, against the plain
    # step on the materialised concatenation of the same data
    shared = None
    if w.scheme == "softlsh" and w.L in (16, 32, 64, 128) and not (args.no_shared or args.core_only):
        shared = shared_leg(hst, w, Wp, dev, stream, capture)
        log(f"shared-prefix step {shared['us']:.2f} us vs {shared['plain_us']:.2f} us "
            f"materialised ({shared['speedup']:.2f}x)")

    # dense attention over every cached key, for the sparse/dense ratio
    dense = None
    if w.B * w.Hkv * w.N <= (1 << 24) and not args.core_only:
        didx = torch.arange(w.N, dtype=torch.int32, device=dev).repeat(w.B, w.Hkv, 1)
        dshape = hst.make_shape(K, w.Hq, sl)
        dout = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        dws = torch.empty(hst.workspace_size(hst._lib.HST_OP_SPARSE_ATTENTION, dshape, k=w.N),
                          dtype=torch.uint8, device=dev)
        dscale = float(w.d ** -0.5)

        def drun(i):
            hst._lib._check(hst._lib._C.hst_sparse_decode_attention(
                ctypes.byref(dshape), q.data_ptr(), sets[i % R][0].data_ptr(),
                sets[i % R][1].data_ptr(), didx.data_ptr(), w.N, dscale, dout.data_ptr(), None,
                dws.data_ptr(), dws.numel(), torch.cuda.current_stream().cuda_stream),
                "dense attention")
        dense_us = time_graph(drun, reps=5)
        dbytes = tot_keys * 2 * w.d * K.element_size() + qo_b
        dense = {"us": dense_us, "alg_bytes": dbytes,
                 "hbm_frac": dbytes / (dense_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                 "sparse_speedup": dense_us / (ms_per_step * 1e3)}
        log(f"dense attention over all keys {dense_us:.1f} us "
            f"({dense['sparse_speedup']:.1f}x the sparse step)")
        del didx, dws

    result = {
        "metric": METRIC,
        "value": w.B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": timed,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "scheme": w.scheme, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "d": w.d, "N": w.N, "kv_dtype": w.kv_dtype,
                   **({"L": w.L, "P": w.P, "tau": w.tau} if w.scheme == "softlsh"
                      else {"code_bits": w.code_bits}),
                   "k": kmax, "ragged": ragged},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "alg_bytes_per_launch": kbytes,
                     "avg_launch_us": kus, "launches": klaunches,
                     "timing": "HIP events on the launch stream around back-to-back replays of a "
                               "captured graph of filter launches over the rotated input copies"},
        "step": {"alg_bytes": step_bytes, "meta_bytes": meta_b, "gathered_bytes": gath_b,
                 "hbm_frac": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "latency_alone_us": {"p10": float(np.percentile(per, 10)),
                                      "p50": float(np.percentile(per, 50)),
                                      "p90": float(np.percentile(per, 90)),
                                      "p99": float(np.percentile(per, 99)), "steps": int(len(per))},
                 "rotated_copies": R,
                 "stages_us": {"prepare": stage_us[0], "filter": stage_us[1],
                               "finish": stage_us[2]}},
        "prefill": prefill,
        "append": append,
        "mass": mass,
        "routed": routed,
        "shared": shared,
        "codes_sweep": codes_sweep,
        "dense": dense,
    }
    if cpu is not None:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu.run()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
