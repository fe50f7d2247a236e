"""Benchmark of the GDN ReplaySSM verify / rollback / flush path on one MI355X.

One step = the whole path over every GDN layer of the model for one batch
("The inference stack behind OCRia", section "Making speculative verification
cheaper": 32 concurrent requests, 24 GDN layers). Three orders of the same work
are timed, each on its own caches built from the same seeded inputs:

  fused     verify_flush on all layers (the periodic flush folded into the
            verify of the next step), then rollback on all layers;
  separate  verify on all layers, rollback on all layers, flush on all layers;
  step      rollback_verify_flush on all layers: one call per layer and step,
            the previous step's rollback and the flush folded into the verify;
  step_norm gdn_replay_step_norm_fp8 on all layers: the step with the gated
            RMSNorm + FP8 of its outputs in the same kernel (codes and scales
            only: the fp32 outputs are not stored), against the step followed
            by the separate norm kernel.

Each layer has its own cache (state + ring + pointers), so the 24 states (1.5 GiB
at 32 requests) do not fit in the 256 MB Infinity Cache and every call streams
its state from HBM.

Timing: HIP events on the launch stream bracket each group of 24 launches of
every timed step. The headline value is the verify + flush time per layer in
microseconds (the fused kernel's time, or verify + flush for the separate
order), averaged over the timed steps; each order also reports its whole step
per layer (rollback included). Algorithmic bytes come from the byte
model below, evaluated with the actual buffer lengths of every call (tracked on
the host from the known schedule).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                    [--path all|fused|separate|step|step_norm]
    python bench.py --sweep [--steps K] [--warmup W]   (replay cost vs buffer length)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN replay verify+flush us/layer and HBM GB/s (% roofline) at 32 reqs"
HBM_PEAK_GBPS = 8000.0
# the sources of the replay kernels whose HBM bytes a profile summary records
KERNEL_SRCS = [os.path.join(ROOT, "gated_deltanet_state_replayssm_amd", "csrc", f)
               for f in ("chunk_ops.h", "chunked.hip", "fused.hip")]
PROFILES = os.path.join(ROOT, "profiles")


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` ("verify", "flush", "verify_flush", ...)
    on `workload`, measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a
    copy of known size) and recorded in a profiles/ summary, or None when no
    summary of that workload matches the current kernel source."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        h.update(open(path, "rb").read())
    sha = h.hexdigest()[:16]
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(path):
            m = re.search(r"traffic source_sha=(\w+) workload=(\w+)((?: \w+_mb_per_launch=[\d.]+)+)",
                          line)
            if m and m.group(1) == sha and m.group(2) == workload:
                vals = dict(re.findall(r"(\w+)_mb_per_launch=([\d.]+)", m.group(3)))
                if kernel in vals:
                    return int(float(vals[kernel]) * 1e6)
    return None


def byte_model(wl, lens_at_verify, folded, drafts=None):
    """Algorithmic HBM bytes of one layer's verify and flush calls.

    verify: state read R*HV*dk*dv*4 (requests with a draft); committed ring read
    sum_r B_r*(HK*dk*ib + HV*dv*ib + HV*8); draft read and ring append
    sum_r D_r*(2*HK*dk*ib + HV*dv*ib + HV*8) each (q is appended too); out write
    sum_r D_r*HV*dv*4. drafts: per-request D_r (default D for every request).
    flush: for each folded slot, state read + write HV*dk*dv*8 and ring read
    n*(HK*dk*ib + HV*dv*ib + HV*8)."""
    ib = wl.in_bytes
    R, HV, HK, dk, dv = wl.num_reqs, wl.hv, wl.hk, wl.dk, wl.dv
    Ds = np.full(R, wl.draft) if drafts is None else np.asarray(drafts)
    with_draft = Ds > 0
    tok_ring = HK * dk * ib + HV * dv * ib + HV * 8
    tok_draft = 2 * HK * dk * ib + HV * dv * ib + HV * 8
    v_bytes = (int(with_draft.sum()) * HV * dk * dv * 4
               + int(np.sum(np.asarray(lens_at_verify)[with_draft])) * tok_ring
               + int(Ds.sum()) * (2 * tok_draft + HV * dv * 4))
    f_bytes = sum(HV * dk * dv * 8 + int(n) * tok_ring for n in folded)
    return v_bytes, f_bytes


def byte_model_fused(wl, lens_at_call, folded, drafts=None):
    """Algorithmic HBM bytes of one layer's verify_flush call: the verify of the
    byte model above with B_r = 0 for the folded slots, whose committed tokens
    are read once by the fold and whose state is written once (HV*dk*dv*4 each)
    but not read a second time (a folded slot without a draft reads its state
    for the fold only)."""
    Ds = np.full(wl.num_reqs, wl.draft) if drafts is None else np.asarray(drafts)
    lens = np.asarray(lens_at_call)
    due = lens >= max(wl.flush_min_len, 1)
    v_bytes, _ = byte_model(wl, np.where(due & (Ds == 0), 0, lens), [], Ds)
    fold_only = int((due & (Ds == 0)).sum())
    tok_ring = wl.hk * wl.dk * wl.in_bytes + wl.hv * wl.dv * wl.in_bytes + wl.hv * 8
    fold_only_ring = int(lens[due & (Ds == 0)].sum()) * tok_ring
    return (v_bytes + len(folded) * wl.hv * wl.dk * wl.dv * 4
            + fold_only * wl.hv * wl.dk * wl.dv * 4 + fold_only_ring)


def norm_leg(wl, layers, steps, warmup):
    """The step after the recurrence: gated RMSNorm + FP8 of one layer's verify
    output ([R * D] rows x HV heads x d_v), timed with HIP events over `steps`
    rounds of `layers` launches, each layer on its own buffers (the 24 layers'
    inputs do not fit in the Infinity Cache), replayed from a HIP graph. Bytes: o
    fp32 + z bf16 read, codes written, one fp32 scale per (row, head), the d_v
    weight."""
    import torch

    from gated_deltanet_state_replayssm_amd import synth
    from gated_deltanet_state_replayssm_amd.cache import to_device
    from gated_deltanet_state_replayssm_amd.norm import gated_rmsnorm_fp8

    rows, H, dv = wl.num_reqs * wl.draft, wl.hv, wl.dv
    rng = np.random.default_rng(synth.seed_for(wl.name, 0, 90))
    w = to_device(rng.uniform(0.5, 1.5, dv).astype(np.float32))
    torch.manual_seed(synth.seed_for(wl.name, 0, 91))
    bufs = []
    for L in range(layers):
        o = torch.randn((rows, H, dv), device="cuda")
        z = torch.randn((rows, H, dv), device="cuda").to(torch.bfloat16)
        q = torch.empty((rows, H, dv), dtype=torch.uint8, device="cuda")
        sc = torch.empty((rows, H), dtype=torch.float32, device="cuda")
        bufs.append((o, z, q, sc))
    # the launches are captured in a HIP graph: a kernel of a few microseconds
    # would otherwise be timed at the rate the host issues launches
    for o, z, q, sc in bufs:
        gated_rmsnorm_fp8(o, z, w, 1e-6, q, sc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for o, z, q, sc in bufs:
            gated_rmsnorm_fp8(o, z, w, 1e-6, q, sc)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    marks = []
    for it in range(warmup + steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        if it >= warmup:
            marks.append((e0, e1))
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in marks) * 1e3 / (len(marks) * layers)
    del g
    nbytes = rows * H * dv * (4 + 2 + 1) + rows * H * 4 + dv * 4
    del bufs
    return {"us": round(us, 2), "bytes": int(nbytes), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "what": f"gated RMSNorm + FP8 of [{rows}][{H}][{dv}] (rows = requests x draft)"}


def conv_leg(wl, layers, steps, warmup, width=4):
    """The step before the recurrence: the causal convolution of the draft block
    over the q, k, v channels (2 HK dk + HV dv), width 4, with its ring history,
    for every layer (each with its own ring and pointers), replayed from a HIP
    graph. Bytes: x read, y written, x appended, K - 1 history rows read, the
    weights and bias."""
    import torch

    from gated_deltanet_state_replayssm_amd import synth
    from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device
    from gated_deltanet_state_replayssm_amd.conv import ConvRing

    R, D, C = wl.num_reqs, wl.draft, wl.cap
    CH = 2 * wl.hk * wl.dk + wl.hv * wl.dv
    rng = np.random.default_rng(synth.seed_for(wl.name, 0, 92))
    torch.manual_seed(synth.seed_for(wl.name, 0, 93))
    slots = to_device(np.arange(R, dtype=np.int32))
    legs = []
    for L in range(layers):
        # the convolution reads only the pointers of the layer's cache
        cache = ReplayCache(wl.num_slots, 1, 1, 16, 16, C, wl.in_dtype)
        cache.head.copy_(to_device(rng.integers(0, C, wl.num_slots).astype(np.int32)))
        cache.len.copy_(to_device(rng.integers(0, C - D + 1, wl.num_slots).astype(np.int32)))
        ring = ConvRing(cache, CH, width)
        ring.ring.normal_()
        x = torch.randn((R, D, CH), device="cuda").to(torch.bfloat16)
        y = torch.empty_like(x)
        w = torch.randn((CH, width), device="cuda") * 0.5
        b = torch.randn((CH,), device="cuda")
        legs.append((ring, x, y, w, b))
    for ring, x, y, w, b in legs:
        ring.update(slots, x, w, b, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for ring, x, y, w, b in legs:
            ring.update(slots, x, w, b, y)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    marks = []
    for it in range(warmup + steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        if it >= warmup:
            marks.append((e0, e1))
    torch.cuda.synchronize()
    assert all(int(ring.cache.err.item()) == 0 for ring, *_ in legs)
    us = sum(a.elapsed_time(b) for a, b in marks) * 1e3 / (len(marks) * layers)
    nbytes = R * D * CH * 2 * 3 + R * (width - 1) * CH * 2 + CH * (width + 1) * 4
    del g, legs
    return {"us": round(us, 2), "bytes": int(nbytes), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "what": f"causal conv width {width} over [{R}][{D}][{CH}] with ring history"}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host's cores
# ---------------------------------------------------------------------------
_CPU = {}   # inputs of the pool's workers, inherited by fork (set before the pool starts)


def _cpu_worker(k):
    """Slots s with s % n == k of one layer, through the steps the GPU timed:
    verify_flush then rollback per step (the fused order), untimed up to the
    first timed step. Returns the seconds spent in the timed steps."""
    from threadpoolctl import threadpool_limits

    from oracle import gdn_oracle as go
    c = _CPU
    wl, n, steps, timed_from = c["wl"], c["n"], c["steps"], c["timed_from"]
    orc = go.ReplayOracle(c["init"], wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, mode="replay")
    spent = 0.0
    with threadpool_limits(limits=1):
        for i, (slots, acc, dl) in enumerate(steps):
            mine = np.array([j for j, sl in enumerate(slots) if sl % n == k], dtype=np.int64)
            if not len(mine):
                continue
            d = c["drafts"][i % 2]
            t0 = time.perf_counter()
            orc.verify_flush(slots[mine], wl.flush_min_len,
                             *(d[x][mine] for x in ("q", "k", "v", "alpha", "beta")),
                             draft_lens=None if dl is None else dl[mine])
            orc.rollback(slots[mine], wl.draft, acc[mine],
                         draft_lens=None if dl is None else dl[mine])
            if i >= timed_from:
                spent += time.perf_counter() - t0
    return spent


def cpu_baseline(wl, init, drafts, steps, warmup, max_cores=16, max_timed=30):
    """The fp64 oracle, as it stands, on the schedule the GPU timed: layer 0's
    cache, its two draft sets alternated as on the GPU, and the same slot
    permutation, accepted counts and draft lengths per step, in the fused order
    (verify_flush then rollback; the lengths at verify and the folded slots are
    therefore those of the GPU's steps). Steps before the GPU's first timed
    step run untimed; the first max_timed of the GPU's timed steps are timed
    (a bounded sample: tens of seconds of CPU work). The slots are split over len(os.sched_getaffinity(0))
    worker processes (at most max_cores; a slot's trajectory is independent of
    the others'), each with one BLAS thread; the value is the slowest worker's
    time per timed step, in us per layer. Runs before the GPU is touched (the
    workers are forked)."""
    import multiprocessing as mp
    n = max(1, min(len(os.sched_getaffinity(0)), max_cores, wl.num_slots))
    steps = steps[:warmup + max_timed]
    _CPU.update(wl=wl, n=n, steps=steps, timed_from=warmup, init=init, drafts=drafts)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        spent = pool.map(_cpu_worker, range(n))
    wall = time.perf_counter() - t0
    timed = len(steps) - warmup
    return {"value": round(max(spent) / timed * 1e6, 1), "unit": "us/layer", "cores": n,
            "kind": "oracle",
            "sample": f"layer 0 of {wl.name}: steps {warmup}..{len(steps) - 1} of the GPU's "
                      f"schedule timed ({warmup} earlier steps untimed), verify_flush + "
                      f"rollback of {wl.num_reqs} requests per step; fp64 NumPy, slots split "
                      f"over {n} processes of 1 thread, slowest process's time; "
                      f"{sum(spent):.1f} s of CPU work timed, {wall:.1f} s wall"}


def cpu_single_thread(workload="r8_hv32_hk16_d128", layers=8):
    """The oracle on one thread for a small workload (8 requests): one verify ->
    rollback -> flush of every request per layer, us per layer."""
    from threadpoolctl import threadpool_limits

    from gated_deltanet_state_replayssm_amd import synth
    from oracle import gdn_oracle as go
    wl = synth.WORKLOADS[workload]
    spent = 0.0
    with threadpool_limits(limits=1):
        for L in range(layers):
            rng = np.random.default_rng(synth.seed_for(wl.name, L, 0))
            init = synth.make_cache_init(wl, rng)
            orc = go.ReplayOracle(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, mode="replay")
            slots = synth.make_slot_idx(wl, rng)
            dr = synth.make_draft(wl, rng)
            acc = synth.sample_accepted(wl, rng)
            t0 = time.perf_counter()
            orc.verify(slots, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
            orc.rollback(slots, wl.draft, acc)
            orc.flush(slots, 1)
            spent += time.perf_counter() - t0
    return {"value": round(spent / layers * 1e6, 1), "unit": "us/layer", "cores": 1,
            "kind": "oracle", "workload": wl.name,
            "sample": f"{layers} layers of {wl.name}: one verify -> rollback -> flush of "
                      f"{wl.num_reqs} requests each; fp64 NumPy, 1 thread"}


def sweep(args, workload="r32_hv32_hk16_d128_f64", buffer_lens=(0, 8, 16, 32, 48, 63),
          fold_lens=(16, 32, 64, 79)):
    """Replay cost against the committed-buffer length (32 requests, ring capacity
    80, D = 16, 24 layer caches): (i) verify with every request's buffer at B,
    (ii) flush alone folding n tokens of every slot. HIP events around each
    group of 24 launches, made through the C entry points with arguments
    marshalled beforehand (flush: every layer's len is reset to n before the
    group); bytes from the byte model."""
    import torch

    from gated_deltanet_state_replayssm_amd import binding, synth
    from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device

    wl = synth.WORKLOADS[workload]
    layers = args.layers or wl.layers
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    slots = to_device(np.arange(wl.num_reqs, dtype=np.int32))
    out = torch.empty((wl.num_reqs, wl.draft, wl.hv, wl.dv), dtype=torch.float32, device="cuda")
    d = {k: to_device(v) for k, v in
         synth.make_draft(wl, np.random.default_rng(synth.seed_for(wl.name, 0, 77))).items()}

    def caches_with(n):
        cs = []
        for L in range(layers):
            rng = np.random.default_rng(synth.seed_for(wl.name, L, 0))
            init = synth.make_cache_init(wl, rng, init_len=np.full(wl.num_slots, n, np.int32))
            cs.append(ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap,
                                             wl.in_dtype))
        torch.cuda.synchronize()
        return cs

    def emit(kind, n, us, nbytes):
        print(json.dumps({
            "metric": f"GDN replay {kind} us/layer at fixed length", "kind": kind,
            "length": int(n), "value": round(us, 2), "unit": "us/layer",
            "hbm_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "bytes_per_layer": int(nbytes), "steps": args.steps, "warmup": args.warmup,
            "config": {"workload": wl.name, "requests": wl.num_reqs, "v_heads": wl.hv,
                       "k_heads": wl.hk, "d_k": wl.dk, "d_v": wl.dv, "draft": wl.draft,
                       "ring_cap": wl.cap, "layers": layers, "inputs": wl.in_dtype}}),
            flush=True)

    lib = binding.load()
    sh = stream.cuda_stream
    dp = tuple(d[x].data_ptr() for x in ("q", "k", "v", "alpha", "beta")) + (out.data_ptr(), sh)
    R, D = wl.num_reqs, wl.draft

    for B in buffer_lens:
        caches = caches_with(B)
        refs = [ctypes.byref(c.struct()) for c in caches]
        marks, status = [], []
        for step in range(args.warmup + args.steps):
            e0, e1 = ev(), ev()
            e0.record(stream)
            # verify leaves state and pointers as they are
            status.extend([lib.gdn_replay_verify(ref, R, slots.data_ptr(), D, *dp)
                           for ref in refs])
            e1.record(stream)
            if step >= args.warmup:
                marks.append((e0, e1))
        torch.cuda.synchronize()
        assert not any(status) and not any(int(c.err.item()) for c in caches)
        us = sum(a.elapsed_time(b) for a, b in marks) * 1e3 / (len(marks) * layers)
        v_bytes, _ = byte_model(wl, np.full(wl.num_reqs, B), [])
        emit("verify", B, us, v_bytes)
        del caches

    for n in fold_lens:
        caches = caches_with(n)
        refs = [ctypes.byref(c.struct()) for c in caches]
        marks, status = [], []
        for step in range(args.warmup + args.steps):
            for c in caches:
                c.len.fill_(n)   # every slot folds n tokens again (head moves on)
            e0, e1 = ev(), ev()
            e0.record(stream)
            status.extend([lib.gdn_replay_flush(ref, R, slots.data_ptr(), 1, sh) for ref in refs])
            e1.record(stream)
            if step >= args.warmup:
                marks.append((e0, e1))
        torch.cuda.synchronize()
        assert not any(status) and not any(int(c.err.item()) for c in caches)
        us = sum(a.elapsed_time(b) for a, b in marks) * 1e3 / (len(marks) * layers)
        _, f_bytes = byte_model(wl, np.zeros(wl.num_reqs), [n] * wl.num_reqs)
        emit("flush", n, us, f_bytes)
        del caches


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="r32_hv32_hk16_d128_f16")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--path", choices=("all", "fused", "separate", "step", "step_norm"),
                    default="all")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step benchmark: verify at fixed committed-buffer "
                         "lengths and flush alone at fixed fold lengths (ring capacity 80 "
                         "workload), one JSON line per point")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many MiB once (a plain "
                         "copy kernel of known size that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the replay path needs no collective and this "
              "build runs on a single MI355X (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    from gated_deltanet_state_replayssm_amd import synth

    wl = synth.WORKLOADS[args.workload]
    layers = args.layers or wl.layers
    total = args.warmup + args.steps
    # host-side inputs first: the CPU baseline runs on them before the GPU is touched
    inits = []
    for L in range(layers):
        inits.append(synth.make_cache_init(wl, np.random.default_rng(synth.seed_for(wl.name, L, 0))))
    init_len = inits[0]["len"].astype(np.int64)
    # two draft sets per layer, alternated: values do not change the work done
    host_drafts = []
    for L in range(layers):
        host_drafts.append([synth.make_draft(wl, np.random.default_rng(synth.seed_for(wl.name, L, 50 + j)))
                            for j in range(2)])
    rng = np.random.default_rng(synth.seed_for(wl.name, 0, 0))
    steps = []
    for _ in range(total):
        slots = synth.make_slot_idx(wl, rng)
        lens = synth.sample_draft_lens(wl, rng)   # None: every request drafts wl.draft
        steps.append((slots, synth.sample_accepted(wl, rng, draft_lens=lens), lens))
    cpu = None
    if not args.no_cpu and not args.sweep:
        cpu = cpu_baseline(wl, inits[0], host_drafts[0], steps, args.warmup)
        cpu["single_thread"] = cpu_single_thread()

    import torch

    from gated_deltanet_state_replayssm_amd import binding
    from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device

    binding.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.sweep:
        sweep(args)
        return
    stream = torch.cuda.current_stream()
    # the step with the norm takes the single-chunk shapes only (its entry point
    # refuses others): bf16 inputs, d in {64, 128}, ring capacity and draft <= 32
    norm_ok = (wl.in_dtype == synth.BF16 and wl.dk == wl.dv and wl.dk in (64, 128)
               and wl.cap <= 32 and wl.draft <= 32)
    paths = (("fused", "separate", "step") + (("step_norm",) if norm_ok else ())
             if args.path == "all" else (args.path,))

    drafts = [[{k: to_device(v) for k, v in d.items()} for d in ds] for ds in host_drafts]
    # each layer writes its own outputs (one shared buffer would stay in the
    # Infinity Cache and understate the write traffic)
    outs = [torch.empty((wl.num_reqs, wl.draft, wl.hv, wl.dv), dtype=torch.float32, device="cuda")
            for _ in range(layers)]
    F = max(wl.flush_min_len, 1)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def run_path(path):
        caches = [ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
                  for init in inits]
        # the host's copy of the schedule (identical on every layer)
        sched = []
        lens = init_len.copy()
        # step order: accepted count and draft length of each slot's previous
        # draft (a slot missing from a batch drops its pending draft: all rejected)
        p_acc = np.zeros(wl.num_slots, np.int32)
        p_len = np.zeros(wl.num_slots, np.int32)
        for slots, acc, dl in steps:
            extra = {}
            if path in ("step", "step_norm"):
                pa, pl = p_acc[slots].copy(), p_len[slots].copy()
                extra = dict(pacc=to_device(pa), plens=None if dl is None else to_device(pl))
                lens[slots] += pa
                p_acc[:] = 0
                p_len[:] = 0
                p_acc[slots] = acc
                p_len[slots] = wl.draft if dl is None else dl
            lv = lens[slots].copy()
            if path in ("fused", "step", "step_norm"):
                due = lv >= F
                folded = lv[due].copy()
                lens[slots] = np.where(due, 0, lv) + acc
            else:
                lens[slots] += acc
                due = lens[slots] >= F
                folded = lens[slots][due].copy()
                lens[slots[due]] = 0
            if path in ("step", "step_norm"):
                lens[slots] = np.where(due, 0, lv)
            sched.append(dict(slots=to_device(slots), acc=to_device(acc), lv=lv, folded=folded,
                              dl=None if dl is None else to_device(dl), drafts=dl, **extra))
        torch.cuda.synchronize()

        # The timed loop calls the C entry points with arguments marshalled
        # beforehand (the cache methods' per-call checks and ctypes set-up cost
        # more host time than a short kernel takes, which would time the host).
        lib = binding.load()
        sh = stream.cuda_stream
        refs = [ctypes.byref(c.struct()) for c in caches]
        ptr = lambda t: None if t is None else t.data_ptr()
        dptr = [[tuple(d[x].data_ptr() for x in ("q", "k", "v", "alpha", "beta")) for d in ds]
                for ds in drafts]
        R, D, FM = wl.num_reqs, wl.draft, wl.flush_min_len
        norms = []
        if path == "step_norm":   # per-layer gate, codes and scales; one weight
            g = torch.Generator(device="cuda").manual_seed(synth.seed_for(wl.name, 0, 94))
            w = torch.rand(wl.dv, device="cuda", generator=g) + 0.5
            for L in range(layers):
                z = torch.randn((R, D, wl.hv, wl.dv), device="cuda",
                                generator=g).to(torch.bfloat16)
                q8 = torch.empty((R, D, wl.hv, wl.dv), dtype=torch.uint8, device="cuda")
                sc = torch.empty((R, D, wl.hv), dtype=torch.float32, device="cuda")
                st = binding.GdnNormFp8(z.data_ptr(), w.data_ptr(), 1e-6, q8.data_ptr(),
                                        sc.data_ptr())
                norms.append((z, q8, sc, st, ctypes.byref(st)))
            norms.append(w)

        def prepared(step):
            sc = sched[step]
            sl, dl = ptr(sc["slots"]), ptr(sc["dl"])
            main, rb, fl = [], [], []
            for L in range(layers):
                dp = dptr[L][step % 2] + (outs[L].data_ptr(), sh)
                if path == "fused":
                    main.append((lib.gdn_replay_verify_flush, (refs[L], R, sl, D, FM) + dp)
                                if dl is None else
                                (lib.gdn_replay_verify_flush_varlen,
                                 (refs[L], R, sl, dl, D, FM) + dp))
                elif path == "step":
                    main.append((lib.gdn_replay_rollback_verify_flush,
                                 (refs[L], R, sl, ptr(sc["pacc"]), ptr(sc["plens"]), D, dl, D,
                                  FM) + dp))
                elif path == "step_norm":
                    main.append((lib.gdn_replay_step_norm_fp8,
                                 (refs[L], R, sl, ptr(sc["pacc"]), ptr(sc["plens"]), D, dl, D,
                                  FM) + dptr[L][step % 2] + (None, norms[L][4], sh)))
                else:
                    main.append((lib.gdn_replay_verify, (refs[L], R, sl, D) + dp)
                                if dl is None else
                                (lib.gdn_replay_verify_varlen, (refs[L], R, sl, dl, D) + dp))
                if path not in ("step", "step_norm"):
                    rb.append((lib.gdn_replay_rollback, (refs[L], R, sl, D, ptr(sc["acc"]), sh))
                              if dl is None else
                              (lib.gdn_replay_rollback_varlen,
                               (refs[L], R, sl, dl, D, ptr(sc["acc"]), sh)))
                if path == "separate":
                    fl.append((lib.gdn_replay_flush, (refs[L], R, sl, FM, sh)))
            return main, rb, fl

        calls = [prepared(step) for step in range(total)]
        status = []

        def run_step(step, marks):
            main, rb, fl = calls[step]
            e = [ev() for _ in range(4)]
            e[0].record(stream)
            status.extend([fn(*a) for fn, a in main])
            e[1].record(stream)
            status.extend([fn(*a) for fn, a in rb])
            e[2].record(stream)
            status.extend([fn(*a) for fn, a in fl])
            e[3].record(stream)
            marks.append(e)

        warm_marks, marks = [], []
        for step in range(args.warmup):
            run_step(step, warm_marks)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for step in range(args.warmup, total):
            run_step(step, marks)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start

        tv = tr = tf = 0.0
        vb = fb = 0
        for step in range(args.warmup, total):
            e = marks[step - args.warmup]
            tv += e[0].elapsed_time(e[1])
            tr += e[1].elapsed_time(e[2])
            tf += e[2].elapsed_time(e[3])
            sc = sched[step]
            if path in ("fused", "step", "step_norm"):
                b_v, b_f = byte_model_fused(wl, sc["lv"], sc["folded"], sc["drafts"]), 0
                if path == "step_norm":   # no fp32 outputs; gate read, codes + scales written
                    nd = wl.num_reqs * wl.draft if sc["drafts"] is None else int(sc["drafts"].sum())
                    b_v += nd * wl.hv * (wl.dv * (2 + 1 - 4) + 4) + wl.dv * 4
            else:
                b_v, b_f = byte_model(wl, sc["lv"], sc["folded"], sc["drafts"])
            vb += b_v * layers          # every layer sees the same lengths
            fb += b_f * layers
        graph_ms = graph_leg(caches, sched, path) if path in ("fused", "step") else None
        assert not any(status), f"{path}: call status {sorted(set(status))}"
        del norms
        errs = [int(c.err.item()) for c in caches]
        assert not any(errs), f"{path}: device error bits set: {errs}"
        del caches
        torch.cuda.synchronize()
        n_launch = args.steps * layers
        r = dict(wall=wall, graph_ms=graph_ms, us_verify=tv * 1e3 / n_launch,
                 us_rollback=tr * 1e3 / n_launch,
                 us_flush=tf * 1e3 / n_launch if path == "separate" else 0.0,
                 v_bytes=vb / n_launch, f_bytes=fb / n_launch)
        r["us_layer"] = r["us_verify"] + r["us_flush"]
        r["us_step_layer"] = r["us_layer"] + r["us_rollback"]
        r["bytes_layer"] = r["v_bytes"] + r["f_bytes"]
        r["gbps"] = r["bytes_layer"] / (r["us_layer"] * 1e-6) / 1e9
        r["v_gbps"] = r["v_bytes"] / (r["us_verify"] * 1e-6) / 1e9
        r["f_gbps"] = r["f_bytes"] / (r["us_flush"] * 1e-6) / 1e9 if r["us_flush"] > 0 else 0.0
        return r

    def graph_leg(caches, sched, path):
        """Secondary figure: one whole step (verify_flush then rollback on every
        layer, or rollback_verify_flush on every layer) captured once in a HIP
        graph and replayed for the timed steps' schedules, whose slot
        permutation, accept counts and lengths are copied into the graph's input
        buffers before each replay. Returns ms per replayed step (HIP events
        around each replay)."""
        clone = lambda key: None if sched[0].get(key) is None else sched[0][key].clone()
        bufs = {key: clone(key) for key in ("slots", "acc", "dl", "pacc", "plens")}
        slots_buf, acc_buf, dl_buf = bufs["slots"], bufs["acc"], bufs["dl"]
        d = drafts
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for L in range(layers):
                dd = d[L][0]
                if path == "step":
                    caches[L].rollback_verify_flush(slots_buf, bufs["pacc"], wl.draft,
                                                    wl.flush_min_len, dd["q"], dd["k"], dd["v"],
                                                    dd["alpha"], dd["beta"], out=outs[L],
                                                    prev_draft_lens=bufs["plens"],
                                                    draft_lens=dl_buf)
                else:
                    caches[L].verify_flush(slots_buf, wl.flush_min_len, dd["q"], dd["k"],
                                           dd["v"], dd["alpha"], dd["beta"], out=outs[L],
                                           draft_lens=dl_buf)
            if path != "step":
                for L in range(layers):
                    caches[L].rollback(slots_buf, wl.draft, acc_buf, draft_lens=dl_buf)
        torch.cuda.synchronize()
        times = []
        for step in range(args.warmup, total):
            for key, buf in bufs.items():
                if buf is not None:
                    buf.copy_(sched[step][key])
            e0, e1 = ev(), ev()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            times.append((e0, e1))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in times) / len(times)
        del g
        return ms

    res = {path: run_path(path) for path in paths}
    if args.copy_calib:
        nbytes = args.copy_calib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    order = next(p for p in ("fused", "separate", "step", "step_norm") if p in res)
    head = res[order]
    kernels = {}
    if "fused" in res:
        f = res["fused"]
        kernels["verify_flush"] = {"us": round(f["us_verify"], 2), "bytes": int(f["v_bytes"]),
                                   "gbps": round(f["v_gbps"], 1)}
        kernels["rollback_fused_order"] = {"us": round(f["us_rollback"], 2)}
    if "step_norm" in res:
        sn = res["step_norm"]
        kernels["step_norm_fp8"] = {"us": round(sn["us_verify"], 2), "bytes": int(sn["v_bytes"]),
                                    "gbps": round(sn["v_gbps"], 1)}
    if "step" in res:
        st = res["step"]
        kernels["rollback_verify_flush"] = {"us": round(st["us_verify"], 2),
                                            "bytes": int(st["v_bytes"]),
                                            "gbps": round(st["v_gbps"], 1)}
    if "separate" in res:
        sp = res["separate"]
        kernels["verify"] = {"us": round(sp["us_verify"], 2), "bytes": int(sp["v_bytes"]),
                             "gbps": round(sp["v_gbps"], 1)}
        kernels["flush"] = {"us": round(sp["us_flush"], 2), "bytes": int(sp["f_bytes"]),
                            "gbps": round(sp["f_gbps"], 1)}
        kernels["rollback"] = {"us": round(sp["us_rollback"], 2)}
    if order == "fused":
        dominant = "verify_flush"
    elif order == "separate":
        dominant = "verify" if kernels["verify"]["us"] >= kernels["flush"]["us"] else "flush"
    elif order == "step":
        dominant = "rollback_verify_flush"
    else:
        dominant = "step_norm_fp8"
    dom = kernels[dominant]
    line = {
        "metric": METRIC,
        "value": round(head["us_layer"], 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall"] * 1e3 / args.steps, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 state, bf16 hi/lo-split MFMA",
        "data": "synthetic",
        "config": {"workload": wl.name, "requests": wl.num_reqs, "v_heads": wl.hv,
                   "k_heads": wl.hk, "d_k": wl.dk, "d_v": wl.dv, "draft": wl.draft,
                   "ring_cap": wl.cap, "flush_min_len": wl.flush_min_len, "layers": layers,
                   "draft_lens": wl.draft_lens,
                   "inputs": wl.in_dtype, "state": "f32",
                   "order": order},
        "hbm_gbps": round(head["gbps"], 1),
        "hbm_frac": round(head["gbps"] / HBM_PEAK_GBPS, 4),
        "bytes_per_layer": int(head["bytes_layer"]),
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": dom["gbps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dom["gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dominant, wl.name),
                     "bytes_per_launch": dom["bytes"], "us_per_launch": dom["us"]},
        "pages_context": {"b200_custom_kernel_us_per_layer": "23-24",
                          "b200_triton_us_per_layer": "72-80"},
    }
    kernels["gated_rmsnorm_fp8"] = norm_leg(wl, layers, max(args.steps // 2, 5), 3)
    kernels["causal_conv_update"] = conv_leg(wl, layers, max(args.steps // 2, 5), 3)
    if "fused" in res and res["fused"]["graph_ms"] is not None:
        gm = res["fused"]["graph_ms"]
        line["graph_step"] = {"ms_per_step": round(gm, 4),
                              "us_per_layer": round(gm * 1e3 / layers, 2),
                              "what": "verify_flush + rollback on every layer, one HIP graph "
                                      "replay per step, HIP events around each replay"}
    line["whole_step_us_per_layer"] = {p: round(r["us_step_layer"], 2) for p, r in res.items()}
    if "step" in res:
        st = res["step"]
        line["one_call_step"] = {"us_per_layer": round(st["us_layer"], 2),
                                 "hbm_gbps": round(st["gbps"], 1),
                                 "bytes_per_layer": int(st["bytes_layer"]),
                                 "graph_ms_per_step": round(st["graph_ms"], 4),
                                 "what": "rollback_verify_flush on every layer: the previous "
                                         "step's rollback and the flush folded into the verify"}
    if "step_norm" in res and "step" in res:
        line["step_with_norm"] = {
            "fused_us_per_layer": round(res["step_norm"]["us_layer"], 2),
            "separate_us_per_layer": round(res["step"]["us_layer"] + kernels["gated_rmsnorm_fp8"]["us"],
                                           2),
            "what": "gdn_replay_step_norm_fp8 (codes and scales only) against "
                    "rollback_verify_flush followed by gdn_gated_rmsnorm_fp8"}
    if "separate" in res:
        sp = res["separate"]
        line["separate_order"] = {"us_per_layer": round(sp["us_layer"], 2),
                                  "hbm_gbps": round(sp["gbps"], 1),
                                  "bytes_per_layer": int(sp["bytes_layer"])}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
