#!/usr/bin/env python3
"""Benchmark of the DSpark per-step verify path on one MI355X.

One step = dspark_plan_pack (STS confidence -> survival -> budget sweep ->
verify_lens -> cu_seqlens, front-packed rows, tier; one launch) +
dspark_accept (vocab-wide argmax over the packed target logits, leading-match
count, bonus, commit, output tokens), on the B=256, gamma=8, V=129280 bf16
workload. Every input, including the packed target logits a forward pass
would have produced, is resident in HBM before the timed region. Three
copies of the packed logits rotate (about 0.56 GB of live rows), so the
256 MB Infinity Cache cannot serve repeated reads.

Prints one JSON line. ``value`` is steps/s (eager launches: K steps between
one HIP event pair, nothing else on the stream). ``roofline`` is
the accept call's achieved HBM bandwidth: algorithmic bytes per launch over
its average launch duration, 100 dedicated accept launches back to back
between one HIP event pair on the stream they run on, whatever ``--steps``
is. The same launches are also bracketed one by one after the step's
plan+pack, and an empty kernel is bracketed the same way, which shows what a
per-launch event pair adds.
``cpu_baseline`` is the untouched CPU oracle on a bounded sample of the same
step, pinned to one host core. ``schedule`` reports the planner's decision
against what the accept committed: b*, the predicted tau(b*) = B + the
selected survivals, the committed tokens, and the tier's padding, for the
timed step and over 16 seeded steps bucketed by tier.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_HBM_GBS = 8000.0
METRIC = "plan+accept steps/s and logit-pass HBM GB/s (% peak) at B=256,γ=8,V=129280"
ACC_EVERY = 4  # of the in-step accept measurement's steps, one in ACC_EVERY is bracketed
N_IN_STEP = 50  # bracketed accept calls inside steps
QUEUE_AHEAD_CYCLES = 200_000  # about 85 us of GPU spin before a timed region


def queue_ahead(torch, cycles=QUEUE_AHEAD_CYCLES):
    """A spin kernel on the current stream just before a timed region's start
    event: while the GPU runs it, the host queues the first timed launches, so
    the region measures the GPU's time and not the host's first enqueue."""
    torch.cuda._sleep(cycles)


# Regions of launches shorter than the host's enqueue of one call (the
# planner's 14 us, the pack's 4 us) are queued whole behind one longer spin:
# about 40 us of spin per launch (a ctypes call and its launch take 10-25 us
# of host time), so the timed launches run back to back on the GPU.
SPIN_CYCLES_PER_LAUNCH = 95_000
N_ACC = 100  # dedicated accept launches behind the roofline figure
N_SCHED = 16  # seeded steps behind the scheduling statistics
TRAFFIC_FILE = ROOT / "profiles" / "accept_b256_g8_v129280_bf16_traffic.json"
# the greedy accept kernels: accept.hip and the unit argmax it includes
ACCEPT_SRCS = [ROOT / "dspark_verify_scheduling_amd" / "csrc" / n
               for n in ("accept.hip", "argmax_unit.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-tv", action="store_true",
                    help="skip the soft accept-rate pass (B=256, gamma=16, V=129280 bf16)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def accept_bytes(total, B, gamma, V, esize):
    """Algorithmic bytes of one accept launch: every packed logit once, plus
    cu_seqlens, drafts, prefix lengths, and the outputs (row argmax, four
    per-request ints, out_tokens, prefix_mask)."""
    logits = total * V * esize
    inputs = (B + 1) * 4 + B * gamma * 4 + B * 4
    outputs = total * 4 + 4 * B * 4 + B * (gamma + 1) * 4 + B * gamma + 2 * 4
    return logits + inputs + outputs


def code_hash(paths):
    """sha256 of C++ sources with // comments and blank lines removed, so that
    a comment edit does not invalidate counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for p in paths:
        for line in p.read_text().splitlines():
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def traffic_for(total_rows):
    """HBM bytes per accept launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    if not TRAFFIC_FILE.exists():
        return None
    rec = json.loads(TRAFFIC_FILE.read_text())
    src_hash = code_hash(ACCEPT_SRCS)
    if rec.get("accept_src_sha256") != src_hash or rec.get("rows") != total_rows:
        return None
    return rec.get("bytes_per_launch")


def tv_bytes(B, gamma, V, esize):
    """Algorithmic bytes of one soft accept-rate call: both logit rows of every
    (draft, target) pair once, plus the accept rates and survivals written."""
    return 2 * B * gamma * V * esize + 2 * B * gamma * 4


def tv_section(dv, torch, dev, stream, reps):
    """The soft accept-rate pass and the chained step that uses it (TV
    accept-rate -> cumprod -> plan in survival mode -> pack -> accept) at
    B=256, gamma=16, V=129280 bf16."""
    from workloads import make

    w = make(4)
    B, G, V = w.B, w.gamma, w.V
    f32 = torch.float32
    q = torch.from_numpy(w.draft_logits.reshape(B * G, V).view(np.int16)).to(dev)
    p = torch.from_numpy(w.target.reshape(B * (G + 1), V).view(np.int16)).to(dev)
    q, p = q.view(torch.bfloat16), p.view(torch.bfloat16)
    a = torch.empty(B * G, dtype=f32, device=dev)
    S = torch.empty(B * G, dtype=f32, device=dev)

    def tv():
        dv.dspark_tv_accept(B, G, V, dv.BF16, q, V, p, V, G + 1, a, S, stream)

    # about 10 ms of warm-up: with only a few calls the first timed ones still
    # ran up to 20% slower
    for _ in range(25):
        tv()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    queue_ahead(torch)
    ev0.record(stream)
    for _ in range(reps):
        tv()
    ev1.record(stream)
    torch.cuda.synchronize()
    tv_us = 1e3 * ev0.elapsed_time(ev1) / reps
    gbs = tv_bytes(B, G, V, 2) / (tv_us * 1e-6) / 1e9

    # chained step on the TV survivals
    def t(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    alpha_t, theta_t = t(w.alpha), t(w.theta)
    anchors_t, drafts_t, prefix_t = t(w.anchors), t(w.drafts), t(w.prefix_lens)
    tiers = [int(x) for x in w.tiers]
    po = dv.alloc_plan_outputs(B, G, dev, survival=False, sweep=False)
    ko = dv.alloc_pack_outputs(B, tiers[-1], dev)

    def plan_pack():
        dv.dspark_plan_pack(B, G, dv.IN_SURVIVAL, S, None, w.min_len, w.max_len, w.eps,
                            w.b_lo, w.b_hi, float(w.bias), alpha_t, theta_t, po,
                            anchors_t, drafts_t, tiers, prefix_t, ko, stream)

    tv()
    plan_pack()
    torch.cuda.synchronize()
    lens = po.verify_lens.cpu().numpy()
    cu = ko.cu_seqlens.cpu().numpy()
    total, tier = int(ko.pack_meta[0].item()), int(ko.pack_meta[1].item())
    req = np.repeat(np.arange(B), lens)
    src = torch.from_numpy(req * (G + 1) + np.arange(total) - np.repeat(cu[:-1], lens)).to(dev)
    packed = torch.zeros(tier, V, dtype=torch.int16, device=dev)
    packed[:total] = p.view(torch.int16).index_select(0, src)
    packed = packed.view(torch.bfloat16)
    ao = dv.alloc_accept_outputs(B, G, tier, V, dv.BF16, dev)

    def chain():
        tv()
        plan_pack()
        dv.dspark_accept(B, G, V, dv.BF16, packed, V, tier, ko.cu_seqlens, drafts_t, prefix_t,
                         ao, stream)

    for _ in range(10):
        chain()
    torch.cuda.synchronize()
    queue_ahead(torch)
    ev0.record(stream)
    for _ in range(reps):
        chain()
    ev1.record(stream)
    torch.cuda.synchronize()
    chain_us = 1e3 * ev0.elapsed_time(ev1) / reps
    assert np.array_equal(po.verify_lens.cpu().numpy(), lens)
    assert int(ao.accept_meta[1].item()) == 0
    return {
        "workload": f"{w.spec.name}: B={B} gamma={G} V={V} bf16",
        "tv_us": tv_us, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS,
        "bytes_per_launch": tv_bytes(B, G, V, 2),
        "chained_step_us": chain_us, "rows": total, "tier": tier,
    }


def host_facts():
    """Logical CPUs this process may use and the host CPU's model name."""
    model = None
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "cpu_model": model}


def schedule_record(po, ao, total, tier):
    """The planner's decision against what the accept committed, for one step:
    b*, the predicted tau(b*) = B + the selected survivals (the expected
    committed tokens under the calibrated survivals), the tokens committed
    (sum of commit_lens, bonus included), and the tier's padding."""
    meta = po.plan_meta.cpu().numpy()
    tau = float(po.plan_val[0].item())
    committed = int(ao.commit_lens.sum().item())
    return {"b_star": int(meta[0]), "n_eligible": int(meta[1]), "rows": total, "tier": tier,
            "padding_ratio": (tier - total) / tier, "predicted_tau": tau,
            "committed": committed, "committed_minus_tau": committed - tau}


SCHED_SHIFTS = (-1.5, 0.0, 1.5, 4.0)  # confidence-logit mean shifts of the seeded steps


def schedule_stats(dv, torch, dev, stream, n):
    """The step on n seeded B=256, gamma=8, V=129280 workloads (metadata seeds
    50000..50000+n-1, the confidence-logit mean shifted by SCHED_SHIFTS in
    turn so that the steps use different tiers): each plans and packs on the
    GPU, its packed rows are filled on the GPU with N(0, 3) clipped to +-15 (a
    seeded torch generator) and the planted maximum 16 at each row's planted
    id (no planted ties), then the accept runs. Records are bucketed by the
    tier the step used."""
    from workloads import make

    gen = torch.Generator(device=dev)
    gen.manual_seed(20260611)
    recs = []
    for i in range(n):
        w = make(3, seed=50000 + i, logits=False, conf_shift=SCHED_SHIFTS[i % len(SCHED_SHIFTS)])
        B, G, V = w.B, w.gamma, w.V
        tiers = [int(x) for x in w.tiers]

        def t(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        po = dv.alloc_plan_outputs(B, G, dev, survival=False, sweep=False)
        ko = dv.alloc_pack_outputs(B, tiers[-1], dev)
        drafts_t, prefix_t = t(w.drafts), t(w.prefix_lens)
        dv.dspark_plan_pack(B, G, dv.IN_CONF_LOGITS, t(w.conf), t(w.temps), w.min_len,
                            w.max_len, w.eps, w.b_lo, w.b_hi, float(w.bias), t(w.alpha),
                            t(w.theta), po, t(w.anchors), drafts_t, tiers, prefix_t, ko, stream)
        torch.cuda.synchronize()
        lens = po.verify_lens.cpu().numpy()
        cu = ko.cu_seqlens.cpu().numpy()
        total, tier = int(ko.pack_meta[0].item()), int(ko.pack_meta[1].item())
        req = np.repeat(np.arange(B), lens)
        jrow = np.arange(total) - np.repeat(cu[:-1], lens)
        top = torch.from_numpy(w.planted_top[req, jrow].astype(np.int64)).to(dev)
        rows = torch.empty(tier, V, dtype=torch.float32, device=dev)
        rows.normal_(0.0, 3.0, generator=gen).clamp_(-15.0, 15.0)
        rows[torch.arange(total, device=dev), top] = 16.0
        packed = rows.to(torch.bfloat16)
        del rows
        ao = dv.alloc_accept_outputs(B, G, tier, V, dv.BF16, dev)
        dv.dspark_accept(B, G, V, dv.BF16, packed, V, tier, ko.cu_seqlens, drafts_t, prefix_t,
                         ao, stream)
        torch.cuda.synchronize()
        assert int(ao.accept_meta[1].item()) == 0
        recs.append(schedule_record(po, ao, total, tier))
        del packed
    buckets = {}
    for r in recs:
        buckets.setdefault(r["tier"], []).append(r)
    out = {}
    for tier, rs in sorted(buckets.items()):
        out[str(tier)] = {
            "steps": len(rs),
            "mean_b_star": statistics.mean(r["b_star"] for r in rs),
            "mean_rows": statistics.mean(r["rows"] for r in rs),
            "mean_padding_ratio": statistics.mean(r["padding_ratio"] for r in rs),
            "mean_predicted_tau": statistics.mean(r["predicted_tau"] for r in rs),
            "mean_committed": statistics.mean(r["committed"] for r in rs),
            "mean_committed_minus_tau": statistics.mean(r["committed_minus_tau"] for r in rs),
        }
    torch.cuda.empty_cache()
    return {"steps": n, "conf_shifts": list(SCHED_SHIFTS), "by_tier": out}


def cpu_baseline(w, lens_ref, packed_host, total, budget_s):
    """The oracle as it stands, pinned to one host core: full plan and pack,
    accept on a 32-row sample of the packed logits, scaled to the step's
    rows."""
    import oracle
    from oracle.accept import as_f32_rows

    facts = host_facts()
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    try:
        res = _cpu_baseline_pinned(oracle, as_f32_rows, w, lens_ref, packed_host, total,
                                   budget_s)
    finally:
        os.sched_setaffinity(0, set(allowed))
    res.update(facts)
    res["pinned_core"] = core
    return res


def _cpu_baseline_pinned(oracle, as_f32_rows, w, lens_ref, packed_host, total, budget_s):
    sample_rows = 32
    t_plan, t_pack, t_row = [], [], []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or not t_plan:
        t0 = time.perf_counter()
        rp = oracle.plan(w.B, w.gamma, oracle.IN_CONF_LOGITS, w.conf, w.temps, w.min_len,
                         w.max_len, w.eps, w.b_lo, w.b_hi, w.bias, w.alpha, w.theta)
        t1 = time.perf_counter()
        rk = oracle.pack(w.B, w.gamma, rp["verify_lens"], w.anchors, w.drafts, w.tiers,
                         w.prefix_lens)
        t2 = time.perf_counter()
        rows = packed_host[:sample_rows]
        oracle.row_argmax(as_f32_rows(rows, "bf16" if rows.dtype == np.uint16 else "f32"))
        t3 = time.perf_counter()
        assert np.array_equal(rp["verify_lens"], lens_ref)
        t_plan.append(t1 - t0)
        t_pack.append(t2 - t1)
        t_row.append((t3 - t2) / sample_rows)
    step = statistics.median(t_plan) + statistics.median(t_pack) + statistics.median(t_row) * total
    return {
        "value": 1.0 / step,
        "unit": "steps/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(t_plan)} repetitions of the full plan + pack and of the row argmax on "
                   f"{sample_rows} of the {total} packed bf16 rows; the per-row time is scaled to "
                   f"{total} rows (median of repetitions); the process pinned to one core"),
        "ms_plan": 1e3 * statistics.median(t_plan),
        "ms_pack": 1e3 * statistics.median(t_pack),
        "ms_accept_per_row": 1e3 * statistics.median(t_row),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; the per-step verify path "
                                   "would shard by request across GPUs, but no multi-GPU run "
                                   "is provided", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import dspark_verify_scheduling_amd as dv
    from workloads import make
    from workloads.gen import sampling_extras

    dev = "cuda"
    dv.load()
    log(f"generating workload {args.config}")
    w = make(args.config)
    B, G, V = w.B, w.gamma, w.V
    dt = dv.BF16 if w.dtype == "bf16" else dv.F32
    tdt = torch.bfloat16 if dt == dv.BF16 else torch.float32
    esize = 2 if dt == dv.BF16 else 4
    cap = int(w.tiers[-1])

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    conf_t, temps_t = t(w.conf), t(w.temps)
    alpha_t, theta_t = t(w.alpha), t(w.theta)
    anchors_t, drafts_t, prefix_t = t(w.anchors), t(w.drafts), t(w.prefix_lens)
    tiers = [int(x) for x in w.tiers]
    po = dv.alloc_plan_outputs(B, G, dev, survival=False, sweep=False)
    ko = dv.alloc_pack_outputs(B, cap, dev)

    # plan once to learn the packed layout; the stand-in for the target
    # forward fills the packed logits for exactly those rows
    dv.dspark_plan(B, G, dv.IN_CONF_LOGITS, conf_t, temps_t, w.min_len, w.max_len, w.eps,
                   w.b_lo, w.b_hi, float(w.bias), alpha_t, theta_t, po)
    dv.dspark_pack(B, G, po.verify_lens, anchors_t, drafts_t, tiers, prefix_t, ko)
    torch.cuda.synchronize()
    lens = po.verify_lens.cpu().numpy()
    cu = ko.cu_seqlens.cpu().numpy()
    total, tier = int(ko.pack_meta[0].item()), int(ko.pack_meta[1].item())
    req = np.repeat(np.arange(B), lens)
    jrow = np.arange(total) - np.repeat(cu[:-1], lens)
    src = torch.from_numpy(req * (G + 1) + jrow).to(dev)
    host_view = w.target.reshape(B * (G + 1), V)
    strided = torch.from_numpy(host_view.view(np.int16) if dt == dv.BF16 else host_view).to(dev)
    if dt == dv.BF16:
        strided = strided.view(torch.bfloat16)
    n_rot = 3
    packed = []
    for _ in range(n_rot):
        buf = torch.zeros(tier, V, dtype=tdt, device=dev)
        buf[:total] = strided.index_select(0, src)
        packed.append(buf)
    packed_host = w.target[req[:64], jrow[:64]]  # rows for the CPU sample
    del strided
    torch.cuda.empty_cache()
    ao = dv.alloc_accept_outputs(B, G, tier, V, dt, dev)
    log(f"B={B} gamma={G} V={V}: total={total} rows, tier={tier}, "
        f"{n_rot} rotating buffers of {total * V * esize / 2**20:.1f} MiB")

    stream = torch.cuda.current_stream()

    def plan_pack(stream=None):
        dv.dspark_plan_pack(B, G, dv.IN_CONF_LOGITS, conf_t, temps_t, w.min_len, w.max_len,
                            w.eps, w.b_lo, w.b_hi, float(w.bias), alpha_t, theta_t, po,
                            anchors_t, drafts_t, tiers, prefix_t, ko, stream)

    def step(i):  # on the current stream (graph capture switches it)
        plan_pack()
        dv.dspark_accept(B, G, V, dt, packed[i % n_rot], V, tier, ko.cu_seqlens, drafts_t,
                         prefix_t, ao)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed: K eager steps, nothing else on the stream between the two
    # events
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    queue_ahead(torch)
    start.record(stream)
    for i in range(args.steps):
        plan_pack(stream)
        dv.dspark_accept(B, G, V, dt, packed[i % n_rot], V, tier, ko.cu_seqlens, drafts_t,
                         prefix_t, ao, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps

    # ---- the accept call inside a step: further steps (after the timed
    # ones) whose accept call every ACC_EVERY-th step is bracketed by an event
    # pair (a pair costs about 3 us, so the other steps run without one)
    n_in = ACC_EVERY * N_IN_STEP
    ev_a0 = [torch.cuda.Event(enable_timing=True) for _ in range(N_IN_STEP)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(N_IN_STEP)]
    torch.cuda.synchronize()
    for i in range(n_in):
        plan_pack(stream)
        if i % ACC_EVERY == 0:
            ev_a0[i // ACC_EVERY].record(stream)
        dv.dspark_accept(B, G, V, dt, packed[i % n_rot], V, tier, ko.cu_seqlens, drafts_t,
                         prefix_t, ao, stream)
        if i % ACC_EVERY == 0:
            ev_a1[i // ACC_EVERY].record(stream)
    torch.cuda.synchronize()
    acc_us = [1e3 * ev_a0[j].elapsed_time(ev_a1[j]) for j in range(N_IN_STEP)]
    acc_mean_us = statistics.mean(acc_us)

    # results of the timed steps must be the planned ones
    assert np.array_equal(po.verify_lens.cpu().numpy(), lens)
    assert int(ao.accept_meta[1].item()) == 0
    sched_step = schedule_record(po, ao, total, tier)

    # ---- the accept roofline: N_ACC dedicated launches, each after the step's
    # plan+pack (as in a step) and bracketed by its own event pair on the
    # accept's stream; then the same launches back to back under one pair
    ea0 = [torch.cuda.Event(enable_timing=True) for _ in range(N_ACC)]
    ea1 = [torch.cuda.Event(enable_timing=True) for _ in range(N_ACC)]
    torch.cuda.synchronize()
    for i in range(N_ACC):
        plan_pack(stream)
        ea0[i].record(stream)
        dv.dspark_accept(B, G, V, dt, packed[i % n_rot], V, tier, ko.cu_seqlens, drafts_t,
                         prefix_t, ao, stream)
        ea1[i].record(stream)
    torch.cuda.synchronize()
    acc_ded_us = [1e3 * ea0[i].elapsed_time(ea1[i]) for i in range(N_ACC)]
    # what one event pair around one launch after plan+pack costs by itself:
    # the same bracket around the smallest kernel torch launches
    floor_buf = torch.empty(1, dtype=torch.float32, device=dev)
    for i in range(N_ACC):
        plan_pack(stream)
        ea0[i].record(stream)
        floor_buf.zero_()
        ea1[i].record(stream)
    torch.cuda.synchronize()
    bracket_floor_us = statistics.median(1e3 * ea0[i].elapsed_time(ea1[i]) for i in range(N_ACC))
    queue_ahead(torch)
    start.record(stream)
    for i in range(N_ACC):
        dv.dspark_accept(B, G, V, dt, packed[i % n_rot], V, tier, ko.cu_seqlens, drafts_t,
                         prefix_t, ao, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    acc_b2b_us = 1e3 * start.elapsed_time(stop) / N_ACC
    assert int(ao.accept_meta[1].item()) == 0

    # ---- plan+pack, plan and pack alone (events), and one step as a HIP graph replay
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    reps = 50
    regions = [lambda: plan_pack(stream),
               lambda: dv.dspark_plan(B, G, dv.IN_CONF_LOGITS, conf_t, temps_t, w.min_len,
                                      w.max_len, w.eps, w.b_lo, w.b_hi, float(w.bias), alpha_t,
                                      theta_t, po, stream),
               lambda: dv.dspark_pack(B, G, po.verify_lens, anchors_t, drafts_t, tiers, prefix_t,
                                      ko, stream)]
    for j, launch in enumerate(regions):
        torch.cuda.synchronize()
        queue_ahead(torch, reps * SPIN_CYCLES_PER_LAUNCH)
        ev[2 * j].record(stream)
        for _ in range(reps):
            launch()
        ev[2 * j + 1].record(stream)
    torch.cuda.synchronize()
    plan_pack_us, plan_us, pack_us = (1e3 * ev[2 * j].elapsed_time(ev[2 * j + 1]) / reps
                                      for j in range(3))

    # launch floor of the latency-bound planner: one event pair around a single
    # launch, the queue drained before each, for plan+pack and for the smallest
    # kernel torch launches (a one-element fill); medians of 50
    floor_t = torch.empty(1, dtype=torch.float32, device=dev)

    def single_launch_us(launch):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        out = []
        for _ in range(50):
            torch.cuda.synchronize()
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(1e3 * e0.elapsed_time(e1))
        return statistics.median(out)

    plan_pack_single_us = single_launch_us(lambda: plan_pack(stream))
    launch_floor_us = single_launch_us(floor_t.zero_)

    graphs = []
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        step(0)
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    for i in range(n_rot):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % n_rot].replay()
    torch.cuda.synchronize()
    queue_ahead(torch)
    start.record(stream)
    for i in range(args.steps):
        graphs[i % n_rot].replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step_graph = start.elapsed_time(stop) / args.steps
    assert np.array_equal(po.verify_lens.cpu().numpy(), lens)
    # the three rotating steps in one graph: the replay boundary (the GPU idles
    # between two graph launches) is paid once per three steps
    g3 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g3):
        for i in range(n_rot):
            step(i)
    for _ in range(max(1, args.warmup // n_rot)):
        g3.replay()
    torch.cuda.synchronize()
    reps3 = max(1, args.steps // n_rot)
    queue_ahead(torch)
    start.record(stream)
    for _ in range(reps3):
        g3.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step_graph3 = start.elapsed_time(stop) / (reps3 * n_rot)
    assert np.array_equal(po.verify_lens.cpu().numpy(), lens)

    # ---- fixed-shape roofline: static mode, every request verifies gamma + 1 rows
    static_rows = B * (G + 1)
    cu_static = torch.arange(0, static_rows + 1, G + 1, dtype=torch.int32, device=dev)
    stat_bufs = []
    host_all = w.target.reshape(static_rows, V)
    for _ in range(2):
        tb = torch.from_numpy(host_all.view(np.int16) if dt == dv.BF16 else host_all).to(dev)
        stat_bufs.append(tb.view(torch.bfloat16) if dt == dv.BF16 else tb)
    ao_s = dv.alloc_accept_outputs(B, G, static_rows, V, dt, dev)
    for i in range(5):
        dv.dspark_accept(B, G, V, dt, stat_bufs[i % 2], V, static_rows, cu_static, drafts_t,
                         prefix_t, ao_s, stream)
    torch.cuda.synchronize()
    queue_ahead(torch)
    start.record(stream)
    n_static = 50
    for i in range(n_static):
        dv.dspark_accept(B, G, V, dt, stat_bufs[i % 2], V, static_rows, cu_static, drafts_t,
                         prefix_t, ao_s, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    static_us = 1e3 * start.elapsed_time(stop) / n_static
    static_gbs = accept_bytes(static_rows, B, G, V, esize) / (static_us * 1e-6) / 1e9

    # ---- cap-accept on the same strided rows (full block verified, commits
    # capped by the planned lengths) and the scatter of the planned packed rows
    # back to stride
    co = dv.alloc_cap_accept_outputs(B, G, V, dt, dev)
    lens_t = po.verify_lens

    def cap(i):
        dv.dspark_cap_accept(B, G, V, dt, stat_bufs[i % 2], V, lens_t, drafts_t, prefix_t, co,
                             stream)

    for i in range(5):
        cap(i)
    torch.cuda.synchronize()
    queue_ahead(torch)
    start.record(stream)
    for i in range(n_static):
        cap(i)
    stop.record(stream)
    torch.cuda.synchronize()
    cap_us = 1e3 * start.elapsed_time(stop) / n_static
    assert int(co.accept_meta[1].item()) == 0
    cap_gbs = accept_bytes(static_rows, B, G, V, esize) / (cap_us * 1e-6) / 1e9
    del stat_bufs
    torch.cuda.empty_cache()
    dst = torch.empty(static_rows, V, dtype=tdt, device=dev)
    smeta = torch.empty(2, dtype=torch.int32, device=dev)

    def scat(i):
        dv.dspark_scatter_to_strided(B, G + 1, ko.cu_seqlens, packed[i % n_rot], dst, V, smeta,
                                     stream)

    for i in range(5):
        scat(i)
    torch.cuda.synchronize()
    queue_ahead(torch)
    start.record(stream)
    for i in range(n_static):
        scat(i)
    stop.record(stream)
    torch.cuda.synchronize()
    scat_us = 1e3 * start.elapsed_time(stop) / n_static
    assert smeta.tolist() == [total, 0]
    scat_bytes = 2 * total * V * esize + (B + 1) * 4
    scat_gbs = scat_bytes / (scat_us * 1e-6) / 1e9
    # its practical ceiling: torch's device copy of the same rows, contiguous
    for i in range(5):
        dst[:total].copy_(packed[i % n_rot][:total])
    torch.cuda.synchronize()
    queue_ahead(torch)
    start.record(stream)
    for i in range(n_static):
        dst[:total].copy_(packed[i % n_rot][:total])
    stop.record(stream)
    torch.cuda.synchronize()
    copy_us = 1e3 * start.elapsed_time(stop) / n_static
    copy_gbs = 2 * total * V * esize / (copy_us * 1e-6) / 1e9
    del dst
    torch.cuda.empty_cache()

    # ---- chain speculative-sampling accept on the same planned layout: every
    # request samples (temperatures 0.6..1.4); draft rows drawn with the
    # draft-logit recipe of the generator, two copies rotating
    log("sampling accept on the planned layout")
    ex = sampling_extras(w)
    n_drot = 2
    dl_host = ex.draft_logits.reshape(B * G, V)
    drf_bufs = []
    for _ in range(n_drot):
        tb = torch.from_numpy(dl_host.view(np.int16) if dt == dv.BF16 else dl_host).to(dev)
        drf_bufs.append(tb.view(torch.bfloat16) if dt == dv.BF16 else tb)
    del dl_host
    stemps_t = t(ex.temps)
    ra_t = t(ex.rand_accept.view(np.int32))
    rs_t = t(ex.rand_sample.view(np.int32))
    so = dv.alloc_sampling_outputs(B, G, V, dt, dev)

    def samp(i):
        dv.dspark_accept_sampling(B, G, V, dt, packed[i % n_rot], V, tier, ko.cu_seqlens,
                                  drf_bufs[i % n_drot], V, drafts_t, stemps_t, ra_t, rs_t,
                                  prefix_t, so, stream)

    for i in range(5):
        samp(i)
    torch.cuda.synchronize()
    n_samp = 50
    queue_ahead(torch)
    start.record(stream)
    for i in range(n_samp):
        samp(i)
    stop.record(stream)
    torch.cuda.synchronize()
    samp_us = 1e3 * start.elapsed_time(stop) / n_samp
    assert so.accept_meta.tolist() == [total, 0]
    live_drafts = int(np.sum(lens - 1))  # every request samples
    samp_bytes = (total + live_drafts) * V * esize
    samp_gbs = samp_bytes / (samp_us * 1e-6) / 1e9
    samp_res = {"rows_target": total, "rows_draft": live_drafts, "us": samp_us, "GB/s": samp_gbs,
                "frac": samp_gbs / PEAK_HBM_GBS, "bytes": samp_bytes,
                "mean_correct": float(so.num_correct.float().mean().item())}
    del drf_bufs
    torch.cuda.empty_cache()

    acc_bytes = accept_bytes(total, B, G, V, esize)
    acc_ded_mean_us = statistics.mean(acc_ded_us)
    achieved = acc_bytes / (acc_b2b_us * 1e-6) / 1e9

    log(f"scheduling statistics over {N_SCHED} seeded steps")
    sched_seeded = schedule_stats(dv, torch, dev, stream, N_SCHED)

    # ---- STS fitter: 65536 records of gamma = 8, 64 grid temperatures, 15 bins
    rng = np.random.default_rng(5)
    n_rec = 65536
    z_rec = (rng.normal(1.2, 1.2, (n_rec, G)) - 0.3 * np.arange(1, G + 1)).astype(np.float32)
    p_acc = 1.0 / (1.0 + np.exp(-z_rec.astype(np.float64) / 1.3))
    y_rec = np.cumprod(rng.random((n_rec, G)) < p_acc, axis=1).astype(np.uint8)
    z_t, y_t = t(z_rec), t(y_rec)
    sts_grid = np.exp(np.linspace(np.log(0.25), np.log(4.0), 64)).astype(np.float32)
    for _ in range(2):
        fit = dv.dspark_sts_fit(z_t, y_t, sts_grid, 15, ece_grid=False, stream=stream)
    torch.cuda.synchronize()
    queue_ahead(torch)
    start.record(stream)
    for _ in range(5):
        fit = dv.dspark_sts_fit(z_t, y_t, sts_grid, 15, ece_grid=False, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    sts_us = 1e3 * start.elapsed_time(stop) / 5
    sts_res = {"records": n_rec, "gamma": G, "grid": int(sts_grid.size), "bins": 15,
               "us": sts_us, "temps": [round(float(x), 4) for x in fit.temps.cpu()]}

    tv_res = None
    if not args.no_tv:
        log("soft accept-rate pass at B=256, gamma=16, V=129280 bf16")
        tv_res = tv_section(dv, torch, dev, stream, 20)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(w, lens, packed_host, total, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": 1e3 / ms_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.spec.name}: B={B} gamma={G} V={V} {w.dtype}, planned packed rows",
                   "B": B, "gamma": G, "V": V, "rows": total, "tier": tier, "seed": w.seed,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_for(total),
                     "kernel": "dspark_accept: accept_argmax_kernel<bf16> then accept_finalize_kernel",
                     "bytes_per_launch": acc_bytes,
                     "mean_us": acc_b2b_us,
                     "timed_launches": N_ACC,
                     "timing": "back to back between one event pair on the accept's stream",
                     "per_launch_after_plan": {
                         "mean_us": acc_ded_mean_us,
                         "p10_us": float(np.percentile(acc_ded_us, 10)),
                         "p50_us": float(np.percentile(acc_ded_us, 50)),
                         "p90_us": float(np.percentile(acc_ded_us, 90)),
                         "frac": acc_bytes / (acc_ded_mean_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                         "empty_kernel_same_bracket_us": bracket_floor_us,
                         "launches": len(acc_ded_us)},
                     "in_step_mean_us": acc_mean_us,
                     "in_step_timed_launches": len(acc_us)},
        "cpu_baseline": cpu,
        "schedule": {"step": sched_step, "seeded_steps": sched_seeded},
        "steps_per_s_graph": 1e3 / ms_step_graph,
        "ms_per_step_graph": ms_step_graph,
        "steps_per_s_graph_3_steps": 1e3 / ms_step_graph3,
        "ms_per_step_graph_3_steps": ms_step_graph3,
        "plan_pack_us": plan_pack_us,
        "plan_us": plan_us,
        "pack_us": pack_us,
        "plan_pack_single_launch_us": plan_pack_single_us,
        "launch_floor_us": launch_floor_us,
        "accept_us_median": statistics.median(acc_us),
        "accept_static": {"rows": static_rows, "us": static_us, "GB/s": static_gbs,
                          "frac": static_gbs / PEAK_HBM_GBS},
        "cap_accept": {"rows": static_rows, "us": cap_us, "GB/s": cap_gbs,
                       "frac": cap_gbs / PEAK_HBM_GBS},
        "scatter_to_strided": {"rows": total, "us": scat_us, "GB/s": scat_gbs,
                               "frac": scat_gbs / PEAK_HBM_GBS, "bytes": scat_bytes,
                               "torch_copy_same_rows_us": copy_us,
                               "torch_copy_GB/s": copy_gbs},
        "sampling_accept": samp_res,
        "sts_fit": sts_res,
        "tv_pass": tv_res,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
