#!/usr/bin/env python3
"""Benchmark of the DiffKV hot path on one MI355X.

Workload: one Llama3-8B-shaped attention layer -- 32 q / 8 KV heads, d = 128,
batch 32, 4096-token contexts, fp16 K/V ~ N(0,1) with 4 outlier channels x8
per KV head, importance scores Zipf(1.1) with a per-unit random permutation,
alpha_h = 1.0, alpha_l = 0.2, W = 64, a pool of 1.25x the conservative need.

A timed step is one decode step of the whole batch on the compacted cache:
generation-step compaction, then decode attention with the score update, as
one diffkv_decode_step call: one kernel that commits each unit's step and
attends over it when every unit is one workgroup.  Each replica's steps are
chained (a step's score update plans the next one into the workspace; the
first step of a chain runs a plan kernel first, done in the warmup).  The
prompt side of the path (classification and prompt compaction) and the
release are timed in the same run on the same caches and reported beside it.
Caches rotate over several independent replicas (one per simulated layer) so
that the 256 MB Infinity Cache cannot hold the working set.

value = batch * steps / (time of the timed region): request-tokens per second
of complete decode steps (timed as 8 back-to-back segments; their spread is
reported as p10/p50/p90 per step).  Three kinds of segments are timed with HIP events on the
stream the library launches on, each over back-to-back launches while a spin
kernel issued before the start event holds the stream (so the events measure
the device, not the host's launch rate): the K complete steps (value), K
attention launches alone on the final caches (attn_us, roofline), and K more
compaction steps alone through the separate kernels (compaction_us_per_step).
The compaction's share of a step is (step - attention alone) / step.  The
roofline object
describes the attention kernel: algorithmic bytes per launch (codes +
metadata of every retained token, q, out, table entries, and the 8-byte
read-modify-write of each retained token's score) over its mean duration;
stream_read_GBps is the box's achievable read rate (a reduction over 4 GiB),
the practical ceiling beside the 8 TB/s peak.  The oracle baseline runs first
(before the process touches the GPU), on one thread and as several processes.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed decode-attn tokens/s + compaction µs/step; % peak HBM GB/s"
WORKLOAD_NAMES = {"llama3_8b": "llama3_8b_layer", "long": "long_context", "churn": "decode_churn",
                  "stress_gqa7": "stress_gqa7_lo_off", "stress_gqa8": "stress_gqa8", "tiny": "tiny"}
PEAK_HBM_GBS = 8000.0


def algorithmic_attn_bytes(tier_state, B, H, G, d):
    """Bytes the attention with score update must move: per retained hi token
    1.5d + 8 (codes + K/V scale/zero), per lo token 0.75d + 8, q (fp16) and out
    (fp32) rows, 4 bytes per page-table entry read, and 8 bytes per retained
    token for the score read-modify-write."""
    ts = tier_state.reshape(-1, 4).astype("int64")
    n_hi, n_lo, ph, pl = ts[:, 0].sum(), ts[:, 1].sum(), ts[:, 2].sum(), ts[:, 3].sum()
    return int(n_hi * (1.5 * d + 8) + n_lo * (0.75 * d + 8) + B * H * G * d * (2 + 4) + 4 * (ph + pl)
               + 8 * (n_hi + n_lo))


KERNEL_SOURCES = ("compressed_paged_attention_amd/csrc/attention.hip",
                  "compressed_paged_attention_amd/csrc/dkv_common.hpp",
                  "compressed_paged_attention_amd/csrc/dkv_step.hpp",
                  "compressed_paged_attention_amd/csrc/dkv_launch.hpp")
TRAFFIC_FILE = "profiles/attn_kernel_llama3_8b_traffic.txt"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when the summary is missing or the kernel sources changed since."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and not line.startswith((" ", "#", "|")):
                kv[parts[0]] = parts[1]
    if kv.get("source_sha256") != kernel_source_hash() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def stream_read_gbps(gib=4, reps=10):
    """Achievable HBM read rate on this machine: row sums over a `gib` GiB
    buffer viewed as 4096-float rows (torch's own kernel; the fastest
    torch reduction measured here, 6.2 TB/s against 3.8 for a full sum),
    best of `reps`."""
    import torch
    x = torch.ones(gib << 28, dtype=torch.float32, device="cuda:0")
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        x.view(-1, 4096).sum(dim=1)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    del x
    torch.cuda.empty_cache()
    return (gib << 30) / best / 1e9


def copy_probe(mib):
    """One elementwise copy of a known size (reads and writes `mib` MiB):
    the calibration point for the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y
    torch.cuda.empty_cache()
    print(f"[bench] copy probe: {mib} MiB read + {mib} MiB written", file=sys.stderr, flush=True)


def _oracle_steps(cfg, n_req, n_steps, barrier=None):
    """Prompt compaction, then n_steps decode steps of the oracle on n_req
    requests of the workload; returns (prompt s, step s)."""
    import numpy as np

    import oracle
    from workloads import synth
    c = dict(cfg, batch=n_req)
    lens = synth.seq_lens(c)
    pr = synth.make_prompt(c, lens=lens)
    P = synth.pool_pages(c, lens, oracle.page_bytes(c))
    st = oracle.State(c, n_req, P)
    cu = pr["cu_seqlens"].numpy()
    t0 = time.perf_counter()
    tiers, _ = oracle.classify(c, cu, pr["scores"].numpy())
    st.compact_prompt(cu, pr["k"].numpy(), pr["v"].numpy(), pr["scores"].numpy(), tiers)
    t_prompt = time.perf_counter() - t0
    seq = lens.numpy().astype(np.int32)
    decs = [synth.make_decode(c, s, batch=n_req) for s in range(n_steps)]
    if barrier is not None:
        barrier.wait()
    t0 = time.perf_counter()
    for s in range(n_steps):
        dec = decs[s]
        st.compact_step(seq, dec["k_new"].numpy(), dec["v_new"].numpy())
        st.decode_attn(dec["q"].numpy(), seq, update_scores=True)
        seq += 1
    t_step = (time.perf_counter() - t0) / n_steps
    return t_prompt, t_step


_BARRIER = None


def _pool_init(b):
    global _BARRIER
    _BARRIER = b


def _oracle_worker_b(args):
    import torch
    torch.set_num_threads(1)
    cfg, n_req, n_steps = args
    return _oracle_steps(cfg, n_req, n_steps, _BARRIER)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(cfg, n_req, n_steps, workers):
    """The oracle timed on this host on a bounded sample of the same workload:
    once on one thread, once as `workers` processes (each n_req / 4 requests
    of its own, steps started together).  Runs before the process touches
    the GPU (the workers are forked)."""
    import multiprocessing as mp
    t_prompt, t_step = _oracle_steps(cfg, n_req, n_steps)
    single = dict(value=n_req / t_step, cores=1,
                  sample=f"{n_req} of {cfg['batch']} requests ({n_req * cfg['num_kv_heads']} units, "
                         f"{cfg['seq'][0]} tokens each): prompt compaction once "
                         f"({t_prompt:.2f} s, not in value), then {n_steps} decode steps "
                         f"(step compaction + fp64 attention + score update), "
                         f"{t_step * 1e3:.1f} ms per step")
    per = max(1, n_req // 4)
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers)
    with ctx.Pool(workers, initializer=_pool_init, initargs=(barrier,)) as pool:
        res = pool.map(_oracle_worker_b, [(cfg, per, n_steps)] * workers)
    value = sum(per / ts for _, ts in res)
    return dict(value=value, unit="request-tokens/s", cores=workers, kind="oracle",
                sample=f"{workers} processes, each {per} requests ({per * cfg['num_kv_heads']} units, "
                       f"{cfg['seq'][0]} tokens each) through prompt compaction, then {n_steps} decode "
                       f"steps (step compaction + fp64 attention + score update) started together; "
                       f"value = sum of the processes' request-tokens/s",
                single_thread=single, cpu=cpu_model(),
                nproc=os.cpu_count())


def churn_schedule(args):
    """Decode churn as the workload defines it: 128 requests with contexts
    U[1K, 16K] and output budgets U[1, 512]; every step appends one token per
    request (diffkv_decode_step with the score update); a request that has
    used its budget is released in the same step and its slot re-admitted
    with a fresh prompt (U[1K, 16K] tokens, Zipf(1.1) scores): release, then
    classify + prompt compaction of the admitted requests.  Every input is
    drawn before the timed region; each step's decode and each admission are
    bracketed by HIP events on a held stream.  Prints one JSON line."""
    import numpy as np
    import torch

    import compressed_paged_attention_amd as dk
    from workloads import synth

    dev = torch.device("cuda:0")
    cfg = synth.config("churn")
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    S = args.steps
    rng = np.random.default_rng(synth.SEED_BASE + 4000)
    lens = synth.seq_lens(cfg)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    st = dk.DiffKVState(cfg, B, P, max_total_tokens=int(lens.sum()), device=dev)
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    cu = pr["cu_seqlens"].to(dev)
    tiers, _ = st.classify(cu, pr["scores"])
    st.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], tiers)
    torch.cuda.synchronize()
    del pr, tiers
    # the schedule, drawn up front
    lo, hi = cfg["seq"]
    blo, bhi = cfg["budget"]
    seq = lens.numpy().astype(np.int64).copy()
    budget = rng.integers(blo, bhi + 1, B)
    gen = np.zeros(B, np.int64)
    steps = []
    for s_ in range(S):
        seq_s = seq.astype(np.int32).copy()
        seq += 1
        gen += 1
        done = gen >= budget
        adm = None
        if done.any():
            nl = np.where(done, rng.integers(lo, hi + 1, B), 0)
            adm = (done.astype(np.uint8), nl)
            seq[done] = nl[done]
            gen[done] = 0
            budget[done] = rng.integers(blo, bhi + 1, int(done.sum()))
        steps.append((seq_s, adm))
    dec = [synth.make_decode(cfg, s_, device=dev) for s_ in range(S)]
    seq_d = [torch.from_numpy(x).to(dev) for x, _ in steps]
    adm_in = {}
    for s_, (_, adm) in enumerate(steps):
        if adm is None:
            continue
        mask, nl = adm
        lens_a = torch.from_numpy(nl.astype(np.int64))
        pa = synth.make_prompt(cfg, device=dev, salt=1 + s_, lens=lens_a)
        adm_in[s_] = (torch.from_numpy(mask).to(dev), pa["cu_seqlens"].to(dev), pa["k"], pa["v"], pa["scores"])
    torch.cuda.synchronize()
    print(f"[bench] churn: {len(adm_in)} admission events, {sum(int(a[0].sum()) for _, a in steps if a)} "
          f"requests replaced", file=sys.stderr, flush=True)
    out = torch.empty(B, H * G, d, dtype=torch.float32, device=dev)
    # warm the classify outputs' allocations of the first admission
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    e_dec = [(ev(), ev()) for _ in range(S)]
    e_adm = {s_: (ev(), ev()) for s_ in adm_in}
    torch.cuda.synchronize()
    torch.cuda._sleep(args.hold_cycles)
    for s_ in range(S):
        e_dec[s_][0].record()
        st.decode_step(dec[s_]["q"], seq_d[s_], dec[s_]["k_new"], dec[s_]["v_new"], update_scores=1, out=out)
        e_dec[s_][1].record()
        if s_ in adm_in:
            mask, cu_a, k_a, v_a, sc_a = adm_in[s_]
            e_adm[s_][0].record()
            st.release(mask)
            t_a, _ = st.classify(cu_a, sc_a)
            st.compact_prompt(cu_a, k_a, v_a, sc_a, t_a)
            e_adm[s_][1].record()
    torch.cuda.synchronize()
    status = int(st.pool.status.item())
    assert status == 0, f"status bits set during the churn run: {status}"
    dec_us = np.array([a.elapsed_time(b) * 1e3 for a, b in e_dec])
    adm_us = np.array([e_adm[s_][0].elapsed_time(e_adm[s_][1]) * 1e3 for s_ in sorted(adm_in)])
    total_us = e_dec[0][0].elapsed_time(e_dec[-1][1]) * 1e3
    ptr = st.pool.ptr.cpu().numpy().view(np.uint64)
    res = {
        "metric": "decode churn: per-step decode time and admissions",
        "workload": "decode_churn_schedule", "batch": B, "q_heads": H * G, "kv_heads": H, "head_dim": d,
        "steps": S, "pool_pages": P,
        "decode_step_us": {"p50": float(np.percentile(dec_us, 50)), "p99": float(np.percentile(dec_us, 99)),
                           "mean": float(dec_us.mean())},
        "admission_events": int(len(adm_us)),
        "requests_replaced": int(sum(int(a[0].sum()) for _, a in steps if a)),
        "admission_us": {"p50": float(np.percentile(adm_us, 50)) if len(adm_us) else None,
                         "p99": float(np.percentile(adm_us, 99)) if len(adm_us) else None},
        "request_tokens_per_s": B * S / (total_us * 1e-6),
        "timed_region_us": total_us,
        "pointer_laps": [float(ptr[0]) / P, float(ptr[1]) / P],
        "data": "synthetic",
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch")
    ap.add_argument("--context", type=int, default=0, help="override with one fixed context length")
    ap.add_argument("--cpu-requests", type=int, default=8)
    ap.add_argument("--cpu-steps", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=min(16, os.cpu_count() or 1),
                    help="oracle processes for the all-cores baseline")
    ap.add_argument("--hold-cycles", type=int, default=100_000_000,
                    help="spin-kernel length that holds the stream while a timed segment is enqueued")
    ap.add_argument("--churn-schedule", action="store_true",
                    help="run the decode-churn schedule (releases and admissions) instead; one JSON line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one elementwise copy of this size first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; the path has no cross-GPU exchange "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.churn_schedule:
        churn_schedule(args)
        return

    import numpy as np
    import torch

    from workloads import synth

    # the oracle baseline first: its worker processes fork from a process
    # that has not touched the GPU
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(synth.config(args.workload), args.cpu_requests, args.cpu_steps, args.cpu_workers)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)

    import compressed_paged_attention_amd as dk

    dev = torch.device("cuda:0")
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    over = {}
    if args.batch > 0:
        over["batch"] = args.batch
    if args.context > 0:
        over["seq"] = (args.context, args.context)
        over["max_seq_len"] = args.context + 256
    cfg = synth.config(args.workload, **over)
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    R = args.replicas
    lens = synth.seq_lens(cfg)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    total = int(lens.sum())

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---- prompt side on every replica: classify + prompt compaction ----
    reps, seqs0, prompt_ms = [], [], []
    for r in range(R):
        pr = synth.make_prompt(cfg, device=dev, salt=r, lens=lens)
        st = dk.DiffKVState(cfg, B, P, max_total_tokens=total, device=dev)
        cu = pr["cu_seqlens"].to(dev)
        # classification has no side effects: one untimed call allocates its
        # outputs, then classify + prompt compaction are timed on a held
        # stream (device time, not the host's launch rate)
        st.classify(cu, pr["scores"])
        torch.cuda.synchronize()
        torch.cuda._sleep(args.hold_cycles)
        e0, e1 = ev(), ev()
        e0.record()
        tiers, counts = st.classify(cu, pr["scores"])
        st.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], tiers)
        e1.record()
        torch.cuda.synchronize()
        prompt_ms.append(e0.elapsed_time(e1))
        assert int(st.pool.status.item()) == 0, "prompt compaction reported a status bit"
        reps.append(st)
        del pr, tiers, counts
        print(f"[bench] replica {r}: prompt compaction {prompt_ms[-1] * 1e3:.0f} us", file=sys.stderr,
              flush=True)
    torch.cuda.empty_cache()

    # steps: warmup, the timed full steps, then the compaction-only segment
    nsteps = args.warmup + 2 * args.steps
    dec = [synth.make_decode(cfg, s, device=dev) for s in range(nsteps)]
    seq_per_step = [(lens + s // R).to(torch.int32).to(dev) for s in range(nsteps)]
    out = torch.empty(B, H * G, d, dtype=torch.float32, device=dev)
    ts_before = [st.tier_state.cpu().numpy() for st in reps]

    def step_compact(s):
        reps[s % R].compact_step(seq_per_step[s], dec[s]["k_new"], dec[s]["v_new"])

    def step_attn(s):
        reps[s % R].decode_attn(dec[s]["q"], seq_per_step[s], update_scores=1, out=out)

    def timed(fn, first, count):
        """GPU time of `count` back-to-back calls.  The stream is held by a
        spin kernel issued before the start event while the host enqueues, so
        the events see the device's own pace, not Python's launch rate."""
        torch.cuda.synchronize()
        torch.cuda._sleep(args.hold_cycles)
        e0, e1 = ev(), ev()
        e0.record()
        for k in range(count):
            fn(first + k)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def full_step(s):
        # compaction then attention with the score update, one library call
        # (chained: the replica's previous step planned this one)
        reps[s % R].decode_step(dec[s]["q"], seq_per_step[s], dec[s]["k_new"], dec[s]["v_new"],
                                update_scores=1, out=out)

    # warmup: the separate kernels, then one full step per replica (which
    # starts each replica's chain of planned steps)
    for s in range(args.warmup):
        if s < args.warmup - R:
            step_compact(s)
            step_attn(s)
        else:
            full_step(s)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # headline: K complete decode steps (compaction + attention with score
    # update), timed as 8 back-to-back segments (their spread: p10/p50/p90)
    nseg = 8 if args.steps % 8 == 0 else 1
    seg_ms = [timed(full_step, args.warmup + k * (args.steps // nseg), args.steps // nseg) for k in range(nseg)]
    total_ms = float(sum(seg_ms))
    ts_after = [st.tier_state.cpu().numpy() for st in reps]
    # attention alone: the same K launches again on the final caches
    last = args.warmup + args.steps - R
    attn_ms = timed(lambda s: step_attn(last + (s % R)), 0, args.steps)
    # compaction alone: K further generation steps
    comp_ms = timed(step_compact, args.warmup + args.steps, args.steps)
    status = [int(st.pool.status.item()) for st in reps]
    assert all(x == 0 for x in status), f"status bits set during the run: {status}"
    attn = np.array([attn_ms / args.steps])
    comp = np.array([comp_ms / args.steps])
    print("[bench] timed steps done", file=sys.stderr, flush=True)

    # ---- release (every replica) ----
    rel_ms = []
    mask = torch.ones(B, dtype=torch.uint8, device=dev)
    for st in reps:
        e0, e1 = ev(), ev()
        e0.record()
        st.release(mask)
        e1.record()
        torch.cuda.synchronize()
        rel_ms.append(e0.elapsed_time(e1))

    # the attention-only segment runs on the caches as the headline segment left them
    attn_bytes = float(np.mean([algorithmic_attn_bytes(a, B, H, G, d) for a in ts_after]))
    t_attn_s = float(attn.mean()) * 1e-3
    achieved = attn_bytes / t_attn_s / 1e9
    ts = np.stack(ts_before).reshape(-1, 4).astype(np.int64)
    n_hi, n_lo = int(ts[:, 0].sum()), int(ts[:, 1].sum())
    ctx = R * total * H
    step_ms = total_ms / args.steps
    res = {
        "metric": METRIC,
        "value": B * args.steps / (total_ms * 1e-3),
        "unit": "request-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "step_us_p10_p50_p90": [float(np.percentile(np.array(seg_ms) * 1e3 / (args.steps // nseg), x))
                                for x in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES.get(args.workload, args.workload), "q_heads": H * G,
                   "kv_heads": H, "head_dim": d, "batch": B,
                   "context": int(lens[0]) if int(lens.min()) == int(lens.max()) else
                   [int(lens.min()), int(lens.max())],
                   "score": "zipf(%g)" % cfg["zipf"][0] if cfg["zipf"][0] == cfg["zipf"][1] else
                   "zipf(U[%g,%g])" % tuple(cfg["zipf"]), "alpha_h": cfg["alpha_h"],
                   "alpha_l": cfg["alpha_l"], "window": cfg["window"], "replicas": R,
                   "pool_pages": P, "page_bytes": dk.diffkv_page_bytes(cfg),
                   "attn_splits": dk.diffkv_attn_splits(cfg, B)},
        "attn_tokens_per_s": B / t_attn_s,
        "attn_us": float(attn.mean()) * 1e3,
        "compaction_us_per_step": float(comp.mean()) * 1e3,
        # the compaction's cost inside a step: the step minus attention alone
        "step_minus_attention_us": step_ms * 1e3 - float(attn.mean()) * 1e3,
        "compaction_share": float((step_ms - attn.mean()) / step_ms),
        "prompt_compaction_us": float(np.mean(prompt_ms)) * 1e3,
        "prompt_input_GBps": (total * H * d * 4 + total * H * 4) / (np.mean(prompt_ms) * 1e-3) / 1e9,
        "release_us": float(np.mean(rel_ms)) * 1e3,
        "retained": {"hi_frac": n_hi / ctx, "lo_frac": n_lo / ctx,
                     "kv_compression_vs_fp16": (ctx * 4 * d) / (n_hi * (1.5 * d + 16) + n_lo * (0.75 * d + 16))},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": measured_traffic() if args.workload == "llama3_8b" else None,
                     "kernel": ("attn_kernel<%d, 1, %s, false>" % (d, "true" if 2 * G <= 16 else "false"))
                     if dk.diffkv_attn_splits(cfg, B) == 1 else
                     "attn_kernel<%d, 2, ...> + attn_merge_kernel + score_kernel" % d,
                     "bytes_per_launch": int(attn_bytes),
                     "stream_read_GBps": stream_read_gbps()},
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
