#!/usr/bin/env python3
"""Benchmark of the DiffKV hot path on one MI355X.

Headline workload (the largest single-GPU configuration): the high-GQA
stress case -- 64 q / 8 KV heads (GQA 8), d = 128, batch 64, ragged contexts
U[2000, 64000], fp16 K/V ~ N(0,1) with 4 outlier channels x8 per KV head,
importance scores Zipf(1.1) with a per-unit random permutation, alpha_h = 1.0,
alpha_l = 0.2, W = 64, a page pool of 200 GB.  Its working set (~630 MB per
step) is far beyond the 256 MB Infinity Cache, so one cache replica is used.
The Llama3-8B-shaped layer (32 q / 8 KV heads, batch 32, 4096 tokens, 8
replicas so the Infinity Cache cannot hold the working set) is measured in
the same run and reported under "extra".

A timed step is one decode step of the whole batch on the compacted cache:
generation-step compaction, then decode attention with the score update, as
one diffkv_decode_step call -- with one workgroup per unit, one kernel that
commits each unit's step and attends over it.  Each replica's steps are
chained (a step's score update plans the next one into the workspace); every
replica's chain is started (its first step runs the plan kernel) before the
warmup steps, so the timed region holds chained steps only.

value = batch * steps / (time of the timed region): request-tokens per second
of complete decode steps, timed as up to 8 back-to-back segments of
near-equal length (their spread: p10/p50/p90 per step).  Three kinds of
segments are timed with HIP events on the stream the library launches on,
each over back-to-back launches while a spin kernel issued before the start
event holds the stream (so the events measure the device, not the host's
launch rate): the K chained steps (value, roofline), K attention launches
alone on the final caches (attn_us, attention_roofline), and K more
compaction steps alone through the separate kernels (compaction_us_per_step).
The compaction's share of a step is (step - attention alone) / step.

roofline describes the dominant kernel, the fused decode step (a chained
step is one launch of it): algorithmic bytes per launch -- codes + metadata
of every retained token, q, out, table entries, the 8-byte read-modify-write
of each retained token's score, and per unit the step's new K/V row, up to
three high-precision token slots, its tier state and one table entry -- over
the mean step time.  attention_roofline is the same for the attention
kernel alone.  traffic is the counters' HBM bytes per launch from the
committed profile of that workload and kernel, null when the sources changed
since.  stream_read_GBps is the box's achievable read rate (a reduction over
4 GiB), the practical ceiling beside the 8 TB/s peak.  The oracle baseline
runs first (before the process touches the GPU), on one thread and as
several processes, on a bounded sample of the headline workload.
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

def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_traffic.txt")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when the summary is missing, covers another kernel,
    or the kernel sources changed since it was taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith(("#", " ", "|")) or ":" not in line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    key = "traffic_bytes_per_launch " + kernel
    return float(kv[key]) if key in kv else None


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
    if "pool_bytes" in c:
        # the workload's 200 GB pool would not fit in host memory: the
        # sample's own need with the same headroom as the other workloads
        c.pop("pool_bytes")
        c["pool_factor"] = 1.25
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
    return t_prompt, t_step, int(lens.sum())


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
    once on one thread, once as `workers` processes (each a sample of its
    own, steps started together).  Runs before the process touches the GPU
    (the workers are forked)."""
    import multiprocessing as mp
    t_prompt, t_step, ntok = _oracle_steps(cfg, n_req, n_steps)
    H = cfg["num_kv_heads"]
    single = dict(value=n_req / t_step, cores=1,
                  sample=f"{n_req} of {cfg['batch']} requests ({n_req * H} units, {ntok} context tokens in "
                         f"all): prompt compaction once ({t_prompt:.2f} s, not in value), then {n_steps} decode "
                         f"steps (step compaction + fp64 attention + score update), {t_step * 1e3:.1f} ms per step")
    per = max(1, n_req // 2)
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers)
    with ctx.Pool(workers, initializer=_pool_init, initargs=(barrier,)) as pool:
        res = pool.map(_oracle_worker_b, [(cfg, per, n_steps)] * workers)
    value = sum(per / ts for _, ts, _ in res)
    return dict(value=value, unit="request-tokens/s", cores=workers, kind="oracle",
                sample=f"{workers} processes, each the first {per} requests of the workload ({per * H} units, "
                       f"{res[0][2]} context tokens) through prompt compaction, then {n_steps} decode steps "
                       f"(step compaction + fp64 attention + score update) started together; value = sum of "
                       f"the processes' request-tokens/s",
                single_thread=single, cpu=cpu_model(), nproc=os.cpu_count())


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


def step_extra_bytes(tier_state, H, d):
    """Bytes a generation step moves per active unit beyond the attention:
    the new token's fp16 K and V rows (4d), up to three high-precision token
    slots (the new token written, a demoted token read and its low copy
    written: 3 (1.5d + 16)), the tier state (16) and one table entry (4)."""
    U = tier_state.reshape(-1, 4).shape[0]
    return int(U * (4 * d + 3 * (1.5 * d + 16) + 16 + 4))


def measure(args, name, R, steps, warmup, dk):
    """Prompt side, chained decode steps, attention alone, compaction alone
    and release of one workload on R cache replicas; returns a dict."""
    import numpy as np
    import torch

    from workloads import synth

    dev = torch.device("cuda:0")
    over = {}
    if args.batch > 0:
        over["batch"] = args.batch
    if args.context > 0:
        over["seq"] = (args.context, args.context)
        over["max_seq_len"] = args.context + 256
    cfg = synth.config(name, **over)
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    lens = synth.seq_lens(cfg)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    total = int(lens.sum())

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---- prompt side on every replica: classify + prompt compaction ----
    reps, prompt_ms = [], []
    for r in range(R):
        pr = synth.make_prompt(cfg, device=dev, salt=r, lens=lens)
        print(f"[bench] {name} replica {r}: inputs drawn", file=sys.stderr, flush=True)
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
        print(f"[bench] {name} replica {r}: prompt compaction {prompt_ms[-1] * 1e3:.0f} us", file=sys.stderr,
              flush=True)
    torch.cuda.empty_cache()

    # decode inputs for every step: R chain starts, warmup, timed, compaction-only
    nsteps = R + warmup + 2 * steps
    dec = [synth.make_decode(cfg, s % 64, device=dev) for s in range(nsteps)]
    seq_per_step = [(lens + s // R).to(torch.int32).to(dev) for s in range(nsteps)]
    out = torch.empty(B, H * G, d, dtype=torch.float32, device=dev)
    ts_before = [st.tier_state.cpu().numpy() for st in reps]

    def full_step(s):
        # compaction then attention with the score update, one library call
        # (chained: the replica's previous step planned this one)
        reps[s % R].decode_step(dec[s]["q"], seq_per_step[s], dec[s]["k_new"], dec[s]["v_new"],
                                update_scores=1, out=out)

    def step_compact(s):
        reps[s % R].compact_step(seq_per_step[s], dec[s]["k_new"], dec[s]["v_new"])

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

    # every replica's chain starts here (its first step runs the plan kernel),
    # then `warmup` chained steps
    for s in range(R + warmup):
        full_step(s)
    torch.cuda.synchronize()
    assert all(st.chain > 0 for st in reps)
    print(f"[bench] {name} warmup done", file=sys.stderr, flush=True)

    # headline: `steps` chained decode steps, timed as up to 8 back-to-back
    # segments of near-equal length (their spread: p10/p50/p90 per step)
    nseg = max(1, min(8, steps))
    bounds = [R + warmup + (k * steps) // nseg for k in range(nseg + 1)]
    seg_ms = [timed(full_step, bounds[k], bounds[k + 1] - bounds[k]) for k in range(nseg)]
    seg_us_per_step = [m * 1e3 / (bounds[k + 1] - bounds[k]) for k, m in enumerate(seg_ms)]
    total_ms = float(sum(seg_ms))
    ts_after = [st.tier_state.cpu().numpy() for st in reps]
    # attention alone (with the score update) on the caches the steps left
    last = R + warmup + steps - R
    attn_ms = timed(lambda s: reps[(last + s) % R].decode_attn(dec[last + s % R]["q"], seq_per_step[last + s % R],
                                                               update_scores=1, out=out), 0, steps)
    # compaction alone through the separate kernels: `steps` further steps
    comp_ms = timed(step_compact, R + warmup + steps, steps)
    status = [int(st.pool.status.item()) for st in reps]
    assert all(x == 0 for x in status), f"status bits set during the run: {status}"
    print(f"[bench] {name} timed steps done", file=sys.stderr, flush=True)

    # ---- release (every replica) ----
    rel_ms = []
    mask = torch.ones(B, dtype=torch.uint8, device=dev)
    for st in reps:
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        st.release(mask)
        e1.record()
        torch.cuda.synchronize()
        rel_ms.append(e0.elapsed_time(e1))
    del reps, dec
    torch.cuda.empty_cache()

    attn_bytes = float(np.mean([algorithmic_attn_bytes(a, B, H, G, d) for a in ts_after]))
    step_bytes = attn_bytes + float(np.mean([step_extra_bytes(a, H, d) for a in ts_after]))
    step_us = total_ms * 1e3 / steps
    attn_us = attn_ms * 1e3 / steps
    ts = np.stack(ts_before).reshape(-1, 4).astype(np.int64)
    n_hi, n_lo = int(ts[:, 0].sum()), int(ts[:, 1].sum())
    ctx = R * total * H
    one_split = dk.diffkv_attn_splits(cfg, B) == 1
    gp = 4 if G <= 4 else (8 if G <= 8 else 16)  # the kernel's softmax layout (G rounded up)
    step_kernel = "attn_kernel<%d, 1, %d, true>" % (d, gp) if one_split else "step + attention kernels"
    attn_kernel = ("attn_kernel<%d, 1, %d, false>" % (d, gp)) if one_split else \
        "attn_kernel<%d, 2, ...> + score_kernel (merging the splits) + score_finish_kernel" % d
    cfg_out = {"workload": WORKLOAD_NAMES.get(name, name), "q_heads": H * G, "kv_heads": H, "head_dim": d,
               "batch": B,
               "context": int(lens[0]) if int(lens.min()) == int(lens.max()) else [int(lens.min()), int(lens.max())],
               "score": "zipf(%g)" % cfg["zipf"][0] if cfg["zipf"][0] == cfg["zipf"][1] else
               "zipf(U[%g,%g])" % tuple(cfg["zipf"]), "alpha_h": cfg["alpha_h"], "alpha_l": cfg["alpha_l"],
               "window": cfg["window"], "lo_enabled": cfg["lo_enabled"], "replicas": R, "pool_pages": P,
               "page_bytes": dk.diffkv_page_bytes(cfg), "attn_splits": dk.diffkv_attn_splits(cfg, B)}
    return {
        "cfg": cfg, "config": cfg_out, "B": B,
        "value": B * steps / (total_ms * 1e-3),
        "ms_per_step": step_us * 1e-3,
        "step_us_p10_p50_p90": [float(np.percentile(seg_us_per_step, x)) for x in (10, 50, 90)],
        "attn_us": attn_us,
        "attn_tokens_per_s": B / (attn_us * 1e-6),
        "compaction_us_per_step": comp_ms * 1e3 / steps,
        # the compaction's cost inside a step: the step minus attention alone
        "step_minus_attention_us": step_us - attn_us,
        "compaction_share": (step_us - attn_us) / step_us,
        "prompt_compaction_us": float(np.mean(prompt_ms)) * 1e3,
        "prompt_input_GBps": (total * H * d * 4 + total * H * 4) / (np.mean(prompt_ms) * 1e-3) / 1e9,
        "release_us": float(np.mean(rel_ms)) * 1e3,
        "retained": {"hi_frac": n_hi / ctx, "lo_frac": n_lo / ctx,
                     "kv_compression_vs_fp16": (ctx * 4 * d) / (n_hi * (1.5 * d + 16) + n_lo * (0.75 * d + 16))},
        "step_kernel": step_kernel, "step_bytes": step_bytes,
        "attn_kernel": attn_kernel, "attn_bytes": attn_bytes,
    }


PEAK_FP16_MFMA_TFLOPS = 2500.0


def importance_timing(args, name, dk):
    """Prompt-side importance (diffkv_importance, causal: every prompt query
    against its earlier keys, twice -- softmax statistics, then the column
    means) on the workload's prompt shape with seeded N(0,1) queries; one
    warmup call, then one call timed with HIP events on a held stream.
    Algorithmic flops: 2 passes x 2d per (query, key <= query) pair and q
    head; bound by the fp16 matrix peak."""
    import torch

    from workloads import synth
    dev = torch.device("cuda:0")
    cfg = synth.config(name)
    H, G, d = cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    lens = synth.seq_lens(cfg)
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    gq = torch.Generator(device=dev)
    gq.manual_seed(synth.SEED_BASE + 999)
    q = torch.randn(int(lens.sum()), H * G, d, generator=gq, device=dev).to(torch.float16).view(torch.int16)
    cu = pr["cu_seqlens"].to(dev)
    total = int(lens.sum())
    ws = torch.empty(dk.diffkv_workspace_bytes(cfg, dk.IMPORTANCE, cfg["batch"], total), dtype=torch.uint8,
                     device=dev)
    scores = torch.empty(H, total, dtype=torch.float32, device=dev)
    dk.diffkv_importance(cfg, dk.IMP_CAUSAL, cu, q, pr["k"], scores, ws)
    torch.cuda.synchronize()
    torch.cuda._sleep(args.hold_cycles)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dk.diffkv_importance(cfg, dk.IMP_CAUSAL, cu, q, pr["k"], scores, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    pairs = sum(int(n) * (int(n) + 1) // 2 for n in lens.tolist())
    flops = 2 * 2 * d * pairs * H * G
    del pr, q, ws, scores
    torch.cuda.empty_cache()
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": WORKLOAD_NAMES.get(name, name), "us": us, "tokens": total,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP16_MFMA_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_FP16_MFMA_TFLOPS, "flops_per_launch": flops,
                         "kernel": "imp_stats_kernel + imp_sum_kernel"}}


def side_timings(args, name, dk):
    """Query-free importance (diffkv_keydiff_scores) on the workload's prompt
    keys, and per-page key bounds (diffkv_page_bounds) and page scores
    (diffkv_page_scores) over its compacted cache; each a warmup call, then
    8 calls timed with HIP events on a held stream.  Algorithmic bytes:
    KeyDiff reads each key once and writes one fp32 score (2d + 4 per token
    and head); the bounds read the K codes and metadata of every retained
    token (d + 4 high, d/2 + 4 low) and write 2d fp32 per live page; the page
    scores read the bounds and the queries and write one fp32 per table
    entry."""
    import torch

    from workloads import synth
    dev = torch.device("cuda:0")
    cfg = synth.config(name)
    B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
    lens = synth.seq_lens(cfg)
    P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
    total = int(lens.sum())
    pr = synth.make_prompt(cfg, device=dev, lens=lens)
    st = dk.DiffKVState(cfg, B, P, max_total_tokens=total, device=dev)
    cu = pr["cu_seqlens"].to(dev)
    t, _ = st.classify(cu, pr["scores"])
    st.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], t)
    q = synth.make_decode(cfg, 0, device=dev)["q"]
    seq = lens.to(torch.int32).to(dev)
    n = 8

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        torch.cuda._sleep(args.hold_cycles)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def line(kernel, nbytes, us):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us": us, "bytes_per_launch": int(nbytes),
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": gbs / PEAK_HBM_GBS, "kernel": kernel}}

    k = pr["k"]
    us_kd = timed(lambda: dk.keydiff_scores(cfg, cu, k))
    bounds = torch.zeros(P, 2, d, dtype=torch.float32, device=dev)
    us_pb = timed(lambda: st.page_bounds(bounds))
    us_ps = timed(lambda: st.page_scores(q, seq, bounds))
    ts = st.tier_state.view(-1, 4).to(torch.int64).sum(0).tolist()
    n_hi, n_lo, p_hi, p_lo = ts
    out = {"workload": WORKLOAD_NAMES.get(name, name),
           "keydiff_scores": line("kd_partial/anchor/score/norm kernels", total * H * (2 * d + 4), us_kd),
           "page_bounds": line("page_bounds_kernel",
                               n_hi * (d + 4) + n_lo * (d // 2 + 4) + (p_hi + p_lo) * 8 * d, us_pb),
           "page_scores": line("page_scores_kernel",
                               (p_hi + p_lo) * 8 * d + B * H * G * d * 2 + B * H * st.L * 4, us_ps)}
    del pr, st, bounds
    torch.cuda.empty_cache()
    return out


# (K, V) high, (K, V) low: the ablation's K4V8/K2V4 and K8V2/K4V1; then three
# precision levels K8V8 / K8V4 / K4V2 (thresholds alpha_h, 0.5, alpha_l)
CODEC_VARIANTS = (((4, 8, 2, 4), {}), ((8, 2, 4, 1), {}),
                  ((8, 8, 4, 2), dict(num_levels=3, alpha_mid=[0.5], mid_k_bits=[8], mid_v_bits=[4])))


def codec_timings(args, name, dk):
    """Tier codec variants and three precision levels (plain layout) at the
    workload's shape: decode attention with the score update
    (diffkv_decode_attn) and the generation step (diffkv_compact STEP) on
    the compacted cache; each a warmup call,
    then 8 calls timed with HIP events on a held stream (the steps advance
    the cache).  Algorithmic bytes of the attention: per retained token its
    K and V codes (d (b_K + b_V) / 8) and scale/zero words (8), 8 for the
    score read-modify-write, 4 per page-table entry, q (fp16) and out (fp32)
    rows."""
    import torch

    from workloads import synth
    dev = torch.device("cuda:0")
    out = {"workload": WORKLOAD_NAMES.get(name, name)}
    for codec, extra in CODEC_VARIANTS:
        hk, hv, lk, lv = codec
        cfg = dict(synth.config(name), hi_k_bits=hk, hi_v_bits=hv, lo_k_bits=lk, lo_v_bits=lv, **extra)
        K = int(extra.get("num_levels", 2))
        bits = [(hk, hv)] + [(a, b) for a, b in zip(extra.get("mid_k_bits", []), extra.get("mid_v_bits", []))]
        bits += [(lk, lv)]
        B, H, G, d = cfg["batch"], cfg["num_kv_heads"], cfg["gqa_group"], cfg["head_dim"]
        lens = synth.seq_lens(cfg)
        P = synth.pool_pages(cfg, lens, dk.diffkv_page_bytes(cfg))
        total = int(lens.sum())
        pr = synth.make_prompt(cfg, device=dev, lens=lens)
        st = dk.DiffKVState(cfg, B, P, max_total_tokens=total, device=dev)
        cu = pr["cu_seqlens"].to(dev)
        t, _ = st.classify(cu, pr["scores"])
        st.compact_prompt(cu, pr["k"], pr["v"], pr["scores"], t)
        del pr
        dec = synth.make_decode(cfg, 0, device=dev)
        seq = lens.to(torch.int32).to(dev)
        n = 8

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            torch.cuda._sleep(args.hold_cycles)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        ts = st.tier_state.view(-1, 2 * K).to(torch.int64).sum(0).tolist()
        ntok, npg = ts[:K], ts[K:]
        nbytes = (sum(ntok[l] * (d * (bits[l][0] + bits[l][1]) // 8 + 8 + 8) for l in range(K)) + 4 * sum(npg)
                  + B * H * G * d * (2 + 4))
        us_attn = timed(lambda: st.decode_attn(dec["q"], seq, update_scores=1))
        seqs = [seq + i for i in range(n + 1)]  # each step one token further
        it = iter(seqs)
        us_step = timed(lambda: st.compact_step(next(it), dec["k_new"], dec["v_new"]))
        assert int(st.pool.status[0]) == 0, "codec variant step status"
        gbs = nbytes / (us_attn * 1e-6) / 1e9
        out["_".join(f"K{a}V{b}" for a, b in bits)] = {
            "attn_us": us_attn, "step_us": us_step, "page_bytes": dk.diffkv_page_bytes(cfg),
            "retained_tokens_per_level": ntok,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "kernel": "plain_attn_kernel + merge + plain_score_kernel",
                         "bytes_per_launch": int(nbytes)}}
        del st
        torch.cuda.empty_cache()
    return out


def roofline(kernel, nbytes, us, workload, stream_gbps):
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(workload, kernel),
            "kernel": kernel, "bytes_per_launch": int(nbytes), "launch_us": us,
            "stream_read_GBps": stream_gbps}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="stress_gqa8")
    ap.add_argument("--replicas", type=int, default=0,
                    help="cache replicas (0: 8, or 1 for the workloads with a 200 GB pool, whose working set "
                         "is far beyond the 256 MB Infinity Cache)")
    ap.add_argument("--extra-workload", default="llama3_8b",
                    help="a second workload measured in the same run and reported as extra keys ('none': skip)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch")
    ap.add_argument("--context", type=int, default=0, help="override with one fixed context length")
    ap.add_argument("--cpu-requests", type=int, default=0, help="oracle sample (0: 8, or 2 with contexts > 4096)")
    ap.add_argument("--cpu-steps", type=int, default=0, help="oracle decode steps (0: 8, or 4 with contexts > 4096)")
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

    from workloads import synth

    def replicas_for(name):
        if args.replicas > 0:
            return args.replicas
        return 1 if "pool_bytes" in synth.config(name) else 8

    # the oracle baseline first: its worker processes fork from a process
    # that has not touched the GPU
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        c0 = synth.config(args.workload)
        short = c0["seq"][1] <= 4096
        nreq = args.cpu_requests or (8 if short else 2)
        cpu = cpu_baseline(c0, nreq, args.cpu_steps or (8 if short else 4), args.cpu_workers)
        print("[bench] cpu baseline done", file=sys.stderr, flush=True)

    import compressed_paged_attention_amd as dk

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    m = measure(args, args.workload, replicas_for(args.workload), args.steps, args.warmup, dk)
    stream = stream_read_gbps()
    res = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "request-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "step_us_p10_p50_p90": m["step_us_p10_p50_p90"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic",
        "config": m["config"],
    }
    for k in ("attn_tokens_per_s", "attn_us", "compaction_us_per_step", "step_minus_attention_us",
              "compaction_share", "prompt_compaction_us", "prompt_input_GBps", "release_us", "retained"):
        res[k] = m[k]
    # the dominant kernel: the fused decode step (one launch per chained step)
    res["roofline"] = roofline(m["step_kernel"], m["step_bytes"], m["ms_per_step"] * 1e3, args.workload, stream)
    res["attention_roofline"] = roofline(m["attn_kernel"], m["attn_bytes"], m["attn_us"], args.workload, stream)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    if args.extra_workload and args.extra_workload != "none" and args.extra_workload != args.workload:
        e = measure(args, args.extra_workload, replicas_for(args.extra_workload), args.steps, args.warmup, dk)
        ex = {k: e[k] for k in ("value", "ms_per_step", "step_us_p10_p50_p90", "attn_us", "attn_tokens_per_s",
                                "compaction_us_per_step", "step_minus_attention_us", "compaction_share",
                                "prompt_compaction_us", "release_us", "retained", "config")}
        ex["roofline"] = roofline(e["step_kernel"], e["step_bytes"], e["ms_per_step"] * 1e3, args.extra_workload,
                                  stream)
        ex["attention_roofline"] = roofline(e["attn_kernel"], e["attn_bytes"], e["attn_us"], args.extra_workload,
                                            stream)
        res["extra"] = {WORKLOAD_NAMES.get(args.extra_workload, args.extra_workload): ex}
        res["extra"]["prompt_importance"] = importance_timing(args, args.extra_workload, dk)
        res["extra"]["key_bounds_and_keydiff"] = side_timings(args, args.extra_workload, dk)
        res["extra"]["codec_variants"] = codec_timings(args, args.extra_workload, dk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
