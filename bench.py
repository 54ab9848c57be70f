#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

One step = one pass of the whole path over one batch: lightning-indexer scores for every
query token, top-k selection, sparse MLA (MQA mode) with its split combine; for an
IndexShare workload, the attention runs once per layer of the group with the same indices.
Inputs are synthetic (seeded), resident in HBM before timing starts, and rotate over
several independent batches so that no step re-reads rows a previous step left in cache.

Prints ONE JSON line. Default workload: decode, batch 32, 128K-token paged caches.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 matrix cores
BF16_PEAK_TFLOPS = 2500.0
METRIC = "sparse-attn decode tokens/s and HBM GB/s at 128K ctx; prefill indexer TFLOPS"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_b32_128k_paged")
    ap.add_argument("--rotate", type=int, default=3, help="independent input batches cycled through")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill-index", action="store_true",
                    help="skip the prefill indexer figure timed after the decode workloads")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (reference for HBM byte counters)")
    return ap.parse_args()


def scan_runs(wl):
    """Whether a step runs the indexer scan: compressed attention whose k covers every compressed
    row (HCA) keeps every visible entry without scores."""
    return not (wl.ratio and (wl.k == 0 or wl.k >= wl.rows))


def index_work(wl):
    """Algorithmic bytes and FLOPs of one index-score launch (every visible key read once per
    sequence; with compressed attention the keys are the visible compressed entries)."""
    if not scan_runs(wl):
        return 0, 0
    B, Q, Hi = wl.B, wl.Q, wl.Hi
    rows = 1 if wl.share_first_query else Q
    keys = sum(wl.n_visible(n) for n in wl.lens) * 128
    scores = B * rows * wl.rows * 4
    qw = B * rows * Hi * (128 + 4)
    table = B * wl.max_pages * 4 if wl.page_size else 0
    flops = 0
    for n in wl.lens:
        for j in range(rows):
            flops += wl.n_visible(n, j) * Hi * 128 * 2
    return keys + scores + qw + table, flops


def mla_work(wl):
    """Algorithmic bytes and FLOPs of one sparse-MLA call (rows gathered once per query token);
    with compressed attention: the selected compressed rows and the window's raw rows, attended
    in one softmax."""
    rows = wl.B * wl.Q
    pos = [n - wl.Q + j for n in wl.lens for j in range(wl.Q)]
    if wl.ratio:
        sel = sum(min(wl.k, (p + 1) // wl.ratio) + min(wl.window, p + 1) for p in pos)
        idx = rows * (wl.k + wl.window) * 4
    else:
        sel = sum(min(wl.k, p + 1) for p in pos)
        idx = rows * wl.k * 4
    row_bytes = 576 if wl.latent_fp8 else 1152          # E4M3 codes or bf16 per latent row
    byts = sel * row_bytes + rows * wl.H * (576 * 2 + 512 * 4 + 4) + idx
    flops = sel * wl.H * 2 * (576 + 512)
    return byts, flops


def prefill_index_figure(dsa, synth, torch, dev, warmup=3, reps=10):
    """FP8 matrix-core rate of the indexer on the prefill chunk (4096 query tokens appended to a
    126976-token prefix, causal): HIP events on the launch stream around each of `reps` launches
    of dsa_index_score after `warmup` untimed ones."""
    wl = synth.WORKLOADS["prefill_4096_at_128k"]
    g = synth.generate(wl, seed=0, device=dev, with_mla=False)
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    scores = torch.empty((wl.B, wl.Q, wl.lmax), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dsa.index_score(g.q_idx, g.w, keys, g.seq_lens, wl.lmax, scores=scores, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        dsa.index_score(g.q_idx, g.w, keys, g.seq_lens, wl.lmax, scores=scores, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
    _, flops = index_work(wl)
    del g, scores
    torch.cuda.empty_cache()
    return {"workload": wl.name, "kernel": "index_score (multi-query form)", "us_per_launch": us,
            "tflops": flops / us / 1e6, "peak_tflops": FP8_PEAK_TFLOPS, "frac": flops / us / 1e6 / FP8_PEAK_TFLOPS,
            "flop_per_launch": flops, "launches": reps,
            "note": "causal pairs x Hi x 128 x 2 FLOP over the mean event-timed launch, after the timed region"}


def traffic_from_profile(wl_name):
    """HBM bytes per index-score launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (matched by hash); else None."""
    path = os.path.join(ROOT, "profiles", f"index_score_{wl_name}_counters.json")
    src = os.path.join(ROOT, "sparse_attention_lightning_amd", "csrc", "index_score.hip")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if rec.get("source_sha256_16") != h:
            return None
        return rec["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(batches, wl, budget_s):
    """The oracle as it stands, timed on a bounded sample of the same workload on host cores: the
    plain C reference (OpenMP over keys and heads) for the DSA workloads, the numpy oracle for
    compressed sparse attention."""
    import numpy as np
    import torch

    import oracle
    from oracle import cref
    import synth

    cores = len(os.sched_getaffinity(0))
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    cref.build()
    done_tokens, done_rows, elapsed, seqs = 0, 0, 0.0, 0
    rows_per_seq = 1 if wl.share_first_query else wl.Q
    wall0 = time.perf_counter()
    # the batches in turn, again from the first while the budget lasts (bounded in wall time too:
    # copying a long sequence's caches to the host is not timed but takes time)
    work = [(gi, b) for gi in range(len(batches)) for b in range(wl.B)]
    for it in range(16 * len(work)):
        gi, b = work[it % len(work)]
        if it > 0 and (elapsed >= budget_s or time.perf_counter() - wall0 >= 3 * budget_s):
            break
        g = batches[gi]
        # inputs of sequence b in logical token order (input preparation, not timed)
        def seq_rows(data, table):
            if data.dtype == torch.bfloat16:
                data = data.view(torch.int16)
            if table is None:
                return data[b:b + 1].cpu().numpy()
            return data[table[b].long()].reshape(1, -1, data.shape[-1]).cpu().numpy()
        keys = oracle.Cache(seq_rows(g.keys, g.key_table))
        lats = [oracle.Cache(r.view(np.uint16) if r.dtype == np.int16 else r)
                for r in (seq_rows(g.latent[l], g.latent_table[l]) for l in range(len(g.latent)))]
        if wl.ratio:
            win = (oracle.Cache(seq_rows(g.window_latent, g.window_table).view(np.uint16))
                   if g.window_latent is not None else oracle.Cache(np.zeros((1, 1, 576), dtype=np.uint16)))
        q_idx = g.q_idx[b].cpu().numpy()
        w = g.w[b].cpu().numpy()
        q_src = synth.draft_queries(g, wl.draft_steps) if wl.draft_steps else g.q_mla
        q_mla = [t[b].view(torch.int16).cpu().numpy().view(np.uint16) for t in q_src]
        lat_of = (lambda i: lats[0]) if wl.draft_steps else (lambda i: lats[i])
        n = wl.lens[b]
        seqs += 1
        for j in range(rows_per_seq):        # the budget is checked after every query token
            p = n - wl.Q + j
            t0 = time.perf_counter()
            if wl.ratio:             # compressed sparse attention: selection, window and attention in one
                oracle.csa.csa_one(q_idx[j], w[j], keys, lats[0], win, 0, p, wl.ratio, wl.k, wl.window, q_mla[0][j],
                                   wl.scale, wl.rows)
            else:
                s = cref.index_scores(q_idx[j], w[j], keys.data[0], p, wl.lmax)
                idx = cref.select_topk(s.astype(np.float32), p, wl.k)
                sel = idx[idx >= 0]
                users = range(wl.Q) if wl.share_first_query else [j]
                for c in range(len(q_mla)):          # every layer, or every draft step of an MTP loop
                    rows = lat_of(c).data[0][sel]
                    for u in users:
                        cref.sparse_mla(q_mla[c][u], rows, wl.scale, latent_scale=1.0)
            elapsed += time.perf_counter() - t0
            done_tokens += (wl.Q if wl.share_first_query else 1) * max(1, wl.draft_steps)
            done_rows += 1
            if elapsed >= budget_s:
                break
    form = "numpy float64 (compressed sparse attention oracle)" if wl.ratio else \
        "plain C, float64, OpenMP over keys and heads (oracle/dsa_ref.c)"
    return {"value": done_tokens / elapsed, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done_rows} selections over {seqs} sequence visits ({len(batches)} batches of {wl.B} sequences) "
                      f"of {wl.name} ({done_tokens} query or "
                      f"draft tokens: index scores over every visible key, top-{wl.k}, sparse MLA over {wl.H} heads x "
                      f"{len(q_mla)} layer(s) or draft step(s)); {elapsed:.1f} s of oracle time; {form}; "
                      f"threads={threads}, affinity cores={cores}"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the DSA path on one GPU; runs on more than one GPU are not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    import sparse_attention_lightning_amd as dsa

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hot = wl.n_slots > 0
    # A hot-buffer workload decodes consecutive steps over one cache, its indexer query
    # drifting from step to step; the others cycle through independent batches.
    batches = [synth.generate(wl, seed=s, device=dev) for s in range(1 if hot else args.rotate)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    rows_sel = wl.B * (1 if wl.share_first_query else wl.Q)
    scores = torch.empty((wl.B, 1 if wl.share_first_query else wl.Q, wl.rows), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.B, scores.shape[1], wl.k), dtype=torch.int32, device=dev)
    outs = [torch.empty((wl.B, wl.Q, wl.H, 512), dtype=torch.float32, device=dev) for _ in range(wl.n_layers)]
    lses = [torch.empty((wl.B, wl.Q, wl.H), dtype=torch.float32, device=dev) for _ in range(wl.n_layers)]
    ws_topk = torch.empty(dsa.workspace_size(dsa.OP_TOPK, wl.B, scores.shape[1], wl.lmax, k=wl.k), dtype=torch.uint8,
                          device=dev)
    n_mla = dsa.workspace_size(dsa.OP_SPARSE_MLA, wl.B, wl.Q, wl.lmax, H=wl.H, k=wl.k)
    ws_mla = torch.empty(max(n_mla, 1), dtype=torch.uint8, device=dev)
    # A group of layers sharing one index set (IndexShare) runs as one dsa_forward_shared call,
    # which launches every layer's MLA together; a single layer runs as the three stage calls.
    group = wl.n_layers > 1
    ws_fs = None
    if group:
        n_fs = dsa.workspace_size(dsa.OP_FORWARD_SHARED, wl.B, wl.Q, wl.lmax, H=wl.H, k=wl.k, n_layers=wl.n_layers)
        ws_fs = torch.empty(n_fs, dtype=torch.uint8, device=dev)
        idx_fs = torch.empty((wl.B, 1 if wl.share_first_query else wl.Q, wl.k), dtype=torch.int32, device=dev)
    q_pos = None
    if wl.share_first_query:   # scores + top-k for query token 0 of each sequence only
        q_pos = torch.tensor([[n - wl.Q] for n in wl.lens], dtype=torch.int32, device=dev)
    if wl.ratio:
        # compressed sparse attention: one dsa_csa_forward call per step. The breakdown after the
        # timed region also calls the scan and top-k over the compressed entries separately (each
        # query at its last visible one); the attention over the union of the selected compressed
        # rows and the window's raw rows is the call minus those two
        ws_csa = torch.empty(max(1, dsa.csa_workspace_size(wl.B, wl.Q, wl.lmax, wl.H, wl.ratio, wl.k, wl.window)),
                             dtype=torch.uint8, device=dev)
        pos = [[n - wl.Q + j for j in range(wl.Q)] for n in wl.lens]
        q_pos = torch.tensor([[(p + 1) // wl.ratio - 1 for p in r] for r in pos], dtype=torch.int32, device=dev)
    ev = {k: [] for k in ("index", "topk", "mla", "group", "swap")}
    n_all_steps = args.warmup + args.steps + 3
    if hot:
        # HiSparse: the latent pages of every sequence in pinned host memory, logical order;
        # the device keeps n_slots slots per sequence (state -1: empty before the warm-up)
        g0 = batches[0]
        host_pool = g0.latent[0][g0.latent_table[0].long()].cpu().pin_memory()
        hb = dsa.HotBuffer(
            block_table=torch.full((wl.B, wl.max_pages), -1, dtype=torch.int32, device=dev),
            slot_page=torch.full((wl.B, wl.n_slots), -1, dtype=torch.int32, device=dev),
            slot_clock=torch.full((wl.B, wl.n_slots), -1, dtype=torch.int32, device=dev),
            page_clock=torch.full((wl.B, wl.max_pages), -1, dtype=torch.int32, device=dev),
            device_pool=torch.zeros((wl.B * wl.n_slots, wl.page_size, 576), dtype=host_pool.dtype, device=dev),
            page_size=wl.page_size)
        hot_lat = hb.latent_cache()
        drift = synth.drift_queries(g0, n_all_steps)
        copied = torch.zeros((n_all_steps, wl.B), dtype=torch.int32, device=dev)
        ws_swap = torch.empty(dsa.workspace_size(dsa.OP_HISPARSE_SWAP_IN, wl.B, wl.Q, 1, k=wl.k), dtype=torch.uint8,
                              device=dev)
        torch.cuda.synchronize()
    # per-batch call arguments, built once (nothing but the library calls runs in a step)
    prepared = []
    if wl.draft_steps:      # an MTP draft loop: one latent cache, a query per draft step
        outs = [torch.empty((wl.B, wl.Q, wl.H, 512), dtype=torch.float32, device=dev) for _ in range(wl.draft_steps)]
        lses = [torch.empty((wl.B, wl.Q, wl.H), dtype=torch.float32, device=dev) for _ in range(wl.draft_steps)]
    for g in batches:
        lats = [dsa.Cache(g.latent[layer], g.latent_table[layer], wl.page_size) for layer in range(wl.n_layers)]
        if wl.draft_steps:
            mla_calls = [(q, lats[0]) for q in synth.draft_queries(g, wl.draft_steps)]
        else:
            mla_calls = [(g.q_mla[layer], lats[layer]) for layer in range(wl.n_layers)]
        prepared.append({
            "win": (dsa.Cache(g.window_latent, g.window_table, wl.page_size) if g.window_latent is not None
                    else None),
            "keys": dsa.Cache(g.keys, g.key_table, wl.page_size),
            "lats": lats,
            "mla_calls": mla_calls,
            "qi": g.q_idx[:, :1].contiguous() if wl.share_first_query else g.q_idx,
            "wi": g.w[:, :1].contiguous() if wl.share_first_query else g.w,
            "g": g,
        })

    def group_call(pr, g):
        dsa.forward_shared(g.q_idx, g.w, pr["keys"], wl.k, g.q_mla, pr["lats"], wl.scale, g.seq_lens, wl.lmax,
                           share_first_query=bool(wl.share_first_query), outs=outs, lses=lses, idx=idx_fs, ws=ws_fs,
                           stream=stream, latent_scales=[1.0] * wl.n_layers if wl.latent_fp8 else None)

    kRepeat = 8      # back-to-back calls per timed interval of the group and CSA breakdowns, so that
                     # the queue never drains inside an interval and the first launch's start-up is shared

    def csa_call(pr, g):
        dsa.csa_forward(g.q_idx, g.w, pr["keys"], pr["lats"][0], pr["win"], wl.ratio, wl.k, wl.window, g.q_mla[0],
                        wl.scale, g.seq_lens, wl.lmax, out=outs[0], lse=lses[0], idx=idx if wl.k else None, ws=ws_csa,
                        stream=stream)

    def step(i, record):
        """One pass of the hot path. record = "index": timing events around the index scan only (an event
        record costs a few microseconds of queue time, so only every fourth timed step carries these two);
        "all": events around every stage."""
        pr = prepared[i % len(prepared)]
        g = pr["g"]
        if wl.ratio:
            if record == "all":
                e = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
                e[0].record(stream)
                for _ in range(kRepeat if scan_runs(wl) else 0):
                    dsa.index_score(g.q_idx, g.w, pr["keys"], g.seq_lens, wl.rows, q_pos=q_pos, scores=scores,
                                    stream=stream)
                e[1].record(stream)
                for _ in range(kRepeat if scan_runs(wl) else 0):
                    dsa.topk(scores, g.seq_lens, wl.k, q_pos=q_pos, idx=idx, ws=ws_topk, stream=stream)
                e[2].record(stream)
                e[4].record(stream)
                for _ in range(kRepeat):
                    csa_call(pr, g)
                e[5].record(stream)
                if scan_runs(wl):                  # HCA: no scan or top-k to time
                    ev["index"].append((e[0], e[1]))
                    ev["topk"].append((e[1], e[2]))
                ev["group"].append((e[4], e[5]))
            else:
                csa_call(pr, g)
            return
        if group:
            if record == "all":
                # breakdown: index scan and top-k as separate calls, then the whole group call; the MLA
                # launches are the group call minus those two stages
                e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                e[0].record(stream)
                for _ in range(kRepeat):
                    dsa.index_score(pr["qi"], pr["wi"], pr["keys"], g.seq_lens, wl.lmax, q_pos=q_pos, scores=scores,
                                    stream=stream)
                e[1].record(stream)
                for _ in range(kRepeat):
                    dsa.topk(scores, g.seq_lens, wl.k, q_pos=q_pos, idx=idx, ws=ws_topk, stream=stream)
                e[2].record(stream)
                e[3].record(stream)
                for _ in range(kRepeat):
                    group_call(pr, g)
                e[4].record(stream)
                ev["index"].append((e[0], e[1]))
                ev["topk"].append((e[1], e[2]))
                ev["group"].append((e[3], e[4]))
            else:
                group_call(pr, g)
            return
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            e[0].record(stream)
        qi = drift[i] if hot else pr["qi"]
        dsa.index_score(qi, pr["wi"], pr["keys"], g.seq_lens, wl.lmax, q_pos=q_pos, scores=scores, stream=stream)
        if record:
            e[1].record(stream)
        dsa.topk(scores, g.seq_lens, wl.k, q_pos=q_pos, idx=idx, ws=ws_topk, stream=stream)
        if record == "all":
            e[2].record(stream)
        if hot:     # the step's selected pages into the device slots, then attention over them
            dsa.hisparse_swap_in(idx, i, hb, host_pool, copied=copied[i], ws=ws_swap, stream=stream)
            if record == "all":
                e[4].record(stream)
                ev["swap"].append((e[2], e[4]))
        # every layer of the step (or every draft step of an MTP loop) attends over the one index set
        for c, (q_mla, lat) in enumerate(pr["mla_calls"]):
            dsa.sparse_mla_fwd(q_mla, hot_lat if hot else lat, idx,
                               wl.k, wl.scale, g.seq_lens, wl.lmax, idx_q_stride=0 if wl.share_first_query else wl.k,
                               out=outs[c], lse=lses[c], ws=ws_mla if n_mla else None, stream=stream,
                               latent_scale=1.0 if wl.latent_fp8 else None)
        if record == "all":
            e[3].record(stream)
            ev["topk"].append((e[1], e[2]))
            ev["mla"].append((e[4] if hot else e[2], e[3]))
        if record:
            ev["index"].append((e[0], e[1]))

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, "index" if i % 4 == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    index_us = sum(a.elapsed_time(b) for a, b in ev["index"]) / len(ev["index"]) * 1e3 if ev["index"] else None
    # stage breakdown, outside the timed region: a few steps with events around every stage
    ev = {k: [] for k in ("index", "topk", "mla", "group", "swap")}
    for i in range(3):
        step(args.warmup + args.steps + i, "all")
    torch.cuda.synchronize()
    avg = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) * 1e3 for k, v in ev.items() if v}   # microseconds
    if wl.ratio or group:
        for key in ("index", "topk", "group"):
            if key in avg:
                avg[key] /= kRepeat
    if wl.ratio:
        # the attention over the union of the two lists is what the one call spends beyond the stages
        avg.setdefault("index", 0.0)
        avg.setdefault("topk", 0.0)
        avg["mla"] = max(0.0, avg["group"] - avg["index"] - avg["topk"])
    elif group:
        avg["mla"] = avg["group"] - avg["index"] - avg["topk"]
    else:
        avg["index"] = index_us

    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tokens = wl.B * wl.Q * max(1, wl.draft_steps)      # an MTP loop yields a draft token per draft step
    value = tokens / (ms_per_step / 1e3)
    ibytes, iflops = index_work(wl)
    mbytes, mflops = mla_work(wl)
    index_s = avg["index"] * 1e-6
    n_mla_calls = wl.draft_steps or wl.n_layers
    if not scan_runs(wl):
        # no scan in the step (every visible compressed entry is kept): the latent gather dominates
        mla_s = avg["mla"] * 1e-6 / n_mla_calls
        roof = {"bound": "hbm", "achieved": mbytes / mla_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "traffic": None, "kernel": "sparse_mla (+ combine): latent-row gather"}
    elif args.workload.startswith("prefill"):
        roof = {"bound": "mfma", "achieved": iflops / index_s / 1e12, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": ibytes / index_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if scan_runs(wl):
        roof["traffic"] = traffic_from_profile(args.workload)
        roof["kernel"] = "index_score (lightning indexer scan)"
    step_bytes = ibytes + mbytes * n_mla_calls
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3+bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Q": wl.Q, "L": wl.L, "page_size": wl.page_size, "k": wl.k,
                   "Hi": wl.Hi, "H": wl.H, "n_layers": wl.n_layers, "share_first_query": wl.share_first_query,
                   "draft_steps": wl.draft_steps, "hot_buffer_slots": wl.n_slots, "latent_fp8": wl.latent_fp8,
                   "planted": wl.planted, "compression_ratio": wl.ratio, "window": wl.window},
        "roofline": roof,
        "kernels_us": {"index_score": avg["index"], "topk": avg["topk"], "sparse_mla": avg["mla"],
                       "note": ("one dsa_csa_forward call per timed step; breakdown in 3 steps after the timed "
                                "region, each stage timed over %d back-to-back calls between two events: "
                                "index_score and topk as separate calls; sparse_mla (one launch over the selected "
                                "compressed rows and the window rows): the whole call minus those two" % kRepeat
                                if wl.ratio else
                                "one dsa_forward_shared call per timed step (all layers' MLA launched together); "
                                "breakdown in 3 steps after the timed region, each stage timed over %d back-to-back "
                                "calls between two events: index_score and topk as separate calls; sparse_mla: the "
                                "group call minus those two" % kRepeat if group else
                                "index_score: HIP events around the scan in every fourth timed step; topk and sparse_mla: "
                                "events around each stage in 3 steps after the timed region")},
        "step_hbm_GBps_algorithmic": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "index_tflops": iflops / index_s / 1e12 if index_s > 0 else None,
        "mla_tflops": mflops * n_mla_calls / (avg["mla"] * 1e-6) / 1e12,
    }
    if hot:
        # pages pulled from host memory per timed step (the queries drift, so each step misses a part)
        per_step = copied[args.warmup:args.warmup + args.steps].sum(dim=1).float().mean().item()
        page_bytes = wl.page_size * 576 * host_pool.element_size()
        line["kernels_us"]["hisparse_swap_in"] = avg["swap"]
        line["kernels_us"]["note"] += "; hisparse_swap_in: events around the swap-in in the same 3 steps"
        line["hot_buffer"] = {
            "slots_per_sequence": wl.n_slots, "page_tokens": wl.page_size, "pages_per_sequence": wl.max_pages,
            "pages_copied_per_step": per_step, "bytes_copied_per_step": per_step * page_bytes,
            "host_read_GBps": per_step * page_bytes / (avg["swap"] * 1e-6) / 1e9,
            "note": "latent pages read by the copy kernel from pinned host memory; host_read_GBps = bytes copied "
                    "per timed step / swap-in time of the breakdown steps"}
    if not args.workload.startswith("prefill"):
        # the decode gather: sparse MLA and its split combine, against the HBM peak
        mla_s = avg["mla"] * 1e-6 / n_mla_calls
        line["roofline_mla"] = {"bound": "hbm", "achieved": mbytes / mla_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": mbytes / mla_s / 1e9 / HBM_PEAK_GBS, "bytes_per_call": mbytes,
                                "us_per_call": mla_s * 1e6,
                                "kernel": "sparse_mla + mla_combine (latent-row gather, one call per layer or draft step)"}
        if not args.no_prefill_index:
            line["prefill_index"] = prefill_index_figure(dsa, synth, torch, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(batches, wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
