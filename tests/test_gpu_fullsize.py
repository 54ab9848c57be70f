"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

Inputs are drawn on the GPU. The oracle checks sampled sequences / query tokens one by one;
properties that hold at any size are checked on every row (set sizes, ascending order,
causality, planted tokens, run-to-run determinism).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import check_mla, check_scores, check_topk_sets, score_tolerance

pytestmark = pytest.mark.gpu
dsa = pytest.importorskip("sparse_attention_lightning_amd")
DEV = "cuda"


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def seq_cache(data, table, b):
    """Sequence b of a cache, in logical token order, on the host (input relayout only)."""
    if data.dtype == torch.bfloat16:
        data = data.view(torch.int16)
    if table is None:
        x = data[b:b + 1]
    else:
        x = data[table[b].long()].reshape(1, -1, data.shape[-1])
    arr = x.cpu().numpy()
    return oracle.Cache(arr.view(np.uint16) if arr.dtype == np.int16 else arr)


def q_bits(t, b):
    return t[b].view(torch.int16).cpu().numpy().view(np.uint16)


def check_rows_wellformed(idx, wl, share_first=False):
    """Every row: min(k, p+1) ascending positions <= p, then -1."""
    idx = idx.cpu().numpy()
    Qs = 1 if share_first else wl.Q
    for b in range(wl.B):
        for j in range(Qs):
            p = wl.lens[b] - wl.Q + j
            m = min(wl.k, p + 1)
            row = idx[b, j]
            assert np.all(row[m:] == -1)
            assert np.all(np.diff(row[:m]) > 0) and row[0] >= 0 and row[m - 1] <= p


def check_topk_exact(scores, idx, wl, rows, share_first=False):
    """The selection of each (b, j) in rows, bit for bit against the oracle's on the GPU's own fp32
    scores (the top-k is exact given its scores; only the scores carry rounding)."""
    s = scores.cpu().numpy()
    got = idx.cpu().numpy()
    for b, j in rows:
        p = wl.lens[b] - wl.Q + j
        assert np.array_equal(got[b, 0 if share_first else j], oracle.select_topk(s[b, 0 if share_first else j], p, wl.k)), (b, j)


def oracle_check_query(g, wl, b, j, scores_gpu, idx_gpu, outs, lses, share_first=False, layers=None,
                       q_mla=None, latent_scale=None):
    """Oracle for one query token (b, j) of a full-size batch. q_mla: the MLA query of each entry
    of outs (default: the layers' queries); latent_scale: the scale of an E4M3 latent cache."""
    layers = range(wl.n_layers) if layers is None else layers
    p = wl.lens[b] - wl.Q + j
    keys = seq_cache(g.keys, g.key_table, b)
    qi = g.q_idx[b, j].cpu().numpy()
    w = g.w[b, j].cpu().numpy()
    exact = oracle.index_scores(qi, w, keys, 0, p, wl.lmax)
    if scores_gpu is not None:
        tol = score_tolerance(qi, w, keys.rows(0, np.arange(wl.lmax)))
        check_scores(scores_gpu[b, j].cpu().numpy(), exact, tol, p)
    o_idx = oracle.select_topk(exact.astype(np.float32), p, wl.k)
    g_idx = idx_gpu[b, 0 if share_first else j].cpu().numpy()
    swaps = check_topk_sets(g_idx, o_idx, exact, wl.k)
    # the attention oracle takes the GPU's set, so that a permitted near-threshold swap does not
    # count against the output
    users = range(wl.Q) if share_first else [j]
    worst = (0.0, 0.0)
    q_src = g.q_mla if q_mla is None else q_mla
    for layer in layers:
        lat = seq_cache(g.latent[min(layer, len(g.latent) - 1)], g.latent_table[min(layer, len(g.latent) - 1)], b)
        qm = q_bits(q_src[layer], b)
        for u in users:
            ref_o, ref_l = oracle.sparse_mla_one(qm[u], lat, 0, g_idx, wl.scale, latent_scale=latent_scale)
            e = check_mla(outs[layer][b, u].cpu().numpy(), lses[layer][b, u].cpu().numpy(), ref_o, ref_l)
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    print(f"  {wl.name} b={b} j={j}: {swaps} near-threshold swaps, out max abs {worst[0]:.3g} rel L2 {worst[1]:.3g}")
    return swaps


def run_path(g, wl, share_first=False, q_mla=None, latent_scale=None):
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    q_pos = None
    qi, wi = g.q_idx, g.w
    if share_first:
        q_pos = torch.tensor([[n - wl.Q] for n in wl.lens], dtype=torch.int32, device=DEV)
        qi, wi = g.q_idx[:, :1].contiguous(), g.w[:, :1].contiguous()
    scores = dsa.index_score(qi, wi, keys, g.seq_lens, wl.lmax, q_pos=q_pos)
    idx = dsa.topk(scores, g.seq_lens, wl.k, q_pos=q_pos)
    outs, lses = [], []
    q_src = g.q_mla if q_mla is None else q_mla      # one query per layer, or per draft step on one cache
    for c in range(len(q_src)):
        layer = min(c, len(g.latent) - 1)
        lat = dsa.Cache(g.latent[layer], g.latent_table[layer], wl.page_size)
        o, l = dsa.sparse_mla_fwd(q_src[c], lat, idx, wl.k, wl.scale, g.seq_lens, wl.lmax,
                                  idx_q_stride=0 if share_first else wl.k, latent_scale=latent_scale)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    return scores, idx, outs, lses


def test_decode_b32_128k_paged():
    wl = synth.WORKLOADS["decode_b32_128k_paged"]
    g = synth.generate(wl, seed=0, device=DEV)
    scores, idx, outs, lses = run_path(g, wl)
    check_rows_wellformed(idx, wl)
    sets = idx.cpu().numpy()
    for b in range(wl.B):                                   # planted tokens are selected in every sequence
        assert set(g.planted_pos[b].tolist()) <= set(sets[b, 0].tolist())
    s2, i2, o2, l2 = run_path(g, wl)                        # bitwise reproducible
    assert torch.equal(scores, s2) and torch.equal(idx, i2) and torch.equal(outs[0], o2[0])
    check_topk_exact(scores, idx, wl, [(b, 0) for b in range(wl.B)])
    for b in (0, 5, 9, 13, 17, 22, 27, 31):
        oracle_check_query(g, wl, b, 0, scores, idx, outs, lses)


def test_decode_b32_128k_paged_fp8kv():
    """The decode batch over an E4M3 latent cache (576 codes per row, scale 1)."""
    wl = synth.WORKLOADS["decode_b32_128k_paged_fp8kv"]
    g = synth.generate(wl, seed=0, device=DEV)
    assert g.latent[0].dtype == torch.uint8
    scores, idx, outs, lses = run_path(g, wl, latent_scale=1.0)
    check_rows_wellformed(idx, wl)
    s2, i2, o2, l2 = run_path(g, wl, latent_scale=1.0)
    assert torch.equal(idx, i2) and torch.equal(outs[0], o2[0]) and torch.equal(lses[0], l2[0])
    check_topk_exact(scores, idx, wl, [(b, 0) for b in range(wl.B)])
    for b in (0, 11, 31):
        oracle_check_query(g, wl, b, 0, scores, idx, outs, lses, latent_scale=1.0)


def test_mtp_draft_b32_128k_paged():
    """One MTP draft loop at the decode shape: the index set of the base position serves all 7
    draft steps over the one latent cache; each step's attention is checked for two sequences."""
    wl = synth.WORKLOADS["mtp_draft_b32_128k_paged"]
    g = synth.generate(wl, seed=0, device=DEV)
    drafts = synth.draft_queries(g, wl.draft_steps)
    assert len(drafts) == 7 and len(g.latent) == 1
    scores, idx, outs, lses = run_path(g, wl, q_mla=drafts)
    check_rows_wellformed(idx, wl)
    for b in (2, 29):
        oracle_check_query(g, wl, b, 0, scores, idx, outs, lses, layers=range(7), q_mla=drafts)


def test_prefill_4096_at_128k():
    wl = synth.WORKLOADS["prefill_4096_at_128k"]
    g = synth.generate(wl, seed=0, device=DEV)
    scores, idx, outs, lses = run_path(g, wl)
    check_rows_wellformed(idx, wl)
    check_topk_exact(scores, idx, wl, [(0, j) for j in range(0, wl.Q, 32)] + [(0, wl.Q - 1)])
    for j in (0, 1234, 2047, 3001, 4095):
        oracle_check_query(g, wl, 0, j, scores, idx, outs, lses)


def test_indexshare_b8_1m_4layers():
    wl = synth.WORKLOADS["indexshare_b8_1m_4layers"]
    g = synth.generate(wl, seed=0, device=DEV)
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    lats = [dsa.Cache(g.latent[l], g.latent_table[l], wl.page_size) for l in range(4)]
    idx, res = dsa.forward_shared(g.q_idx, g.w, keys, wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax)
    torch.cuda.synchronize()
    check_rows_wellformed(idx, wl)
    # the group selects what separate stage calls select; its four layers match the oracle
    scores = dsa.index_score(g.q_idx, g.w, keys, g.seq_lens, wl.lmax)
    assert torch.equal(idx, dsa.topk(scores, g.seq_lens, wl.k))
    check_topk_exact(scores, idx, wl, [(b, 0) for b in range(wl.B)])
    oracle_check_query(g, wl, 3, 0, scores, idx, [o for o, _ in res], [l for _, l in res])


def test_indexshare_b8_1m_4layers_fp8kv():
    """The 1M-token IndexShare group over four E4M3 latent caches: the group selects what separate
    stage calls select; one sequence against the oracle in every layer."""
    wl = synth.WORKLOADS["indexshare_b8_1m_4layers_fp8kv"]
    g = synth.generate(wl, seed=0, device=DEV)
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    lats = [dsa.Cache(g.latent[l], g.latent_table[l], wl.page_size) for l in range(4)]
    idx, res = dsa.forward_shared(g.q_idx, g.w, keys, wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax,
                                  latent_scales=[1.0] * 4)
    torch.cuda.synchronize()
    check_rows_wellformed(idx, wl)
    scores = dsa.index_score(g.q_idx, g.w, keys, g.seq_lens, wl.lmax)
    assert torch.equal(idx, dsa.topk(scores, g.seq_lens, wl.k))
    oracle_check_query(g, wl, 6, 0, scores, idx, [o for o, _ in res], [l for _, l in res], latent_scale=1.0)


def test_decode_at_the_16m_token_limit():
    """One sequence at the longest context the library accepts (L_max = 2^24 tokens, paged by 64):
    indexer scores at 4096 sampled positions against the oracle, the top-k set bit for bit
    against the oracle's selection on the GPU's own fp32 scores (the long-row top-k form), the
    planted tokens in it, and the attention against the oracle on that set."""
    L = 1 << 24
    wl = synth.Workload("decode_16m", B=1, Q=1, L=L, page_size=64, planted=16)
    g = synth.generate(wl, seed=0, device=DEV)
    scores, idx, outs, lses = run_path(g, wl)
    check_rows_wellformed(idx, wl)
    p = L - 1
    rng = np.random.default_rng(0)
    t = np.unique(np.concatenate([rng.integers(0, L, 4096), g.planted_pos[0].cpu().numpy(), [0, p]]))
    key_rows = g.keys[g.key_table[0][torch.from_numpy(t // 64).to(DEV).long()].long(),
                      torch.from_numpy(t % 64).to(DEV).long()].cpu().numpy()
    qi, wi = g.q_idx[0, 0].cpu().numpy(), g.w[0, 0].cpu().numpy()
    sub = oracle.Cache(key_rows[None])
    exact = oracle.index_scores(qi, wi, sub, 0, t.size - 1, t.size)
    got = scores[0, 0, torch.from_numpy(t).to(DEV).long()].cpu().numpy()
    tol = score_tolerance(qi, wi, key_rows)
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= tol), float(err.max())
    s32 = scores[0, 0].cpu().numpy()
    assert np.array_equal(idx[0, 0].cpu().numpy(), oracle.select_topk(s32, p, wl.k))
    assert set(g.planted_pos[0].tolist()) <= set(idx[0, 0].cpu().tolist())
    sel = idx[0, 0].cpu().numpy()
    tab = g.latent_table[0][0].long()
    rows = g.latent[0].view(torch.int16)[tab[torch.from_numpy(sel // 64).to(DEV).long()],
                                         torch.from_numpy(sel % 64).to(DEV).long()].cpu().numpy().view(np.uint16)
    ref_o, ref_l = oracle.sparse_mla(q_bits(g.q_mla[0], 0)[0], rows, wl.scale)
    check_mla(outs[0][0, 0].cpu().numpy(), lses[0][0, 0].cpu().numpy(), ref_o, ref_l)


@pytest.mark.parametrize("name", ["verify_b64_q8_32k", "verify_b64_q8_32k_draftshare"])
def test_verify_b64_q8_32k(name):
    wl = synth.WORKLOADS[name]
    share = bool(wl.share_first_query)
    g = synth.generate(wl, seed=0, device=DEV)
    scores, idx, outs, lses = run_path(g, wl, share_first=share)
    check_rows_wellformed(idx, wl, share_first=share)
    check_topk_exact(scores, idx, wl, [(b, j) for b in range(wl.B) for j in range(1 if share else wl.Q)],
                     share_first=share)
    if share:
        oracle_check_query(g, wl, 5, 0, scores, idx, outs, lses, share_first=True)
    else:
        for j in (0, 3, 7):
            oracle_check_query(g, wl, 5, j, scores, idx, outs, lses)


@pytest.mark.parametrize("name", ["hisparse_b8_1m_decode", "hisparse_b8_1m_decode_fp8kv"])
def test_hisparse_b8_1m_decode(name):
    """The hot buffer at the benchmark's size: 8 sequences of 1M tokens, 6144 slots of 16
    tokens each, the latent cache in pinned host memory, three drifting decode steps. After
    each step the library's state equals the oracle's on the same selected sets (every table
    entry), the slots written by the step hold the host bytes of their pages, and sparse MLA
    over the hot buffer gives the bits of sparse MLA over the whole device cache."""
    wl = synth.WORKLOADS[name]
    g = synth.generate(wl, seed=0, device=DEV)
    fp8 = bool(wl.latent_fp8)
    scale8 = 1.0 if fp8 else None
    bits = torch.uint8 if fp8 else torch.int16
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    whole = dsa.Cache(g.latent[0], g.latent_table[0], wl.page_size)
    host = g.latent[0][g.latent_table[0].long()].view(bits).cpu().pin_memory()
    host_np = host.numpy()
    hb = dsa.HotBuffer(
        block_table=torch.full((wl.B, wl.max_pages), -1, dtype=torch.int32, device=DEV),
        slot_page=torch.full((wl.B, wl.n_slots), -1, dtype=torch.int32, device=DEV),
        slot_clock=torch.full((wl.B, wl.n_slots), -1, dtype=torch.int32, device=DEV),
        page_clock=torch.full((wl.B, wl.max_pages), -1, dtype=torch.int32, device=DEV),
        device_pool=torch.zeros((wl.B * wl.n_slots, wl.page_size, 576), dtype=bits, device=DEV),
        page_size=wl.page_size)
    st = oracle.HotBufferState.empty(wl.B, wl.max_pages, wl.n_slots)
    dev_np = np.zeros((wl.B * wl.n_slots, wl.page_size, 576), dtype=host_np.dtype)
    for step, q in enumerate(synth.drift_queries(g, 3)):
        scores = dsa.index_score(q, g.w, keys, g.seq_lens, wl.lmax)
        idx = dsa.topk(scores, g.seq_lens, wl.k)
        if step == 0:
            # the decode scan over 16-token pages and the top-k of a 1M row, against the oracle (sequence 6)
            b, p = 6, wl.lens[6] - 1
            kc = seq_cache(g.keys, g.key_table, b)
            qi, wi = q[b, 0].cpu().numpy(), g.w[b, 0].cpu().numpy()
            exact = oracle.index_scores(qi, wi, kc, 0, p, wl.lmax)
            check_scores(scores[b, 0].cpu().numpy(), exact, score_tolerance(qi, wi, kc.rows(0, np.arange(wl.lmax))), p)
            check_topk_sets(idx[b, 0].cpu().numpy(), oracle.select_topk(exact.astype(np.float32), p, wl.k), exact,
                            wl.k)
            del kc, exact
        del scores
        copied = torch.zeros((wl.B,), dtype=torch.int32, device=DEV)
        dsa.hisparse_swap_in(idx, step, hb, host, copied=copied)
        o1, l1 = dsa.sparse_mla_fwd(g.q_mla[0], hb.latent_cache(), idx, wl.k, wl.scale, g.seq_lens, wl.lmax,
                                    latent_scale=scale8)
        o2, l2 = dsa.sparse_mla_fwd(g.q_mla[0], whole, idx, wl.k, wl.scale, g.seq_lens, wl.lmax,
                                    latent_scale=scale8)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), step
        copies = oracle.swap_in(st, idx.cpu().numpy(), step, wl.page_size, host_np, dev_np)
        for name in ("block_table", "slot_page", "slot_clock", "page_clock"):
            assert np.array_equal(getattr(hb, name).cpu().numpy(), getattr(st, name)), (name, step)
        assert copied.cpu().tolist() == [sum(1 for c in copies if c[0] == b) for b in range(wl.B)], step
        pool = hb.device_pool.view(bits)
        for b, p, s in copies[:: max(1, len(copies) // 64)]:     # a sample of this step's copies
            assert np.array_equal(pool[b * wl.n_slots + s].cpu().numpy(), host_np[b, p]), (step, b, p)


@pytest.mark.parametrize("B,Q,L,lens,page_size", [
    (2, 1024, 200003, (200003, 150001), 0),       # contiguous rows, L_max % 8 != 0: each lane finds its row
    (8, 512, 65536, (65536, 60001, 65000, 33333, 65536, 40000, 65536, 512), 64),   # paged
])
def test_multi_query_scan_in_long_chunks(B, Q, L, lens, page_size):
    """Launches of the multi-query scan that hold 16 or more workgroups per CU at 8192 keys take
    8192-key chunks: scores of sampled query tokens against the oracle (ragged lengths, chunk
    edges inside a row), every score after the query -inf, and the selection of sampled rows bit
    for bit against the oracle's on the GPU's scores."""
    wl = synth.Workload("mq_long", B=B, Q=Q, L=L, L_max=L, seq_lens=lens, page_size=page_size, k=2048)
    g = synth.generate(wl, seed=3, device=DEV, with_mla=False)
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    scores = dsa.index_score(g.q_idx, g.w, keys, g.seq_lens, wl.lmax)
    idx = dsa.topk(scores, g.seq_lens, wl.k)
    torch.cuda.synchronize()
    rows = [(0, 0), (0, Q // 2), (0, Q - 1), (1, 7), (B - 1, Q - 1)]
    check_topk_exact(scores, idx, wl, rows + [(b, j) for b in range(B) for j in (0, Q - 1)])
    for b, j in rows:
        p = wl.lens[b] - wl.Q + j
        kc = seq_cache(g.keys, g.key_table, b)
        qi, wi = g.q_idx[b, j].cpu().numpy(), g.w[b, j].cpu().numpy()
        exact = oracle.index_scores(qi, wi, kc, 0, p, wl.lmax)
        tol = score_tolerance(qi, wi, kc.rows(0, np.arange(wl.lmax)))
        check_scores(scores[b, j].cpu().numpy(), exact, tol, p)
