"""GPU parity of compressed sparse attention (dsa_csa_forward) against the CSA oracle.

Small cases compare every query token: the selected compressed entries against the oracle's
(equal up to near-threshold swaps, with the exact compressed scores), and the attention output
against the oracle evaluated on the GPU's own selection (fixed bars: max abs 2e-2, rel L2
5e-3; lse within 1e-3). The full-size workloads are checked on sampled sequences and by
properties of every row.
"""
import gc
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import csa as ocsa
from oracle.dsa import Cache as OCache
from helpers import bits, check_mla, check_topk_sets, np_

pytestmark = pytest.mark.gpu
dsa = pytest.importorskip("sparse_attention_lightning_amd")
DEV = "cuda"


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def seq_view(data, table, b, page_size):
    """Sequence b of a cache on the host, in logical row order (input relayout only)."""
    if data is None:
        return OCache(np.zeros((1, 1, 576), dtype=np.uint16))
    if data.dtype == torch.bfloat16:
        data = data.view(torch.int16)
    x = data[b:b + 1] if table is None else data[table[b].long()].reshape(1, -1, data.shape[-1])
    arr = x.cpu().numpy()
    return OCache(arr.view(np.uint16) if arr.dtype == np.int16 else arr)


def run_gpu(g, wl):
    keys_c = dsa.Cache(g.keys, g.key_table, wl.page_size)
    lat_c = dsa.Cache(g.latent[0], g.latent_table[0], wl.page_size)
    lat = dsa.Cache(g.window_latent, g.window_table, wl.page_size) if g.window_latent is not None else None
    return dsa.csa_forward(g.q_idx, g.w, keys_c, lat_c, lat, wl.ratio, wl.k, wl.window, g.q_mla[0], wl.scale,
                           g.seq_lens, wl.lmax)


def check_query(g, wl, b, j, idx, out, lse):
    """One query token against the oracle: selection (with exact compressed scores) and output."""
    p = wl.lens[b] - wl.Q + j
    kc = seq_view(g.keys, g.key_table, b, wl.page_size)
    lc = seq_view(g.latent[0], g.latent_table[0], b, wl.page_size)
    lr = seq_view(g.window_latent, g.window_table, b, wl.page_size)
    qi, w = np_(g.q_idx[b, j]), np_(g.w[b, j])
    qm = bits(g.q_mla[0][b, j])
    swaps = 0
    if wl.k > 0:
        o_sel, exact = ocsa.select_compressed(qi, w, kc, 0, p, wl.ratio, wl.k, wl.rows)
        g_sel = np_(idx[b, j])
        n_c = ocsa.visible_compressed(p, wl.ratio)
        if n_c == 0:
            assert np.all(g_sel == -1)
        else:
            swaps = check_topk_sets(g_sel, o_sel, exact, wl.k)
    else:
        g_sel = np.zeros(0, dtype=np.int32)
    _, ref_o, ref_l, _ = ocsa.csa_one(qi, w, kc, lc, lr, 0, p, wl.ratio, wl.k, wl.window, qm, wl.scale, wl.rows,
                                      sel=g_sel)
    check_mla(np_(out[b, j]), np_(lse[b, j]), ref_o, ref_l)
    return swaps


CASES = [
    # decode form over paged caches, a planted set, ragged lengths spanning several key chunks
    ("csa_pro_decode_b32_128k", dict(B=3, L=9000, L_max=9024, planted=4, seq_lens=(9000, 6001, 4097), k=300)),
    # the first raw tokens: no complete block yet (only the window), then exactly one block
    ("csa_pro_decode_b32_128k", dict(B=4, L=4000, L_max=4032, planted=0, seq_lens=(2, 3, 4, 4000), k=64)),
    # the multi-query scan form over a contiguous cache with an odd row stride, H = 64, Hi = 32
    ("csa_pro_decode_b32_128k", dict(B=2, Q=3, L=5001, L_max=5001, page_size=0, planted=0, seq_lens=(5001, 1500),
                                     k=200, H=64, Hi=32, window=96)),
    # a window only (k = 0): sliding-window attention
    ("csa_flash_decode_b8_1m", dict(B=2, L=3000, L_max=3008, planted=0, seq_lens=(3000, 77), k=0)),
    # HCA: compressed by 128, every visible entry kept, no window
    ("hca_decode_b32_128k", dict(B=3, L=40000, L_max=40064, seq_lens=(40000, 20000, 130), k=320)),
    # a window of 2048 (the most a split list holds) and a short selection
    ("csa_flash_decode_b8_1m", dict(B=2, L=6000, L_max=6016, planted=0, seq_lens=(6000, 2500), k=16, window=2048)),
]


@pytest.mark.parametrize("name,kw", CASES)
def test_csa_small(name, kw):
    wl = synth.small(name, **kw)
    cpu = synth.generate(wl, seed=1, device="cpu")
    g = cpu.to(DEV)
    idx, out, lse = run_gpu(g, wl)
    torch.cuda.synchronize()
    swaps = 0
    for b in range(wl.B):
        for j in range(wl.Q):
            swaps += check_query(cpu, wl, b, j, idx, out, lse)
    if wl.planted:
        sets = np_(idx)
        for b in range(wl.B):
            assert set(cpu.planted_pos[b].tolist()) <= set(sets[b, -1].tolist())
    print(f"{name} {kw}: {swaps} near-threshold swaps")


@pytest.mark.parametrize("form", ["radix", "sampled", "row"])
def test_csa_each_topk_form(form):
    wl = synth.small("csa_pro_decode_b32_128k", B=2, L=12000, L_max=12032, planted=4, seq_lens=(12000, 9000), k=500)
    cpu = synth.generate(wl, seed=2, device="cpu")
    g = cpu.to(DEV)
    prev = os.environ.get("DSA_TOPK_FORM")
    os.environ["DSA_TOPK_FORM"] = form
    try:
        idx, out, lse = run_gpu(g, wl)
        torch.cuda.synchronize()
    finally:
        if prev is None:
            del os.environ["DSA_TOPK_FORM"]
        else:
            os.environ["DSA_TOPK_FORM"] = prev
    for b in range(wl.B):
        check_query(cpu, wl, b, 0, idx, out, lse)


def test_csa_ratio_one_without_window_is_the_dsa_path():
    """With ratio 1 and no window, the compressed caches are the raw ones and the call equals the
    DSA stage calls (index scores, top-k, sparse MLA) bit for bit."""
    wl = synth.small("decode_b32_128k_paged", B=2, L=6000, L_max=6016, planted=4, seq_lens=(6000, 4100), k=700)
    g = synth.generate(wl, seed=3, device=DEV)
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    lat = dsa.Cache(g.latent[0], g.latent_table[0], wl.page_size)
    idx, out, lse = dsa.csa_forward(g.q_idx, g.w, keys, lat, None, 1, wl.k, 0, g.q_mla[0], wl.scale, g.seq_lens,
                                    wl.lmax)
    scores = dsa.index_score(g.q_idx, g.w, keys, g.seq_lens, wl.lmax)
    idx2 = dsa.topk(scores, g.seq_lens, wl.k)
    out2, lse2 = dsa.sparse_mla_fwd(g.q_mla[0], lat, idx2, wl.k, wl.scale, g.seq_lens, wl.lmax)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2)


def test_hca_keeps_every_entry_without_indexer_inputs():
    """When k covers every compressed row (HCA), the selection keeps every visible entry whatever
    the scores: the call needs no indexer inputs and gives the same bits without them."""
    wl = synth.small("hca_decode_b32_128k", B=3, L=40000, L_max=40064, seq_lens=(40000, 20000, 130), k=320)
    g = synth.generate(wl, seed=4, device=DEV)
    lat_c = dsa.Cache(g.latent[0], g.latent_table[0], wl.page_size)
    idx, out, lse = run_gpu(g, wl)
    idx2, out2, lse2 = dsa.csa_forward(None, None, None, lat_c, None, wl.ratio, wl.k, 0, g.q_mla[0], wl.scale,
                                       g.seq_lens, wl.lmax)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2)
    for b in range(wl.B):
        n_c = wl.n_visible(wl.lens[b])
        assert np_(idx)[b, 0].tolist() == list(range(n_c)) + [-1] * (wl.k - n_c)


def test_csa_caches_of_different_layouts():
    """The attention runs over two index lists on two caches, each with its own layout: compressed
    caches stored contiguously and the raw cache in pages of 16 under another permutation give the
    bits of the all-paged (64) call, since the same rows are gathered."""
    wl = synth.small("csa_pro_decode_b32_128k", B=2, L=9000, L_max=9024, planted=4, seq_lens=(9000, 5000), k=300)
    g = synth.generate(wl, seed=5, device=DEV)
    idx, out, lse = run_gpu(g, wl)

    def contiguous(pool, table, rows):
        x = pool[table.long()].reshape(wl.B, -1, pool.shape[-1])
        return x[:, :rows].contiguous()

    keys_c = contiguous(g.keys, g.key_table, wl.rows)
    lat_c = contiguous(g.latent[0], g.latent_table[0], wl.rows)
    raw = g.window_latent[g.window_table.long()].reshape(wl.B, -1, 576)          # logical order
    n16 = raw.shape[1] // 16
    perm = torch.randperm(wl.B * n16, generator=torch.Generator().manual_seed(6)).to(DEV)
    pool16 = torch.empty((wl.B * n16, 16, 576), dtype=raw.dtype, device=DEV)
    pool16[perm] = raw.reshape(wl.B * n16, 16, 576)
    table16 = perm.to(torch.int32).view(wl.B, n16).contiguous()
    idx2, out2, lse2 = dsa.csa_forward(g.q_idx, g.w, dsa.Cache(keys_c, None, 0), dsa.Cache(lat_c, None, 0),
                                       dsa.Cache(pool16, table16, 16), wl.ratio, wl.k, wl.window, g.q_mla[0],
                                       wl.scale, g.seq_lens, wl.lmax)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2)


def test_csa_rejects_before_hip():
    wl = synth.small("csa_pro_decode_b32_128k", B=1, L=4096, planted=0)
    g = synth.generate(wl, seed=0, device=DEV)
    keys_c = dsa.Cache(g.keys, g.key_table, wl.page_size)
    lat_c = dsa.Cache(g.latent[0], g.latent_table[0], wl.page_size)
    lat = dsa.Cache(g.window_latent, g.window_table, wl.page_size)
    for kw in (dict(k=0, window=0), dict(ratio=0), dict(k=2049), dict(window=-1)):
        a = dict(ratio=4, k=64, window=128)
        a.update(kw)
        with pytest.raises(dsa.DsaError):
            dsa.csa_forward(g.q_idx, g.w, keys_c, lat_c, lat, a["ratio"], a["k"], a["window"], g.q_mla[0], wl.scale,
                            g.seq_lens, wl.lmax)


# ----------------------------------------------------------------------------- full sizes
@pytest.mark.parametrize("name,sample", [
    ("csa_pro_decode_b32_128k", (0, 13, 31)),
    ("csa_flash_decode_b8_1m", (5,)),
    ("hca_decode_b32_128k", (2, 30)),
])
def test_csa_fullsize(name, sample):
    wl = synth.WORKLOADS[name]
    g = synth.generate(wl, seed=0, device=DEV)
    idx, out, lse = run_gpu(g, wl)
    idx2, out2, lse2 = run_gpu(g, wl)                      # bitwise reproducible
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2)
    del idx2, out2, lse2
    sets = np_(idx)
    for b in range(wl.B):                                  # every row: size, order, visibility
        n_c = wl.n_visible(wl.lens[b])
        m = min(wl.k, n_c)
        row = sets[b, 0]
        assert np.all(row[m:] == -1) and np.all(np.diff(row[:m]) > 0) and row[m - 1] < n_c
        if wl.planted:
            assert set(g.planted_pos[b].tolist()) <= set(row.tolist())
    for b in sample:
        s = check_query(g, wl, b, 0, idx, out, lse)
        print(f"  {name} b={b}: {s} near-threshold swaps")
