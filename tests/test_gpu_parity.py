"""GPU parity of the DSA hot path against the CPU oracle, through the C ABI.

Small cases run the oracle on every output; they span several key chunks, split tiles and
a ragged tail. Tolerances and their derivations are in tests/helpers.py.
"""
import math

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (bits, check_mla, check_scores, check_topk_sets, dsa_cache, integer_e4m3, key_cache,
                     latent_cache, np_, positions, score_tolerance)

pytestmark = pytest.mark.gpu

dsa = pytest.importorskip("sparse_attention_lightning_amd")
DEV = "cuda"


def gpu_batch(wl, seed=0, layers=None, with_mla=True):
    """Draw on the CPU, copy to the GPU (small cases)."""
    cpu = synth.generate(wl, seed=seed, device="cpu", layers=layers, with_mla=with_mla)
    return cpu, cpu.to(DEV)


def keys_arg(g):
    return dsa_cache(g.keys, g.key_table, g.wl.page_size)


def lat_arg(g, layer=0):
    return dsa_cache(g.latent[layer], g.latent_table[layer], g.wl.page_size)


# ----------------------------------------------------------------------------- indexer
@pytest.mark.parametrize("Hi", [64, 32])
@pytest.mark.parametrize("page_size", [0, 64, 16])
def test_index_score_integer_inputs_exact(Hi, page_size):
    wl = synth.Workload("int", B=3, Q=2, L=5000, Hi=Hi, page_size=page_size, L_max=5056,
                        seq_lens=(5000, 4099, 1500))
    cpu, g = gpu_batch(wl, with_mla=False)
    gen = torch.Generator().manual_seed(11)
    cpu.q_idx = integer_e4m3(tuple(cpu.q_idx.shape), gen)
    cpu.keys = integer_e4m3(tuple(cpu.keys.shape), gen)
    g.q_idx, g.keys = cpu.q_idx.to(DEV), cpu.keys.to(DEV)
    scores = np_(dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax))
    torch.cuda.synchronize()
    kc = key_cache(cpu)
    pos = positions(wl)
    for b in range(wl.B):
        for j in range(wl.Q):
            p = pos[b][j]
            exact = oracle.index_scores(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc, b, p, wl.lmax)
            tol = score_tolerance(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc.rows(b, np.arange(wl.lmax)),
                                  integer_inputs=True)
            check_scores(scores[b, j], exact, tol, p)


@pytest.mark.parametrize("Q,page_size,L_max,lens", [
    (1, 16, 5008, (5000, 4099, 1500)),     # decode form over 16-token pages (the hot buffer's page)
    (1, 32, 5024, (5024, 4099, 1500)),
    (1, 48, 5040, (5001, 4099, 47)),       # a page size that is not a power of two; a one-page row
    (1, 0, 5001, (5001, 4099, 1500)),      # contiguous, L_max % 8 != 0: each lane finds its own row
    (2, 0, 5001, (5001, 4099, 1500)),      # the multi-query form of the same
    (3, 0, 4093, (4093, 2050, 17)),
])
def test_index_score_page_sizes_and_odd_row_strides(Q, page_size, L_max, lens):
    """Integer-valued inputs (exact products: only the fp32 head sum rounds), then the top-k sets
    of N(0,1) inputs against the oracle's, on page sizes and row strides the workloads do not use."""
    wl = synth.Workload("odd", B=3, Q=Q, L=max(lens), Hi=64, page_size=page_size, L_max=L_max, seq_lens=lens,
                        k=1000)
    cpu, g = gpu_batch(wl, with_mla=False)
    pos = positions(wl)
    kc = key_cache(cpu)
    # N(0,1) inputs: scores within the truncation bound, sets equal up to near-threshold swaps
    scores = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax)
    idx = np_(dsa.topk(scores, g.seq_lens, wl.k))
    scores = np_(scores)
    for b in range(wl.B):
        for j in range(wl.Q):
            p = pos[b][j]
            exact = oracle.index_scores(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc, b, p, wl.lmax)
            tol = score_tolerance(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc.rows(b, np.arange(wl.lmax)))
            check_scores(scores[b, j], exact, tol, p)
            check_topk_sets(idx[b, j], oracle.select_topk(exact.astype(np.float32), p, wl.k), exact, wl.k)
    # integer inputs: exact up to the fp32 head sum
    gen = torch.Generator().manual_seed(12)
    cpu.q_idx = integer_e4m3(tuple(cpu.q_idx.shape), gen)
    cpu.keys = integer_e4m3(tuple(cpu.keys.shape), gen)
    g.q_idx, g.keys = cpu.q_idx.to(DEV), cpu.keys.to(DEV)
    scores = np_(dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax))
    kc = key_cache(cpu)
    for b in range(wl.B):
        for j in range(wl.Q):
            p = pos[b][j]
            exact = oracle.index_scores(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc, b, p, wl.lmax)
            tol = score_tolerance(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc.rows(b, np.arange(wl.lmax)),
                                  integer_inputs=True)
            check_scores(scores[b, j], exact, tol, p)


@pytest.mark.parametrize("name,kw", [
    ("decode_tiny_8k", {}),                                                   # the 8K tiny decode workload as is
    ("decode_b32_128k_paged", dict(B=2, L=9000, L_max=9024, planted=4, seq_lens=(9000, 7777))),
    ("verify_b64_q8_32k", dict(B=2, L=4200, L_max=4224)),
])
def test_index_score_normal_inputs(name, kw):
    wl = synth.small(name, **kw)
    cpu, g = gpu_batch(wl, with_mla=False)
    scores = np_(dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax))
    kc = key_cache(cpu)
    pos = positions(wl)
    worst = 0.0
    for b in range(wl.B):
        for j in range(wl.Q):
            p = pos[b][j]
            exact = oracle.index_scores(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc, b, p, wl.lmax)
            tol = score_tolerance(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc.rows(b, np.arange(wl.lmax)))
            worst = max(worst, check_scores(scores[b, j], exact, tol, p))
    print(f"{name}: max |score error| {worst:.3g}")


def test_index_score_explicit_positions_and_determinism():
    wl = synth.small("verify_b64_q8_32k", B=2, Q=3, L=3000, L_max=3000, page_size=0)
    cpu, g = gpu_batch(wl, with_mla=False)
    q_pos = torch.tensor([[5, 1000, 2999], [0, 17, 2048]], dtype=torch.int32)
    s1 = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax, q_pos=q_pos.to(DEV))
    s2 = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax, q_pos=q_pos.to(DEV))
    assert torch.equal(s1, s2)
    scores = np_(s1)
    kc = key_cache(cpu)
    for b in range(2):
        for j in range(3):
            p = int(q_pos[b, j])
            exact = oracle.index_scores(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc, b, p, wl.lmax)
            tol = score_tolerance(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc.rows(b, np.arange(wl.lmax)))
            check_scores(scores[b, j], exact, tol, p)


# ----------------------------------------------------------------------------- top-k
# Three top-k forms give identical results; DSA_TOPK_FORM pins one (unset, the library picks by
# shape). Every top-k case runs in each form.
FORMS = ["radix", "sampled", "row"]


def run_topk(scores32, seq_lens, k, q_pos=None, form="radix"):
    scores32 = np.ascontiguousarray(scores32)
    t = torch.from_numpy(scores32).to(DEV)
    sl = torch.tensor(list(seq_lens), dtype=torch.int32, device=DEV)
    qp = None if q_pos is None else torch.tensor(np.asarray(q_pos), dtype=torch.int32, device=DEV)
    prev = os.environ.get("DSA_TOPK_FORM")
    os.environ["DSA_TOPK_FORM"] = form
    try:
        got = np_(dsa.topk(t, sl, k, q_pos=qp))
    finally:
        if prev is None:
            del os.environ["DSA_TOPK_FORM"]
        else:
            os.environ["DSA_TOPK_FORM"] = prev
    return got


def oracle_topk(scores32, seq_lens, k, q_pos=None):
    return oracle.topk_batch(scores32, seq_lens, k, q_pos=q_pos)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("k", [2048, 1, 7, 300])
def test_topk_exact_on_oracle_scores(k, form):
    wl = synth.small("verify_b64_q8_32k", B=3, Q=2, L=20000, L_max=20480, page_size=0, seq_lens=(20000, 9000, 2100))
    cpu = synth.generate(wl, seed=3, with_mla=False)
    s = oracle.index_scores_batch(np_(cpu.q_idx), np_(cpu.w), key_cache(cpu), wl.lens, wl.lmax)
    s32 = s.astype(np.float32)
    got = run_topk(s32, wl.lens, k, form=form)
    assert np.array_equal(got, oracle_topk(s32, wl.lens, k))


@pytest.mark.parametrize("form", FORMS)
def test_topk_exact_ties_and_degenerate_rows(form):
    rng = np.random.default_rng(7)
    L = 13000
    rows = [
        rng.integers(0, 50, L).astype(np.float32),                 # heavy ties at the threshold
        np.full(L, 3.5, np.float32),                                # all equal: the first k positions
        np.where(rng.random(L) < 0.5, -0.0, 0.0).astype(np.float32),  # -0 and +0 tie
        rng.normal(size=L).astype(np.float32),
        np.concatenate([np.full(L - 5000, -np.inf, np.float32), rng.normal(size=5000).astype(np.float32)]),
        (rng.integers(-3, 3, L) * 1e-30).astype(np.float32),        # denormal-scale values
    ]
    s = np.stack(rows)[:, None, :]
    lens = [L, L, L, 12345, L, 4097]
    for k in (2048, 1000, 1):
        got = run_topk(s, lens, k, form=form)
        assert np.array_equal(got, oracle_topk(s, lens, k)), k


@pytest.mark.parametrize("form", FORMS)
def test_topk_rows_shorter_than_k_and_positions(form):
    rng = np.random.default_rng(8)
    L = 6000
    s = rng.normal(size=(2, 4, L)).astype(np.float32)
    lens = [L, 1500]
    q_pos = [[0, 2047, 2048, 5999], [10, 1499, 700, 2047]]
    got = run_topk(s, lens, 2048, q_pos=q_pos, form=form)
    assert np.array_equal(got, oracle_topk(s, lens, 2048, q_pos=np.array(q_pos)))
    assert got[0, 0, 0] == 0 and np.all(got[0, 0, 1:] == -1)


@pytest.mark.parametrize("form", FORMS)
def test_topk_odd_row_length(form):
    # L_max % 4 != 0: rows start unaligned, so every form takes its scalar loads (each clamped
    # into the row); visible lengths end inside and at the row, across chunk and sample edges
    rng = np.random.default_rng(10)
    L = 13001
    s = rng.normal(size=(5, 1, L)).astype(np.float32)
    s[3, 0, :] = np.round(s[3, 0, :] * 4)                       # ties at the threshold
    lens = [L, 9999, 4097, 8193, 3]
    for k in (2048, 1000, 5):
        got = run_topk(s, lens, k, form=form)
        assert np.array_equal(got, oracle_topk(s, lens, k)), k


@pytest.mark.parametrize("form", FORMS)
def test_topk_emission_bucket_edges(form):
    # The ordered emission buckets the kept positions by position >> shift, with shift the least
    # that puts a row's positions below 2048 buckets. Visible lengths on both sides of each shift
    # change; scores rising with position put the whole selection in the last buckets, filled to
    # their width, and a random permutation spreads it.
    rng = np.random.default_rng(11)
    lens = [2048, 2049, 4096, 4097, 131072, 131073, 262144, 262145]
    L = 262160
    rising = np.tile(np.arange(L, dtype=np.float32), (len(lens), 1))
    spread = np.stack([rng.permutation(L).astype(np.float32) for _ in lens])
    middle = rng.normal(size=(len(lens), L)).astype(np.float32)
    for b, n in enumerate(lens):                     # a run of high scores in the middle of the row
        middle[b, max(0, n // 2 - 1500): n // 2 + 1500] += 100.0
    for s in (rising, spread, middle):
        s3 = s[:, None, :]
        for k in (2048, 2047):
            got = run_topk(s3, lens, k, form=form)
            assert np.array_equal(got, oracle_topk(s3, lens, k)), k


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("L", [8192, 8191, 4100])
def test_topk_short_rows(form, L):
    # rows of at most 8192 scores (the tiny decode's length), where the row form's sample is
    # short or skipped (rows up to 4096 keep every score as a candidate): aligned (L % 4 == 0)
    # and unaligned rows, ties, -inf runs, all-equal rows and lengths on both sides of k
    rng = np.random.default_rng(12 + L)
    rows = [
        rng.normal(size=L).astype(np.float32),
        rng.integers(0, 40, L).astype(np.float32),
        np.full(L, -2.5, np.float32),
        np.concatenate([rng.normal(size=L // 2), np.full(L - L // 2, -np.inf)]).astype(np.float32),
        (rng.integers(-3, 3, L) * 1e-30).astype(np.float32),
        rng.normal(size=L).astype(np.float32),
    ]
    s = np.stack(rows)[:, None, :]
    lens = [L, L - 1, L, L, 2049, 2048]
    for k in (2048, 2047, 100, 1):
        got = run_topk(s, lens, k, form=form)
        assert np.array_equal(got, oracle_topk(s, lens, k)), k


@pytest.mark.parametrize("form", FORMS)
def test_topk_deterministic(form):
    rng = np.random.default_rng(9)
    s = rng.integers(0, 1000, size=(4, 1, 70000)).astype(np.float32)
    a = run_topk(s, [70000] * 4, 2048, form=form)
    b = run_topk(s, [70000] * 4, 2048, form=form)
    assert np.array_equal(a, b)
    assert np.array_equal(a, oracle_topk(s, [70000] * 4, 2048))


# ----------------------------------------------------------------------------- sparse MLA
def oracle_idx(cpu, wl, share_first=False):
    Q = 1 if share_first else wl.Q
    pos = np.array(positions(wl))[:, :Q]
    s = oracle.index_scores_batch(np_(cpu.q_idx)[:, :Q], np_(cpu.w)[:, :Q], key_cache(cpu), wl.lens, wl.lmax, q_pos=pos)
    return oracle.topk_batch(s.astype(np.float32), wl.lens, wl.k, q_pos=pos), s


@pytest.mark.parametrize("name,kw", [
    ("decode_tiny_8k", dict(B=2, L=5000, seq_lens=(5000, 3333))),                                 # split path
    ("decode_b32_128k_paged", dict(B=2, L=2600, L_max=2624, planted=0, H=64, seq_lens=(2600, 1000))),  # p+1 < k rows
    ("verify_b64_q8_32k", dict(B=2, L=3000, L_max=3008, k=100)),                                  # k not a multiple of 32
    ("prefill_4096_at_128k", dict(Q=130, L=3000, k=256)),                                          # many rows, no split
])
def test_sparse_mla_on_oracle_indices(name, kw):
    wl = synth.small(name, **kw)
    cpu, g = gpu_batch(wl)
    idx, _ = oracle_idx(cpu, wl)
    idx_g = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[0]), latent_cache(cpu), idx, wl.scale)
    worst = (0.0, 0.0)
    for b in range(wl.B):
        for j in range(wl.Q):
            m = check_mla(out[b, j], lse[b, j], ref_o[b, j], ref_l[b, j])
            worst = (max(worst[0], m[0]), max(worst[1], m[1]))
    print(f"{name}: max abs {worst[0]:.3g} rel L2 {worst[1]:.3g}")


@pytest.mark.parametrize("H", [128, 64])
def test_sparse_mla_logit_jumps_after_the_first_step(H):
    """Each split keeps one softmax reference per head, taken in its first step with a visible
    token. Late tokens whose logits exceed it: by about 30 binades (weights above 1, no rerun),
    by about 130 binades (beyond the headroom: the split is computed again with its exact
    maximum), and a split whose first step is entirely masked."""
    gen = torch.Generator().manual_seed(5)
    B, L, k = 3, 4096, 2048
    scale = 1.0 / 576 ** 0.5
    q = torch.randn((B, 1, H, 576), generator=gen).to(torch.bfloat16)
    lat = torch.randn((B, L, 576), generator=gen).to(torch.bfloat16)
    idx = torch.arange(k, dtype=torch.int32).repeat(B, 1, 1)
    lat[0, 2040] = q[0, 0, 3]                                      # head 3: logit ~ 24
    lat[1, 2040] = (4 * q[1, 0, 5].float()).to(torch.bfloat16)    # head 5: logit ~ 96
    idx[2, 0, :40] = -1                                            # first step of split 0 masked
    lat[2, 1000] = (3 * q[2, 0, 1].float()).to(torch.bfloat16)    # head 1: logit ~ 72
    seq_lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    out, lse = dsa.sparse_mla_fwd(q.to(DEV), dsa.Cache(lat.to(DEV), None, 0), idx.to(DEV), k, scale, seq_lens, L)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(q), oracle.Cache(bits(lat)), idx.numpy(), scale)
    for b in range(B):
        check_mla(out[b, 0], lse[b, 0], ref_o[b, 0], ref_l[b, 0])


@pytest.mark.parametrize("H", [128, 64])
def test_sparse_mla_dominant_rows_with_large_values(H):
    """Rows that dominate a head's softmax and carry values up to about 17, through a launch of
    16 splits per query token: the output is then about that row. P is rounded to bf16 for PV;
    normalising by the sum of the rounded weights makes a dominant token's rounding cancel, and
    fp32 split partials keep the combine exact, so the fixed bars hold at this scale. One planted
    row opens its split (no second pass), two sit in later steps (second pass), and one split
    starts with a masked step."""
    gen = torch.Generator().manual_seed(15)
    B, L, k = 3, 4096, 2048
    scale = 1.0 / 576 ** 0.5
    q = torch.randn((B, 1, H, 576), generator=gen).to(torch.bfloat16)
    lat = torch.randn((B, L, 576), generator=gen).to(torch.bfloat16)
    idx = torch.arange(k, dtype=torch.int32).repeat(B, 1, 1)
    lat[0, 1920] = (5 * q[0, 0, 3].float()).to(torch.bfloat16)    # head 3: logit ~ 120, first token of a split
    lat[1, 2040] = (5 * q[1, 0, 5].float()).to(torch.bfloat16)    # head 5: logit ~ 120, last step of a split
    lat[2, 1000] = (4 * q[2, 0, 1].float()).to(torch.bfloat16)    # head 1: logit ~ 96, a middle split
    idx[2, 0, :40] = -1                                            # first step of split 0 masked
    seq_lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    # 16 splits per query token: the workspace holds 16 fp32 partials of every head of all 3 tokens
    assert dsa.workspace_size(dsa.OP_SPARSE_MLA, B, 1, L, H=H, k=k) >= B * 16 * H * 512 * 4
    out, lse = dsa.sparse_mla_fwd(q.to(DEV), dsa.Cache(lat.to(DEV), None, 0), idx.to(DEV), k, scale, seq_lens, L)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(q), oracle.Cache(bits(lat)), idx.numpy(), scale)
    for b, h in ((0, 3), (1, 5), (2, 1)):
        assert float(np.abs(ref_o[b, 0, h]).max()) >= 10.0, (b, h)
    for b in range(B):
        check_mla(out[b, 0], lse[b, 0], ref_o[b, 0], ref_l[b, 0])


def test_sparse_mla_shared_index_row_and_empty_sets():
    wl = synth.small("verify_b64_q8_32k", B=2, Q=4, L=2500, L_max=2560, k=512)
    cpu, g = gpu_batch(wl)
    idx, _ = oracle_idx(cpu, wl, share_first=True)       # [B, 1, k]
    idx[1, 0, :] = -1                                    # sequence 1: empty set -> out 0, lse -inf
    idx_g = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax, idx_q_stride=0)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[0]), latent_cache(cpu), idx, wl.scale, idx_q_stride_is_k=False)
    for j in range(wl.Q):
        check_mla(out[0, j], lse[0, j], ref_o[0, j], ref_l[0, j])
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_sparse_mla_deterministic_and_paged_equals_contiguous():
    wl = synth.small("decode_b32_128k_paged", B=3, L=4000, L_max=4032, planted=0, seq_lens=(4000, 3000, 2222))
    cpu, g = gpu_batch(wl)
    idx, _ = oracle_idx(cpu, wl)
    idx_g = torch.from_numpy(idx).to(DEV)
    o1, l1 = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax)
    o2, l2 = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    tab = g.latent_table[0].long()
    contig = g.latent[0][tab].reshape(wl.B, wl.lmax, 576).contiguous()
    o3, l3 = dsa.sparse_mla_fwd(g.q_mla[0], dsa_cache(contig, None, 0), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


# ----------------------------------------------------------------------------- whole path
def test_decode_tiny_end_to_end():
    """The 8K tiny decode workload exactly: B=1, Q=1, L=8192 contiguous, seed 0."""
    wl = synth.WORKLOADS["decode_tiny_8k"]
    cpu, g = gpu_batch(wl)
    scores = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax)
    idx = dsa.topk(scores, g.seq_lens, wl.k)
    out, lse = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx, wl.k, wl.scale, g.seq_lens, wl.lmax)
    o_idx, exact = oracle_idx(cpu, wl)
    p = wl.L - 1
    tol = score_tolerance(np_(cpu.q_idx[0, 0]), np_(cpu.w[0, 0]), np_(cpu.keys[0]))
    check_scores(np_(scores)[0, 0], exact[0, 0], tol, p)
    swaps = check_topk_sets(np_(idx)[0, 0], o_idx[0, 0], exact[0, 0], wl.k)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[0]), latent_cache(cpu), o_idx, wl.scale)
    check_mla(np_(out)[0, 0], np_(lse)[0, 0], ref_o[0, 0], ref_l[0, 0])
    print(f"decode_tiny_8k: {swaps} near-threshold swaps")


def random_shape(seed):
    """A seeded random small shape: cache layout, query count, head counts, k and ragged lengths."""
    r = np.random.default_rng(1000 + seed)
    ps = int(r.choice([0, 0, 16, 48, 64, 128]))
    Q = int(r.choice([1, 2, 5, 8]))
    B = int(r.integers(1, 5))
    L_max = int(r.integers(64, 16000))
    lens = tuple(int(x) for x in r.integers(Q, L_max + 1, B))
    return synth.small("verify_b64_q8_32k", B=B, Q=Q, L=max(lens), L_max=L_max, page_size=ps, seq_lens=lens,
                       Hi=int(r.choice([32, 64])), H=int(r.choice([64, 128])), k=int(r.choice([1, 777, 2048, 2048])))


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes_end_to_end(seed):
    """Scan, top-k and attention on a random small shape, each stage against the oracle: scores
    within the tolerance, sets up to near-threshold swaps, attention over the GPU's own set."""
    check_end_to_end(random_shape(seed), seed)


@pytest.mark.parametrize("name,kw", [
    ("one token each", dict(B=3, Q=1, L=1, L_max=1, page_size=0, seq_lens=(1, 1, 1))),
    ("one and seventeen tokens, pages of 16", dict(B=2, Q=1, L=17, L_max=17, page_size=16, seq_lens=(1, 17))),
    ("two queries at positions 0 and 1", dict(B=2, Q=2, L=2, L_max=2, page_size=0, seq_lens=(2, 2))),
    ("k = 1 over pages of 16", dict(B=2, Q=3, L=40, L_max=48, page_size=16, seq_lens=(40, 3), k=1)),
])
def test_degenerate_lengths_end_to_end(name, kw):
    """Sequences of one or a few tokens, rows shorter than every tile, k = 1: the path still
    matches the oracle (one visible token: its score, the set {0}, the output its value row)."""
    check_end_to_end(synth.small("verify_b64_q8_32k", **kw), 0)


def check_end_to_end(wl, seed):
    print(f"seed {seed}: B={wl.B} Q={wl.Q} L_max={wl.lmax} page={wl.page_size} Hi={wl.Hi} H={wl.H} k={wl.k} "
          f"lens={wl.lens}", flush=True)
    cpu, g = gpu_batch(wl, seed=seed)
    scores = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax)
    idx = dsa.topk(scores, g.seq_lens, wl.k)
    out, lse = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx, wl.k, wl.scale, g.seq_lens, wl.lmax)
    o_idx, exact = oracle_idx(cpu, wl)
    kc = key_cache(cpu)
    sc, gi = np_(scores), np_(idx)
    for b in range(wl.B):
        for j, p in enumerate(positions(wl)[b]):
            if j in (0, wl.Q - 1):                  # the tolerance costs host time per key: two queries
                tol = score_tolerance(np_(cpu.q_idx[b, j]), np_(cpu.w[b, j]), kc.rows(b, np.arange(wl.lmax)))
                check_scores(sc[b, j], exact[b, j], tol, p)
            check_topk_sets(gi[b, j], o_idx[b, j], exact[b, j], wl.k)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[0]), latent_cache(cpu), gi, wl.scale)
    out, lse = np_(out), np_(lse)
    for b in range(wl.B):
        for j in range(wl.Q):
            check_mla(out[b, j], lse[b, j], ref_o[b, j], ref_l[b, j])


@pytest.mark.parametrize("share_first", [False, True])
def test_forward_shared_small(share_first):
    if share_first:
        wl = synth.small("verify_b64_q8_32k_draftshare", B=3, L=3000, L_max=3008, seq_lens=(3000, 2900, 2100))
    else:
        wl = synth.small("indexshare_b8_1m_4layers", B=2, L=6000, L_max=6016, seq_lens=(6000, 4444))
    cpu, g = gpu_batch(wl)
    idx, res = dsa.forward_shared(g.q_idx, g.w, keys_arg(g), wl.k, g.q_mla, [lat_arg(g, l) for l in range(wl.n_layers)],
                                  wl.scale, g.seq_lens, wl.lmax, share_first_query=share_first)
    o_idx, exact = oracle_idx(cpu, wl, share_first=share_first)
    idx = np_(idx)
    for b in range(wl.B):
        for j in range(o_idx.shape[1]):
            check_topk_sets(idx[b, j], o_idx[b, j], exact[b, j], wl.k)
    for layer in range(wl.n_layers):
        ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[layer]), latent_cache(cpu, layer), o_idx, wl.scale,
                                               idx_q_stride_is_k=not share_first)
        out, lse = np_(res[layer][0]), np_(res[layer][1])
        for b in range(wl.B):
            for j in range(wl.Q):
                check_mla(out[b, j], lse[b, j], ref_o[b, j], ref_l[b, j])


@pytest.mark.parametrize("H", [128, 64])
@pytest.mark.parametrize("B,n_layers", [(2, 10), (8, 4)])
def test_forward_shared_many_layers(H, B, n_layers):
    """Layers that share one index set: the library launches their MLA eight layers at a time
    (ten layers: two launches) and splits each launch's tokens over all its layers. Every layer
    matches the oracle on the GPU's set, and the group is deterministic."""
    lens = tuple(3000 - 97 * b for b in range(B))
    wl = synth.small("indexshare_b8_1m_4layers", B=B, L=3000, L_max=3008, seq_lens=lens, n_layers=n_layers, H=H)
    cpu, g = gpu_batch(wl)
    lats = [lat_arg(g, l) for l in range(wl.n_layers)]
    idx, res = dsa.forward_shared(g.q_idx, g.w, keys_arg(g), wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax)
    idx2, res2 = dsa.forward_shared(g.q_idx, g.w, keys_arg(g), wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    o_idx, exact = oracle_idx(cpu, wl)
    idx_np = np_(idx)
    for b in range(wl.B):
        check_topk_sets(idx_np[b, 0], o_idx[b, 0], exact[b, 0], wl.k)
    for layer in range(wl.n_layers):
        assert torch.equal(res[layer][0], res2[layer][0]) and torch.equal(res[layer][1], res2[layer][1]), layer
        ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[layer]), latent_cache(cpu, layer), idx_np, wl.scale)
        out_l, lse_l = np_(res[layer][0]), np_(res[layer][1])
        for b in range(wl.B):
            check_mla(out_l[b, 0], lse_l[b, 0], ref_o[b, 0], ref_l[b, 0])


@pytest.mark.parametrize("form", ["sampled", "row"])
@pytest.mark.parametrize("L", [131072, 200000])
def test_topk_when_the_sample_misses(form, L):
    """Both sampled forms read a block-strided sample of each row: up to 512 blocks of 16
    scores (1024 on rows above 128K scores), so one block in `stride`. When
    exactly those blocks, or exactly the blocks between them, carry the high scores, or every
    score is equal, the candidate list misses or overflows and the exact full-row scan must
    produce the set."""
    rng = np.random.default_rng(21)
    n_sample = 1024 if L > 131072 else 512
    stride = -(-(-(-L // 16)) // n_sample)
    s = (1.0 + rng.random((6, 1, L))).astype(np.float32)
    blk = np.arange(L) // 16
    s[0, 0, blk % (2 * stride) == 0] += 100.0      # half of the sampled blocks
    s[1, 0, blk % (2 * stride) != 0] += 100.0      # everything but them
    s[2, 0, :] = np.float32(7.0)                   # every score equal: a flood of candidates
    s[3, 0, blk % 4 == 0] += 100.0                 # every fourth block
    s[4, 0, blk % stride == 0] += 100.0            # exactly the sampled blocks
    s[5, 0, blk % stride != 0] += 100.0            # everything but them
    for k in (2048, 300):
        got = run_topk(s, [L] * 6, k, form=form)
        assert np.array_equal(got, oracle_topk(s, [L] * 6, k)), k


def test_mtp_draft_loop_reuses_the_step1_set():
    """The MTP draft loop (one shared MTP layer unrolled over 7 steps; IndexShare on MTP: only
    step 1 scores and selects): one index scan + top-k, then 7 sequential sparse-MLA calls over
    that set, each with its own query. Every draft step matches the oracle on the step-1 set."""
    wl = synth.small("mtp_draft_b32_128k_paged", B=2, L=4000, L_max=4032, planted=4, seq_lens=(4000, 2900))
    cpu, g = gpu_batch(wl)
    scores = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax)
    idx = dsa.topk(scores, g.seq_lens, wl.k)
    o_idx, exact = oracle_idx(cpu, wl)
    for b in range(wl.B):
        check_topk_sets(np_(idx)[b, 0], o_idx[b, 0], exact[b, 0], wl.k)
    qs_cpu = synth.draft_queries(cpu, wl.draft_steps)
    for s, q in enumerate(qs_cpu):
        out, lse = dsa.sparse_mla_fwd(q.to(DEV), lat_arg(g), idx, wl.k, wl.scale, g.seq_lens, wl.lmax)
        ref_o, ref_l = oracle.sparse_mla_batch(bits(q), latent_cache(cpu), np_(idx), wl.scale)
        for b in range(wl.B):
            check_mla(np_(out)[b, 0], np_(lse)[b, 0], ref_o[b, 0], ref_l[b, 0])


# ----------------------------------------------------------------------------- FP8 latent cache
@pytest.mark.parametrize("name,kw,scale", [
    ("decode_b32_128k_paged", dict(B=2, L=5000, L_max=5056, planted=4, seq_lens=(5000, 3001)), 1.0),       # split, paged
    ("decode_tiny_8k", dict(B=2, L=3000, seq_lens=(3000, 1500), H=64), 0.37),                              # contiguous, H=64
    ("verify_b64_q8_32k", dict(B=2, L=3000, L_max=3008, k=300), 0.5),                                      # many rows, no split
])
def test_sparse_mla_fp8_latent_on_oracle_indices(name, kw, scale):
    """The absolute bar (2e-2) is for values of the workloads' size: scales stay at or below 1."""
    wl = synth.small(name, latent_fp8=1, **kw)
    cpu, g = gpu_batch(wl)
    idx, _ = oracle_idx(cpu, wl)
    idx_g = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax,
                                  latent_scale=scale)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[0]), latent_cache(cpu), idx, wl.scale, latent_scale=scale)
    for b in range(wl.B):
        for j in range(wl.Q):
            check_mla(out[b, j], lse[b, j], ref_o[b, j], ref_l[b, j])


@pytest.mark.parametrize("H", [128, 64])
def test_sparse_mla_fp8_latent_equals_bf16_cache_of_its_values(H):
    """With a power-of-two scale the FP8 path gives the bits of the bf16 path over a bf16 cache
    holding the decoded values (same products, same order)."""
    wl = synth.small("decode_b32_128k_paged", B=2, L=4000, L_max=4032, planted=4, seq_lens=(4000, 2222), H=H,
                     latent_fp8=1)
    cpu, g = gpu_batch(wl)
    scores = dsa.index_score(g.q_idx, g.w, keys_arg(g), g.seq_lens, wl.lmax)
    idx = dsa.topk(scores, g.seq_lens, wl.k)
    as_bf16 = (g.latent[0].view(torch.float8_e4m3fn).to(torch.float32) * 4.0).to(torch.bfloat16)
    o8, l8 = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx, wl.k, wl.scale, g.seq_lens, wl.lmax, latent_scale=4.0)
    ob, lb = dsa.sparse_mla_fwd(g.q_mla[0], dsa_cache(as_bf16, g.latent_table[0], wl.page_size), idx, wl.k, wl.scale,
                                g.seq_lens, wl.lmax)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob) and torch.equal(l8, lb)


def test_sparse_mla_fp8_every_code():
    """Latent rows that hold every E4M3FN code but the two NaNs: the FP8 path converts each
    code on the device and gives the bits of the bf16 path over the decoded values."""
    gen = torch.Generator().manual_seed(13)
    B, L, k, H = 2, 2048, 2048, 128
    codes = (torch.arange(B * L * 576, dtype=torch.int64) * 37 % 256).to(torch.uint8).view(B, L, 576)
    codes[(codes & 0x7F) == 0x7F] = 0
    assert torch.unique(codes).numel() == 254
    q = (torch.randn((B, 1, H, 576), generator=gen) * 0.05).to(torch.bfloat16)
    idx = torch.arange(k, dtype=torch.int32).repeat(B, 1, 1)
    seq_lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    scale, ls = 1.0 / 576 ** 0.5, 2.0 ** -6
    o8, l8 = dsa.sparse_mla_fwd(q.to(DEV), dsa.Cache(codes.to(DEV), None, 0), idx.to(DEV), k, scale, seq_lens, L,
                                latent_scale=ls)
    vals = (codes.view(torch.float8_e4m3fn).to(torch.float32) * ls).to(torch.bfloat16)
    ob, lb = dsa.sparse_mla_fwd(q.to(DEV), dsa.Cache(vals.to(DEV), None, 0), idx.to(DEV), k, scale, seq_lens, L)
    torch.cuda.synchronize()
    assert torch.isfinite(o8).all()
    assert torch.equal(o8, ob) and torch.equal(l8, lb)


def e4m3_codes(x):
    """E4M3FN codes (uint8) of float values (torch's round-to-nearest-even cast)."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


@pytest.mark.parametrize("H", [128, 64])
def test_sparse_mla_fp8_logit_jumps_after_the_first_step(H):
    """The softmax-reference cases of the bf16 test on an E4M3 cache: a late logit about 30
    binades above the reference, one beyond the headroom (the split is computed a second time
    through the FP8 staging and conversion path), and a split whose first step is masked."""
    gen = torch.Generator().manual_seed(6)
    B, L, k = 3, 4096, 2048
    scale = 1.0 / 576 ** 0.5
    q = torch.randn((B, 1, H, 576), generator=gen).to(torch.bfloat16)
    codes = e4m3_codes(torch.randn((B, L, 576), generator=gen))
    idx = torch.arange(k, dtype=torch.int32).repeat(B, 1, 1)
    codes[0, 2040] = e4m3_codes(q[0, 0, 3].float())                # head 3: logit ~ 24
    codes[1, 2040] = e4m3_codes(4 * q[1, 0, 5].float())            # head 5: logit ~ 96
    idx[2, 0, :40] = -1                                            # first step of split 0 masked
    codes[2, 1000] = e4m3_codes(3 * q[2, 0, 1].float())            # head 1: logit ~ 72
    seq_lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    out, lse = dsa.sparse_mla_fwd(q.to(DEV), dsa.Cache(codes.to(DEV), None, 0), idx.to(DEV), k, scale, seq_lens, L,
                                  latent_scale=1.0)
    # every E4M3 value is a bf16 value: the bits of the bf16 path over the decoded rows, second
    # pass included
    vals = codes.view(torch.float8_e4m3fn).to(torch.float32).to(torch.bfloat16)
    ob, lb = dsa.sparse_mla_fwd(q.to(DEV), dsa.Cache(vals.to(DEV), None, 0), idx.to(DEV), k, scale, seq_lens, L)
    torch.cuda.synchronize()
    assert torch.equal(out, ob) and torch.equal(lse, lb)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(q), oracle.Cache(codes.numpy()), idx.numpy(), scale, latent_scale=1.0)
    # the planted rows dominate their heads, whose outputs reach about 10-16, far beyond the
    # workloads' scale (about 0.04 RMS); the bars stay the fixed ones
    assert float(np.abs(ref_o[1, 0, 5]).max()) >= 8.0
    for b in range(B):
        check_mla(out[b, 0], lse[b, 0], ref_o[b, 0], ref_l[b, 0])


@pytest.mark.parametrize("share_first", [False, True])
def test_forward_shared_fp8_layers(share_first):
    """The IndexShare group over E4M3 latent caches, one scale per layer: layers sharing a scale go
    in one launch (here two launches: scales 0.5, 0.5, 2.0). Every layer matches the oracle on
    the GPU's set; with a power-of-two scale the group equals its bf16 form over the decoded values
    bit for bit (same launches, same products)."""
    base = "verify_b64_q8_32k_draftshare" if share_first else "indexshare_b8_1m_4layers"
    wl = synth.small(base, B=2, Q=3 if share_first else 1, L=4000, L_max=4032, seq_lens=(4000, 2900), n_layers=3,
                     latent_fp8=1, page_size=64)
    cpu, g = gpu_batch(wl)
    scales = [0.5, 0.5, 2.0]
    lats = [lat_arg(g, l) for l in range(wl.n_layers)]
    idx, res = dsa.forward_shared(g.q_idx, g.w, keys_arg(g), wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax,
                                  share_first_query=share_first, latent_scales=scales)
    o_idx, exact = oracle_idx(cpu, wl, share_first=share_first)
    idx_np = np_(idx)
    for b in range(wl.B):
        for j in range(idx_np.shape[1]):
            check_topk_sets(idx_np[b, j], o_idx[b, j], exact[b, j], wl.k)
    for layer in range(wl.n_layers):
        out, lse = np_(res[layer][0]), np_(res[layer][1])
        ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[layer]), latent_cache(cpu, layer), idx_np, wl.scale,
                                               idx_q_stride_is_k=not share_first, latent_scale=scales[layer])
        for b in range(wl.B):
            for j in range(wl.Q):
                check_mla(out[b, j], lse[b, j], ref_o[b, j], ref_l[b, j])
    # the bf16 group over the decoded values (same scales grouping: layers 0-1, then layer 2)
    dec = [dsa_cache((g.latent[l].view(torch.float8_e4m3fn).to(torch.float32) * scales[l]).to(torch.bfloat16),
                     g.latent_table[l], wl.page_size) for l in range(wl.n_layers)]
    _, res_a = dsa.forward_shared(g.q_idx, g.w, keys_arg(g), wl.k, g.q_mla[:2], dec[:2], wl.scale, g.seq_lens,
                                  wl.lmax, share_first_query=share_first)
    _, res_b = dsa.forward_shared(g.q_idx, g.w, keys_arg(g), wl.k, g.q_mla[2:], dec[2:], wl.scale, g.seq_lens,
                                  wl.lmax, share_first_query=share_first)
    torch.cuda.synchronize()
    for layer, (o, l) in enumerate(res_a + res_b):
        assert torch.equal(res[layer][0], o) and torch.equal(res[layer][1], l), layer


def test_sparse_mla_fp8_shared_index_row_and_empty_sets():
    wl = synth.small("verify_b64_q8_32k", B=2, Q=4, L=2500, L_max=2560, k=512, latent_fp8=1)
    cpu, g = gpu_batch(wl)
    idx, _ = oracle_idx(cpu, wl, share_first=True)       # [B, 1, k]
    idx[1, 0, :] = -1                                    # sequence 1: empty set -> out 0, lse -inf
    idx_g = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_mla_fwd(g.q_mla[0], lat_arg(g), idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax, idx_q_stride=0,
                                  latent_scale=0.5)
    out, lse = np_(out), np_(lse)
    ref_o, ref_l = oracle.sparse_mla_batch(bits(cpu.q_mla[0]), latent_cache(cpu), idx, wl.scale, idx_q_stride_is_k=False,
                                           latent_scale=0.5)
    for j in range(wl.Q):
        check_mla(out[0, j], lse[0, j], ref_o[0, j], ref_l[0, j])
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_sparse_mla_fp8_deterministic_and_paged_equals_contiguous():
    wl = synth.small("decode_b32_128k_paged", B=3, L=4000, L_max=4032, planted=0, seq_lens=(4000, 3000, 2222),
                     latent_fp8=1)
    cpu, g = gpu_batch(wl)
    idx, _ = oracle_idx(cpu, wl)
    idx_g = torch.from_numpy(idx).to(DEV)
    run = lambda cache: dsa.sparse_mla_fwd(g.q_mla[0], cache, idx_g, wl.k, wl.scale, g.seq_lens, wl.lmax,
                                           latent_scale=1.0)
    o1, l1 = run(lat_arg(g))
    o2, l2 = run(lat_arg(g))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    tab = g.latent_table[0].long()
    contig = g.latent[0][tab].reshape(wl.B, wl.lmax, 576).contiguous()
    o3, l3 = run(dsa_cache(contig, None, 0))
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
