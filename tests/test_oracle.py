"""Pins of the CPU oracle against things other than itself.

What pins each oracle function:
  e4m3_to_f64       every code vs torch's float8_e4m3fn cast; the OCP spec's named values.
  bf16_to_f64       every bit pattern vs torch's bfloat16 cast.
  index_scores      exact rational arithmetic (fractions) on torch-decoded inputs;
                    one-hot head weights reduce it to ReLU of a torch float64 matmul;
                    relu(x) + relu(-x) = |x| under a sign flip of the query codes;
                    linearity in w; causality (keys after p change nothing, score -inf).
  select_topk       Python's sorted() over (-score, position) on tie-heavy inputs;
                    the defining order property; k >= n keeps all; equal scores keep the
                    lowest positions; -0 ties +0; planted high-similarity tokens are kept.
  sparse_mla        torch scaled_dot_product_attention in float64; dense causal attention
                    when k >= L; masked dense attention over the selected set; convex hull;
                    logsumexp (scipy); one row, zero query and empty-set closed forms.
  Cache (paging)    a shuffled block table gives bit-identical results to contiguous.
  forward_shared    equals one score+select followed by per-layer attention; draft reuse.
  cost model        the pages' printed 1.6%, about 1/62 and 0.2% figures.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.dsa import Cache
import synth


def np_(t):
    return t.cpu().numpy()


def bits(t_bf16):
    return t_bf16.cpu().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- formats
def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_f64(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2            # S.1111.111 only: E4M3FN has no infinities


def test_e4m3_spec_values():
    v = oracle.e4m3_to_f64(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x40, 0xB8, 0x80], dtype=np.uint8))
    assert list(v) == [448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 2.0, -1.0, 0.0]
    assert math.copysign(1.0, v[-1]) == -1.0


def test_bf16_all_patterns_match_torch():
    b = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = b.view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_f64(b.numpy().view(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ----------------------------------------------------------------------------- helpers
def tiny_index_inputs(Hi=5, L=37, seed=3):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(Hi, 128, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    keys = torch.randn(1, L, 128, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    w = torch.rand(Hi, generator=g)
    return np_(q), np_(w), Cache(np_(keys))


# ----------------------------------------------------------------------------- step 1 pins
def test_index_scores_exact_rational():
    """Brute force in exact rational arithmetic on torch-decoded values."""
    q, w, keys = tiny_index_inputs(Hi=3, L=9)
    p = 6
    s = oracle.index_scores(q, w, keys, 0, p, 9)
    qv = torch.from_numpy(q).view(torch.float8_e4m3fn).float().tolist()
    kv = torch.from_numpy(keys.data[0]).view(torch.float8_e4m3fn).float().tolist()
    for t in range(9):
        if t > p:
            assert s[t] == -np.inf
            continue
        exact = Fraction(0)
        for h in range(3):
            d = sum(Fraction(qv[h][i]) * Fraction(kv[t][i]) for i in range(128))
            exact += Fraction(float(w[h])) * max(d, Fraction(0))
        assert abs(Fraction(s[t]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_index_scores_one_hot_weight_is_relu_of_torch_matmul():
    q, w, keys = tiny_index_inputs(Hi=6, L=40)
    kd = torch.from_numpy(keys.data[0]).view(torch.float8_e4m3fn).double()
    qd = torch.from_numpy(q).view(torch.float8_e4m3fn).double()
    for h in range(6):
        onehot = np.zeros(6, np.float32)
        onehot[h] = 1.0
        s = oracle.index_scores(q, onehot, keys, 0, 39, 40)
        ref = torch.clamp(kd @ qd[h], min=0).numpy()
        assert np.array_equal(s, ref)


def test_index_scores_relu_sign_identity():
    """s(q) + s(-q) = sum_h w_h |q_h . k_t|: fails if the ReLU is dropped, doubled or mis-signed."""
    q, w, keys = tiny_index_inputs(Hi=7, L=50)
    s_pos = oracle.index_scores(q, w, keys, 0, 49, 50)
    s_neg = oracle.index_scores(q ^ np.uint8(0x80), w, keys, 0, 49, 50)
    kd = torch.from_numpy(keys.data[0]).view(torch.float8_e4m3fn).double()
    qd = torch.from_numpy(q).view(torch.float8_e4m3fn).double()
    ref = ((kd @ qd.T).abs() @ torch.from_numpy(w).double()).numpy()
    np.testing.assert_allclose(s_pos + s_neg, ref, rtol=1e-13, atol=0)
    assert np.all(s_pos >= 0) and np.any(s_pos != s_neg)


def test_index_scores_linear_in_weights():
    q, w, keys = tiny_index_inputs(Hi=4, L=30)
    w2 = np.roll(w, 1) * np.float32(0.5)
    s1 = oracle.index_scores(q, w, keys, 0, 29, 30)
    s2 = oracle.index_scores(q, w2, keys, 0, 29, 30)
    s12 = oracle.index_scores(q, w.astype(np.float64) + w2, keys, 0, 29, 30)
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-14)


def test_index_scores_causal():
    q, w, keys = tiny_index_inputs(Hi=4, L=30)
    p = 11
    s = oracle.index_scores(q, w, keys, 0, p, 30)
    assert np.all(np.isneginf(s[p + 1:])) and np.all(np.isfinite(s[: p + 1]))
    keys.data[0, p + 1:] = np.uint8(0x7E)   # change only tokens after p
    assert np.array_equal(oracle.index_scores(q, w, keys, 0, p, 30), s)


def test_index_scores_heads_and_dims_not_transposed():
    """Asymmetric one-hot construction: head h only sees dim (3h+1); closed form by hand."""
    Hi, L = 5, 8
    q = np.zeros((Hi, 128), np.uint8)
    keys = np.zeros((1, L, 128), np.uint8)
    for h in range(Hi):
        q[h, 3 * h + 1] = 0x40                      # 2.0
    rng = np.random.default_rng(0)
    vals = rng.integers(-6, 7, size=(L, Hi))        # small integers, exact in E4M3
    enc = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for h in range(Hi):
        keys[0, :, 3 * h + 1] = enc[:, h]
    w = np.array([1.0, 0.5, 0.25, 0.125, 0.0625], np.float32)
    s = oracle.index_scores(q, w, Cache(keys), 0, L - 1, L)
    by_hand = [sum(w[h] * max(2.0 * vals[t, h], 0.0) for h in range(Hi)) for t in range(L)]
    assert np.array_equal(s, np.array(by_hand))


# ----------------------------------------------------------------------------- step 2 pins
@pytest.mark.parametrize("seed", range(6))
def test_select_matches_python_sorted(seed):
    rng = np.random.default_rng(seed)
    n_total = int(rng.integers(1, 60))
    p = int(rng.integers(0, n_total))
    k = int(rng.integers(1, 20))
    scores = rng.integers(-3, 4, size=n_total).astype(np.float32)   # many ties
    got = oracle.select_topk(scores, p, k)
    ranked = sorted(range(p + 1), key=lambda t: (-float(scores[t]), t))
    want = sorted(ranked[:k]) + [-1] * max(0, k - (p + 1))
    assert got.tolist() == want


@pytest.mark.parametrize("seed", range(4))
def test_select_defining_property(seed):
    rng = np.random.default_rng(100 + seed)
    n = 300
    scores = rng.normal(size=n).astype(np.float32)
    scores[rng.integers(0, n, 40)] = scores[5]      # plant ties around one value
    k, p = 64, 250
    got = oracle.select_topk(scores, p, k)
    kept = set(got.tolist())
    assert len(kept) == k and min(kept) >= 0 and max(kept) <= p
    assert got.tolist() == sorted(got.tolist())
    for a in kept:
        for b in set(range(p + 1)) - kept:
            assert (scores[a] > scores[b]) or (scores[a] == scores[b] and a < b)


def test_select_small_and_degenerate():
    s = np.array([3, 1, 2], np.float32)
    assert oracle.select_topk(s, 2, 5).tolist() == [0, 1, 2, -1, -1]        # p + 1 <= k keeps all
    assert oracle.select_topk(np.zeros(10, np.float32), 9, 4).tolist() == [0, 1, 2, 3]
    z = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)
    assert oracle.select_topk(z, 3, 2).tolist() == [0, 1]                     # -0 ties +0
    assert oracle.select_topk(np.array([1.0, np.inf, 2.0], np.float32), 2, 1).tolist() == [1]


def test_planted_tokens_selected():
    wl = synth.small("decode_b32_128k_paged", B=2, L=4096, planted=8, k=256)
    batch = synth.generate(wl, seed=0, with_mla=False)
    keys = Cache(np_(batch.keys), np_(batch.key_table), wl.page_size)
    s = oracle.index_scores_batch(np_(batch.q_idx), np_(batch.w), keys, wl.lens, wl.lmax)
    idx = oracle.topk_batch(s.astype(np.float32), wl.lens, wl.k)
    for b in range(wl.B):
        assert set(np_(batch.planted_pos[b]).tolist()) <= set(idx[b, 0].tolist())


# ----------------------------------------------------------------------------- step 3 pins
def mla_inputs(H=4, m=20, seed=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, 576, generator=g).to(torch.bfloat16)
    rows = torch.randn(m, 576, generator=g).to(torch.bfloat16)
    return q, rows


def test_sparse_mla_matches_torch_sdpa():
    q, rows = mla_inputs(H=6, m=33)
    scale = 1 / math.sqrt(576)
    o, lse = oracle.sparse_mla(bits(q), bits(rows), scale)
    qd, kd = q.double()[None, :, None, :], rows.double()[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd.expand(1, 6, 33, 576),
                                                           kd[..., :512].expand(1, 6, 33, 512), scale=scale)
    np.testing.assert_allclose(o, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-14)
    from scipy.special import logsumexp
    z = scale * (q.double() @ rows.double().T).numpy()
    np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-13)


def test_sparse_equals_dense_when_k_covers_context():
    """k >= L: the selector keeps every visible token and DSA is dense causal MLA."""
    L, p = 48, 40
    g = torch.Generator().manual_seed(5)
    q_idx = torch.randn(1, 1, 4, 128, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    w = torch.rand(1, 1, 4, generator=g)
    keys = torch.randn(1, L, 128, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    q_mla, lat = mla_inputs(H=4, m=L, seed=6)
    s = oracle.index_scores_batch(np_(q_idx), np_(w), Cache(np_(keys)), [p + 1], L)
    idx = oracle.topk_batch(s.astype(np.float32), [p + 1], k=64)
    assert idx[0, 0, : p + 1].tolist() == list(range(p + 1))
    o, lse = oracle.sparse_mla_one(bits(q_mla), Cache(bits(lat)[None]), 0, idx[0, 0], 1 / 24)
    od, lsed = oracle.dense_mla_causal(bits(q_mla), bits(lat), p, 1 / 24)
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lsed, rtol=1e-13)


def test_sparse_equals_masked_dense_over_selected():
    L = 64
    q, lat = mla_inputs(H=3, m=L, seed=9)
    sel = np.array(sorted(np.random.default_rng(1).choice(50, 12, replace=False)) + [-1] * 4, np.int32)
    o, lse = oracle.sparse_mla_one(bits(q), Cache(bits(lat)[None]), 0, sel, 0.05)
    od, lsed = oracle.dense_mla_causal(bits(q), bits(lat), 55, 0.05, keep=sel)
    np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lsed, rtol=1e-13)


def test_sparse_mla_invariants_and_closed_forms():
    q, rows = mla_inputs(H=5, m=17, seed=2)
    o, lse = oracle.sparse_mla(bits(q), bits(rows), 0.1)
    c = rows.double().numpy()[:, :512]
    assert np.all(o <= c.max(0) + 1e-12) and np.all(o >= c.min(0) - 1e-12)           # convex hull
    z = 0.1 * (q.double() @ rows.double().T).numpy()
    np.testing.assert_allclose(np.exp(z - lse[:, None]).sum(1), 1.0, rtol=1e-13)   # LSE identity
    o1, l1 = oracle.sparse_mla(bits(q), bits(rows[3:4]), 0.1)                       # one row
    assert np.array_equal(o1, np.broadcast_to(c[3], o1.shape)) and np.allclose(l1, z[:, 3], rtol=1e-14)
    oz, lz = oracle.sparse_mla(np.zeros((2, 576), np.uint16), bits(rows), 0.1)        # zero query
    np.testing.assert_allclose(oz, np.broadcast_to(c.mean(0), oz.shape), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lz, math.log(17), rtol=1e-14)
    oe, le = oracle.sparse_mla(bits(q), np.zeros((0, 576), np.uint16), 0.1)         # empty set
    assert np.all(oe == 0) and np.all(np.isneginf(le))
    perm = np.random.default_rng(0).permutation(17)                                  # order-free
    op, lp = oracle.sparse_mla(bits(q), bits(rows)[perm], 0.1)
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- paging, IndexShare
def test_paged_equals_contiguous():
    wl = synth.small("decode_b32_128k_paged", B=3, L=700, L_max=768, planted=0, k=64, H=4, page_size=64)
    batch = synth.generate(wl, seed=1)
    keys_p = Cache(np_(batch.keys), np_(batch.key_table), 64)
    lat_p = Cache(bits(batch.latent[0]), np_(batch.latent_table[0]), 64)
    # the same logical content, laid out contiguously
    tab = np_(batch.key_table).astype(np.int64)
    keys_c = Cache(np_(batch.keys)[tab].reshape(3, 768, 128))
    lat_c = Cache(bits(batch.latent[0])[tab].reshape(3, 768, 576))
    s_p = oracle.index_scores_batch(np_(batch.q_idx), np_(batch.w), keys_p, wl.lens, wl.lmax)
    s_c = oracle.index_scores_batch(np_(batch.q_idx), np_(batch.w), keys_c, wl.lens, wl.lmax)
    assert np.array_equal(s_p, s_c)
    idx = oracle.topk_batch(s_p.astype(np.float32), wl.lens, wl.k)
    o_p, l_p = oracle.sparse_mla_batch(bits(batch.q_mla[0]), lat_p, idx, wl.scale)
    o_c, l_c = oracle.sparse_mla_batch(bits(batch.q_mla[0]), lat_c, idx, wl.scale)
    assert np.array_equal(o_p, o_c) and np.array_equal(l_p, l_c)


def test_forward_shared_is_one_selection_reused():
    wl = synth.small("indexshare_b8_1m_4layers", B=2, L=300, k=32, H=4)
    batch = synth.generate(wl, seed=0)
    keys = Cache(np_(batch.keys), np_(batch.key_table), 64)
    lats = [Cache(bits(batch.latent[i]), np_(batch.latent_table[i]), 64) for i in range(4)]
    qms = [bits(t) for t in batch.q_mla]
    idx, res = oracle.forward_shared(np_(batch.q_idx), np_(batch.w), keys, wl.lens, wl.lmax, wl.k, qms, lats, wl.scale)
    s = oracle.index_scores_batch(np_(batch.q_idx), np_(batch.w), keys, wl.lens, wl.lmax)
    idx2 = oracle.topk_batch(s.astype(np.float32), wl.lens, wl.k)
    assert np.array_equal(idx, idx2)
    for i in range(4):
        o, l = oracle.sparse_mla_batch(qms[i], lats[i], idx2, wl.scale)
        assert np.array_equal(res[i][0], o) and np.array_equal(res[i][1], l)
    assert not np.array_equal(res[0][0], res[1][0])      # layers really differ


def test_forward_shared_draft_reuses_first_position():
    wl = synth.small("verify_b64_q8_32k_draftshare", B=2, Q=4, L=200, k=16, H=2)
    batch = synth.generate(wl, seed=0)
    keys = Cache(np_(batch.keys), np_(batch.key_table), 64)
    lat = Cache(bits(batch.latent[0]), np_(batch.latent_table[0]), 64)
    idx, res = oracle.forward_shared(np_(batch.q_idx), np_(batch.w), keys, wl.lens, wl.lmax, wl.k,
                                     [bits(batch.q_mla[0])], [lat], wl.scale, share_first_query=True)
    assert idx.shape == (2, 1, 16)
    s0 = oracle.index_scores_batch(np_(batch.q_idx)[:, :1], np_(batch.w)[:, :1], keys, wl.lens, wl.lmax,
                                   q_pos=np.array([[196], [196]]))
    assert np.array_equal(idx[:, 0], oracle.topk_batch(s0.astype(np.float32), wl.lens, 16, q_pos=np.array([[196], [196]]))[:, 0])
    assert np.all(idx[idx >= 0] <= 196)                   # causally valid for every later position
    q = bits(batch.q_mla[0])
    for j in range(4):
        o, _ = oracle.sparse_mla_one(q[1, j], lat, 1, idx[1, 0], wl.scale)
        assert np.array_equal(res[0][0][1, j], o)


# ----------------------------------------------------------------------------- cost-model pins (page figures)
def test_page_complexity_figures(golden):
    k = golden["top_k"]["value"]
    # "128K" read as 128,000 tokens: 2048 / 128000 = 1.6 %, dense / sparse = 62.5 ("about 1/62")
    r = oracle.sparse_to_dense_ratio(128_000, k)
    assert round(100 * r, 1) == 1.6 == 100 * golden["keys_seen_fraction_128k"]["value"]
    assert int(1 / r) == golden["dense_cost_ratio_128k"]["value"]
    assert oracle.sparse_to_dense_ratio(131072, k) == 1 / 64
    # shared-layer attention at 1M context: 2048 / 1,048,576 = 0.195 %, printed as 0.2 %
    r1m = oracle.sparse_to_dense_ratio(1 << 20, k)
    assert round(100 * r1m, 1) == 100 * golden["shared_layer_attention_fraction_1m"]["value"]
    # O(L*k): attention cost is linear in the number of attended tokens, independent of L
    assert oracle.attention_flops(128, 2 * k) == 2 * oracle.attention_flops(128, k)
    assert oracle.attention_flops(128, k) == 2 * 128 * 2048 * 1088
    assert oracle.indexer_flops(64, 1) == 16384


# ----------------------------------------------------------------------------- FP8 latent rows
def test_fp8_latent_rows_equal_bf16_rows_of_their_values():
    """A latent cache of E4M3 codes with a power-of-two scale is a bf16 cache of the decoded
    values: every E4M3 value times a power of two is a bf16 value (torch's casts decide), so
    attention over the codes equals attention over those bf16 rows."""
    g = torch.Generator().manual_seed(5)
    codes = (torch.randn((40, 576), generator=g) * 3).to(torch.float8_e4m3fn)
    q = torch.randn((8, 576), generator=g).to(torch.bfloat16)
    for s in (1.0, 0.25, 8.0):
        vals = codes.to(torch.float32) * s
        as_bf16 = vals.to(torch.bfloat16)
        assert torch.equal(as_bf16.to(torch.float32), vals)
        o1, l1 = oracle.sparse_mla(bits(q), codes.view(torch.uint8).numpy(), 0.05, latent_scale=s)
        o2, l2 = oracle.sparse_mla(bits(q), bits(as_bf16), 0.05)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), s


def test_fp8_latent_values_follow_the_code_table():
    codes = np.arange(256, dtype=np.uint8)
    ok = ~np.isnan(oracle.e4m3_to_f64(codes))
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.latent_values(codes, 0.5)[ok], 0.5 * ref[ok])
