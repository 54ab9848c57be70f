"""Pins of the compressed sparse attention oracle (oracle/csa.py).

What fixes each part, independently of the oracle's own code:
  * ratio 1 without a window: the compressed cache is the raw cache and CSA is DSA itself
    (the DSA oracle, pinned in test_oracle.py, bit for bit);
  * a selection that covers every visible entry: dense attention over the whole compressed
    cache and the whole raw cache, with the visibility and window masks written out here
    from their definitions (a block is visible once its last raw token is; the window is the
    last `window` raw tokens up to p) - this is HCA when the ratio is 128 and there is no window;
  * no selection: sliding-window attention, through the dense masked path of the DSA oracle;
  * one softmax over the union equals the log-sum-exp merge of the two partial attentions;
  * the selected entries are the k best by (score, then lower entry), by Python's sort.
Positions cover every residue modulo the ratio and the first tokens (no complete block yet).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import csa
from oracle.dsa import Cache

SCALE = 1.0 / math.sqrt(576)


def draw(B, L, ratio, H=8, Hi=4, Q=1, seed=0, window=0):
    """Small inputs: E4M3(N(0,1)) indexer query and keys, U(0,1) weights, bf16(N(0,1)) latents."""
    g = torch.Generator().manual_seed(seed)
    Lc = -(-L // ratio)
    e4 = lambda *s: torch.randn(s, generator=g).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bf = lambda *s: torch.randn(s, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return dict(q_idx=e4(B, Q, Hi, 128), w=torch.rand((B, Q, Hi), generator=g).numpy(),
                keys_c=Cache(e4(B, Lc, 128)), latent_c=Cache(bf(B, Lc, 576)), latent=Cache(bf(B, L, 576)),
                q_mla=bf(B, Q, H, 576), Lc=Lc)


def dense_union(q_bits, lat_c_rows, lat_rows, p, ratio, window, scale):
    """Dense attention of one query over every compressed row and every raw row of a sequence,
    masked from the definitions: compressed entry c is kept when all of its raw tokens
    ratio*c .. ratio*c + ratio - 1 are at or before p; raw token t when p - window < t <= p."""
    q = oracle.bf16_to_f64(q_bits)
    rows = np.concatenate([oracle.bf16_to_f64(lat_c_rows), oracle.bf16_to_f64(lat_rows)])
    keep_c = [all(t <= p for t in range(ratio * c, ratio * c + ratio)) for c in range(lat_c_rows.shape[0])]
    keep_r = [(t <= p and t > p - window) for t in range(lat_rows.shape[0])]
    keep = np.array(keep_c + keep_r)
    z = scale * (q @ rows.T)
    z[:, ~keep] = -np.inf
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return (e @ rows[:, :512]) / e.sum(axis=1, keepdims=True), m[:, 0] + np.log(e.sum(axis=1))


def test_ratio_one_without_window_is_dsa():
    B, L, k = 2, 300, 40
    d = draw(B, L, 1, Q=3, seed=1)
    lens = [300, 177]
    idx, out, lse, s = csa.csa_batch(d["q_idx"], d["w"], d["keys_c"], d["latent_c"], d["latent"], lens, 1, k, 0,
                                     d["q_mla"], SCALE, d["Lc"])
    s_dsa = oracle.index_scores_batch(d["q_idx"], d["w"], d["keys_c"], lens, L)
    idx_dsa = oracle.topk_batch(s_dsa.astype(np.float32), lens, k)
    out_dsa, lse_dsa = oracle.sparse_mla_batch(d["q_mla"], d["latent_c"], idx_dsa, SCALE)
    np.testing.assert_array_equal(s, s_dsa)
    np.testing.assert_array_equal(idx, idx_dsa)
    np.testing.assert_array_equal(out, out_dsa)
    np.testing.assert_array_equal(lse, lse_dsa)


@pytest.mark.parametrize("ratio,window", [(4, 128), (4, 16), (4, 0), (128, 0), (3, 7)])
def test_full_selection_is_dense_attention_over_the_union(ratio, window):
    L = 700 if ratio < 128 else 1100
    d = draw(1, L, ratio, seed=2)
    k = d["Lc"]                                   # keeps every visible entry
    positions = list(range(0, 2 * ratio + 3)) + [L - 9, L - 4, L - 3, L - 2, L - 1]
    for p in positions:
        sel, o, l, _ = csa.csa_one(d["q_idx"][0, 0], d["w"][0, 0], d["keys_c"], d["latent_c"], d["latent"], 0, p, ratio,
                                   k, window, d["q_mla"][0, 0], SCALE, d["Lc"])
        if csa.visible_compressed(p, ratio) == 0 and window == 0:
            assert np.all(o == 0) and np.all(np.isneginf(l))
            continue
        ref_o, ref_l = dense_union(d["q_mla"][0, 0], d["latent_c"].data[0], d["latent"].data[0], p, ratio, window,
                                   SCALE)
        np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [1, 128, 5000])
def test_no_selection_is_sliding_window_attention(window):
    L = 900
    d = draw(1, L, 4, seed=3)
    for p in (0, 5, 127, 128, 500, L - 1):
        _, o, l, _ = csa.csa_one(d["q_idx"][0, 0], d["w"][0, 0], d["keys_c"], d["latent_c"], d["latent"], 0, p, 4, 0,
                                 window, d["q_mla"][0, 0], SCALE, d["Lc"])
        keep = [t for t in range(p + 1) if p - t < window]
        ref_o, ref_l = oracle.dense_mla_causal(d["q_mla"][0, 0], d["latent"].data[0], p, SCALE, keep=np.array(keep))
        np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)
        if window > p:                            # the window holds every token: dense causal attention
            full_o, full_l = oracle.dense_mla_causal(d["q_mla"][0, 0], d["latent"].data[0], p, SCALE)
            np.testing.assert_allclose(o, full_o, rtol=0, atol=1e-12)


def test_one_softmax_equals_the_merge_of_two_partials():
    L, ratio, k, window = 1000, 4, 24, 64
    d = draw(2, L, ratio, seed=4)
    for b, p in ((0, 999), (1, 130), (0, 2), (1, 3)):
        sel, o, l, _ = csa.csa_one(d["q_idx"][b, 0], d["w"][b, 0], d["keys_c"], d["latent_c"], d["latent"], b, p,
                                   ratio, k, window, d["q_mla"][b, 0], SCALE, d["Lc"])
        o1, l1 = oracle.sparse_mla_one(d["q_mla"][b, 0], d["latent_c"], b, sel, SCALE)
        o2, l2 = oracle.sparse_mla_one(d["q_mla"][b, 0], d["latent"], b, csa.window_positions(p, window), SCALE)
        lt = np.logaddexp(l1, l2)
        merged = np.exp(l1 - lt)[:, None] * np.nan_to_num(o1) + np.exp(l2 - lt)[:, None] * o2
        np.testing.assert_allclose(o, merged, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lt, rtol=0, atol=1e-12)


@pytest.mark.parametrize("ratio", [4, 128])
def test_visibility_needs_a_complete_block(ratio):
    assert [csa.visible_compressed(p, 4) for p in range(10)] == [0, 0, 0, 1, 1, 1, 1, 2, 2, 2]
    L = 6 * ratio + 5
    d = draw(1, L, ratio, seed=5)
    for p in range(L):
        n_c = csa.visible_compressed(p, ratio)
        assert n_c == sum(1 for c in range(d["Lc"]) if ratio * c + ratio - 1 <= p)
        for k in (1, 3, 100):
            sel, s = csa.select_compressed(d["q_idx"][0, 0], d["w"][0, 0], d["keys_c"], 0, p, ratio, k, d["Lc"])
            got = sel[sel >= 0]
            assert got.size == min(k, n_c) and np.all(got < n_c) and np.all(np.diff(got) > 0)
            assert np.all(np.isneginf(s[n_c:])) and np.all(np.isfinite(s[:n_c]))


def test_selection_is_the_best_scores_by_python_sort():
    L, ratio, k = 4000, 4, 50
    d = draw(1, L, ratio, seed=6)
    # plant compressed keys aligned with the weighted query: they must be among the chosen
    q = oracle.e4m3_to_f64(d["q_idx"][0, 0])
    gsum = (d["w"][0, 0][:, None] * q).sum(axis=0)
    planted = torch.tensor(3.0 * gsum / np.linalg.norm(gsum) * math.sqrt(128))
    codes = planted.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for c in (0, 17, 500, 998):
        d["keys_c"].data[0, c] = codes
    p = L - 1
    sel, s = csa.select_compressed(d["q_idx"][0, 0], d["w"][0, 0], d["keys_c"], 0, p, ratio, k, d["Lc"])
    n_c = csa.visible_compressed(p, ratio)
    s32 = s[:n_c].astype(np.float32)
    best = sorted(range(n_c), key=lambda c: (-float(s32[c]), c))[:k]
    assert sel.tolist() == sorted(best)
    assert {0, 17, 500, 998} <= set(sel.tolist())
