"""The plain C reference (oracle/dsa_ref.c) computes what the numpy oracle computes.

The numpy oracle is pinned by tests/test_oracle.py (exact rational brute force, torch's casts,
SDPA, dense attention, Python's sort, the pages' printed figures); the C reference is tied to
it here: selections bit for bit, index scores and attention to float64 rounding (the products
and their order differ only in the last bits of double sums). Every E4M3 code and every bf16
class (normal, subnormal, zero, both signs) passes through both decoders.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import cref


def e4m3_codes(shape, gen):
    return torch.randn(shape, generator=gen).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_bits(shape, gen, scale=1.0):
    return (scale * torch.randn(shape, generator=gen)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("Hi,n,p", [(64, 3000, 2999), (32, 700, 345), (64, 1, 0)])
def test_index_scores_equal(Hi, n, p):
    gen = torch.Generator().manual_seed(n + Hi)
    q = e4m3_codes((Hi, 128), gen)
    keys = e4m3_codes((n, 128), gen)
    w = torch.rand(Hi, generator=gen).numpy()
    got = cref.index_scores(q, w, keys, p, n + 5)
    ref = oracle.index_scores(q, w, oracle.Cache(keys[None]), 0, p, n + 5)
    assert np.all(np.isneginf(got[p + 1:])) and np.all(np.isneginf(ref[p + 1:]))
    np.testing.assert_allclose(got[: p + 1], ref[: p + 1], rtol=1e-13, atol=1e-300)


def test_every_e4m3_code_decodes_alike():
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                  # the two NaN codes are never generated
    # query = one-hot per head, so score_t = w_h * max(code value, 0) for the head's dim
    n = codes.size
    keys = np.zeros((n, 128), dtype=np.uint8)
    keys[:, 5] = codes
    q = np.zeros((1, 128), dtype=np.uint8)
    q[0, 5] = 0x38                                         # 1.0 in E4M3
    got = cref.index_scores(q, np.array([1.0], np.float32), keys, n - 1, n)
    ref = np.maximum(oracle.e4m3_to_f64(codes), 0.0)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("k", [1, 7, 300, 2048])
def test_select_topk_equal_on_ties_and_signed_zeros(k):
    rng = np.random.default_rng(k)
    rows = [rng.integers(0, 40, 5000).astype(np.float32),
            np.where(rng.random(5000) < 0.5, -0.0, 0.0).astype(np.float32),
            rng.normal(size=5000).astype(np.float32),
            np.full(5000, 2.5, np.float32)]
    for s in rows:
        for p in (0, 5, 2047, 2048, 4999):
            np.testing.assert_array_equal(cref.select_topk(s, p, k), oracle.select_topk(s, p, k))


@pytest.mark.parametrize("m,H", [(300, 16), (1, 8), (0, 4), (2048, 2)])
def test_sparse_mla_equal(m, H):
    gen = torch.Generator().manual_seed(m * 7 + H)
    q = bf16_bits((H, 576), gen)
    rows = bf16_bits((m, 576), gen, scale=3.0)
    if m:
        rows[0, :3] = np.array([0x0001, 0x8000, 0x0000], dtype=np.uint16)   # subnormal, -0, +0
    o, l = cref.sparse_mla(q, rows, 0.04)
    ro, rl = oracle.sparse_mla(q, rows, 0.04)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l, rl, rtol=1e-12, atol=0)
    if m == 0:
        assert np.all(o == 0) and np.all(np.isneginf(l))


def test_sparse_mla_equal_on_e4m3_rows():
    gen = torch.Generator().manual_seed(99)
    q = bf16_bits((8, 576), gen)
    rows = e4m3_codes((500, 576), gen)
    o, l = cref.sparse_mla(q, rows, 0.04, latent_scale=0.375)
    ro, rl = oracle.sparse_mla(q, rows, 0.04, latent_scale=0.375)
    np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l, rl, rtol=1e-12, atol=0)
