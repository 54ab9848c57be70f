"""Shared pieces of the GPU parity tests: oracle views of synthetic batches and the
comparison rules with their tolerances.

Tolerances
  scores (integer-valued E4M3 inputs): the FP8 matrix cores are exact on them (every product
    is an integer and the internal grid of a group is at most 2^-7), so only the fp32 head sum
    rounds: |ds| <= 2^-17 * sum_h |w_h| |d_h|  (64 fp32 additions, 2^-24 each, with margin).
  scores (general E4M3 inputs): the FP8 matrix cores truncate each product of a group of 8 to
    a grid 13 binades below the group's largest product (measured on gfx950: 256 + 2^-5 is
    kept, 256 + 2^-6 comes back as 256). Per group that is < 8 * 2^-13 * max|p| <= 2^-10 *
    sum|p|, so |d_gpu - d| <= 2^-10 * sum_i |q_i k_i| per head, and
    |ds| <= 2^-10 * sum_h |w_h| sum_i |q_hi k_ti| + 2^-16 * sum_h |w_h| |d_h|.
  top-k sets: equal, except that tokens whose exact score lies within 1e-3 * |s_k| of the
    exact k-th largest score s_k may swap; the set sizes are equal.
  top-k on identical float32 scores: bit-exact (integer work).
  sparse MLA outputs: max abs error <= 2e-2 and relative L2 error <= 5e-3 against the
    float64 oracle, per query token; lse within 1e-3 (the logits are fp32 sums of bf16
    products, error ~1e-5; the bf16 rounding of P does not enter lse).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle.dsa import Cache as OCache

SCORE_REL_GENERAL = 2.0 ** -10
SCORE_REL_FP32 = 2.0 ** -16
SCORE_REL_INT = 2.0 ** -17
TOPK_SWAP_REL = 1e-3
MLA_MAX_ABS = 2e-2
MLA_REL_L2 = 5e-3
LSE_ABS = 1e-3


def np_(t):
    return t.detach().cpu().numpy()


def bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def key_cache(batch):
    wl = batch.wl
    return OCache(np_(batch.keys), None if batch.key_table is None else np_(batch.key_table), wl.page_size)


def latent_cache(batch, layer=0):
    """The oracle's view of a latent cache: bf16 bits, or E4M3 codes for an FP8 cache."""
    wl = batch.wl
    tab = batch.latent_table[layer]
    lat = batch.latent[layer]
    data = np_(lat) if lat.dtype == torch.uint8 else bits(lat)
    return OCache(data, None if tab is None else np_(tab), wl.page_size)


def score_tolerance(q_codes, w, key_rows_codes, integer_inputs=False):
    """Per-token tolerance of GPU scores for one query (see module docstring)."""
    q = oracle.e4m3_to_f64(q_codes)
    k = oracle.e4m3_to_f64(key_rows_codes)
    aw = np.abs(np.asarray(w, dtype=np.float64))
    d = k @ q.T
    mag = np.abs(d) @ aw
    if integer_inputs:
        return SCORE_REL_INT * mag
    l1 = np.abs(k) @ np.abs(q).T
    return SCORE_REL_GENERAL * (l1 @ aw) + SCORE_REL_FP32 * mag


def check_scores(gpu_row, exact_row, tol, p):
    """gpu_row, exact_row: [L_max]; entries after p must be -inf."""
    g = np.asarray(gpu_row, dtype=np.float64)
    assert np.all(np.isneginf(g[p + 1:])), "scores after the query position must be -inf"
    err = np.abs(g[: p + 1] - exact_row[: p + 1])
    bad = np.nonzero(err > tol[: p + 1])[0]
    assert bad.size == 0, f"{bad.size} scores out of tolerance, first t={bad[0]}: gpu {g[bad[0]]} exact {exact_row[bad[0]]} tol {tol[bad[0]]}"
    return float(err.max()) if err.size else 0.0


def check_topk_sets(gpu_idx, oracle_idx, exact_scores, k):
    """Equal sets up to swaps of near-threshold tokens; both ascending and -1 padded."""
    g = np.asarray(gpu_idx)
    o = np.asarray(oracle_idx)
    mg, mo = int((g >= 0).sum()), int((o >= 0).sum())
    assert mg == mo, f"set sizes differ: gpu {mg} oracle {mo}"
    assert np.all(g[mg:] == -1) and np.all(np.diff(g[:mg]) > 0), "gpu indices not ascending / padded"
    diff = np.setxor1d(g[:mg], o[:mo])
    if diff.size:
        s = np.asarray(exact_scores, dtype=np.float64)
        sk = np.sort(s[o[:mo]])[0]                 # the oracle's k-th largest score
        far = diff[np.abs(s[diff] - sk) > TOPK_SWAP_REL * abs(sk)]
        assert far.size == 0, f"tokens {far[:8]} differ beyond the swap band (s_k={sk})"
    return int(diff.size)


def check_mla(out_gpu, lse_gpu, out_ref, lse_ref):
    """One query token: out [H, 512], lse [H]; the fixed bars max abs <= 2e-2, rel L2 <= 5e-3."""
    og = np.asarray(out_gpu, dtype=np.float64)
    err = np.abs(og - out_ref)
    max_abs = float(err.max())
    rel_l2 = float(np.linalg.norm(og - out_ref) / max(np.linalg.norm(out_ref), 1e-30))
    assert max_abs <= MLA_MAX_ABS, f"max abs error {max_abs}"
    assert rel_l2 <= MLA_REL_L2, f"relative L2 error {rel_l2}"
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.all(np.abs(lg[fin] - lse_ref[fin]) <= LSE_ABS), float(np.abs(lg[fin] - lse_ref[fin]).max())
    return max_abs, rel_l2


def dsa_cache(data, table, page_size):
    import sparse_attention_lightning_amd as dsa
    return dsa.Cache(data, table, page_size)


def integer_e4m3(shape, gen, lo=-8, hi=8, device="cpu"):
    """E4M3 codes of small integers (exactly representable)."""
    v = torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32).to(torch.float32)
    return v.to(torch.float8_e4m3fn).view(torch.uint8).to(device)


def positions(wl):
    return [[n - wl.Q + j for j in range(wl.Q)] for n in wl.lens]


def scale_of(wl):
    return 1.0 / math.sqrt(576)
