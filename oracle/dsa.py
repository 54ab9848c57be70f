"""CPU oracle of the DeepSeek Sparse Attention (DSA) hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module. The GPU library never calls it, and it shares
no code, tables or constants with the GPU library.

What it computes, step by step, in the order the pages give ("LLM architecture survey",
section 2.2 DeepSeek-V3.2: a two-stage pipeline that selects first and attends second):

1. Lightning indexer. For each query token at position p, a scalar relevance score for
   every preceding token t <= p:  s_t = sum_h w_h * ReLU(q_h . k_t), with Hi heads of
   dim 128 in FP8 (section 2.2; GLM-5.2's indexer with 32 heads in section 7.2 is the
   same computation with another head count). Tokens t > p score -inf.
2. Token selector. Each query keeps the k (= 2048) highest-scoring tokens; equal scores
   go to the lower position; when p + 1 <= k every visible token is kept. The kept
   positions are returned in ascending order and padded with -1 up to k.
3. Sparse MLA in MQA mode. MLA caches one latent row per token: 512 latent dims plus a
   64-dim RoPE part (section 2.1 DeepSeek-V3). In MQA mode every query head attends the
   same rows: z_i = scale * q_h . c_{t_i} over all 576 dims, P = softmax(z),
   o_h = sum_i P_i c_{t_i}[0:512], lse_h = log sum_i exp z_i (natural log, scale included).
4. IndexShare (section 7.2 and Fig. 7-2): steps 1-2 run once per group of consecutive
   sparse layers; every layer of the group runs step 3 with its own query and latent cache
   and the same index set. The draft-reuse form ("GLM-5.2 inference deployment" page,
   MTP draft + verify: only draft step 1 computes the top-K indices) runs steps 1-2 for
   the first query token of each sequence and uses that set for all its query tokens.

Readings where the pages are silent (all listed with their reasons in the design notes):
the weighted-ReLU head sum is the score; "preceding" is inclusive (t <= p); ties go to the
lower position; softmax scale is a parameter (1/sqrt(576) in the workloads); the value is
the first 512 dims of the latent row; FP8 is OCP E4M3FN with unit scale.

Precision: the indexer dot products are exact in float64 (every E4M3 value is an integer
multiple of 2^-9, so every product is a multiple of 2^-18 below 448^2 and any sum of 128
of them stays below 2^43 on that grid). Everything else runs in float64. The selector
decides on scores rounded to float32, the precision the GPU library stores them in.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

DI = 128
DQK = 576
DV = 512


# ----------------------------------------------------------------------------- formats
def _e4m3_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3FN code: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN;
    there are no infinities, so the largest magnitude is 1.75 * 2^8 = 448."""
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = sign * m * 2.0 ** -9
        else:
            tab[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3 = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3[np.asarray(codes, dtype=np.uint8)]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32: shift the 16 bits up and reinterpret."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- caches
@dataclass
class Cache:
    """Token-major cache of one tensor kind (indexer keys or latent rows).

    Contiguous: data [B, L_max, D]. Paged: data [n_pages, page_size, D] and
    table [B, max_pages]; token t of sequence b lives at data[table[b, t // page_size], t % page_size].
    """
    data: np.ndarray
    table: Optional[np.ndarray] = None
    page_size: int = 0

    def rows(self, b: int, positions: np.ndarray) -> np.ndarray:
        positions = np.asarray(positions, dtype=np.int64)
        if self.table is None:
            return self.data[b, positions]
        pages = self.table[b, positions // self.page_size].astype(np.int64)
        return self.data[pages, positions % self.page_size]


def query_positions(seq_lens: Sequence[int], Q: int, q_pos: Optional[np.ndarray] = None) -> np.ndarray:
    """Position of query token j of sequence b: given, or the last Q cache entries."""
    if q_pos is not None:
        return np.asarray(q_pos, dtype=np.int64)
    return np.array([[int(n) - Q + j for j in range(Q)] for n in seq_lens], dtype=np.int64)


# ----------------------------------------------------------------------------- step 1
def index_scores(q_codes: np.ndarray, w: np.ndarray, keys: Cache, b: int, p: int, L_max: int) -> np.ndarray:
    """Scores of one query token (sequence b, position p) against tokens 0..L_max-1.

    q_codes [Hi, 128] E4M3 codes, w [Hi] per-head weights. Returns float64 [L_max]:
    s_t = sum_h w_h * max(q_h . k_t, 0) for t <= p and -inf for t > p.
    """
    q = e4m3_to_f64(q_codes)                                    # [Hi, 128]
    k = e4m3_to_f64(keys.rows(b, np.arange(p + 1)))             # [p+1, 128]
    d = k @ q.T                                                 # [p+1, Hi], exact
    s = np.maximum(d, 0.0) @ np.asarray(w, dtype=np.float64)    # weighted ReLU head sum
    out = np.full(L_max, -np.inf)
    out[: p + 1] = s
    return out


def index_scores_batch(q_idx, w, keys: Cache, seq_lens, L_max: int, q_pos=None) -> np.ndarray:
    """[B, Q, L_max] float64 scores for every query token of the batch."""
    B, Q = q_idx.shape[:2]
    pos = query_positions(seq_lens, Q, q_pos)
    out = np.empty((B, Q, L_max))
    for b in range(B):
        for j in range(Q):
            out[b, j] = index_scores(q_idx[b, j], w[b, j], keys, b, int(pos[b, j]), L_max)
    return out


# ----------------------------------------------------------------------------- step 2
def select_topk(scores: np.ndarray, p: int, k: int) -> np.ndarray:
    """Top-k token positions of one query at position p, ascending, -1 padded to k.

    Ranks tokens 0..p by (score descending, position ascending) with a library sort and
    keeps the first min(k, p+1). Scores are compared as IEEE values (-0 == +0).
    """
    n = p + 1
    m = min(k, n)
    s = np.asarray(scores[:n], dtype=np.float64)
    order = np.lexsort((np.arange(n), -s))      # last key is primary: -score, then position
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = np.sort(order[:m])
    return out


def topk_batch(scores32: np.ndarray, seq_lens, k: int, q_pos=None) -> np.ndarray:
    """[B, Q, k] int32 index sets from float32 scores [B, Q, L_max]."""
    B, Q = scores32.shape[:2]
    pos = query_positions(seq_lens, Q, q_pos)
    out = np.empty((B, Q, k), dtype=np.int32)
    for b in range(B):
        for j in range(Q):
            out[b, j] = select_topk(scores32[b, j], int(pos[b, j]), k)
    return out


# ----------------------------------------------------------------------------- step 3
def latent_values(rows: np.ndarray, latent_scale: float = 1.0) -> np.ndarray:
    """Latent rows as float64: bf16 bits (uint16), or E4M3FN codes (uint8) times the cache's
    scale. The FP8 form reads the inference page's fp8_e4m3 KV-cache option; the pages give
    no scale convention, so one scale per cache is the reading taken."""
    if rows.dtype == np.uint8:
        return e4m3_to_f64(rows) * float(latent_scale)
    return bf16_to_f64(rows)


def sparse_mla(q_bits: np.ndarray, rows_bits: np.ndarray, scale: float, latent_scale: float = 1.0):
    """MQA-mode attention of H query heads over m selected latent rows.

    q_bits [H, 576] bf16 bits, rows_bits [m, 576] bf16 bits or E4M3 codes (m may be 0).
    Returns (o [H, 512] float64, lse [H] float64). With no rows: o = 0, lse = -inf.
    """
    H = q_bits.shape[0]
    if rows_bits.shape[0] == 0:
        return np.zeros((H, DV)), np.full(H, -np.inf)
    q = bf16_to_f64(q_bits)
    c = latent_values(rows_bits, latent_scale)
    z = scale * (q @ c.T)                       # [H, m] logits over all 576 dims
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    Z = e.sum(axis=1, keepdims=True)
    o = (e @ c[:, :DV]) / Z                     # value = first 512 dims
    lse = zmax[:, 0] + np.log(Z[:, 0])
    return o, lse


def sparse_mla_one(q_bits, latent: Cache, b: int, idx_row: np.ndarray, scale: float, latent_scale: float = 1.0):
    """Sparse MLA for one query token: gather the rows named by idx_row (skipping -1)."""
    sel = np.asarray(idx_row)
    sel = sel[sel >= 0]
    return sparse_mla(q_bits, latent.rows(b, sel), scale, latent_scale)


def sparse_mla_batch(q_mla, latent: Cache, idx: np.ndarray, scale: float, idx_q_stride_is_k: bool = True,
                     latent_scale: float = 1.0):
    """[B, Q, H, 512] outputs and [B, Q, H] lse. idx is [B, Q, k] (one set per query token)
    or, when idx_q_stride_is_k is False, [B, 1, k] shared by all query tokens of a sequence."""
    B, Q, H = q_mla.shape[:3]
    out = np.empty((B, Q, H, DV))
    lse = np.empty((B, Q, H))
    for b in range(B):
        for j in range(Q):
            row = idx[b, j] if idx_q_stride_is_k else idx[b, 0]
            out[b, j], lse[b, j] = sparse_mla_one(q_mla[b, j], latent, b, row, scale, latent_scale)
    return out, lse


# ----------------------------------------------------------------------------- step 4
def forward_shared(q_idx, w, keys: Cache, seq_lens, L_max: int, k: int,
                   q_mla_layers: List[np.ndarray], latent_layers: List[Cache], scale: float,
                   share_first_query: bool = False, q_pos=None):
    """One IndexShare group: score + select once, attend in every layer with that set.

    Returns (idx, [(out, lse) per layer]). With share_first_query the index set of the
    first query token of each sequence serves all its query tokens (idx is [B, 1, k]).
    """
    B, Q = q_idx.shape[:2]
    pos = query_positions(seq_lens, Q, q_pos)
    if share_first_query:
        s = index_scores_batch(q_idx[:, :1], w[:, :1], keys, seq_lens, L_max, q_pos=pos[:, :1])
        idx = topk_batch(s.astype(np.float32), seq_lens, k, q_pos=pos[:, :1])
    else:
        s = index_scores_batch(q_idx, w, keys, seq_lens, L_max, q_pos=pos)
        idx = topk_batch(s.astype(np.float32), seq_lens, k, q_pos=pos)
    results = [sparse_mla_batch(qm, lat, idx, scale, idx_q_stride_is_k=not share_first_query)
               for qm, lat in zip(q_mla_layers, latent_layers)]
    return idx, results


# ----------------------------------------------------------------------------- dense reference path
def dense_mla_causal(q_bits: np.ndarray, latent_rows_bits: np.ndarray, p: int, scale: float,
                     keep: Optional[np.ndarray] = None):
    """Masked dense MLA-MQA attention of one query at position p over rows 0..n-1.

    A separate code path from sparse_mla: it materialises the full [H, n] logit matrix,
    masks t > p (and, when `keep` is given, every t not in keep) with -inf, and applies
    softmax over the whole row. With keep = the selected set it must equal sparse_mla;
    with k >= p + 1 the selector keeps everything and sparse == dense causal attention.
    """
    q = bf16_to_f64(q_bits)
    c = bf16_to_f64(latent_rows_bits)
    n = c.shape[0]
    z = scale * (q @ c.T)
    mask = np.arange(n) > p
    if keep is not None:
        allowed = np.zeros(n, dtype=bool)
        allowed[np.asarray(keep)[np.asarray(keep) >= 0]] = True
        mask |= ~allowed
    z[:, mask] = -np.inf
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    Z = e.sum(axis=1, keepdims=True)
    return (e @ c[:, :DV]) / Z, zmax[:, 0] + np.log(Z[:, 0])


# ----------------------------------------------------------------------------- cost model
def attention_flops(H: int, n_keys: int) -> int:
    """Multiply-add FLOPs of MLA-MQA for one query over n_keys latent rows:
    2*H*n*576 for the logits plus 2*H*n*512 for the weighted value sum."""
    return 2 * H * n_keys * (DQK + DV)


def indexer_flops(Hi: int, n_keys: int) -> int:
    """FLOPs of the indexer dot products for one query over n_keys keys."""
    return 2 * Hi * n_keys * DI


def sparse_to_dense_ratio(L: int, k: int, H: int = 128) -> float:
    """Attention cost with top-k selection relative to dense attention over L tokens."""
    return attention_flops(H, min(k, L)) / attention_flops(H, L)
