"""CPU oracle of compressed sparse attention (CSA), DeepSeek-V4's attention over a KV cache
compressed along the sequence.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module. The GPU library never calls it, and it shares
no code, tables or constants with the GPU library.

What it computes ("LLM architecture survey", section 2.3 DeepSeek-V4): the KV cache is
compressed along the sequence by a ratio of 4; DSA's sparse selection runs on top of the
compressed entries (top-1024 in the Pro model, top-512 in Flash); a sliding window of the
last 128 raw tokens is added to keep locality. HCA, the heavily compressed variant in the
same section, compresses by 128 and attends densely: the same computation with a selection
that keeps every visible compressed entry and no window.

For one query token at raw position p:
1. Visible compressed entries. Entry c summarises raw tokens ratio*c .. ratio*c + ratio - 1;
   it is visible once its last token is: ratio*c + ratio - 1 <= p, so n_c = (p + 1) // ratio
   entries (a partly filled block is not yet an entry).
2. Selection (DSA's two steps on the compressed entries): lightning-indexer scores of the
   query against the n_c compressed indexer keys, then the k highest (ties to the lower
   entry, every entry when n_c <= k). k = 0 selects nothing.
3. Window: the raw tokens t with p - window < t <= p (fewer near the start).
4. Attention: one MQA-mode softmax over the union of the selected compressed latent rows and
   the window's raw latent rows, the same row format and formula as DSA's sparse MLA. A raw
   token that both lies in the window and belongs to a selected compressed block contributes
   both rows: the compressed entry and the raw token are different rows.

Readings where the page is silent (listed with the others in the design notes): the
compression itself is a learned map of the model, so the compressed caches are inputs;
compressed entries use the indexer key and latent row formats of the uncompressed path;
visibility needs a complete block; the window counts p itself; window and selection share
one softmax (equal, by the log-sum-exp identity, to merging two partial attentions).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .dsa import Cache, index_scores, query_positions, select_topk, sparse_mla


def visible_compressed(p: int, ratio: int) -> int:
    """Compressed entries whose whole block of raw tokens lies at or before position p."""
    return (p + 1) // ratio


def window_positions(p: int, window: int) -> np.ndarray:
    """Raw positions of the sliding window of a query at position p, ascending."""
    return np.arange(max(0, p - window + 1), p + 1, dtype=np.int64)


def select_compressed(q_codes, w, keys_c: Cache, b: int, p: int, ratio: int, k: int, Lc_max: int):
    """Steps 1-2: ids of the selected compressed entries (ascending, -1 padded to k) and the
    float64 scores of every compressed entry (-inf past the visible ones)."""
    n_c = visible_compressed(p, ratio)
    if n_c == 0:
        return np.full(k, -1, dtype=np.int32), np.full(Lc_max, -np.inf)
    s = index_scores(q_codes, w, keys_c, b, n_c - 1, Lc_max)
    if k == 0:
        return np.zeros(0, dtype=np.int32), s
    return select_topk(s.astype(np.float32), n_c - 1, k), s


def csa_one(q_idx_codes, w, keys_c: Cache, latent_c: Cache, latent: Cache, b: int, p: int, ratio: int, k: int,
            window: int, q_bits, scale: float, Lc_max: int, sel: Optional[np.ndarray] = None):
    """One query token: (selected entry ids [k], o [H, 512], lse [H], scores [Lc_max]).

    `sel` overrides the selection (to evaluate attention over another valid selection)."""
    if sel is None:
        sel, s = select_compressed(q_idx_codes, w, keys_c, b, p, ratio, k, Lc_max)
    else:
        s = None
    chosen = np.asarray(sel)
    chosen = chosen[chosen >= 0]
    rows = np.concatenate([latent_c.rows(b, chosen), latent.rows(b, window_positions(p, window))], axis=0)
    o, lse = sparse_mla(q_bits, rows, scale)
    return sel, o, lse, s


def csa_batch(q_idx, w, keys_c: Cache, latent_c: Cache, latent: Cache, seq_lens, ratio: int, k: int, window: int,
              q_mla, scale: float, Lc_max: int, q_pos=None):
    """Every query token of a batch: idx [B, Q, k], out [B, Q, H, 512], lse [B, Q, H],
    scores [B, Q, Lc_max] (float64)."""
    B, Q = q_idx.shape[:2]
    H = q_mla.shape[2]
    pos = query_positions(seq_lens, Q, q_pos)
    idx = np.full((B, Q, k), -1, dtype=np.int32)
    out = np.empty((B, Q, H, 512))
    lse = np.empty((B, Q, H))
    scores = np.empty((B, Q, Lc_max))
    for b in range(B):
        for j in range(Q):
            sel, out[b, j], lse[b, j], scores[b, j] = csa_one(q_idx[b, j], w[b, j], keys_c, latent_c, latent, b,
                                                              int(pos[b, j]), ratio, k, window, q_mla[b, j], scale,
                                                              Lc_max)
            idx[b, j, :len(sel)] = sel
    return idx, out, lse, scores
