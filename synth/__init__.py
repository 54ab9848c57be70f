"""Seeded synthetic inputs for the DSA hot path (indexer -> top-k -> sparse MLA).

This module only draws random inputs and lays them out in memory; it holds none of
the method's arithmetic. It is shared by the CPU oracle's tests, the GPU parity tests,
the smoke check and the benchmark, so both sides see the same bytes.

Distributions follow the workloads of the DeepSeek-V3.2 / GLM-5.2 pages:
  * indexer query and keys: N(0,1) rounded to OCP FP8 E4M3FN (round-to-nearest-even),
    64 heads x head dim 128 ("LLM architecture survey", section 2.2 DeepSeek-V3.2);
  * per-head indexer weights w ~ U(0,1), one vector per query token;
  * MLA query and latent rows: N(0,1) rounded to bf16, 576 = 512 latent + 64 RoPE dims,
    128 query heads (same survey, section 2.1 DeepSeek-V3);
  * paged caches: pages of `page_size` tokens, a seeded random permutation as the
    block table (the KV page / slot unit of the GLM-5.2 inference page, HiSparse section);
  * optional "planted" tokens whose indexer key is aligned with the query's weighted
    head sum, so that the selected set is not trivial.

Every tensor comes from its own torch.Generator seeded by (seed, stream, layer), so a
tensor does not depend on which other tensors were drawn before it. Values are
reproducible on one device type; CPU and GPU draws differ, so a test draws once and
copies to the other side.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import torch

DI = 128        # indexer head dim
DQK = 576       # latent row: 512 latent + 64 RoPE
DV = 512        # value part of the latent row

# generator streams
S_QIDX, S_KEYS, S_W, S_QMLA, S_LATENT, S_TABLE, S_PLANT_POS, S_PLANT_NOISE, S_DRIFT, S_DRAFT = (1, 2, 3, 4, 5, 6, 7, 8,
                                                                                          9, 10)
S_WINDOW, S_WINDOW_TABLE = 11, 12


@dataclass(frozen=True)
class Workload:
    """Shape of one batch of the hot path.

    B sequences, Q query tokens per sequence placed at the last Q cache positions,
    cache length L per sequence (the Q new tokens included), L_max the allocated length.
    page_size 0 means contiguous caches [B, L_max, D]; otherwise paged pools
    [n_pages, page_size, D] addressed through a block table [B, L_max / page_size].
    """
    name: str
    B: int
    Q: int
    L: int
    Hi: int = 64
    H: int = 128
    k: int = 2048
    page_size: int = 0
    planted: int = 0
    n_layers: int = 1
    share_first_query: int = 0
    L_max: int = 0                       # 0 -> L
    seq_lens: Optional[tuple] = None     # ragged lengths; None -> all L
    n_slots: int = 0                     # > 0: latent pages live in host memory, n_slots device slots per sequence
    drift_heads: int = 0                 # indexer query heads redrawn from one decode step to the next
    draft_steps: int = 0                 # > 0: an MTP draft loop of this many sequential steps per index set
    latent_fp8: int = 0                  # 1: latent rows as 576 E4M3FN codes (uint8) instead of bf16
    ratio: int = 0                       # > 0: compressed sparse attention; keys and latent rows are compressed
                                         # entries, one per `ratio` raw tokens (ceil(L_max / ratio) per sequence)
    window: int = 0                      # raw tokens of the sliding window (compressed sparse attention)

    @property
    def lmax(self) -> int:
        return self.L_max if self.L_max else self.L

    @property
    def lens(self) -> List[int]:
        return list(self.seq_lens) if self.seq_lens is not None else [self.L] * self.B

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(DQK)

    @property
    def rows(self) -> int:
        """Rows per sequence of the key and latent caches: raw tokens, or compressed entries."""
        return -(-self.lmax // self.ratio) if self.ratio else self.lmax

    @property
    def max_pages(self) -> int:
        """Pages per sequence of the key and latent caches."""
        return -(-self.rows // self.page_size) if self.page_size else 0

    @property
    def max_pages_raw(self) -> int:
        """Pages per sequence of the raw latent cache that a sliding window reads."""
        return -(-self.lmax // self.page_size) if self.page_size else 0

    def n_visible(self, n: int, j: int = None) -> int:
        """Rows of a sequence of n raw tokens visible to its query token j (the last by default)."""
        p = n - self.Q + (self.Q - 1 if j is None else j)
        return (p + 1) // self.ratio if self.ratio else p + 1


# The five workloads of the DSA hot path, at full size.
WORKLOADS = {
    "decode_tiny_8k": Workload("decode_tiny_8k", B=1, Q=1, L=8192),
    "decode_b32_128k_paged": Workload("decode_b32_128k_paged", B=32, Q=1, L=131072, page_size=64, planted=32),
    "prefill_4096_at_128k": Workload("prefill_4096_at_128k", B=1, Q=4096, L=131072),
    "indexshare_b8_1m_4layers": Workload("indexshare_b8_1m_4layers", B=8, Q=1, L=1048576, page_size=64, n_layers=4),
    "verify_b64_q8_32k": Workload("verify_b64_q8_32k", B=64, Q=8, L=32768, page_size=64),
    "verify_b64_q8_32k_draftshare": Workload("verify_b64_q8_32k_draftshare", B=64, Q=8, L=32768, page_size=64,
                                             share_first_query=1),
    # HiSparse: 1M-token decode with the latent cache in pinned host memory and a device
    # buffer of 6144 slots of one 16-token page per sequence (the GLM-5.2 inference page gives
    # 4096-6144 slots and a host : device ratio of 8-10; 65536 pages / 6144 slots = 10.7).
    # Consecutive decode steps redraw 4 of the 64 indexer query heads.
    "hisparse_b8_1m_decode": Workload("hisparse_b8_1m_decode", B=8, Q=1, L=1048576, page_size=16,
                                      n_slots=6144, drift_heads=4),
    # The same with E4M3 latent rows in both pools: half the bytes over the host link per page.
    "hisparse_b8_1m_decode_fp8kv": Workload("hisparse_b8_1m_decode_fp8kv", B=8, Q=1, L=1048576, page_size=16,
                                            n_slots=6144, drift_heads=4, latent_fp8=1),
    # MTP draft loop (GLM-5.2 inference page, MTP section): one MTP layer unrolled 7 times;
    # KVShare: every draft step reads the main model's cache; IndexShare on MTP: the top-2048
    # set is computed at step 1 and reused by the next 6 steps. Decode shape of the 128K batch.
    # The default decode batch over an FP8 latent cache (the inference page's fp8_e4m3 KV option):
    # rows of 576 E4M3FN(N(0,1)) codes, scale 1.
    "decode_b32_128k_paged_fp8kv": Workload("decode_b32_128k_paged_fp8kv", B=32, Q=1, L=131072, page_size=64,
                                            planted=32, latent_fp8=1),
    "mtp_draft_b32_128k_paged": Workload("mtp_draft_b32_128k_paged", B=32, Q=1, L=131072, page_size=64,
                                         planted=32, draft_steps=7),
    # The IndexShare group over E4M3 latent caches (one scale per layer's cache, 1 here).
    "indexshare_b8_1m_4layers_fp8kv": Workload("indexshare_b8_1m_4layers_fp8kv", B=8, Q=1, L=1048576, page_size=64,
                                               n_layers=4, latent_fp8=1),
    # Compressed sparse attention (architecture survey, DeepSeek-V4): compressed entries of 4 raw
    # tokens (keys and latent rows drawn like the uncompressed ones; the compression map is the
    # model's), top-1024 (V4-Pro) or top-512 (V4-Flash) of them, and a 128-token raw window.
    "csa_pro_decode_b32_128k": Workload("csa_pro_decode_b32_128k", B=32, Q=1, L=131072, page_size=64, planted=32,
                                        k=1024, ratio=4, window=128),
    "csa_flash_decode_b8_1m": Workload("csa_flash_decode_b8_1m", B=8, Q=1, L=1048576, page_size=64, planted=32,
                                       k=512, ratio=4, window=128),
    # HCA: compressed by 128, dense attention over every visible compressed entry, no window.
    "hca_decode_b32_128k": Workload("hca_decode_b32_128k", B=32, Q=1, L=131072, page_size=64, k=1024, ratio=128),
}


def _gen(seed: int, stream: int, layer: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 24) ^ (int(stream) << 8) ^ int(layer))
    return g


def _normal_chunks(shape, g, device, out_dtype, chunk=1 << 26):
    """N(0,1) draws rounded to out_dtype, generated in float32 chunks to bound memory."""
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=out_dtype, device=device)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        out[lo:hi] = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32).to(out_dtype)
    return out.view(*shape)


def e4m3_normal(shape, g, device) -> torch.Tensor:
    """uint8 codes of OCP E4M3FN(N(0,1)) (torch's float32 -> float8_e4m3fn cast, RNE)."""
    return _normal_chunks(shape, g, device, torch.float8_e4m3fn).view(torch.uint8)


def bf16_normal(shape, g, device) -> torch.Tensor:
    return _normal_chunks(shape, g, device, torch.bfloat16)


def block_table(wl: Workload, seed: int, layer: int, device) -> torch.Tensor:
    """[B, max_pages] int32: a seeded permutation of the B*max_pages physical pages."""
    n_pages = wl.B * wl.max_pages
    perm = torch.randperm(n_pages, generator=_gen(seed, S_TABLE, layer, "cpu"), dtype=torch.int64)
    return perm.to(torch.int32).view(wl.B, wl.max_pages).to(device)


def cache_shape(wl: Workload, dim: int):
    if wl.page_size:
        return (wl.B * wl.max_pages, wl.page_size, dim)
    return (wl.B, wl.rows, dim)


def raw_cache_shape(wl: Workload, dim: int):
    if wl.page_size:
        return (wl.B * wl.max_pages_raw, wl.page_size, dim)
    return (wl.B, wl.lmax, dim)


@dataclass
class Batch:
    wl: Workload
    seq_lens: torch.Tensor                 # [B] int32
    q_idx: torch.Tensor                    # [B, Q, Hi, 128] uint8 (E4M3FN codes)
    w: torch.Tensor                        # [B, Q, Hi] float32
    keys: torch.Tensor                     # contiguous [B, L_max, 128] or pool [P, page, 128] uint8
    key_table: Optional[torch.Tensor]      # [B, max_pages] int32 or None
    q_mla: List[torch.Tensor] = field(default_factory=list)     # per layer [B, Q, H, 576] bf16
    latent: List[torch.Tensor] = field(default_factory=list)    # per layer contiguous or pool, bf16
    latent_table: List[Optional[torch.Tensor]] = field(default_factory=list)
    planted_pos: Optional[torch.Tensor] = None                   # [B, planted] int64 (rows of the key cache)
    window_latent: Optional[torch.Tensor] = None                 # compressed attention: the raw latent cache
    window_table: Optional[torch.Tensor] = None                  # [B, max_pages_raw] int32 or None

    def to(self, device) -> "Batch":
        mv = lambda t: None if t is None else t.to(device)
        return Batch(self.wl, mv(self.seq_lens), mv(self.q_idx), mv(self.w), mv(self.keys), mv(self.key_table),
                     [mv(t) for t in self.q_mla], [mv(t) for t in self.latent],
                     [mv(t) for t in self.latent_table], mv(self.planted_pos), mv(self.window_latent),
                     mv(self.window_table))


def token_slot(table: Optional[torch.Tensor], page_size: int, b: int, t: torch.Tensor):
    """(page or sequence index, row) of token positions t of sequence b in a cache."""
    if table is None:
        return torch.full_like(t, b), t
    return table[b, t // page_size].to(torch.int64), t % page_size


def generate(wl: Workload, seed: int = 0, device="cpu", layers: Optional[int] = None,
             with_mla: bool = True) -> Batch:
    """Draw one batch of inputs for workload `wl`.

    Layer l of an IndexShare group uses seed `seed + l` for its MLA query, latent cache
    and block table; the indexer inputs use `seed`. The key cache is paged with layer 0's
    block table (one slot holds a token's latent row and its indexer key).
    """
    dev = torch.device(device)
    n_layers = wl.n_layers if layers is None else layers
    lens = torch.tensor(wl.lens, dtype=torch.int32, device=dev)
    q_idx = e4m3_normal((wl.B, wl.Q, wl.Hi, DI), _gen(seed, S_QIDX, 0, dev), dev)
    w = torch.rand((wl.B, wl.Q, wl.Hi), generator=_gen(seed, S_W, 0, dev), device=dev, dtype=torch.float32)
    keys = e4m3_normal(cache_shape(wl, DI), _gen(seed, S_KEYS, 0, dev), dev)
    key_table = block_table(wl, seed, 0, dev) if wl.page_size else None
    batch = Batch(wl, lens, q_idx, w, keys, key_table)

    if wl.planted:
        gp = _gen(seed, S_PLANT_POS, 0, "cpu")
        pos = torch.stack([torch.randperm(wl.n_visible(wl.lens[b]), generator=gp)[: wl.planted] for b in range(wl.B)])
        batch.planted_pos = pos.to(dev)
        # key = e4m3(2 * g_hat + 0.25 * eps) with g = sum_h w_h q_h (query token 0), |g_hat| = sqrt(128)
        qd = q_idx[:, 0].view(torch.float8_e4m3fn).to(torch.float32)          # [B, Hi, 128]
        g = torch.einsum("bh,bhi->bi", w[:, 0], qd)
        g_hat = g * (math.sqrt(DI) / g.norm(dim=1, keepdim=True))
        eps = torch.randn((wl.B, wl.planted, DI), generator=_gen(seed, S_PLANT_NOISE, 0, dev), device=dev)
        pk = (2.0 * g_hat[:, None, :] + 0.25 * eps).to(torch.float8_e4m3fn).view(torch.uint8)
        for b in range(wl.B):
            page, row = token_slot(key_table, wl.page_size, b, batch.planted_pos[b])
            keys[page, row] = pk[b]

    if with_mla:
        for layer in range(n_layers):
            s = seed + layer
            batch.q_mla.append(bf16_normal((wl.B, wl.Q, wl.H, DQK), _gen(s, S_QMLA, layer, dev), dev))
            if wl.latent_fp8:
                batch.latent.append(e4m3_normal(cache_shape(wl, DQK), _gen(s, S_LATENT, layer, dev), dev))
            else:
                batch.latent.append(bf16_normal(cache_shape(wl, DQK), _gen(s, S_LATENT, layer, dev), dev))
            if wl.page_size:
                batch.latent_table.append(key_table if layer == 0 else block_table(wl, s, layer, dev))
            else:
                batch.latent_table.append(None)
        if wl.ratio and wl.window:
            batch.window_latent = bf16_normal(raw_cache_shape(wl, DQK), _gen(seed, S_WINDOW, 0, dev), dev)
            if wl.page_size:
                n_pages = wl.B * wl.max_pages_raw
                perm = torch.randperm(n_pages, generator=_gen(seed, S_WINDOW_TABLE, 0, "cpu"), dtype=torch.int64)
                batch.window_table = perm.to(torch.int32).view(wl.B, wl.max_pages_raw).to(dev)
    return batch


def small(name: str, **kw) -> Workload:
    """A scaled-down variant of a named workload (same structure, smaller sizes)."""
    return replace(WORKLOADS[name], **kw)


def drift_queries(batch: Batch, n_steps: int, seed: int = 0) -> List[torch.Tensor]:
    """Indexer queries of n_steps consecutive decode steps: step 0 is the batch's own query;
    each later step redraws wl.drift_heads heads (chosen at random) of the step before with
    fresh E4M3FN(N(0,1)) values, so consecutive selected sets overlap without being equal."""
    wl = batch.wl
    dev = batch.q_idx.device
    qs = [batch.q_idx]
    gsel = _gen(seed, S_DRIFT, 0, "cpu")
    for t in range(1, n_steps):
        q = qs[-1].clone()
        fresh = e4m3_normal((wl.B, wl.Q, wl.drift_heads, DI), _gen(seed, S_DRIFT, t, dev), dev)
        for b in range(wl.B):
            heads = torch.randperm(wl.Hi, generator=gsel)[: wl.drift_heads].to(dev)
            q[b, :, heads] = fresh[b]
        qs.append(q)
    return qs


def draft_queries(batch: Batch, n_steps: int, seed: int = 0) -> List[torch.Tensor]:
    """MLA queries of the n_steps draft steps of an MTP loop ([B, Q, H, 576] bf16 each, N(0,1)):
    one shared MTP layer, so one latent cache, and a fresh query per step."""
    wl = batch.wl
    dev = batch.q_idx.device
    return [bf16_normal((wl.B, wl.Q, wl.H, DQK), _gen(seed, S_DRAFT, s, dev), dev) for s in range(n_steps)]
