"""ctypes binding of libdsa.so, the C ABI declared in include/dsa.h.

Argument marshalling only: every step of the hot path runs in the library's HIP kernels.
Torch tensors supply device memory and the current stream. Importing this module fails
loudly when the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
OP_INDEX_SCORE, OP_TOPK, OP_SPARSE_MLA, OP_FORWARD_SHARED, OP_HISPARSE_SWAP_IN = range(5)

# every symbol include/dsa.h declares
EXPORTS = ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_sparse_mla_fwd_fp8", "dsa_forward_shared",
           "dsa_forward_shared_fp8", "dsa_forward_shared_noalloc", "dsa_csa_forward", "dsa_csa_workspace_size", "dsa_hisparse_swap_in",
           "dsa_workspace_size", "dsa_status_str", "dsa_last_error")


class CacheT(C.Structure):
    _fields_ = [("base", C.c_void_p), ("block_table", C.c_void_p), ("max_pages", C.c_int32),
                ("page_size", C.c_int32)]


class BatchT(C.Structure):
    _fields_ = [("B", C.c_int32), ("Q", C.c_int32), ("L_max", C.c_int32), ("seq_lens", C.c_void_p),
                ("q_pos", C.c_void_p)]


class HotBufferT(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("slot_page", C.c_void_p), ("slot_clock", C.c_void_p),
                ("page_clock", C.c_void_p), ("max_pages", C.c_int32), ("n_slots", C.c_int32),
                ("page_size", C.c_int32), ("row_bytes", C.c_int32)]


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
                4: "DSA_ERR_HIP"}


def load_library(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_lightning_amd.build` "
                          "(the DSA path has no non-HIP fallback)")
    lib = C.CDLL(path)
    P, I, F, S = C.c_void_p, C.c_int, C.c_float, C.c_size_t
    lib.dsa_index_score.argtypes = [C.POINTER(BatchT), P, P, I, C.POINTER(CacheT), P, P]
    lib.dsa_topk.argtypes = [C.POINTER(BatchT), P, I, P, P, S, P]
    lib.dsa_sparse_mla_fwd.argtypes = [C.POINTER(BatchT), P, I, C.POINTER(CacheT), P, I, I, F, P, P, P, S, P]
    lib.dsa_sparse_mla_fwd_fp8.argtypes = [C.POINTER(BatchT), P, I, C.POINTER(CacheT), F, P, I, I, F, P, P, P, S, P]
    lib.dsa_forward_shared.argtypes = [C.POINTER(BatchT), P, P, I, C.POINTER(CacheT), I, I, I, P, I,
                                       C.POINTER(CacheT), F, P, P, P, P, S, P]
    lib.dsa_forward_shared_fp8.argtypes = [C.POINTER(BatchT), P, P, I, C.POINTER(CacheT), I, I, I, P, I,
                                           C.POINTER(CacheT), P, F, P, P, P, P, S, P]
    lib.dsa_forward_shared_noalloc.argtypes = [C.POINTER(BatchT), P, P, I, C.POINTER(CacheT), I, I, I, P, I,
                                               C.POINTER(CacheT), F, P, P, P, P]
    lib.dsa_csa_forward.argtypes = [C.POINTER(BatchT), P, P, I, C.POINTER(CacheT), C.POINTER(CacheT),
                                    C.POINTER(CacheT), I, I, I, P, I, F, P, P, P, P, S, P]
    lib.dsa_csa_workspace_size.argtypes = [C.POINTER(BatchT), I, I, I, I]
    lib.dsa_csa_workspace_size.restype = S
    lib.dsa_hisparse_swap_in.argtypes = [I, P, I, I, I, C.POINTER(HotBufferT), P, P, P, P, S, P]
    lib.dsa_workspace_size.argtypes = [I, C.POINTER(BatchT), I, I, I, I]
    lib.dsa_workspace_size.restype = S
    lib.dsa_status_str.argtypes = [I]
    lib.dsa_status_str.restype = C.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = C.c_char_p
    for name in ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_fwd", "dsa_sparse_mla_fwd_fp8", "dsa_forward_shared",
                 "dsa_forward_shared_fp8", "dsa_forward_shared_noalloc", "dsa_csa_forward", "dsa_hisparse_swap_in"):
        getattr(lib, name).restype = C.c_int
    return lib


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, lib().dsa_last_error().decode())


# ----------------------------------------------------------------------------- torch-facing API
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass
class Cache:
    """A token-major cache: contiguous [B, L_max, D] or a paged pool [n_pages, page_size, D]
    with block_table [B, max_pages] (int32)."""
    data: "object"
    block_table: "object" = None
    page_size: int = 0

    def c(self) -> CacheT:
        if self.block_table is None:
            return CacheT(self.data.data_ptr(), None, 0, 0)
        return CacheT(self.data.data_ptr(), self.block_table.data_ptr(), self.block_table.shape[1], self.page_size)


def batch_t(B: int, Q: int, L_max: int, seq_lens, q_pos=None) -> BatchT:
    return BatchT(B, Q, L_max, seq_lens.data_ptr(), _ptr(q_pos))


def workspace_size(op: int, B: int, Q: int, L_max: int, Hi: int = 64, H: int = 128, k: int = 2048,
                   n_layers: int = 1) -> int:
    bt = BatchT(B, Q, L_max, None, None)
    return lib().dsa_workspace_size(op, C.byref(bt), Hi, H, k, n_layers)


def _workspace(nbytes: int, device, ws=None):
    import torch
    if nbytes == 0:
        return None
    if ws is not None:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def index_score(q, w, keys: Cache, seq_lens, L_max: int, q_pos=None, scores=None, stream=None):
    """q [B,Q,Hi,128] uint8 (E4M3FN codes), w [B,Q,Hi] float32 -> scores [B,Q,L_max] float32."""
    import torch
    B, Q, Hi = q.shape[:3]
    if scores is None:
        scores = torch.empty((B, Q, L_max), dtype=torch.float32, device=q.device)
    bt = batch_t(B, Q, L_max, seq_lens, q_pos)
    kc = keys.c()
    _check(lib().dsa_index_score(C.byref(bt), q.data_ptr(), w.data_ptr(), Hi, C.byref(kc), scores.data_ptr(),
                                 _stream(stream)))
    return scores


def topk(scores, seq_lens, k: int, q_pos=None, idx=None, ws=None, stream=None):
    """scores [B,Q,L_max] float32 -> idx [B,Q,k] int32 (ascending, -1 padded)."""
    import torch
    B, Q, L_max = scores.shape
    if idx is None:
        idx = torch.empty((B, Q, k), dtype=torch.int32, device=scores.device)
    bt = batch_t(B, Q, L_max, seq_lens, q_pos)
    n = lib().dsa_workspace_size(OP_TOPK, C.byref(bt), 64, 128, k, 1)
    ws = _workspace(n, scores.device, ws)
    _check(lib().dsa_topk(C.byref(bt), scores.data_ptr(), k, idx.data_ptr(), _ptr(ws), n, _stream(stream)))
    return idx


def sparse_mla_fwd(q, latent: Cache, idx, k: int, scale: float, seq_lens, L_max: int, idx_q_stride: Optional[int] = None,
                   q_pos=None, out=None, lse=None, want_lse: bool = True, ws=None, stream=None,
                   latent_scale: Optional[float] = None):
    """q [B,Q,H,576] bf16 -> (out [B,Q,H,512] float32, lse [B,Q,H] float32). With latent_scale
    the latent cache holds 576 E4M3 codes per row (uint8), value = latent_scale x code."""
    import torch
    B, Q, H = q.shape[:3]
    if idx_q_stride is None:
        idx_q_stride = k if idx.shape[1] == Q else 0      # one set per query token, or one per sequence
    if out is None:
        out = torch.empty((B, Q, H, 512), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    bt = batch_t(B, Q, L_max, seq_lens, q_pos)
    n = lib().dsa_workspace_size(OP_SPARSE_MLA, C.byref(bt), 64, H, k, 1)
    ws = _workspace(n, q.device, ws)
    lc = latent.c()
    if latent_scale is None:
        _check(lib().dsa_sparse_mla_fwd(C.byref(bt), q.data_ptr(), H, C.byref(lc), idx.data_ptr(), k, idx_q_stride,
                                        float(scale), out.data_ptr(), _ptr(lse), _ptr(ws), n, _stream(stream)))
    else:
        _check(lib().dsa_sparse_mla_fwd_fp8(C.byref(bt), q.data_ptr(), H, C.byref(lc), float(latent_scale),
                                            idx.data_ptr(), k, idx_q_stride, float(scale), out.data_ptr(), _ptr(lse),
                                            _ptr(ws), n, _stream(stream)))
    return out, lse


def forward_shared(q_idx, w, keys: Cache, k: int, q_mla: Sequence, latents: Sequence[Cache], scale: float,
                   seq_lens, L_max: int, share_first_query: bool = False, q_pos=None,
                   outs: Optional[List] = None, lses: Optional[List] = None, idx=None, ws=None, stream=None,
                   latent_scales: Optional[Sequence[float]] = None):
    """One IndexShare group: scores + top-k once, sparse MLA per layer with the same indices.
    With latent_scales (one per layer) the latent caches hold 576 E4M3 codes per row (uint8),
    value = latent_scales[l] x code. Returns (idx, [(out, lse) per layer])."""
    import torch
    B, Q, Hi = q_idx.shape[:3]
    H = q_mla[0].shape[2]
    nl = len(q_mla)
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, 1 if share_first_query else Q, k), dtype=torch.int32, device=dev)
    if outs is None:
        outs = [torch.empty((B, Q, H, 512), dtype=torch.float32, device=dev) for _ in range(nl)]
    if lses is None:
        lses = [torch.empty((B, Q, H), dtype=torch.float32, device=dev) for _ in range(nl)]
    bt = batch_t(B, Q, L_max, seq_lens, q_pos)
    n = lib().dsa_workspace_size(OP_FORWARD_SHARED, C.byref(bt), Hi, H, k, nl)
    ws = _workspace(n, dev, ws)
    qs = (C.c_void_p * nl)(*[t.data_ptr() for t in q_mla])
    lats = (CacheT * nl)(*[c.c() for c in latents])
    os_ = (C.c_void_p * nl)(*[t.data_ptr() for t in outs])
    ls = (C.c_void_p * nl)(*[(t.data_ptr() if t is not None else None) for t in lses])
    kc = keys.c()
    if latent_scales is None:
        _check(lib().dsa_forward_shared(C.byref(bt), q_idx.data_ptr(), w.data_ptr(), Hi, C.byref(kc), k,
                                        int(share_first_query), nl, qs, H, lats, float(scale), os_, ls, idx.data_ptr(),
                                        _ptr(ws), n, _stream(stream)))
    else:
        sc = (C.c_float * nl)(*[float(x) for x in latent_scales])
        _check(lib().dsa_forward_shared_fp8(C.byref(bt), q_idx.data_ptr(), w.data_ptr(), Hi, C.byref(kc), k,
                                            int(share_first_query), nl, qs, H, lats, sc, float(scale), os_, ls,
                                            idx.data_ptr(), _ptr(ws), n, _stream(stream)))
    return idx, list(zip(outs, lses))


NOALLOC_SCRATCH_BYTES = 128 << 20     # DSA_NOALLOC_SCRATCH_BYTES


def forward_shared_noalloc(q_idx, w, keys: Cache, k: int, q_mla: Sequence, latents: Sequence[Cache], scale: float,
                           seq_lens, L_max: int, outs: List, lses: List, idx, share_first_query: bool = False,
                           q_pos=None, stream=None):
    """forward_shared without a workspace: the library's own per-device scratch serves the call,
    which allocates nothing (outputs are the caller's: outs, lses, idx must be given)."""
    B, Q, Hi = q_idx.shape[:3]
    H = q_mla[0].shape[2]
    nl = len(q_mla)
    bt = batch_t(B, Q, L_max, seq_lens, q_pos)
    qs = (C.c_void_p * nl)(*[t.data_ptr() for t in q_mla])
    lats = (CacheT * nl)(*[c.c() for c in latents])
    os_ = (C.c_void_p * nl)(*[t.data_ptr() for t in outs])
    ls = (C.c_void_p * nl)(*[(t.data_ptr() if t is not None else None) for t in lses])
    kc = keys.c()
    _check(lib().dsa_forward_shared_noalloc(C.byref(bt), q_idx.data_ptr(), w.data_ptr(), Hi, C.byref(kc), k,
                                            int(share_first_query), nl, qs, H, lats, float(scale), os_, ls,
                                            idx.data_ptr(), _stream(stream)))
    return idx, list(zip(outs, lses))


def csa_workspace_size(B: int, Q: int, L_max: int, H: int, ratio: int, k: int, window: int) -> int:
    bt = BatchT(B, Q, L_max, None, None)
    return lib().dsa_csa_workspace_size(C.byref(bt), H, ratio, k, window)


def csa_forward(q_idx, w, keys_c: Optional[Cache], latent_c: Optional[Cache], latent: Optional[Cache], ratio: int,
                k: int, window: int, q_mla, scale: float, seq_lens, L_max: int, q_pos=None, out=None, lse=None,
                idx=None, ws=None, stream=None):
    """Compressed sparse attention: top-k over the compressed entries (keys_c, latent_c: ceil(L_max /
    ratio) rows per sequence) plus a window of raw rows (latent), one softmax over both.
    Returns (idx [B,Q,k] int32 compressed entry ids or None when k == 0, out [B,Q,H,512], lse [B,Q,H])."""
    import torch
    B, Q, H = q_mla.shape[:3]
    dev = q_mla.device
    if out is None:
        out = torch.empty((B, Q, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    if idx is None and k > 0:
        idx = torch.empty((B, Q, k), dtype=torch.int32, device=dev)
    bt = batch_t(B, Q, L_max, seq_lens, q_pos)
    n = lib().dsa_csa_workspace_size(C.byref(bt), H, ratio, k, window)
    ws = _workspace(n, dev, ws)
    empty = CacheT(None, None, 0, 0)
    kc = keys_c.c() if keys_c is not None else empty
    lc = latent_c.c() if latent_c is not None else empty
    lr = latent.c() if latent is not None else empty
    Hi = q_idx.shape[2] if q_idx is not None else 64
    _check(lib().dsa_csa_forward(C.byref(bt), _ptr(q_idx), _ptr(w), Hi, C.byref(kc), C.byref(lc), C.byref(lr), ratio, k,
                                 window, q_mla.data_ptr(), H, float(scale), out.data_ptr(), _ptr(lse), _ptr(idx),
                                 _ptr(ws), n, _stream(stream)))
    return idx, out, lse


@dataclass
class HotBuffer:
    """HiSparse hot buffer of B sequences: device slots of one page each over a latent cache
    kept whole in host memory. Every state tensor is int32 on the device, -1 before the first
    step: block_table [B, max_pages], slot_page [B, n_slots], slot_clock [B, n_slots],
    page_clock [B, max_pages]. device_pool [B * n_slots, page_size, 576]: bf16 rows, or uint8
    E4M3 rows (for sparse_mla_fwd with latent_scale)."""
    block_table: "object"
    slot_page: "object"
    slot_clock: "object"
    page_clock: "object"
    device_pool: "object"
    page_size: int

    def c(self) -> HotBufferT:
        return HotBufferT(self.block_table.data_ptr(), self.slot_page.data_ptr(), self.slot_clock.data_ptr(),
                          self.page_clock.data_ptr(), self.block_table.shape[1], self.slot_page.shape[1],
                          self.page_size, 576 * self.device_pool.element_size())

    def latent_cache(self) -> Cache:
        """The latent cache that sparse MLA reads once the step's pages are resident."""
        return Cache(self.device_pool, self.block_table, self.page_size)


def hisparse_swap_in(idx, step: int, hb: HotBuffer, host_pool, copied=None, ws=None, stream=None):
    """idx [B, n_sets, k] int32 from topk; host_pool [B, max_pages, page_size, 576] pinned, the
    device pool's dtype (bf16, or uint8 E4M3 codes);
    copied: optional device [B] int32 that receives the pages copied per sequence."""
    B, n_sets, k = idx.shape
    if host_pool.element_size() != hb.device_pool.element_size():
        raise ValueError("host_pool and device_pool must hold rows of the same type")
    bt = BatchT(B, n_sets, 1, None, None)
    n = lib().dsa_workspace_size(OP_HISPARSE_SWAP_IN, C.byref(bt), 0, 0, k, 0)
    ws = _workspace(n, idx.device, ws)
    h = hb.c()
    _check(lib().dsa_hisparse_swap_in(B, idx.data_ptr(), n_sets, k, int(step), C.byref(h), host_pool.data_ptr(),
                                      hb.device_pool.data_ptr(), _ptr(copied), _ptr(ws), n, _stream(stream)))
