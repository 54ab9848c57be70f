"""CPU-only checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments on the host with the documented status before touching HIP."""
import ctypes as C
import os
import re

import pytest

import sparse_attention_lightning_amd as dsa
from sparse_attention_lightning_amd._binding import BatchT, CacheT

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
A = 1 << 20          # a fake, well-aligned "device address": never dereferenced by these calls


def header_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(dsa.EXPORTS)
    lib = dsa.load_library()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = dsa.lib()
    assert [lib.dsa_status_str(i).decode() for i in range(5)] == [
        "DSA_OK", "DSA_ERR_INVALID_ARG", "DSA_ERR_UNSUPPORTED", "DSA_ERR_WORKSPACE", "DSA_ERR_HIP"]


def batch(B=2, Q=1, L=4096, seq=A, q_pos=None):
    return BatchT(B, Q, L, seq, q_pos)


def cache(base=A, table=None, max_pages=0, page=0):
    return CacheT(base, table, max_pages, page)


def call_index(bt, q=A, w=A, Hi=64, kc=None, scores=A):
    kc = kc or cache()
    lib = dsa.lib()
    return lib.dsa_index_score(C.byref(bt) if bt is not None else None, q, w, Hi, C.byref(kc), scores, None)


@pytest.mark.parametrize("case,expect", [
    (dict(bt=None), INVALID),
    (dict(bt=batch(B=0)), INVALID),
    (dict(bt=batch(Q=0)), INVALID),
    (dict(bt=batch(L=0)), INVALID),
    (dict(bt=batch(Q=5000, L=4096)), INVALID),
    (dict(bt=batch(seq=None)), INVALID),
    (dict(bt=batch(seq=A + 2)), INVALID),
    (dict(bt=batch(), Hi=48), UNSUPPORTED),
    (dict(bt=batch(), Hi=128), UNSUPPORTED),
    (dict(bt=batch(), q=None), INVALID),
    (dict(bt=batch(), q=A + 8), INVALID),
    (dict(bt=batch(), w=A + 2), INVALID),
    (dict(bt=batch(), scores=None), INVALID),
    (dict(bt=batch(), kc=cache(base=None)), INVALID),
    (dict(bt=batch(), kc=cache(base=A + 4)), INVALID),
    (dict(bt=batch(), kc=cache(table=A, max_pages=64, page=24)), UNSUPPORTED),
    (dict(bt=batch(), kc=cache(table=A, max_pages=64, page=0)), UNSUPPORTED),
    (dict(bt=batch(L=4096), kc=cache(table=A, max_pages=63, page=64)), INVALID),
    (dict(bt=batch(B=(1 << 24) + 1, L=4096)), UNSUPPORTED),  # B*Q above 2^24
    (dict(bt=batch(L=(1 << 24) + 16)), UNSUPPORTED),         # L_max above 2^24
    (dict(bt=batch(B=1 << 13, L=1 << 24)), UNSUPPORTED),     # B*Q*L_max = 2^37 scores
])
def test_index_score_rejects(case, expect):
    assert call_index(**case) == expect
    assert dsa.lib().dsa_last_error().decode().startswith("dsa_index_score")


def test_topk_rejects():
    lib = dsa.lib()
    bt = batch()
    need = dsa.workspace_size(dsa.OP_TOPK, 2, 1, 4096, k=2048)
    assert need > 0
    for k in (0, -1, 2049, 4096):
        assert lib.dsa_topk(C.byref(bt), A, k, A, A, need, None) == UNSUPPORTED
    assert lib.dsa_topk(C.byref(bt), A, 2048, A, None, need, None) == WORKSPACE
    assert lib.dsa_topk(C.byref(bt), A, 2048, A, A + 128, need, None) == WORKSPACE
    assert lib.dsa_topk(C.byref(bt), A, 2048, A, A, need - 1, None) == WORKSPACE
    assert lib.dsa_topk(C.byref(bt), A + 1, 2048, A, A, need, None) == INVALID
    assert lib.dsa_topk(C.byref(bt), A, 2048, None, A, need, None) == INVALID
    big = batch(B=1 << 12, L=1 << 24)                        # B*Q*L_max = 2^36 scores: accepted shape
    assert lib.dsa_topk(C.byref(big), A, 2048, A, None, 0, None) == WORKSPACE
    big = batch(B=(1 << 12) + 1, L=1 << 24)                  # one row more
    assert lib.dsa_topk(C.byref(big), A, 2048, A, None, 0, None) == UNSUPPORTED


def test_sparse_mla_rejects():
    lib = dsa.lib()
    bt = batch(B=1, L=8192)
    kc = cache()
    need = dsa.workspace_size(dsa.OP_SPARSE_MLA, 1, 1, 8192, H=128, k=2048)
    ok = dict(q=A, H=128, k=2048, stride=2048, scale=0.04, out=A, lse=A, ws=A, n=need)

    def call(**kw):
        a = {**ok, **kw}
        return lib.dsa_sparse_mla_fwd(C.byref(bt), a["q"], a["H"], C.byref(kc), A, a["k"], a["stride"], a["scale"],
                                      a["out"], a["lse"], a["ws"], a["n"], None)
    assert call(H=96) == UNSUPPORTED
    assert call(H=256) == UNSUPPORTED
    assert call(k=0) == UNSUPPORTED
    assert call(stride=5) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(scale=float("inf")) == INVALID
    # the kernel takes the maximum of the raw logits and scales it afterwards: only a
    # non-negative scale commutes with that maximum
    assert call(scale=-0.04) == INVALID
    assert call(scale=-1e-30) == INVALID
    assert call(q=A + 4) == INVALID
    assert call(out=A + 4) == INVALID
    assert call(lse=A + 2) == INVALID
    if need:
        assert call(ws=None) == WORKSPACE
        assert call(n=need - 1) == WORKSPACE


def test_sparse_mla_fp8_rejects_scales():
    lib = dsa.lib()
    bt = batch(B=1, L=8192)
    kc = cache()
    need = dsa.workspace_size(dsa.OP_SPARSE_MLA, 1, 1, 8192, H=128, k=2048)

    def call(scale=0.04, latent_scale=1.0):
        return lib.dsa_sparse_mla_fwd_fp8(C.byref(bt), A, 128, C.byref(kc), latent_scale, A, 2048, 2048, scale, A, A,
                                          A, need, None)
    assert call(scale=-0.04) == INVALID
    assert call(scale=float("-inf")) == INVALID
    assert call(latent_scale=0.0) == INVALID
    assert call(latent_scale=-1.0) == INVALID
    assert call(latent_scale=float("nan")) == INVALID


def test_forward_shared_rejects():
    lib = dsa.lib()
    bt = batch(B=1, L=8192)
    kc = cache()
    lat = (CacheT * 4)(*[cache() for _ in range(4)])
    ptrs = (C.c_void_p * 4)(A, A, A, A)
    need = dsa.workspace_size(dsa.OP_FORWARD_SHARED, 1, 1, 8192, k=2048, n_layers=4)

    def call(share=0, nl=4, qs=ptrs, lats=lat, outs=ptrs, ws=A, n=need, Hi=64, H=128, scale=0.04):
        return lib.dsa_forward_shared(C.byref(bt), A, A, Hi, C.byref(kc), 2048, share, nl, qs, H, lats, scale, outs,
                                      None, A, ws, n, None)
    assert call(scale=-0.04) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(share=2) == INVALID
    assert call(nl=0) == INVALID
    assert call(qs=None) == INVALID
    assert call(outs=(C.c_void_p * 4)(A, A, None, A)) == INVALID
    assert call(Hi=16) == UNSUPPORTED
    assert call(H=32) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(n=need - 1) == WORKSPACE


def test_forward_shared_fp8_rejects_scales():
    lib = dsa.lib()
    bt = batch(B=1, L=8192)
    kc = cache()
    lat = (CacheT * 2)(cache(), cache())
    ptrs = (C.c_void_p * 2)(A, A)
    need = dsa.workspace_size(dsa.OP_FORWARD_SHARED, 1, 1, 8192, k=2048, n_layers=2)

    def call(scales):
        sc = None if scales is None else (C.c_float * 2)(*scales)
        return lib.dsa_forward_shared_fp8(C.byref(bt), A, A, 64, C.byref(kc), 2048, 0, 2, ptrs, 128, lat, sc, 0.04,
                                          ptrs, None, A, A, need, None)
    assert call(None) == INVALID
    assert call([1.0, 0.0]) == INVALID
    assert call([-1.0, 1.0]) == INVALID
    assert call([1.0, float("inf")]) == INVALID
    assert dsa.lib().dsa_last_error().decode().startswith("dsa_forward_shared_fp8")


def test_forward_shared_noalloc_rejects_before_hip():
    """The allocation-free group call checks its arguments as dsa_forward_shared does, and refuses
    a call whose workspace would not fit the library's scratch, all before any HIP call."""
    lib = dsa.lib()
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    assert "#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in text
    assert dsa.NOALLOC_SCRATCH_BYTES == 128 << 20
    kc = cache()
    lat = (CacheT * 4)(*[cache() for _ in range(4)])
    ptrs = (C.c_void_p * 4)(A, A, A, A)

    def call(bt, nl=4, share=0, Hi=64, H=128, scale=0.04, outs=ptrs):
        return lib.dsa_forward_shared_noalloc(C.byref(bt), A, A, Hi, C.byref(kc), 2048, share, nl, ptrs, H, lat,
                                              scale, outs, None, A, None)
    # 64 sequences x 8 query tokens at 128K keep 256 MiB of scores alone
    big = batch(B=64, Q=8, L=1 << 17)
    assert dsa.workspace_size(dsa.OP_FORWARD_SHARED, 64, 8, 1 << 17, n_layers=4) > dsa.NOALLOC_SCRATCH_BYTES
    assert call(big) == UNSUPPORTED
    assert "scratch" in dsa.lib().dsa_last_error().decode()
    ok = batch(B=1, L=8192)
    assert call(ok, share=2) == INVALID
    assert call(ok, nl=0) == INVALID
    assert call(ok, Hi=16) == UNSUPPORTED
    assert call(ok, H=32) == UNSUPPORTED
    assert call(ok, scale=-1.0) == INVALID
    assert call(ok, outs=(C.c_void_p * 4)(A, A, None, A)) == INVALID
    assert call(batch(B=0)) == INVALID
    assert dsa.lib().dsa_last_error().decode().startswith("dsa_forward_shared_noalloc")


def test_workspace_sizes_scale_with_batch():
    small = dsa.workspace_size(dsa.OP_TOPK, 1, 1, 8192)
    big = dsa.workspace_size(dsa.OP_TOPK, 32, 1, 131072)
    assert 0 < small < big
    assert dsa.workspace_size(dsa.OP_INDEX_SCORE, 32, 1, 131072) == 0
    shared = dsa.workspace_size(dsa.OP_FORWARD_SHARED, 32, 1, 131072)
    assert shared >= 32 * 131072 * 4 + big
    # layers that share an index set are launched together (up to 8), each with its own split
    # partials, and a launch splits its tokens over all its layers: 8 tokens x 1 layer take 16
    # splits; bf16 rows at 8 x 4 take 4 splits x 2 head groups, FP8 rows 8 splits x 1 group, and
    # the size covers the larger (8 x 4: 8 splits, 8 x 8: 4); 20 layers go as 8 + 8 + 4
    P = 8 * 128 * 512 * 4 + 2 * 8 * 128 * 4      # fp32 partial, lse and factor of one split of 8 tokens x 128 heads
    base = dsa.workspace_size(dsa.OP_FORWARD_SHARED, 8, 1, 1 << 20, n_layers=1) - \
        dsa.workspace_size(dsa.OP_SPARSE_MLA, 8, 1, 1 << 20)
    mla1 = dsa.workspace_size(dsa.OP_SPARSE_MLA, 8, 1, 1 << 20)
    assert mla1 == 16 * P
    for nl, splits in ((4, 8), (8, 4), (20, 4)):
        assert dsa.workspace_size(dsa.OP_FORWARD_SHARED, 8, 1, 1 << 20, n_layers=nl) - base == min(nl, 8) * splits * P


# ----------------------------------------------------------------------------- HiSparse swap-in
def hot(table=A, slot_page=A, slot_clock=A, page_clock=A, max_pages=64, n_slots=4096, page=16, row_bytes=1152):
    from sparse_attention_lightning_amd._binding import HotBufferT
    return HotBufferT(table, slot_page, slot_clock, page_clock, max_pages, n_slots, page, row_bytes)


def call_swap(B=2, idx=A, n_sets=1, k=2048, step=0, hb="default", host=A, dev=A, copied=None, ws=A, ws_bytes=1 << 30):
    hb = hot() if hb == "default" else hb
    lib = dsa.lib()
    return lib.dsa_hisparse_swap_in(B, idx, n_sets, k, step, C.byref(hb) if hb is not None else None, host, dev,
                                    copied, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(B=0), INVALID),
    (dict(n_sets=0), INVALID),
    (dict(k=0), UNSUPPORTED),
    (dict(k=2049), UNSUPPORTED),
    (dict(step=-1), INVALID),
    (dict(hb=None), INVALID),
    (dict(idx=None), INVALID),
    (dict(idx=A + 2), INVALID),
    (dict(hb=hot(table=None)), INVALID),
    (dict(hb=hot(slot_page=A + 1)), INVALID),
    (dict(hb=hot(slot_clock=None)), INVALID),
    (dict(hb=hot(page_clock=None)), INVALID),
    (dict(hb=hot(page=8)), UNSUPPORTED),
    (dict(hb=hot(page=24)), UNSUPPORTED),
    (dict(hb=hot(max_pages=0)), INVALID),
    (dict(hb=hot(row_bytes=1024)), UNSUPPORTED),
    (dict(hb=hot(row_bytes=0)), UNSUPPORTED),
    (dict(hb=hot(n_slots=2047)), UNSUPPORTED),             # one step's selected set must fit
    (dict(n_sets=3, hb=hot(n_slots=6143)), UNSUPPORTED),
    (dict(dev=None), INVALID),
    (dict(dev=A + 8), INVALID),
    (dict(host=None), INVALID),
    (dict(copied=A + 2), INVALID),
    (dict(ws=None), WORKSPACE),
    (dict(ws=A + 64), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE),
])
def test_swap_in_rejects_before_hip(case, expect):
    assert call_swap(**case) == expect


def test_swap_in_workspace_size():
    n1 = dsa.workspace_size(dsa.OP_HISPARSE_SWAP_IN, 8, 1, 1, k=2048)
    n2 = dsa.workspace_size(dsa.OP_HISPARSE_SWAP_IN, 8, 2, 1, k=2048)
    assert n1 >= 2 * 8 * 2048 * 4 and n2 > n1 and n1 % 256 == 0
