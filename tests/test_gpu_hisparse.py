"""GPU parity of the HiSparse swap-in (dsa_hisparse_swap_in) against the CPU oracle.

Every case runs several steps on one state and compares, after each step, the four state
tables bit for bit and the device pool byte for byte with oracle.swap_in on the same inputs.
The host pool is pinned host memory (torch pin_memory) unless a case says otherwise.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_lightning_amd as dsa
from oracle.hisparse import HotBufferState

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 576


def make(B, max_pages, n_slots, ps, seed, pinned=True, fp8=False):
    """Pools of bf16 rows (int16 bit patterns), or of E4M3 rows (uint8 codes) when fp8."""
    g = torch.Generator().manual_seed(seed)
    if fp8:
        host = torch.randint(0, 256, (B, max_pages, ps, D), dtype=torch.uint8, generator=g)
    else:
        host = torch.randint(-32768, 32767, (B, max_pages, ps, D), dtype=torch.int16, generator=g)
    if pinned:
        host = host.pin_memory()
    else:
        host = host.to(DEV)
    hb = dsa.HotBuffer(block_table=torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV),
                       slot_page=torch.full((B, n_slots), -1, dtype=torch.int32, device=DEV),
                       slot_clock=torch.full((B, n_slots), -1, dtype=torch.int32, device=DEV),
                       page_clock=torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV),
                       device_pool=torch.zeros((B * n_slots, ps, D), dtype=host.dtype, device=DEV), page_size=ps)
    st = HotBufferState.empty(B, max_pages, n_slots)
    dev_np = np.zeros((B * n_slots, ps, D), dtype=np.uint8 if fp8 else np.int16)
    return host, hb, st, dev_np


def compare(hb, st, dev_np, step):
    torch.cuda.synchronize()
    for name in ("block_table", "slot_page", "slot_clock", "page_clock"):
        got = getattr(hb, name).cpu().numpy()
        assert np.array_equal(got, getattr(st, name)), (name, step)
    assert np.array_equal(hb.device_pool.cpu().numpy(), dev_np), ("device_pool", step)


def random_sets(rng, B, n_sets, k, L, n_valid, prev=None, keep=0.0):
    """Selected positions, ascending then -1 padded like dsa_topk output; a fraction `keep` of
    each set is drawn from the previous step's set (consecutive decode steps overlap)."""
    idx = np.full((B, n_sets, k), -1, np.int32)
    for b in range(B):
        for j in range(n_sets):
            n = int(n_valid[b])
            take = []
            if prev is not None and keep > 0:
                old = prev[b, j][prev[b, j] >= 0]
                take = list(rng.choice(old, size=min(len(old), int(keep * n)), replace=False))
            pool = np.setdiff1d(np.arange(L), take)
            take += list(rng.choice(pool, size=n - len(take), replace=False))
            idx[b, j, :n] = np.sort(np.array(take, np.int32))
    return idx


@pytest.mark.parametrize("B,n_sets,k,ps,max_pages,n_slots,steps,keep,fp8", [
    (3, 1, 40, 16, 64, 48, 10, 0.5, False),       # pressure: 40 selected tokens on 48 slots
    (2, 2, 24, 16, 50, 48, 8, 0.7, False),        # two index sets per sequence, exactly full buffer
    (2, 1, 300, 32, 80, 320, 6, 0.8, False),      # pages of 32 tokens, several tokens per page
    (1, 1, 2048, 16, 1024, 2048, 4, 0.9, False),  # one decode row at k = 2048 on the smallest legal buffer
    (3, 1, 40, 16, 64, 48, 10, 0.5, True),        # E4M3 rows (576 bytes): the pressure case
    (2, 1, 300, 48, 80, 320, 6, 0.8, True),       # E4M3 rows, pages of 48 tokens
])
def test_swap_in_matches_oracle(B, n_sets, k, ps, max_pages, n_slots, steps, keep, fp8):
    host, hb, st, dev_np = make(B, max_pages, n_slots, ps, seed=k, fp8=fp8)
    host_np = host.numpy()
    rng = np.random.default_rng(k + B)
    L = max_pages * ps
    prev = None
    for step in range(steps):
        n_valid = rng.integers(max(1, k // 2), k + 1, size=B)
        idx = random_sets(rng, B, n_sets, k, L, n_valid, prev, keep)
        prev = idx
        copied = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        dsa.hisparse_swap_in(torch.from_numpy(idx).to(DEV), step, hb, host, copied=copied)
        copies = oracle.swap_in(st, idx, step, ps, host_np, dev_np)
        compare(hb, st, dev_np, step)
        assert copied.cpu().tolist() == [sum(1 for c in copies if c[0] == b) for b in range(B)], step


def test_step_clocks_across_every_radix_level():
    """The victim select is a radix select over slot clocks + 1, 8 bits per level from the top;
    levels above the step's top bit hold nothing and are skipped. Step numbers that grow through
    every byte exercise each level, with slot clocks spread over them (ties broken by slot)."""
    B, n_sets, k, ps, max_pages, n_slots = 2, 1, 40, 16, 64, 48
    host, hb, st, dev_np = make(B, max_pages, n_slots, ps, seed=21)
    host_np = host.numpy()
    rng = np.random.default_rng(22)
    L = max_pages * ps
    prev = None
    steps = [0, 1, 255, 256, 257, 65535, 65536, 70000, (1 << 24) - 1, 1 << 24, (1 << 24) + 3, (1 << 30) + 7]
    for step in steps:
        n_valid = rng.integers(k // 2, k + 1, size=B)
        idx = random_sets(rng, B, n_sets, k, L, n_valid, prev, 0.5)
        prev = idx
        dsa.hisparse_swap_in(torch.from_numpy(idx).to(DEV), step, hb, host)
        oracle.swap_in(st, idx, step, ps, host_np, dev_np)
        compare(hb, st, dev_np, step)


def test_repeated_positions_and_empty_sets():
    B, ps, max_pages, n_slots, k = 2, 16, 20, 32, 16
    host, hb, st, dev_np = make(B, max_pages, n_slots, ps, seed=5)
    host_np = host.numpy()
    sets = [
        [[0, 1, 2, 3, 17, 17, 300, -1] + [-1] * 8, [-1] * 16],        # several tokens of one page
        [[-1] * 16, [-1] * 16],                                       # nothing selected
        [[5, 40, 41, 42, 80, 319] + [-1] * 10, [319] * 16],
    ]
    for step, s in enumerate(sets):
        idx = np.array(s, np.int32).reshape(B, 1, k)
        dsa.hisparse_swap_in(torch.from_numpy(idx).to(DEV), 10 * step + 3, hb, host)
        oracle.swap_in(st, idx, 10 * step + 3, ps, host_np, dev_np)
        compare(hb, st, dev_np, step)


def test_host_pool_in_device_memory():
    B, ps, max_pages, n_slots, k = 2, 16, 40, 40, 32
    host, hb, st, dev_np = make(B, max_pages, n_slots, ps, seed=9, pinned=False)
    host_np = host.cpu().numpy()
    rng = np.random.default_rng(3)
    prev = None
    for step in range(5):
        idx = random_sets(rng, B, 1, k, max_pages * ps, [k, k // 2], prev, 0.5)
        prev = idx
        dsa.hisparse_swap_in(torch.from_numpy(idx).to(DEV), step, hb, host)
        oracle.swap_in(st, idx, step, ps, host_np, dev_np)
        compare(hb, st, dev_np, step)


def test_pool_types_must_match():
    _, hb, _, _ = make(1, 8, 16, 16, seed=1)
    host8 = torch.zeros((1, 8, 16, D), dtype=torch.uint8).pin_memory()
    with pytest.raises(ValueError):
        dsa.hisparse_swap_in(torch.zeros((1, 1, 4), dtype=torch.int32, device=DEV), 0, hb, host8)


def test_pageable_host_memory_is_refused():
    B, ps, max_pages, n_slots, k = 1, 16, 8, 16, 4
    _, hb, _, _ = make(B, max_pages, n_slots, ps, seed=1)
    pageable = torch.zeros((B, max_pages, ps, D), dtype=torch.int16)
    idx = torch.zeros((B, 1, k), dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.hisparse_swap_in(idx, 0, hb, pageable)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert (hb.block_table == -1).all()                  # nothing ran


def test_attention_over_the_hot_buffer_equals_the_whole_cache():
    """Top-k positions -> swap-in -> sparse MLA through the hot buffer's block table gives the
    bits that sparse MLA over the whole cache gives (the rows are the same, only their place
    in memory differs)."""
    B, Q, L, k, ps, H = 2, 1, 4096, 512, 16, 128
    max_pages, n_slots = L // ps, 512
    gen = torch.Generator().manual_seed(11)
    lat_full = (torch.randn((B, L, D), generator=gen) * 0.5).to(torch.bfloat16)
    host = lat_full.view(B, max_pages, ps, D).contiguous().pin_memory()
    q = (torch.randn((B, Q, H, D), generator=gen) * 0.5).to(torch.bfloat16).to(DEV)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    hb = dsa.HotBuffer(block_table=torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV),
                       slot_page=torch.full((B, n_slots), -1, dtype=torch.int32, device=DEV),
                       slot_clock=torch.full((B, n_slots), -1, dtype=torch.int32, device=DEV),
                       page_clock=torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV),
                       device_pool=torch.zeros((B * n_slots, ps, D), dtype=torch.bfloat16, device=DEV), page_size=ps)
    whole = dsa.Cache(lat_full.to(DEV), None, 0)
    rng = np.random.default_rng(2)
    scale = 1.0 / np.sqrt(D)
    for step in range(3):
        scores = torch.from_numpy(rng.standard_normal((B, Q, L)).astype(np.float32)).to(DEV)
        idx = dsa.topk(scores, lens, k)
        dsa.hisparse_swap_in(idx, step, hb, host)
        o1, l1 = dsa.sparse_mla_fwd(q, hb.latent_cache(), idx, k, scale, lens, L)
        o2, l2 = dsa.sparse_mla_fwd(q, whole, idx, k, scale, lens, L)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), step


def test_fp8_attention_over_the_hot_buffer_equals_the_whole_cache():
    """The same over an E4M3 latent cache: the hot buffer moves 576-byte rows and sparse MLA
    over its block table gives the bits of sparse MLA over the whole FP8 cache."""
    B, Q, L, k, ps, H = 2, 1, 4096, 512, 16, 64
    max_pages, n_slots = L // ps, 640
    gen = torch.Generator().manual_seed(12)
    codes = torch.randint(0, 256, (B, L, D), dtype=torch.uint8, generator=gen)
    codes[(codes & 0x7F) == 0x7F] = 0x38            # no NaN codes (0x38 = 1.0)
    host = codes.view(B, max_pages, ps, D).contiguous().pin_memory()
    q = (torch.randn((B, Q, H, D), generator=gen) * 0.5).to(torch.bfloat16).to(DEV)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    hb = dsa.HotBuffer(block_table=torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV),
                       slot_page=torch.full((B, n_slots), -1, dtype=torch.int32, device=DEV),
                       slot_clock=torch.full((B, n_slots), -1, dtype=torch.int32, device=DEV),
                       page_clock=torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV),
                       device_pool=torch.zeros((B * n_slots, ps, D), dtype=torch.uint8, device=DEV), page_size=ps)
    whole = dsa.Cache(codes.to(DEV), None, 0)
    rng = np.random.default_rng(4)
    scale = 1.0 / np.sqrt(D)
    for step in range(3):
        scores = torch.from_numpy(rng.standard_normal((B, Q, L)).astype(np.float32)).to(DEV)
        idx = dsa.topk(scores, lens, k)
        dsa.hisparse_swap_in(idx, step, hb, host)
        o1, l1 = dsa.sparse_mla_fwd(q, hb.latent_cache(), idx, k, scale, lens, L, latent_scale=0.02)
        o2, l2 = dsa.sparse_mla_fwd(q, whole, idx, k, scale, lens, L, latent_scale=0.02)
        torch.cuda.synchronize()
        assert torch.isfinite(o1).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), step
