"""Pins of the hot-buffer oracle (oracle/hisparse.py) against things other than itself.

What pins swap_in:
  - a trace worked out by hand from the page's three steps (tests/golden/hisparse_trace.json);
  - the textbook LRU page-replacement example: the reference string 7 0 1 2 0 3 0 4 2 3 0 3 2
    1 2 0 1 7 0 1 with 3 frames takes 12 faults under LRU (one page selected per step);
  - an independent LRU cache (collections.OrderedDict, least recent first) on random
    one-page-per-step traces: the same faults and the same resident pages after every step;
  - the defining LRU property on random many-page steps: every victim is at least as old as
    every unneeded slot that stays;
  - invariants after every step: each selected page is resident, the page table and the
    slot table are inverse maps, the device buffer holds the host bytes of every resident
    page, and pages only move on a miss;
  - with room for every page, the copies equal the distinct pages ever selected.
"""
import json
import os
from collections import OrderedDict

import numpy as np
import pytest

import oracle
from oracle.hisparse import HotBufferState

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hisparse_trace.json")


def pools(B, max_pages, n_slots, page_size, D=4, seed=0):
    rng = np.random.default_rng(seed)
    host = rng.integers(0, 1 << 16, size=(B, max_pages, page_size, D), dtype=np.uint16)
    dev = np.zeros((B * n_slots, page_size, D), dtype=np.uint16)
    return host, dev


def check_invariants(st, idx, page_size, host, dev):
    B, n_slots = st.slot_page.shape
    for b in range(B):
        for p in oracle.selected_pages(idx[b], page_size):
            assert st.block_table[b, p] >= 0, (b, p)
        for p in np.nonzero(st.block_table[b] >= 0)[0]:
            s = st.block_table[b, p] - b * n_slots
            assert 0 <= s < n_slots and st.slot_page[b, s] == p
            assert np.array_equal(dev[b * n_slots + s], host[b, p])
        for s in np.nonzero(st.slot_page[b] >= 0)[0]:
            assert st.block_table[b, st.slot_page[b, s]] == b * n_slots + s


def test_hand_worked_trace():
    g = json.load(open(GOLDEN))
    ps, n_slots, max_pages = g["page_size"], g["n_slots"], g["max_pages"]
    st = HotBufferState.empty(1, max_pages, n_slots)
    host, dev = pools(1, max_pages, n_slots, ps)
    for s in g["steps"]:
        idx = np.array([[s["positions"]]], dtype=np.int32)
        copies = oracle.swap_in(st, idx, s["step"], ps, host, dev)
        e = s["expect"]
        assert st.block_table[0].tolist() == e["block_table"], s["step"]
        assert st.slot_page[0].tolist() == e["slot_page"], s["step"]
        assert st.slot_clock[0].tolist() == e["slot_clock"], s["step"]
        assert len(copies) == e["misses"], s["step"]
        check_invariants(st, idx, ps, host, dev)
    assert st.page_clock[0].tolist() == g["final_page_clock"]


def run_one_page_per_step(refs, frames, page_size=16):
    max_pages = max(refs) + 1
    st = HotBufferState.empty(1, max_pages, frames)
    host, dev = pools(1, max_pages, frames, page_size)
    faults, resident = 0, []
    for t, p in enumerate(refs):
        idx = np.array([[[p * page_size + (t % page_size)]]], dtype=np.int32)
        faults += len(oracle.swap_in(st, idx, t, page_size, host, dev))
        resident.append(set(np.nonzero(st.block_table[0] >= 0)[0].tolist()))
    return faults, resident


def test_textbook_lru_reference_string():
    refs = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]
    faults, _ = run_one_page_per_step(refs, 3)
    assert faults == 12


def lru_cache_trace(refs, frames):
    cache, faults, resident = OrderedDict(), 0, []
    for p in refs:
        if p in cache:
            cache.move_to_end(p)
        else:
            faults += 1
            if len(cache) == frames:
                cache.popitem(last=False)
            cache[p] = True
        resident.append(set(cache))
    return faults, resident


@pytest.mark.parametrize("seed", range(6))
def test_one_page_per_step_matches_an_lru_cache(seed):
    rng = np.random.default_rng(seed)
    frames = int(rng.integers(2, 9))
    refs = rng.integers(0, frames * 3, size=200).tolist()
    assert run_one_page_per_step(refs, frames) == lru_cache_trace(refs, frames)


@pytest.mark.parametrize("seed", range(4))
def test_victims_are_least_recently_used(seed):
    rng = np.random.default_rng(100 + seed)
    B, ps, max_pages, n_slots, k = 3, 16, 40, 12, 6
    st = HotBufferState.empty(B, max_pages, n_slots)
    host, dev = pools(B, max_pages, n_slots, ps, seed=seed)
    for t in range(30):
        idx = np.full((B, 1, k), -1, np.int32)
        for b in range(B):
            n = int(rng.integers(1, k + 1))
            idx[b, 0, :n] = np.sort(rng.choice(max_pages * ps, size=n, replace=False))
        before = st.copy()
        copies = oracle.swap_in(st, idx, t, ps, host, dev)
        for b in range(B):
            need = set(oracle.selected_pages(idx[b], ps).tolist())
            victims = {s for (bb, _, s) in copies if bb == b}
            stay = [s for s in range(n_slots) if s not in victims and before.slot_page[b, s] not in need]
            for v in victims:
                assert before.slot_page[b, v] not in need or before.slot_page[b, v] < 0
                for s in stay:      # every victim precedes every unneeded slot that stays in (clock, slot)
                    assert (before.slot_clock[b, v], v) < (before.slot_clock[b, s], s)
            # pages only move on a miss: every resident page not copied keeps its slot
            for p in np.nonzero(before.block_table[b] >= 0)[0]:
                if st.block_table[b, p] >= 0:
                    assert st.block_table[b, p] == before.block_table[b, p]
        check_invariants(st, idx, ps, host, dev)


def test_room_for_every_page_copies_each_page_once():
    rng = np.random.default_rng(7)
    B, ps, max_pages, k = 2, 16, 20, 8
    st = HotBufferState.empty(B, max_pages, max_pages)
    host, dev = pools(B, max_pages, max_pages, ps)
    seen = [set(), set()]
    n_copies = 0
    for t in range(25):
        idx = rng.integers(-1, max_pages * ps, size=(B, 2, k)).astype(np.int32)
        n_copies += len(oracle.swap_in(st, idx, t, ps, host, dev))
        for b in range(B):
            seen[b] |= set(oracle.selected_pages(idx[b], ps).tolist())
        check_invariants(st, idx, ps, host, dev)
    assert n_copies == len(seen[0]) + len(seen[1])


def test_a_selected_set_larger_than_the_buffer_is_refused():
    st = HotBufferState.empty(1, 8, 2)
    host, dev = pools(1, 8, 2, 16)
    with pytest.raises(ValueError):
        oracle.swap_in(st, np.array([[[0, 16, 32]]], np.int32), 0, 16, host, dev)
