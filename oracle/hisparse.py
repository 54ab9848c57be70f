"""CPU oracle of the HiSparse hot buffer: top-k driven swap-in of latent pages.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline may import or run this module. The GPU library never calls it, and it shares
no code, tables or constants with the GPU library.

What it follows ("GLM-5.2 inference deployment" page, section on HiSparse's GPU <-> CPU KV
swap path): the full KV cache lives in pinned host memory and the GPU keeps a buffer of
hot slots, one slot per KV page. After the indexer and selector of a step have produced
the top-k positions, the swap-in runs three steps:
  1. miss detection: the pages of the selected positions that the device buffer does not
     hold;
  2. LRU eviction: victims are taken from the device buffer, least recently used first;
  3. H2D pull: the page table is updated and the missing entries are copied from host
     memory into the freed slots.
The page moves the latent rows that attention reads (not up-projected keys and values).

Readings where the page is silent (listed with their reasons in the design notes):
  - every sequence owns its own buffer of n_slots slots; physical page b * n_slots + s is
    slot s of sequence b;
  - "recently used" counts steps: a slot's clock is the last step whose selected set held
    its page (a hit or the step that pulled it in); a slot never used has clock -1;
  - a slot whose page the current step selected is never a victim, so the buffer must hold
    the step's whole selected set (n_slots >= the positions selected per sequence);
  - among equally old slots the lower slot index goes first; the page fixes which slots are
    evicted, not which freed slot each missing page takes: the i-th missing page in ascending
    page order takes the i-th victim in ascending slot order;
  - the state also records, per logical page, the last step that selected it (page clock).

State of one batch (all int32, -1 = none), as returned and consumed by swap_in():
  block_table [B][max_pages]: physical page of each logical page, or -1 when not resident
  slot_page   [B][n_slots]:   logical page held by each slot, or -1
  slot_clock  [B][n_slots]:   last step that used the slot, or -1
  page_clock  [B][max_pages]: last step whose selected set held the page, or -1
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class HotBufferState:
    block_table: np.ndarray
    slot_page: np.ndarray
    slot_clock: np.ndarray
    page_clock: np.ndarray

    @staticmethod
    def empty(B: int, max_pages: int, n_slots: int) -> "HotBufferState":
        return HotBufferState(np.full((B, max_pages), -1, np.int32), np.full((B, n_slots), -1, np.int32),
                              np.full((B, n_slots), -1, np.int32), np.full((B, max_pages), -1, np.int32))

    def copy(self) -> "HotBufferState":
        return HotBufferState(self.block_table.copy(), self.slot_page.copy(), self.slot_clock.copy(),
                              self.page_clock.copy())


def selected_pages(idx_b: np.ndarray, page_size: int) -> np.ndarray:
    """Distinct logical pages of the valid (>= 0) positions in one sequence's index sets."""
    pos = np.asarray(idx_b).reshape(-1)
    pos = pos[pos >= 0]
    return np.unique(pos // page_size)


def swap_in(state: HotBufferState, idx: np.ndarray, step: int, page_size: int, host_pool: np.ndarray,
            device_pool: np.ndarray):
    """One swap-in step, in place on `state` and `device_pool`.

    idx [B][sets][k] int32 selected positions (-1 padded); host_pool [B][max_pages][page_size][D];
    device_pool [B * n_slots][page_size][D]. Returns the list of (b, page, slot) copies made,
    in the order the pages were paired with their slots."""
    B, n_slots = state.slot_page.shape
    copies = []
    for b in range(B):
        need = selected_pages(idx[b], page_size)
        if len(need) > n_slots:
            raise ValueError(f"sequence {b}: {len(need)} selected pages exceed {n_slots} slots")
        # 1. miss detection (hits refresh their slot's clock)
        missing = []
        for p in need:
            state.page_clock[b, p] = step
            phys = state.block_table[b, p]
            if phys >= 0:
                state.slot_clock[b, phys - b * n_slots] = step
            else:
                missing.append(int(p))
        # 2. LRU eviction among the slots this step does not use
        free = [s for s in range(n_slots) if state.slot_clock[b, s] < step]
        free.sort(key=lambda s: (int(state.slot_clock[b, s]), s))
        victims = sorted(free[:len(missing)])
        # 3. page-table update and H2D pull
        for p, s in zip(missing, victims):
            old = state.slot_page[b, s]
            if old >= 0:
                state.block_table[b, old] = -1
            state.block_table[b, p] = b * n_slots + s
            state.slot_page[b, s] = p
            state.slot_clock[b, s] = step
            device_pool[b * n_slots + s] = host_pool[b, p]
            copies.append((b, p, s))
    return copies
