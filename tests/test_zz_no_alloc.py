"""The allocation-free IndexShare group call (dsa_forward_shared_noalloc) against the same call
with a caller workspace (dsa_forward_shared), through the C ABI.

Both run the same kernels in the same order on the same inputs, so their results must be
bitwise equal. Two calls follow each other on the library's one scratch array: the second,
smaller one must not depend on what the first left there. Collected last: a failure here hides
no other test."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
dsa = pytest.importorskip("sparse_attention_lightning_amd")
DEV = "cuda"


def both_calls(wl, seed=0, share_first=False):
    g = synth.generate(wl, seed=seed, device=DEV)
    keys = dsa.Cache(g.keys, g.key_table, wl.page_size)
    lats = [dsa.Cache(g.latent[l], g.latent_table[l], wl.page_size) for l in range(wl.n_layers)]
    n_sets = 1 if share_first else wl.Q
    idx_ref, res_ref = dsa.forward_shared(g.q_idx, g.w, keys, wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax,
                                          share_first_query=share_first)
    # outputs start as garbage, so that an unwritten entry cannot pass
    outs = [torch.full((wl.B, wl.Q, wl.H, 512), float("nan"), device=DEV) for _ in range(wl.n_layers)]
    lses = [torch.full((wl.B, wl.Q, wl.H), float("nan"), device=DEV) for _ in range(wl.n_layers)]
    idx = torch.full((wl.B, n_sets, wl.k), -7, dtype=torch.int32, device=DEV)
    before = torch.cuda.memory_allocated()
    dsa.forward_shared_noalloc(g.q_idx, g.w, keys, wl.k, g.q_mla, lats, wl.scale, g.seq_lens, wl.lmax, outs=outs,
                               lses=lses, idx=idx, share_first_query=share_first)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(idx, idx_ref)
    for layer in range(wl.n_layers):
        assert torch.equal(outs[layer], res_ref[layer][0]), layer
        assert torch.equal(lses[layer], res_ref[layer][1]), layer
    return idx


def test_noalloc_group_call_equals_workspace_call_then_a_smaller_one():
    # the decode batch at its full size (83 MiB of scratch), then a smaller two-layer group
    big = synth.WORKLOADS["decode_b32_128k_paged"]
    print("noalloc: decode B=32 L=131072", flush=True)
    both_calls(big)
    small = synth.small("indexshare_b8_1m_4layers", B=2, L=6000, L_max=6016, seq_lens=(6000, 4444), n_layers=2)
    print("noalloc: B=2 L=6000, 2 layers", flush=True)
    both_calls(small, seed=3)


def test_noalloc_draft_form_twice():
    wl = synth.small("verify_b64_q8_32k_draftshare", B=6, L=9000, L_max=9024)
    both_calls(wl, share_first=True)
    both_calls(synth.small("verify_b64_q8_32k_draftshare", B=3, L=3000, L_max=3008), seed=1, share_first=True)
