"""CPU oracle of the DSA hot path: plain numpy in float64 (dsa.py, hisparse.py, csa.py) and the
same DSA steps as plain C (dsa_ref.c through cref.py), tied to the numpy form by tests.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU baseline
may import this package. The GPU library and its Python binding never do.

Pinned functions and what pins them are listed at the top of tests/test_oracle.py.
"""
from .dsa import (E4M3, Cache, attention_flops, bf16_to_f64, dense_mla_causal, e4m3_to_f64,  # noqa: F401
                  forward_shared, index_scores, index_scores_batch, indexer_flops, latent_values, query_positions,
                  select_topk, sparse_mla, sparse_mla_batch, sparse_mla_one, sparse_to_dense_ratio,
                  topk_batch)
from .hisparse import HotBufferState, selected_pages, swap_in  # noqa: F401,E402
from . import csa  # noqa: F401,E402
