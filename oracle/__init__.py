"""CPU oracle for the causal lightning indexer and its group-shared variant.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything under this directory: only the test-suite, the smoke check
in the repository's entry module and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library and does not import it.

Everything here is plain NumPy in float64, written for a reader to check by
eye against the definitions it cites.  See ``indexer.py`` for the method and
``formats.py`` for the independent bf16 / OCP-e4m3fn decoders.
"""

from .formats import (bf16_bits_to_f64, e4m3fn_bits_to_f64, f64_to_bf16_bits_rne,
                      real_values)
from .indexer import (causal_scores, dense_scores, select_topk, dense_topk, proxy_means,
                      round_proxy, proxy_limits, proxy_scores, proxy_candidates,
                      refine_topk, reuse_topk, grouped_reference, recall,
                      group_bounds, block_means, block_limits, block_route, block_reference,
                      ivf_store, ivf_assign, ivf_update, ivf_build, ivf_visible_end,
                      ivf_route, ivf_reference)

__all__ = [
    "bf16_bits_to_f64", "e4m3fn_bits_to_f64", "f64_to_bf16_bits_rne", "real_values",
    "causal_scores", "dense_scores", "select_topk", "dense_topk", "proxy_means", "round_proxy",
    "proxy_limits", "proxy_scores", "proxy_candidates", "refine_topk",
    "reuse_topk", "grouped_reference", "recall", "group_bounds",
    "block_means", "block_limits", "block_route", "block_reference",
    "ivf_store", "ivf_assign", "ivf_update", "ivf_build", "ivf_visible_end",
    "ivf_route", "ivf_reference",
]
