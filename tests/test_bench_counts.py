"""The bench's own FLOP counts (CPU only): its closed-form and numpy pair counts agree with the
oracle's masks, so that `value` and `roofline.achieved` divide the right amount of work."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402


def test_allowed_pairs_match_the_oracle_masks():
    for n, causal, window in [(1, False, (-1, -1)), (37, True, (-1, -1)), (100, False, (5, 3)),
                              (64, True, (10, 0)), (129, False, (-1, 7))]:
        ref = int(oracle.cross_allowed_mask(n, n, causal, window).sum())
        assert bench.allowed_pairs(n, causal, window) == ref, (n, causal, window)


def test_block_workload_pairs_match_the_oracle_masks():
    """A smaller block workload of the same kind (queries at the end of a longer key range)."""
    w = W.BlockWorkload("t", 2, 3, 192, 448, 64, "bf16", seed=4)
    allowed = oracle.cross_allowed_mask(w.n_q, w.n_k, True)
    blocks = W.draw_blocks(w.H, w.n_q, w.n_k, 0.5, w.seed)
    kpm = W.key_padding_case(w.B, w.n_k, w.seed + 7, density=0.3)
    assert bench.block_workload_pairs(w) == w.B * w.H * int(allowed.sum())
    ref = sum(int((allowed & oracle.block_allowed(w.n_q, w.n_k, blocks[h])).sum())
              for h in range(w.H)) * w.B
    assert bench.block_workload_pairs(w, blocks) == ref
    ref = sum(int((allowed & oracle.block_allowed(w.n_q, w.n_k, blocks[h]) & ~kpm[b][None, :]).sum())
              for b in range(w.B) for h in range(w.H))
    assert bench.block_workload_pairs(w, blocks, kpm) == ref
    ref = w.H * sum(int((allowed & ~kpm[b][None, :]).sum()) for b in range(w.B))
    assert bench.block_workload_pairs(w, None, kpm) == ref
