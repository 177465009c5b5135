"""The sharing hint derived from block tables (workloads/hints.py), on small
hand-made tables (CPU)."""
import numpy as np

from workloads import make_workload, share_prev_hint


def test_hint_counts_common_leading_blocks_within_both_contexts():
    bs = 4
    tables = np.array([[7, 8, 9, 10],
                       [7, 8, 9, 11],    # 3 common blocks with row 0
                       [7, 8, 5, 6],     # 2 common with row 1
                       [1, 2, 3, 4],     # none
                       [1, 2, 3, 4]], np.int32)
    lens = np.array([16, 16, 16, 16, 6], np.int32)
    h = share_prev_hint(tables, lens, bs)
    assert h.tolist() == [0, 12, 8, 0, 6]   # the last is capped by its own length


def test_hint_on_the_shared_prefix_workload():
    w = make_workload("prefix", num_prompts=3, samples=4, prefix_len=1032, max_suffix=200,
                      num_q_heads=8, num_kv_heads=2)
    h = share_prev_hint(w.block_tables, w.context_lens, w.block_size)
    # the samples of a prompt share its 64 whole blocks; the half-full 65th
    # block was copied on each sample's first write (all but the last)
    assert (h.reshape(3, 4)[:, 0] == 0).all()
    assert (h.reshape(3, 4)[:, 1:] == 1024).all()
