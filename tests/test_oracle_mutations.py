"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies the oracle, the input generator and the pin tests into a
temporary directory, plants one mistake in the copied oracle (a dropped scale,
a wrong index, a transposed slice, an off-by-one limit, a flipped sign, a
missing write, a missing snapshot, a missing rescale), and runs the pins there
in a fresh interpreter. Every planted mistake must make some pin fail. The
repository's own oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (text in oracle/paged_attention.py, replacement)
MUTATIONS = {
    "drop_scale": ("s = sigma * (K @ qv)\n    m = s.max()", "s = (K @ qv)\n    m = s.max()"),
    "v_slot_slice_swapped": ("v = vview[blk, g, off // 4, :, off % 4]",
                             "v = vview[blk, g, off % 4, :, off // 4]"),
    "k_slice_transposed": ("k = kview[blk, g, :, off, :].reshape(n, head_dim)",
                           "k = kview[blk, g, :, off, :].transpose(0, 2, 1).reshape(n, head_dim)"),
    "gqa_strided_heads": ("for h in range(g * G, (g + 1) * G):\n                out[b, h]",
                          "for h in [x for x in range(Hq) if x % num_kv_heads == g]:\n"
                          "                out[b, h]"),
    "causal_off_by_one": ("a = n - L + i\n                for h in range(g * G, (g + 1) * G):\n"
                          "                    out[",
                          "a = n - L + i - 1\n                for h in range(g * G, (g + 1) * G):\n"
                          "                    out["),
    "slot_offset_wrong": ("off = t % block_size", "off = (t // block_size) % block_size"),
    "softmax_sign": ("w = np.exp(s - m)\n    return", "w = np.exp(m - s)\n    return"),
    "append_drops_v": ("        vview[blk, :, off // 4, :, off % 4] = v_new[i]\n", "        pass\n"),
    "copy_without_snapshot": ("out[int(dst)] = snap[int(src)]", "out[int(dst)] = out[int(src)]"),
    "merge_without_rescale": ("l = sum(p[1] * np.exp(p[0] - M) for p in finite)",
                              "l = sum(p[1] for p in finite)"),
    "moments_unnormalised": ("    w = w / w.sum()\n    o = w @ V", "    o = w @ V / w.sum()"),
    "moments_deviation_signed": ("w @ np.abs(V - o)", "np.abs(w @ (V - o))"),
}

# name -> (text in oracle/scheduler.py, replacement); caught by test_sched_oracle.py
SCHED_MUTATIONS = {
    "copy_on_write_skipped": ("elif self.ref[table[j]] > 1:", "elif False:"),
    "free_list_first_in_first_out": ("b = self.free.pop()", "b = self.free.pop(0)"),
    "evicts_the_oldest": ("self._evict(self.running[-1], plan)",
                          "self._evict(self.running[0], plan)"),
    "finished_blocks_kept": ("self._release_table(s.table)\n                        s.released",
                             "s.released"),
    "static_batch_ends_at_first_finish": ("if self.running and all(self.reqs[rid].state",
                                          "if self.running and any(self.reqs[rid].state"),
    "chunk_overruns_budget": ("L = min(r.prompt - r.prefilled, cfg.max_chunk, budget)\n        if",
                              "L = min(r.prompt - r.prefilled, cfg.max_chunk, budget + 1)\n        if"),
    "fork_without_reference": ("                    for b in r.table:\n                        self.ref[b] += 1\n",
                               ""),
    "prefill_token_not_counted": ("self.gen = 1 ", "self.gen = 0 "),
    "swap_in_forgets_sharing": ("self.ref[b] = sum(q.table.count(b) for q in live)", "pass"),
    "swap_out_skips_host_order": ("where[b] = self.host_free.pop()", "where[b] = self.host_free.pop(0)"),
    "cache_evicts_newest": ("key = next(k for k in self.lru if", "key = next(k for k in self.lru[::-1] if"),
    "cache_hit_past_a_miss": (
        "        while (len(hits) + 1) * bs <= limit and (r.prefix_id, len(hits)) in self.cache:\n"
        "            hits.append(self.cache[(r.prefix_id, len(hits))])\n",
        "        hits = [self.cache[(r.prefix_id, j)] for j in range(limit // bs)\n"
        "                if (r.prefix_id, j) in self.cache]\n"),
    "cache_takes_partial_block": ("if (j + 1) * bs <= r.prefix_len and key not in self.cache:",
                                  "if j * bs < r.prefix_len and key not in self.cache:"),
}


def _copy_tree(dst):
    for d in ("oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in ("__init__.py", "conftest.py", "pool_writer.py", "test_oracle_pins.py",
              "test_sched_oracle.py"):
        src = os.path.join(ROOT, "tests", f)
        if os.path.exists(src):
            shutil.copy(src, os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    _copy_tree(str(tmp_path))
    path = os.path.join(str(tmp_path), "oracle", "paged_attention.py")
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, f"the oracle no longer contains the text {name} mutates"
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=str(tmp_path), capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 1, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(SCHED_MUTATIONS))
def test_planted_scheduler_mistake_is_caught(name, tmp_path):
    old, new = SCHED_MUTATIONS[name]
    _copy_tree(str(tmp_path))
    path = os.path.join(str(tmp_path), "oracle", "scheduler.py")
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, f"the oracle no longer contains the text {name} mutates"
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_sched_oracle.py", "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu", "--timeout", "120"],
                       cwd=str(tmp_path), capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 1, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"
