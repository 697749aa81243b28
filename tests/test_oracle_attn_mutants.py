"""The sparse-attention oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/sparse_attn.py (a dropped factor, a
wrong index or grouping, a missing mask) and runs the pin suite
(tests/test_oracle_attn.py) against that copy in a subprocess. The suite must fail for
every variant, and pass for the unmodified source.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "sparse_attn.py")

MUTANTS = {
    "scale_dropped": ("s = scale * (keys @ qf[t, j])", "s = (keys @ qf[t, j])"),
    "interleaved_head_groups": ("for j in range(h * G, (h + 1) * G):",
                                "for j in range(h, HG, H):"),
    "single_token_rows_skipped": ("if c == 0:", "if c <= 1:"),
    "whole_last_page": ("i = np.arange(c)", "i = np.arange(-(-c // 16) * 16)"),
    "no_max_shift": ("e = np.exp(s - s.max())", "e = np.exp(s)"),
    "bad_keys_read_page_0": ("keys[~ok] = 0.0", "pass"),
    "bad_values_read_page_0": ("vals[~ok] = 0.0", "pass"),
    "key_slot_and_dim_group_swapped": (
        "k_cache[pg[:, None], h, d[None, :] // 8, slots[:, None], d[None, :] % 8]",
        "k_cache[pg[:, None], h, slots[:, None], d[None, :] // 8, d[None, :] % 8]"),
    "page_of_next_token": ("pages = table[t, h, i // TOKENS_PER_PAGE]",
                           "pages = table[t, h, np.minimum(i + 1, c - 1) // TOKENS_PER_PAGE]"),
    "ctx_not_clamped_to_width": ("c = min(max(int(ctx[t, h]), 0), TOKENS_PER_PAGE * W)",
                                 "c = max(int(ctx[t, h]), 0) % (TOKENS_PER_PAGE * W + 1)"),
    "uniform_weights": ("w = e / e.sum()", "w = np.ones_like(e) / e.size"),
    "cache_of_another_kv_head": ("i % TOKENS_PER_PAGE, h)",
                                 "i % TOKENS_PER_PAGE, (h + 1) % H)"),
}


def _run_suite(src_path):
    env = dict(os.environ, KVBT_ATTN_ORACLE_SRC=src_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_attn.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_unmodified_source_passes(tmp_path):
    p = tmp_path / "original.py"
    with open(SRC) as f:
        p.write_text(f.read())
    code, out = _run_suite(str(p))
    assert code == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation anchor not unique: %s" % name
    p = tmp_path / ("%s.py" % name)
    p.write_text(text.replace(old, new))
    code, out = _run_suite(str(p))
    assert code != 0, "pins did not catch mutant %s:\n%s" % (name, out)
