"""The index-score oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/index_scores.py and runs the pin suite
(tests/test_oracle_index.py) against that copy in a subprocess. The suite must fail for
every variant, and pass for the unmodified source.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "index_scores.py")

MUTANTS = {
    "scale_dropped": ("s = scale * (keys @ qf[t, h])", "s = (keys @ qf[t, h])"),
    "causal_length_is_position": (
        "c = max(int(seq_lens[req]) - q + (t - req * q) + 1, 0)",
        "c = max(int(seq_lens[req]) - q + (t - req * q), 0)"),
    "row_request_interleaved": ("req = t // q", "req = t % B"),
    "whole_last_block": ("n = min(BLOCK_TOKENS, c - BLOCK_TOKENS * b)", "n = BLOCK_TOKENS"),
    "lse_without_shift": ("return float(m + np.log(np.exp(s - m).sum()))",
                          "return float(np.log(np.exp(s).sum()))"),
    "mean_for_lse": ("return float(m + np.log(np.exp(s - m).sum()))",
                     "return float(s.mean())"),
    "block_table_ignored": ("keys = block_keys(k_cache, int(block_table[req, b]), h, n, k_scale)",
                            "keys = block_keys(k_cache, b, h, n, k_scale)"),
    "slot_and_dim_group_swapped": (
        "k_cache[page[:, None], h, d[None, :] // 8, slot[:, None], d[None, :] % 8]",
        "k_cache[page[:, None], h, slot[:, None], d[None, :] // 8, d[None, :] % 8]"),
    "pages_of_block_not_scaled": ("page = phys * PAGES_PER_BLOCK + tok // PAGE_TOKENS",
                                  "page = phys + tok // PAGE_TOKENS"),
    "invalid_block_clamped": (
        "    if phys < 0 or (phys + 1) * PAGES_PER_BLOCK > P:\n        return np.zeros((n, D))\n",
        "    phys = min(max(phys, 0), P // PAGES_PER_BLOCK - 1)\n"),
    "max_blocks_ignored": ("nvp = min(-(-c // BLOCK_TOKENS), max_blocks, M)",
                           "nvp = min(-(-c // BLOCK_TOKENS), M)"),
    "another_heads_keys": ("keys = block_keys(k_cache, int(block_table[req, b]), h, n, k_scale)",
                           "keys = block_keys(k_cache, int(block_table[req, b]), (h + 1) % H, n, k_scale)"),
    "e4m3_exponent_bias_8": ("(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    "e4m3_subnormal_as_normal": ("np.where(e == 0, m / 8.0 * 2.0 ** -6,", "np.where(e < 0, m / 8.0 * 2.0 ** -6,"),
    "fp8_scale_ignored": ("return e4m3_value(codes) * k_scale[page, h, slot].astype(np.float64)[:, None]",
                          "return e4m3_value(codes)"),
    "fp8_scale_of_first_token": ("return e4m3_value(codes) * k_scale[page, h, slot].astype(np.float64)[:, None]",
                                 "return e4m3_value(codes) * k_scale[page, h, 0].astype(np.float64)[:, None]"),
    "fp8_dims_in_groups_of_8": ("codes = k_cache[page[:, None], h, d[None, :] // 16, slot[:, None], d[None, :] % 16]",
                                "codes = k_cache[page[:, None], h, (d[None, :] // 8) % 8, slot[:, None], d[None, :] % 8 + 8 * (d[None, :] // 64)]"),
}


def _run_suite(src_path):
    env = dict(os.environ, KVBT_INDEX_ORACLE_SRC=src_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_index.py")],
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
