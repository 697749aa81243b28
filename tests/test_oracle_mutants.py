"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a dropped term, a
wrong sign or index, a reversed comparison), builds it with gcc into a temporary
directory, and runs the pin suite (tests/test_oracle.py) against that build in a
subprocess. The suite must fail for every variant, and pass for the unmodified
source.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "kvbt_oracle.c")

MUTANTS = {
    "signed_zero_equal": (
        "if (x_neg != y_neg) return x_neg ? -1 : 1;      /* clause (b): -0 < +0 */",
        "if (x_neg != y_neg) return 0;"),
    "nan_lowest": (
        "if (x_nan && !y_nan) return x_neg ? -1 : 1;",
        "if (x_nan && !y_nan) return -1;"),
    "nan_payload_sign": ("return x_neg ? -c : c;", "return c;"),
    "tie_to_higher_id": (
        "return (a->block > b->block) - (a->block < b->block);",
        "return (a->block < b->block) - (a->block > b->block);"),
    "local_window_off_by_one": ("(b >= nvp - num_local)", "(b > nvp - num_local)"),
    "init_window_dropped": ("(b < num_init) || ", ""),
    "forced_sorted_by_score": ("    if (!a->forced) {\n", "    {\n"),
    "ascending_scores": ("if (c != 0) return -c;", "if (c != 0) return c;"),
    "pad_with_zero": ("? buf[r].block : -1;", "? buf[r].block : 0;"),
    "partial_block_index": ("c - (int64_t)TOKENS_PER_BLOCK * b;",
                            "c - (int64_t)TOKENS_PER_BLOCK * (b + 1) + 1;"),
    "page_id_without_scale": ("phys * (uint32_t)PAGES_PER_BLOCK + (uint32_t)j",
                              "phys + (uint32_t)j"),
    "pages_floor": ("cdiv64(t_b, TOKENS_PER_PAGE)", "(t_b / TOKENS_PER_PAGE)"),
    "ctx_counts_pages": ("ctx += t_b;", "ctx += pages * TOKENS_PER_PAGE;"),
    "decode_position": ("pos = (int64_t)seq_lens[req] - q + local_q;",
                        "pos = (int64_t)seq_lens[req] - 1 + local_q;"),
    "table_in_selector_order": (
        "qsort(kept, (size_t)n, sizeof(int32_t), cmp_i32);", ""),
    "no_dedupe": ("if (!seen) kept[n++] = b;", "kept[n++] = (seen, b);"),
    "causal_count_floor": (
        "const int64_t nvp = clamp64(cdiv64(c, TOKENS_PER_BLOCK), 0, max_k_tiles);",
        "const int64_t nvp = clamp64(c / TOKENS_PER_BLOCK, 0, max_k_tiles);"),
    "block_limit_ignores_max_blocks": (
        "const int64_t limit = nvp < max_blocks ? nvp : max_blocks;",
        "const int64_t limit = nvp;"),
}


def _run_suite(lib_path):
    env = dict(os.environ, KVBT_ORACLE_LIB=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def _build(tmp_path, text, name):
    import oracle
    src = tmp_path / ("%s.c" % name)
    src.write_text(text)
    return oracle.build(force=True, src=str(src), out=str(tmp_path / ("lib%s.so" % name)))


def test_unmodified_source_passes(tmp_path):
    with open(SRC) as f:
        text = f.read()
    code, out = _run_suite(_build(tmp_path, text, "original"))
    assert code == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation anchor not unique: %s" % name
    code, out = _run_suite(_build(tmp_path, text.replace(old, new), name))
    assert code != 0, "pins did not catch mutant %s:\n%s" % (name, out)
