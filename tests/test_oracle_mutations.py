"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (no GPU).

Each mutant is a textual edit of ``oracle/oracle.c`` (a swapped index, a
dropped term, a transposed operand, a wrong group rule), compiled with gcc
into a temporary library and run against ``oracle_pins`` in a child process.
A mutant passes the test when the pins FAIL on it (or it crashes).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, old text, new text, which occurrence)
MUTANTS = [
    ("seq_offset_t_h_swapped", "((r * Bl + bl) * St + t) * H + h) * d + e",
     "((r * Bl + bl) * H + h) * St + t) * d + e", 0),
    ("seq_offset_drops_batch_stride", "(((r * Bl + bl) * St + t)", "(((r + bl) * St + t)", 0),
    ("head_major_s_hl_swapped", "return (((r * Bl + bl) * Hl + hl) * S + s) * d + e;",
     "return (((r * Bl + bl) * S + s) * Hl + hl) * d + e;", 0),
    ("token_major_s_hl_swapped", "return (((r * Bl + bl) * S + s) * Hl + hl) * d + e;",
     "return (((r * Bl + bl) * Hl + hl) * S + s) * d + e;", 0),
    ("s2h_group_member_swapped", "const int64_t g = r / P, j = r % P;",
     "const int64_t g = r % P, j = r / P;", 0),
    ("h2s_group_member_swapped", "const int64_t g = r / P, j = r % P;",
     "const int64_t g = r % P, j = r / P;", 1),
    ("s2h_heads_strided", "const int64_t h = j * Hl + hl;", "const int64_t h = hl * P + j;", 0),
    ("s2h_src_rank_drops_group", "const int64_t src_rank = g * P + s / St;",
     "const int64_t src_rank = s / St;", 0),
    ("s2h_tokens_strided", "const int64_t src_rank = g * P + s / St;\n                    const int64_t t = s % St;",
     "const int64_t src_rank = g * P + s % P;\n                    const int64_t t = s / P;", 0),
    ("h2s_tokens_strided", "const int64_t s = j * St + t;", "const int64_t s = t * P + j;", 0),
    ("h2s_src_rank_strided_heads", "const int64_t src_rank = g * P + h / Hl;\n                    const int64_t hl = h % Hl;",
     "const int64_t src_rank = g * P + h % P;\n                    const int64_t hl = h / P;", 0),
    ("h2s_src_rank_drops_group", "const int64_t src_rank = g * P + h / Hl;",
     "const int64_t src_rank = h / Hl;", 0),
    ("basp_groups_transposed", "*G = B;\n        *P = N / B;", "*G = N / B;\n        *P = B;", 0),
    ("basp_keeps_whole_batch", "*P = N / B;\n        *Bl = 1;", "*P = N / B;\n        *Bl = B;", 0),
    ("fallback_rule_wrong", "*G = N;\n    *P = 1;\n    *Bl = B / N;", "*G = 1;\n    *P = 1;\n    *Bl = B;", 0),
    ("no_divisibility_check", "if (N % B != 0) /* N = K*B */\n            return -1;", "", 0),
    ("head_check_dropped", "if (S % *P != 0 || H % *P != 0)", "if (S % *P != 0)", 0),
    ("element_size_ignored", "memcpy((char *)dst + di * es, (const char *)src + si * es, (size_t)es);",
     "memcpy((char *)dst + di * es, (const char *)src + si * es, 2);", 0),
    ("one_element_token_rule_swapped", "src[i] = seq_offset(g * P + s / St, bl, s % St, j * Hl + hl, e, Bl, St, H, d);",
     "src[i] = seq_offset(g * P + s % P, bl, s / P, j * Hl + hl, e, Bl, St, H, d);", 0),
    ("one_element_head_rule_swapped", "src[i] = head_offset(layout, g * P + h / Hl, bl, h % Hl, j * St + t, e, Bl, Hl, S, d);",
     "src[i] = head_offset(layout, g * P + h % P, bl, h / P, j * St + t, e, Bl, Hl, S, d);", 0),
    ("groups_members_from_batch", "*P = N / G_req;", "*P = B / G_req;", 0),
    ("groups_whole_batch_per_group", "*Bl = B / G_req;", "*Bl = B;", 0),
    ("groups_one_sequence_per_group", "*Bl = B / G_req;", "*Bl = 1;", 0),
    ("groups_batch_divisibility_dropped", " || B % G_req != 0", "", 0),
    ("groups_count_from_ranks", "*G = G_req;", "*G = N / G_req;", 0),
    ("source_index_off_by_one_channel", "in, seq_offset(src_rank, bl, t, h, e, Bl, St, H, d), es);",
     "in, seq_offset(src_rank, bl, t, h, (e + 1) % d, Bl, St, H, d), es);", 0),
]


def _mutate(text, old, new, occurrence):
    pos = -1
    for _ in range(occurrence + 1):
        pos = text.find(old, pos + 1)
        assert pos >= 0, "mutation site not found: %r" % old
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, occ):
    src = _mutate(open(SRC).read(), old, new, occ)
    c = tmp_path / "oracle_mut.c"
    c.write_text(src)
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(c), "-o", str(lib)],
                   check=True)
    code = ("import sys; sys.path.insert(0, %r); import oracle; oracle._use_library(%r); "
            "from tests import oracle_pins; oracle_pins.run_all()" % (ROOT, str(lib)))
    # two OpenMP threads per child: with several test workers at once, a
    # child per worker with a thread per core oversubscribes the CPUs, and
    # the oracle's many small parallel loops then crawl
    env = dict(os.environ, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode != 0, "mutant %s survived every pin" % name
