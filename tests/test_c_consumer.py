"""include/basp.h is a C header: a C11 program compiles against it, links
libbasp.so and uses the host-side calls (no GPU); the last-error status is
per thread."""
import os
import subprocess
import threading

from sequence_re_layout_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sequence_re_layout_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "basp.h"

static int fail(const char *what) { printf("FAIL %s\n", what); return 1; }

int main(void)
{
    basp_plan *p = basp_plan_create(8, 2, 16384, 32, 8, 64, BASP_BF16, BASP_MODE_BASP);
    if (!p) return fail("create");
    basp_plan_info info;
    memset(&info, 0, sizeof(info));
    if (basp_plan_query(p, &info) != BASP_OK) return fail("query");
    if (info.G != 2 || info.P != 4 || info.Bl != 1 || info.peers_per_rank != 3) return fail("groups");
    if (info.tokens_per_rank * 8 != 2 * 16384) return fail("tokens");
    basp_tuning t;
    memset(&t, 0, sizeof(t));
    t.tile_heads = 2;
    if (basp_plan_set_direction_tuning(p, BASP_HEAD_TO_SEQ, &t) != BASP_OK) return fail("tuning");
    basp_tuning back;
    if (basp_plan_get_tuning(p, BASP_HEAD_TO_SEQ, &back) != BASP_OK || back.tile_heads != 2) return fail("get");
    if (basp_plan_create(8, 3, 24, 24, 24, 8, BASP_BF16, BASP_MODE_BASP) != NULL) return fail("indivisible");
    if (basp_last_error() != BASP_ERR_INDIVISIBLE) return fail("last error");
    if (strncmp(basp_status_str(BASP_ERR_ALIAS), "BASP_ERR_ALIAS", 14) != 0) return fail("status str");
    if (basp_seq_to_head(p, NULL, NULL, NULL, NULL, NULL) != BASP_ERR_INVALID) return fail("null ptrs");
    basp_plan_destroy(p);
    basp_plan_destroy(NULL);
    printf("OK\n");
    return 0;
}
"""


def test_c_program_uses_the_abi(tmp_path):
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-L", PKG, "-lbasp", "-Wl,-rpath," + PKG, "-Wl,-rpath,/opt/rocm/lib",
                    "-Wl,--allow-shlib-undefined", "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip() == "OK", res.stdout + res.stderr


def test_last_error_is_per_thread():
    """Each thread sees the status of its own last call."""
    lib = b.library()
    barrier = threading.Barrier(8)
    seen = {}

    def worker(i):
        barrier.wait()
        for _ in range(200):
            if i % 2:
                h = lib.basp_plan_create(8, 3, 24, 24, 24, 8, 0, 1)        # N % B != 0
                want = b.BASP_ERR_INDIVISIBLE
            else:
                h = lib.basp_plan_create(8, 2, 16, 8, 8, 8, 0, 1)
                want = b.BASP_OK
            got = b.basp_last_error()
            if h:
                lib.basp_plan_destroy(h)
                if want == b.BASP_OK:
                    got_after = b.basp_last_error()   # destroy records OK as well
                    assert got_after == b.BASP_OK
            if got != want:
                seen[i] = (got, want)
                return
        seen.setdefault(i, None)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(v is None for v in seen.values()), seen
