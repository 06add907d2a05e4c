// Host sanitizer run of the library's host code (plan.cpp, launch.cpp) and
// the kernels' index arithmetic (launch.hpp) through the CPU emulator
// (tests/emu/kernel_emu.cpp), built with -fsanitize=address,undefined.
//
// Every case fills Q, K, V with distinct tags and checks, without the
// oracle: no in-tile access outside a descriptor, every output element a
// distinct input tag (a bijection), the fused head->seq inverse and the
// head->seq of the Q part giving the inputs back, and the unfused baseline
// agreeing with the fused call.  It also walks the plan validation paths.
// Exit status 0 when every check holds; the sanitizers abort on any error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <unordered_set>
#include <vector>

#include "basp.h"

extern "C" {
int emu_seq_to_head(const basp_plan *p, const void *q, const void *k, const void *v, void *out,
                    uint64_t *bad, int *vw);
int emu_head_to_seq(const basp_plan *p, const void *o, void *out, uint64_t *bad, int *vw);
int emu_head_to_seq_qkv(const basp_plan *p, const void *in, void *dq, void *dk, void *dv,
                        uint64_t *bad, int *vw);
int emu_seq_to_head_unfused(const basp_plan *p, const void *q, const void *k, const void *v,
                            void *out, void *ws, uint64_t *bad, int *vw);
}

namespace {

int failures = 0;

void expect(bool ok, const char *what, int line)
{
    if (!ok) {
        std::printf("FAIL line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

struct Shape {
    int N, B;
    int64_t S;
    int Hq, Hkv, d;
    basp_mode mode;
    basp_layout layout;
    int G;   // groups of BASP_MODE_GROUPS
};

void run_case(const Shape &s, const basp_tuning *t)
{
    basp_plan *p = s.mode == BASP_MODE_GROUPS
                       ? basp_plan_create_groups(s.N, s.B, s.S, s.Hq, s.Hkv, s.d, BASP_INT32, s.G, s.layout)
                       : basp_plan_create_ex(s.N, s.B, s.S, s.Hq, s.Hkv, s.d, BASP_INT32, s.mode, s.layout);
    EXPECT(p != nullptr);
    if (!p)
        return;
    if (t)
        EXPECT(basp_plan_set_tuning(p, t) == BASP_OK);
    basp_plan_info info;
    EXPECT(basp_plan_query(p, &info) == BASP_OK);
    const size_t nq = size_t(info.q_elems), nkv = size_t(info.kv_elems), nqkv = size_t(info.qkv_elems);
    std::vector<int32_t> q(nq), k(nkv), v(nkv), out(nqkv, -1), out2(nqkv, -1);
    for (size_t i = 0; i < nq; ++i)
        q[i] = int32_t(i);
    for (size_t i = 0; i < nkv; ++i) {
        k[i] = int32_t(nq + i);
        v[i] = int32_t(nq + nkv + i);
    }
    uint64_t bad = 0;
    int vw = 0;
    EXPECT(emu_seq_to_head(p, q.data(), k.data(), v.data(), out.data(), &bad, &vw) == BASP_OK);
    EXPECT(bad == 0);
    std::unordered_set<int32_t> seen;
    bool distinct = true;
    for (int32_t x : out)
        distinct = distinct && x >= 0 && size_t(x) < nqkv && seen.insert(x).second;
    EXPECT(distinct);
    std::vector<int32_t> dq(nq, -1), dk(nkv, -1), dv(nkv, -1), o(nq, -1);
    EXPECT(emu_head_to_seq_qkv(p, out.data(), dq.data(), dk.data(), dv.data(), &bad, &vw) == BASP_OK);
    EXPECT(dq == q && dk == k && dv == v);
    EXPECT(emu_head_to_seq(p, out.data(), o.data(), &bad, &vw) == BASP_OK);
    EXPECT(o == q);
    // basp_unfused_workspace_bytes lives with the kernels: packed and
    // exchanged copies of all three tensors
    std::vector<unsigned char> ws(2 * nqkv * sizeof(int32_t));
    EXPECT(emu_seq_to_head_unfused(p, q.data(), k.data(), v.data(), out2.data(), ws.data(), &bad, &vw) ==
           BASP_OK);
    EXPECT(out2 == out);
    EXPECT(bad == 0);
    basp_plan_destroy(p);
}

}  // namespace

int main()
{
    const Shape shapes[] = {
        {4, 2, 4 * 37, 8, 4, 8, BASP_MODE_BASP, BASP_LAYOUT_HEAD_MAJOR},
        {6, 3, 6 * 11, 12, 6, 5, BASP_MODE_ULYSSES, BASP_LAYOUT_HEAD_MAJOR},
        {6, 3, 6 * 11, 12, 6, 5, BASP_MODE_BASP, BASP_LAYOUT_TOKEN_MAJOR},
        {8, 16, 40, 8, 8, 4, BASP_MODE_BASP, BASP_LAYOUT_HEAD_MAJOR},   // data-parallel fallback
        {8, 1, 8 * 13, 16, 8, 16, BASP_MODE_BASP, BASP_LAYOUT_TOKEN_MAJOR},
        {1, 1, 29, 3, 3, 7, BASP_MODE_ULYSSES, BASP_LAYOUT_HEAD_MAJOR},
        {6, 4, 3 * 9, 6, 3, 40, BASP_MODE_GROUPS, BASP_LAYOUT_HEAD_MAJOR, 2},   // 3 members, 2 sequences
        {8, 16, 2 * 7, 4, 2, 3, BASP_MODE_GROUPS, BASP_LAYOUT_TOKEN_MAJOR, 4},  // 2 members, 4 sequences
    };
    basp_tuning staged = {};
    staged.stage = 2;
    staged.tile_heads = 2;
    basp_tuning small = {};
    small.tile_tokens = 3;
    small.tile_heads = 3;
    small.max_grid = 5;
    small.block_size = 64;
    small.lane_order = 1;
    small.tile_order = 1;
    small.xcd_remap = 2;
    small.batch_order = 2;
    for (const Shape &s : shapes) {
        run_case(s, nullptr);
        run_case(s, &staged);
        run_case(s, &small);
    }
    // validation paths
    EXPECT(basp_plan_create(8, 3, 24, 24, 24, 8, BASP_BF16, BASP_MODE_BASP) == nullptr);
    EXPECT(basp_last_error() == BASP_ERR_INDIVISIBLE);
    EXPECT(basp_plan_create(0, 1, 8, 8, 8, 8, BASP_BF16, BASP_MODE_BASP) == nullptr);
    EXPECT(basp_last_error() == BASP_ERR_INVALID);
    EXPECT(basp_plan_create(8, 2, int64_t(1) << 60, 8, 8, 8, BASP_BF16, BASP_MODE_BASP) == nullptr);
    EXPECT(basp_last_error() == BASP_ERR_UNSUPPORTED);
    EXPECT(basp_plan_create_groups(8, 6, 24, 24, 24, 8, BASP_BF16, 4, BASP_LAYOUT_HEAD_MAJOR) == nullptr);
    EXPECT(basp_last_error() == BASP_ERR_INDIVISIBLE);
    EXPECT(basp_plan_create_groups(8, 8, 24, 24, 24, 8, BASP_BF16, 0, BASP_LAYOUT_HEAD_MAJOR) == nullptr);
    EXPECT(basp_last_error() == BASP_ERR_INVALID);
    EXPECT(std::strlen(basp_status_str(basp_status(99))) > 0);
    std::printf("%s (%d failures)\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}
