// plan.cpp -- host side of libbasp: plan creation and validation, the plan
// query, tuning, and status reporting.  No device calls.
//
// Group structure (BASP review page, "Summary" and "Frequently asked
// questions"; the general G-group form of its "Strengths", the paper's
// Sec. IV.C):
//   Ulysses            G = 1, P = N,   Bl = B
//   BASP, B <= N       G = B, P = N/B, Bl = 1     (N = K*B, K = P)
//   BASP, B >  N       G = N, P = 1,   Bl = B/N   (data-parallel fallback)
//   G groups           G,     P = N/G, Bl = B/G   (G divides N and B)
// Tokens and heads split evenly over the P members of a group.
#include <climits>
#include <cstring>
#include <new>

#include "plan_internal.hpp"

namespace basp {

static thread_local basp_status t_last = BASP_OK;

basp_status record(basp_status s)
{
    t_last = s;
    return s;
}

}  // namespace basp

using basp::record;

namespace {

int elem_size(basp_dtype t)
{
    switch (t) {
    case BASP_BF16:
    case BASP_FP16:
        return 2;
    case BASP_FP32:
    case BASP_INT32:
        return 4;
    }
    return 0;
}

// a * b, or -1 when the product exceeds 2^62 (operands non-negative).
int64_t mul_capped(int64_t a, int64_t b)
{
    if (a < 0 || b < 0)
        return -1;
    if (a == 0 || b == 0)
        return 0;
    if (a > (int64_t{1} << 62) / b)
        return -1;
    return a * b;
}

}  // namespace

namespace {

// A plan with the group structure (G, P, Bl) already chosen: checks the
// even splits of tokens and heads and the sizes, then fills the plan.
basp_plan *make_plan(int N, int B, int64_t S, int Hq, int Hkv, int d, basp_dtype dtype, basp_mode mode,
                     basp_layout layout, int G, int P, int Bl)
{
    const int es = elem_size(dtype);
    if (S % P != 0 || Hq % P != 0 || Hkv % P != 0) {
        record(BASP_ERR_INDIVISIBLE);
        return nullptr;
    }

    // every byte count below 2^62, so sums of a few of them stay in int64
    const int64_t row = int64_t{d} * es;
    const int64_t q_elems = mul_capped(mul_capped(mul_capped(B, S), Hq), d);
    const int64_t kv_elems = mul_capped(mul_capped(mul_capped(B, S), Hkv), d);
    if (q_elems < 0 || kv_elems < 0 || mul_capped(q_elems + 2 * kv_elems, 2 * es) < 0) {
        record(BASP_ERR_UNSUPPORTED);
        return nullptr;
    }

    basp_plan *p = new (std::nothrow) basp_plan;
    if (!p) {
        record(BASP_ERR_UNSUPPORTED);
        return nullptr;
    }
    p->N = N;
    p->B = B;
    p->S = S;
    p->Hq = Hq;
    p->Hkv = Hkv;
    p->d = d;
    p->dtype = dtype;
    p->mode = mode;
    p->layout = layout;
    p->es = es;
    p->G = G;
    p->P = P;
    p->Bl = Bl;
    p->St = S / P;
    p->Hl_q = Hq / P;
    p->Hl_kv = Hkv / P;
    p->row_bytes = row;
    p->q_elems = q_elems;
    p->kv_elems = kv_elems;
    std::memset(p->tuning, 0, sizeof(p->tuning));

    const basp_status lim = basp::check_launch_limits(*p, p->tuning[0]);
    if (lim != BASP_OK) {
        delete p;
        record(lim);
        return nullptr;
    }
    record(BASP_OK);
    return p;
}

bool args_valid(int N, int B, int64_t S, int Hq, int Hkv, int d, basp_dtype dtype, basp_layout layout)
{
    return N >= 1 && B >= 1 && S >= 0 && Hq >= 1 && Hkv >= 1 && d >= 1 && elem_size(dtype) != 0 &&
           (layout == BASP_LAYOUT_HEAD_MAJOR || layout == BASP_LAYOUT_TOKEN_MAJOR);
}

}  // namespace

extern "C" basp_plan *basp_plan_create_ex(int N, int B, int64_t S, int Hq, int Hkv, int d,
                                          basp_dtype dtype, basp_mode mode, basp_layout layout)
{
    if (!args_valid(N, B, S, Hq, Hkv, d, dtype, layout) ||
        (mode != BASP_MODE_ULYSSES && mode != BASP_MODE_BASP)) {
        record(BASP_ERR_INVALID);
        return nullptr;
    }

    int G, P, Bl;
    if (mode == BASP_MODE_ULYSSES) {
        G = 1;
        P = N;
        Bl = B;
    } else if (B <= N) {
        if (N % B != 0) {
            record(BASP_ERR_INDIVISIBLE);
            return nullptr;
        }
        G = B;
        P = N / B;
        Bl = 1;
    } else {
        if (B % N != 0) {
            record(BASP_ERR_INDIVISIBLE);
            return nullptr;
        }
        G = N;
        P = 1;
        Bl = B / N;
    }
    return make_plan(N, B, S, Hq, Hkv, d, dtype, mode, layout, G, P, Bl);
}

extern "C" basp_plan *basp_plan_create_groups(int N, int B, int64_t S, int Hq, int Hkv, int d,
                                              basp_dtype dtype, int G, basp_layout layout)
{
    // the general form of the per-GPU work equality (review page,
    // "Strengths"; the paper's Sec. IV.C): G groups of N/G consecutive ranks,
    // each owning B/G consecutive sequences
    if (!args_valid(N, B, S, Hq, Hkv, d, dtype, layout) || G < 1) {
        record(BASP_ERR_INVALID);
        return nullptr;
    }
    if (N % G != 0 || B % G != 0) {
        record(BASP_ERR_INDIVISIBLE);
        return nullptr;
    }
    return make_plan(N, B, S, Hq, Hkv, d, dtype, BASP_MODE_GROUPS, layout, G, N / G, B / G);
}

extern "C" basp_plan *basp_plan_create(int N, int B, int64_t S, int Hq, int Hkv, int d,
                                       basp_dtype dtype, basp_mode mode)
{
    return basp_plan_create_ex(N, B, S, Hq, Hkv, d, dtype, mode, BASP_LAYOUT_HEAD_MAJOR);
}

extern "C" void basp_plan_destroy(basp_plan *plan)
{
    delete plan;
    record(BASP_OK);
}

extern "C" basp_status basp_plan_query(const basp_plan *p, basp_plan_info *info)
{
    if (!p || !info)
        return record(BASP_ERR_INVALID);
    basp_plan_info r;
    std::memset(&r, 0, sizeof(r));
    r.N = p->N;
    r.B = p->B;
    r.Hq = p->Hq;
    r.Hkv = p->Hkv;
    r.d = p->d;
    r.elem_size = p->es;
    r.S = p->S;
    r.mode = p->mode;
    r.layout = p->layout;
    r.dtype = p->dtype;
    r.G = p->G;
    r.P = p->P;
    r.Bl = p->Bl;
    r.St = p->St;
    r.Hl_q = p->Hl_q;
    r.Hl_kv = p->Hl_kv;
    r.tokens_per_rank = int64_t{p->Bl} * p->St;
    r.peers_per_rank = p->P - 1;
    r.q_elems = p->q_elems;
    r.kv_elems = p->kv_elems;
    r.q_elems_per_rank = p->q_elems / p->N;
    r.kv_elems_per_rank = p->kv_elems / p->N;
    r.qkv_elems = p->q_elems + 2 * p->kv_elems;
    r.qkv_offset_q = 0;
    r.qkv_offset_k = p->q_elems;
    r.qkv_offset_v = p->q_elems + p->kv_elems;
    // one peer's chunk: Bl sequences x St tokens x Hl heads x d channels
    r.per_peer_bytes_q = int64_t{p->Bl} * p->St * p->Hl_q * p->row_bytes;
    r.per_peer_bytes_kv = int64_t{p->Bl} * p->St * p->Hl_kv * p->row_bytes;
    // every rank receives P chunks, one of them from itself
    r.cross_rank_bytes_q = int64_t{p->N} * (p->P - 1) * r.per_peer_bytes_q;
    r.cross_rank_bytes_kv = int64_t{p->N} * (p->P - 1) * r.per_peer_bytes_kv;
    r.qkv_bytes_moved = 2 * r.qkv_elems * p->es;
    r.o_bytes_moved = 2 * p->q_elems * p->es;
    // the foil: Ulysses over groups of K = N/B ranks, each group holding all B
    // sequences, so every rank keeps B*S/K = B*B*S/N tokens.  K divides the
    // plan's group size P, so S/K is whole whenever the plan exists.
    if (p->B <= p->N && p->N % p->B == 0)
        r.tokens_per_rank_foil = int64_t{p->B} * (p->S / (p->N / p->B));
    *info = r;
    return record(BASP_OK);
}

namespace basp {

bool tuning_in_range(const basp_tuning &t)
{
    const int v = t.vectors_per_thread;
    return (v == 0 || v == 1 || v == 2 || v == 4 || v == 8) && t.tile_tokens >= 0 &&
           t.tile_heads >= 0 && t.cache_policy >= 0 && t.cache_policy <= 5 && t.max_grid >= 0 &&
           t.lane_order >= 0 && t.lane_order <= 2 && t.xcd_remap >= 0 && t.xcd_remap <= 2 &&
           t.tile_order >= 0 && t.tile_order <= 3 && t.stage >= 0 && t.stage <= 2 &&
           (t.block_size == 0 || t.block_size == 64 || t.block_size == 128 || t.block_size == 256) &&
           t.batch_order >= 0 && t.batch_order <= 2;
}

}  // namespace basp

extern "C" basp_status basp_plan_set_direction_tuning(basp_plan *p, basp_direction dir,
                                                      const basp_tuning *t)
{
    if (!p || !t || (dir != BASP_SEQ_TO_HEAD && dir != BASP_HEAD_TO_SEQ) || !basp::tuning_in_range(*t))
        return record(BASP_ERR_INVALID);
    const basp_status lim = basp::check_launch_limits(*p, *t);
    if (lim != BASP_OK)
        return record(lim);
    p->tuning[dir] = *t;
    return record(BASP_OK);
}

extern "C" basp_status basp_plan_set_tuning(basp_plan *p, const basp_tuning *t)
{
    if (!p || !t || !basp::tuning_in_range(*t))
        return record(BASP_ERR_INVALID);
    const basp_status lim = basp::check_launch_limits(*p, *t);
    if (lim != BASP_OK)
        return record(lim);
    p->tuning[0] = p->tuning[1] = *t;
    return record(BASP_OK);
}

extern "C" basp_status basp_plan_get_tuning(const basp_plan *p, basp_direction dir, basp_tuning *t)
{
    if (!p || !t || (dir != BASP_SEQ_TO_HEAD && dir != BASP_HEAD_TO_SEQ))
        return record(BASP_ERR_INVALID);
    *t = p->tuning[dir];
    return record(BASP_OK);
}

extern "C" basp_status basp_last_error(void)
{
    return basp::t_last;
}

extern "C" const char *basp_status_str(basp_status s)
{
    switch (s) {
    case BASP_OK:
        return "BASP_OK";
    case BASP_ERR_INVALID:
        return "BASP_ERR_INVALID: NULL plan or pointer, size out of range, or unknown enum";
    case BASP_ERR_INDIVISIBLE:
        return "BASP_ERR_INDIVISIBLE: N must be a multiple of B (or B of N when B > N), "
               "and S, Hq, Hkv multiples of the group size";
    case BASP_ERR_UNSUPPORTED:
        return "BASP_ERR_UNSUPPORTED: sizes beyond the library's index limits";
    case BASP_ERR_ALIGN:
        return "BASP_ERR_ALIGN: pointer not aligned to the element size";
    case BASP_ERR_ALIAS:
        return "BASP_ERR_ALIAS: an output overlaps an input or another output";
    case BASP_ERR_HIP:
        return "BASP_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown basp_status";
}
