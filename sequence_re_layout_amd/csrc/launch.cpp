// launch.cpp -- host-side planning of every kernel launch: pointer checks,
// vector width, tile shape, descriptors and grid.  Plain C++ with no device
// calls, so that the same code can also drive a CPU emulation of the kernels.
#include <algorithm>
#include <cstring>

#ifndef BASP_HD
#define BASP_HD
#endif
#include "launch.hpp"
#include "plan_internal.hpp"

namespace basp {
namespace {

constexpr uint32_t kGridCap = 1u << 22;  // work-groups per launch at most

// Launch shape of one tile launch: the plan's tuning where set, else the
// defaults below, chosen on MI355X over every named workload of at least
// 256 MiB (Llama/Qwen shapes, 128- and 256-byte rows, both modes, both
// directions, rotating buffers) as the launch shape whose worst ratio to
// each workload's best was highest (0.94-0.95 in sweeps of two builds, 0.98
// on average): direct (no LDS staging), 256 threads per work-group, one
// vector per lane, head blocks fastest in work-group order, lanes along
// heads, non-temporal loads and non-temporal device-scope stores; 8 heads
// per tile for 128-byte rows, one head for longer rows.
//
// Smaller calls, bound by start-up and drain more than by bandwidth, got a
// rule of their own, chosen the same way over the named workloads' calls of
// 4 to 384 MiB (HIP graph replays, 1 296 shapes per call), which lifted the
// worst ratio there from 0.87-0.89 to 0.95-0.96:
// * rows of at most 128 bytes, calls of at most 32 MiB: 128 threads, two
//   vectors per lane, 4 heads per tile, token blocks fastest within a source
//   member (tile order 3), lanes along tokens, XCD-contiguous tiles;
// * longer rows, calls of at most 160 MiB: token blocks fastest (tile order
//   1), the rest as for large calls.
// basp_plan_autotune replaces these by measurement.
constexpr uint64_t kSmallCallShortRows = uint64_t{32} << 20;
constexpr uint64_t kSmallCallLongRows = uint64_t{160} << 20;

// a + b, or the largest value where that overflows (call sizes of plans
// near the 2^62-byte buffer limit only need to compare as large)
uint64_t add_sat(uint64_t a, uint64_t b) { return a > ~uint64_t{0} - b ? ~uint64_t{0} : a + b; }
struct Shape {
    int vpt, policy;
    int block;                          // threads per work-group
    uint32_t tile_tokens, tile_heads;   // tile_tokens 0: derived
    bool heads_given;                   // tile_heads set by the tuning
    bool s_fast;
    int order;                          // tile order 1, 2 or 3 (launch.hpp)
    uint32_t grid_cap;
    bool xcd;
    bool stage;
    bool batch_x;
};

// call_bytes: the bytes the launch reads and writes (the algorithmic bytes
// of the call), which picks between the rules above.
Shape resolve(const basp_plan &p, const basp_tuning &t, uint64_t call_bytes)
{
    const bool short_rows = p.row_bytes <= 128;
    const bool small = call_bytes <= (short_rows ? kSmallCallShortRows : kSmallCallLongRows);
    const bool small_short = small && short_rows;
    Shape s;
    s.vpt = t.vectors_per_thread ? t.vectors_per_thread : (small_short ? 2 : 1);
    s.policy = t.cache_policy ? t.cache_policy : 4;
    s.block = t.block_size ? t.block_size : (small_short ? 128 : kBlock);
    s.tile_tokens = uint32_t(t.tile_tokens);
    s.tile_heads = t.tile_heads ? uint32_t(t.tile_heads) : (short_rows ? (small ? 4 : 8) : 1);
    s.heads_given = t.tile_heads != 0;
    s.s_fast = t.lane_order ? t.lane_order == 1 : small_short;
    s.order = t.tile_order ? t.tile_order : (small ? (short_rows ? 3 : 1) : 2);
    s.grid_cap = t.max_grid ? uint32_t(t.max_grid) : kGridCap;
    s.xcd = t.xcd_remap ? t.xcd_remap == 2 : small_short;
    s.stage = t.stage == 2;
    s.batch_x = t.batch_order == 2;
    return s;
}

// The launch shape a vector width runs with.  The tuned work-group size and
// vectors per lane, and LDS staging (for rows of at most one pass of the
// work-group), exist for 16-byte vectors; narrower vectors run the direct
// kernel with 256 threads and 4 vectors per lane.
Shape for_vector_width(Shape sh, int vw, uint32_t A)
{
    if (vw != 16) {
        sh.block = kBlock;
        sh.vpt = 4;
    }
    sh.stage = sh.stage && vw == 16 && A <= uint32_t(sh.block * sh.vpt);
    return sh;
}

uint64_t addr(const void *p) { return reinterpret_cast<uint64_t>(p); }

// Widest vector (16, 8, 4 or 2 bytes, never below the element size) that
// divides the row.  The addresses need only the element alignment the entry
// points check: compute queues run in the unaligned access mode, in which a
// buffer access of any width may start at any byte (compilers emit 16-byte
// loads for byte-aligned copies on this target), and rows that straddle
// cache lines cost less that way than split into narrower vectors.
int vector_width(const basp_plan &p)
{
    int vw = 16;
    while (vw > p.es && p.row_bytes % vw != 0)
        vw /= 2;
    return vw;
}

struct TileShape {
    uint32_t Ts, Th, ntb, nhb;
    uint64_t ntiles;   // tiles of one (member, batch index) plane
};

// Tile of one tensor with Hl heads per rank and A vectors per row: about one
// pass of the work-group (block * vpt vectors) unless the tile extent is given.
TileShape tile_shape(const basp_plan &p, const Shape &sh, uint32_t Hl, uint32_t A)
{
    const uint64_t rows = std::max<uint64_t>(1, uint64_t(sh.block) * sh.vpt / A);
    uint64_t th = std::min<uint64_t>(sh.tile_heads, Hl);
    if (sh.stage)   // a staged tile is one pass of the work-group: at most `rows` rows
        th = std::min<uint64_t>(th, rows);
    uint64_t ts = sh.tile_tokens ? uint64_t(sh.tile_tokens) : std::max<uint64_t>(1, rows / th);
    if (sh.stage)
        ts = std::min<uint64_t>(ts, std::max<uint64_t>(1, rows / th));
    ts = std::min<uint64_t>(ts, uint64_t(std::max<int64_t>(p.St, 1)));
    TileShape s;
    s.Ts = uint32_t(ts);
    s.Th = uint32_t(th);
    s.ntb = uint32_t((uint64_t(p.St) + ts - 1) / ts);
    s.nhb = uint32_t((Hl + th - 1) / th);
    s.ntiles = uint64_t(s.nhb) * p.P * s.ntb;
    return s;
}

struct Strides {
    uint64_t seq_tok, head_tok, head_head;
};

// Byte strides inside a tile, for a tensor of H heads (basp.h, "Memory layouts").
Strides strides(const basp_plan &p, uint32_t H)
{
    const uint64_t row = p.row_bytes, Hl = H / p.P, S = p.S;
    Strides s;
    s.seq_tok = H * row;
    if (p.layout == BASP_LAYOUT_HEAD_MAJOR) {
        s.head_tok = row;
        s.head_head = S * row;
    } else {
        s.head_head = row;
        s.head_tok = Hl * row;
    }
    return s;
}

constexpr uint32_t kGridYZ = 65535;   // work-groups along y and along z at most

// What the tile launch grid and tile_origin assume of a plan: every tensor
// holds fewer than 2^32 rows (tile bases are 32-bit row indices, and S fits
// 32 bits), and P and B fit the grid's y and z extents.
bool grid_fits(const basp_plan &p)
{
    const uint64_t H = uint64_t(std::max(p.Hq, p.Hkv));
    return uint64_t(p.S) <= 0xffffffffull / (uint64_t(p.B) * H) && uint32_t(p.P) <= kGridYZ &&
           uint32_t(p.B) <= kGridYZ;
}

// Every offset a lane computes inside a tile stays below kI31Max.
bool tile_offsets_fit(const basp_plan &p, uint32_t H, const TileShape &ts)
{
    const Strides s = strides(p, H);
    const uint64_t seq_max = (ts.Ts - 1) * s.seq_tok + uint64_t(ts.Th) * p.row_bytes;
    const uint64_t head_max = (ts.Ts - 1) * s.head_tok + (ts.Th - 1) * s.head_head + p.row_bytes;
    return seq_max <= kI31Max && head_max <= kI31Max && s.seq_tok <= kI31Max &&
           s.head_tok <= kI31Max && (ts.Th == 1 || s.head_head <= kI31Max);
}

// Tile shape of a tensor of H heads whose in-tile offsets fit; a built-in
// multi-head tile falls back to one head per tile (the head stride of a very
// long head-major sequence is too large for 31-bit offsets).
bool fitted_shape(const basp_plan &p, Shape sh, uint32_t H, uint32_t A, TileShape &ts)
{
    ts = tile_shape(p, sh, H / p.P, A);
    if (tile_offsets_fit(p, H, ts) && uint64_t(ts.Ts) * ts.Th * A <= kI31Max)
        return true;
    if (sh.heads_given || ts.Th == 1)
        return false;
    sh.tile_heads = 1;
    ts = tile_shape(p, sh, H / p.P, A);
    return tile_offsets_fit(p, H, ts) && uint64_t(ts.Ts) * ts.Th * A <= kI31Max;
}

struct SegSpec {
    uint64_t seq, head;   // addresses
    uint32_t H;           // heads of this tensor
};

int build_tiles(const basp_plan &p, const SegSpec *segs, int nseg, bool s2h, TileLaunch &L)
{
    std::memset(&L, 0, sizeof(L));
    if (!grid_fits(p))
        return BASP_ERR_UNSUPPORTED;
    const int vw = vector_width(p);
    const uint32_t A = uint32_t(p.row_bytes / vw);
    uint64_t call_bytes = 0;        // read once and written once
    for (int i = 0; i < nseg; ++i)
        call_bytes = add_sat(call_bytes, 2 * (uint64_t(p.B) * p.S * segs[i].H * p.row_bytes));
    const Shape sh = for_vector_width(
        resolve(p, p.tuning[s2h ? BASP_SEQ_TO_HEAD : BASP_HEAD_TO_SEQ], call_bytes), vw, A);
    TileDesc &D = L.D;
    D.St = uint32_t(p.St);
    D.S = uint32_t(p.S);
    D.token_major = p.layout == BASP_LAYOUT_TOKEN_MAJOR;
    D.row = uint32_t(p.row_bytes);
    D.s_fast = sh.s_fast;
    // staged loads run along the source's contiguous axis, stores along the
    // destination's: heads in the sequence-sharded layout and in the
    // token-major head layout, tokens in the head-major one
    const bool head_major = p.layout == BASP_LAYOUT_HEAD_MAJOR;
    D.load_s_fast = s2h ? 0 : head_major;
    D.store_s_fast = s2h ? head_major : 0;
    D.order = uint32_t(sh.order);
    D.P = make_fastdiv(p.P);
    D.Bl = uint32_t(p.Bl);
    D.gstride = uint32_t(p.P - 1) * uint32_t(p.Bl);
    D.Blf = make_fastdiv(uint32_t(p.Bl));
    D.A = make_fastdiv(A);
    uint64_t total = 0;
    uint32_t end[3];                // each tensor's end in the plane's tiles
    for (int i = 0; i < 3; ++i) {
        TileSeg &sg = D.seg[i];
        if (i >= nseg) {            // unused slot: an empty range after the last tensor
            sg = D.seg[i - 1];
            sg.tile_begin = end[i] = end[i - 1];
            continue;
        }
        const uint32_t H = segs[i].H, Hl = H / p.P;
        TileShape ts;
        if (!fitted_shape(p, sh, H, A, ts))
            return BASP_ERR_UNSUPPORTED;
        const Strides st = strides(p, H);
        sg.seq = segs[i].seq;
        sg.head = segs[i].head;
        sg.bytes = uint64_t(p.B) * p.S * H * p.row_bytes;
        sg.seq_tok = uint32_t(st.seq_tok);
        sg.head_tok = uint32_t(st.head_tok);
        sg.head_head_lane = ts.Th == 1 ? 0u : uint32_t(st.head_head);
        sg.Hl = Hl;
        sg.Ts = make_fastdiv(ts.Ts);
        sg.Th = make_fastdiv(ts.Th);
        sg.fast = make_fastdiv(sh.order == 2 ? ts.nhb : ts.ntb);
        sg.mid = make_fastdiv(sh.order == 3 ? ts.nhb : uint32_t(p.P));
        sg.tile_begin = uint32_t(total);
        total += ts.ntiles;
        if (total > kI31Max)
            return BASP_ERR_UNSUPPORTED;
        end[i] = uint32_t(total);
    }
    D.plane = uint32_t(total);
    D.batch_x = sh.batch_x && p.B > 1;
    D.nb = make_fastdiv(uint32_t(p.B));
    if (D.batch_x && total * uint64_t(p.B) > kI31Max)
        return BASP_ERR_UNSUPPORTED;
    D.xbound = D.batch_x ? uint32_t(total * uint64_t(p.B)) : uint32_t(total);
    D.seg_end0 = end[0];
    D.seg_end1 = end[1];
    D.xcd_span = sh.xcd ? uint32_t(total / kXcds) : 0;
    L.grid = uint32_t(std::min<uint64_t>(D.xbound, sh.grid_cap));
    L.nseg = nseg;
    L.grid_y = uint32_t(p.P);
    L.grid_z = D.batch_x ? 1u : uint32_t(p.B);
    L.vw = vw;
    L.vpt = sh.vpt;
    L.block = sh.block;
    L.policy = sh.policy;
    L.s2h = s2h;
    L.staged = sh.stage;
    return BASP_OK;
}

bool overlaps(uint64_t a, uint64_t na, uint64_t b, uint64_t nb)
{
    return na && nb && a < b + nb && b < a + na;
}

struct Buf {
    const void *ptr;
    uint64_t bytes;
};

// NULL, alignment and aliasing checks (basp.h, "Conventions").
int check_buffers(const basp_plan &p, const Buf *ins, int nin, const Buf *outs, int nout)
{
    for (int i = 0; i < nin + nout; ++i) {
        const Buf &b = i < nin ? ins[i] : outs[i - nin];
        if (b.bytes && !b.ptr)
            return BASP_ERR_INVALID;
        if (addr(b.ptr) % p.es)
            return BASP_ERR_ALIGN;
    }
    for (int o = 0; o < nout; ++o) {
        for (int i = 0; i < nin; ++i)
            if (overlaps(addr(outs[o].ptr), outs[o].bytes, addr(ins[i].ptr), ins[i].bytes))
                return BASP_ERR_ALIAS;
        for (int j = 0; j < o; ++j)
            if (overlaps(addr(outs[o].ptr), outs[o].bytes, addr(outs[j].ptr), outs[j].bytes))
                return BASP_ERR_ALIAS;
    }
    return BASP_OK;
}

struct PermSpec {
    uint64_t src, dst, src_bytes, dst_bytes;
    uint32_t ext[5];       // digit extents, d0 slowest
    uint32_t sstride[5];   // source strides in rows
    uint64_t rows;
};

int build_perm(const basp_plan &p, const PermSpec *ps, int n, int vw, PermLaunch &L)
{
    std::memset(&L, 0, sizeof(L));
    PermDesc &D = L.D;
    const uint32_t A = uint32_t(p.row_bytes / vw);
    D.row = uint32_t(p.row_bytes);
    D.A = make_fastdiv(A);
    uint64_t chunks = 0;
    for (int i = 0; i < 3; ++i) {
        PermSeg &sg = D.seg[i];
        if (i >= n) {
            sg = D.seg[i - 1];
            sg.chunk_begin = sg.chunk_end;
            continue;
        }
        const uint64_t nvec = ps[i].rows * A;
        if (nvec > kI31Max || ps[i].src_bytes > kI31Max || ps[i].dst_bytes > kI31Max)
            return BASP_ERR_UNSUPPORTED;
        sg.src = ps[i].src;
        sg.dst = ps[i].dst;
        sg.src_bytes = ps[i].src_bytes;
        sg.dst_bytes = ps[i].dst_bytes;
        for (int j = 0; j < 4; ++j)
            sg.ext[j] = make_fastdiv(ps[i].ext[j + 1]);
        for (int j = 0; j < 5; ++j)
            sg.sstride[j] = ps[i].sstride[j];
        sg.nvec = uint32_t(nvec);
        sg.chunk_begin = uint32_t(chunks);
        chunks += (nvec + kBlock * kPermVpt - 1) / (kBlock * kPermVpt);
        sg.chunk_end = uint32_t(chunks);
    }
    D.nchunks = uint32_t(chunks);
    L.grid = uint32_t(std::min<uint64_t>(chunks, kGridCap));
    L.vw = vw;
    return BASP_OK;
}

}  // namespace

basp_status check_launch_limits(const basp_plan &p, const basp_tuning &t)
{
    if (p.St > int64_t(kI31Max) || p.row_bytes > int64_t(kI31Max) ||
        int64_t(p.Hq) * p.row_bytes > int64_t(kI31Max) || !grid_fits(p))
        return BASP_ERR_UNSUPPORTED;
    const uint32_t heads[3] = {uint32_t(p.Hq), uint32_t(p.Hkv), uint32_t(p.Hkv)};
    // the built-in choices depend on the call's size: those of a one-tensor
    // call (O, dO) and of a fused one (Q, K, V)
    const uint64_t one = 2 * (uint64_t(p.q_elems) * p.es);
    const uint64_t fused = add_sat(one, add_sat(2 * (uint64_t(p.kv_elems) * p.es), 2 * (uint64_t(p.kv_elems) * p.es)));
    for (const uint64_t call_bytes : {one, fused}) {
        const Shape resolved = resolve(p, t, call_bytes);
        // every vector width a launch may pick, with the tile it then uses
        for (int vw = 16; vw >= p.es; vw /= 2) {
            if (p.row_bytes % vw)
                continue;
            const uint32_t A = uint32_t(p.row_bytes / vw);
            const Shape sh = for_vector_width(resolved, vw, A);
            uint64_t total = 0;
            for (int i = 0; i < 3; ++i) {
                TileShape ts;
                if (!fitted_shape(p, sh, heads[i], A, ts))
                    return BASP_ERR_UNSUPPORTED;
                total += ts.ntiles;
            }
            if (total * (sh.batch_x ? uint64_t(p.B) : 1u) > kI31Max)
                return BASP_ERR_UNSUPPORTED;
        }
    }
    return BASP_OK;
}

int prepare_seq_to_head(const basp_plan &p, const void *q, const void *k, const void *v, void *out,
                        TileLaunch &L)
{
    std::memset(&L, 0, sizeof(L));
    const uint64_t qb = uint64_t(p.q_elems) * p.es, kb = uint64_t(p.kv_elems) * p.es;
    const Buf ins[3] = {{q, qb}, {k, kb}, {v, kb}};
    const Buf outs[1] = {{out, qb + 2 * kb}};
    const int s = check_buffers(p, ins, 3, outs, 1);
    if (s != BASP_OK || p.S == 0)
        return s;
    const uint64_t o = addr(out);
    const SegSpec segs[3] = {{addr(q), o, uint32_t(p.Hq)},
                             {addr(k), o + qb, uint32_t(p.Hkv)},
                             {addr(v), o + qb + kb, uint32_t(p.Hkv)}};
    return build_tiles(p, segs, 3, true, L);
}

int prepare_head_to_seq(const basp_plan &p, const void *o, void *out, TileLaunch &L)
{
    std::memset(&L, 0, sizeof(L));
    const uint64_t qb = uint64_t(p.q_elems) * p.es;
    const Buf ins[1] = {{o, qb}};
    const Buf outs[1] = {{out, qb}};
    const int s = check_buffers(p, ins, 1, outs, 1);
    if (s != BASP_OK || p.S == 0)
        return s;
    const SegSpec segs[1] = {{addr(out), addr(o), uint32_t(p.Hq)}};
    return build_tiles(p, segs, 1, false, L);
}

int prepare_seq_to_head_o(const basp_plan &p, const void *dout, void *out, TileLaunch &L)
{
    std::memset(&L, 0, sizeof(L));
    const uint64_t qb = uint64_t(p.q_elems) * p.es;
    const Buf ins[1] = {{dout, qb}};
    const Buf outs[1] = {{out, qb}};
    const int s = check_buffers(p, ins, 1, outs, 1);
    if (s != BASP_OK || p.S == 0)
        return s;
    const SegSpec segs[1] = {{addr(dout), addr(out), uint32_t(p.Hq)}};
    return build_tiles(p, segs, 1, true, L);
}

int prepare_head_to_seq_qkv(const basp_plan &p, const void *in, void *dq, void *dk, void *dv,
                            TileLaunch &L)
{
    std::memset(&L, 0, sizeof(L));
    const uint64_t qb = uint64_t(p.q_elems) * p.es, kb = uint64_t(p.kv_elems) * p.es;
    const Buf ins[1] = {{in, qb + 2 * kb}};
    const Buf outs[3] = {{dq, qb}, {dk, kb}, {dv, kb}};
    const int s = check_buffers(p, ins, 1, outs, 3);
    if (s != BASP_OK || p.S == 0)
        return s;
    const uint64_t i = addr(in);
    const SegSpec segs[3] = {{addr(dq), i, uint32_t(p.Hq)},
                             {addr(dk), i + qb, uint32_t(p.Hkv)},
                             {addr(dv), i + qb + kb, uint32_t(p.Hkv)}};
    return build_tiles(p, segs, 3, false, L);
}

int check_autotune_buffers(const basp_plan &p, const void *q, const void *k, const void *v,
                           void *qkv, const void *o, void *o_out)
{
    // autotune runs both directions back to back on these buffers, so each
    // output must be clear of every input of either call and of the other
    // output, not only of its own call's input
    const uint64_t qb = uint64_t(p.q_elems) * p.es, kb = uint64_t(p.kv_elems) * p.es;
    const Buf ins[4] = {{q, qb}, {k, kb}, {v, kb}, {o, qb}};
    const Buf outs[2] = {{qkv, qb + 2 * kb}, {o_out, qb}};
    return check_buffers(p, ins, 4, outs, 2);
}

int prepare_seq_to_head_unfused(const basp_plan &p, const void *q, const void *k, const void *v,
                                void *out, void *ws, PermLaunch L[3])
{
    std::memset(L, 0, 3 * sizeof(PermLaunch));
    const uint64_t qb = uint64_t(p.q_elems) * p.es, kb = uint64_t(p.kv_elems) * p.es;
    const uint64_t tot = qb + 2 * kb;
    const Buf ins[3] = {{q, qb}, {k, kb}, {v, kb}};
    const Buf outs[2] = {{out, tot}, {ws, 2 * tot}};
    int s = check_buffers(p, ins, 3, outs, 2);
    if (s != BASP_OK || p.S == 0)
        return s;

    const uint64_t w1 = addr(ws), w2 = w1 + tot, o = addr(out);
    const uint64_t src[3] = {addr(q), addr(k), addr(v)};
    const uint64_t off[3] = {0, qb, qb + kb};
    const uint64_t bytes[3] = {qb, kb, kb};
    const uint32_t heads[3] = {uint32_t(p.Hq), uint32_t(p.Hkv), uint32_t(p.Hkv)};
    const int vw = vector_width(p);

    const uint32_t N = p.N, P = p.P, Bl = p.Bl, St = uint32_t(p.St), G = p.G;
    PermSpec pack[3], xchg[3], unpack[3];
    for (int i = 0; i < 3; ++i) {
        const uint32_t H = heads[i], Hl = H / P;
        const uint64_t rows = bytes[i] / p.row_bytes;
        const uint32_t C = Bl * St * Hl;  // rows of one per-peer chunk
        // (1) pack each rank's shard by destination member:
        //     [r][Bl][St][P*Hl] -> [r][jh][Bl][St][Hl]
        pack[i] = {src[i], w1 + off[i], bytes[i], bytes[i],
                   {N, P, Bl, St, Hl}, {Bl * St * H, Hl, St * H, H, 1}, rows};
        // (2) exchange: chunk jh of rank (g, js) becomes chunk js of rank (g, jh)
        xchg[i] = {w1 + off[i], w2 + off[i], bytes[i], bytes[i],
                   {G, P, P, C, 1}, {P * P * C, C, P * C, 1, 0}, rows};
        // (3) unpack [r][js][Bl][St][Hl] into the head-sharded layout
        if (p.layout == BASP_LAYOUT_HEAD_MAJOR)
            unpack[i] = {w2 + off[i], o + off[i], bytes[i], bytes[i],
                         {N, Bl, Hl, P, St}, {P * C, St * Hl, 1, C, Hl}, rows};
        else
            unpack[i] = {w2 + off[i], o + off[i], bytes[i], bytes[i],
                         {N, Bl, P, St, Hl}, {P * C, St * Hl, C, Hl, 1}, rows};
    }
    if ((s = build_perm(p, pack, 3, vw, L[0])) != BASP_OK)
        return s;
    if ((s = build_perm(p, xchg, 3, vw, L[1])) != BASP_OK)
        return s;
    return build_perm(p, unpack, 3, vw, L[2]);
}

}  // namespace basp
