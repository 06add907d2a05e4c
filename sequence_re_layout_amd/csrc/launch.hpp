// launch.hpp -- launch descriptors of the re-layout kernels and the index
// arithmetic every lane runs, as plain C++ shared by the HIP kernels and the
// host-side planning code.
//
// The exchange at the attention boundary (BASP review page, "Summary";
// "Scope & Claims") moves (token, head) rows of d*es bytes: member js of
// group g holds tokens [js*St, (js+1)*St) of every head before attention,
// member jh holds heads [jh*Hl, (jh+1)*Hl) of every token after it.
//
// Tile kernel.  A work tile is the rectangle
//     tokens [t0, t0+Ts) of source member js  x  heads [hl0, hl0+Th) of
//     destination member jh,  for one group g and local sequence bl.
// Inside a tile both layouts are 2-D strided arrays of rows:
//     sequence-sharded  t*H*row + h*row
//     head-major        h*S*row + t*row
//     token-major       t*Hl*row + h*row
// so a work-group computes the tile's two base addresses once and each lane
// only adds 32-bit offsets.
//
// Launch grid.  blockIdx.z is the batch index b, blockIdx.y one group member
// and blockIdx.x a tile of the (y, z) plane, Q, K and V planes one after the
// other; optionally the batch index is folded into x instead (tile_and_batch).
// Three tile orders, x running over (slow, middle, fast) digits:
//   1, token blocks fastest (the head-sharded layout's order): y = jh and x
//     runs over (hb, js, tb), so neighbouring tiles continue one destination
//     head across source members;
//   2, head blocks fastest (the sequence-sharded layout's order): y = js and
//     x runs over (tb, jh, hb), so neighbouring tiles continue one source
//     token across destination members;
//   3, token blocks fastest within a source member: y = js and x runs over
//     (jh, hb, tb), so neighbouring tiles continue one head through the
//     member's token chunk, and the tiles that run at one time take the
//     neighbouring heads of the same tokens.
// Neighbouring tiles run at the same time and share the DRAM pages of one
// side.  Optionally each XCD takes one contiguous eighth of a plane
// (xcd_tile).  The staged variant passes each tile through LDS in one pass:
// loads in the source's contiguous order, stores in the destination's
// (tile_vector with an explicit lane order).
//
// Perm kernel (unfused baseline).  Writes its destination linearly; row i of
// the destination has digits (d0..d4), d4 fastest, and is read from source
// row sum(d_k * sstride_k).
#pragma once

#include <cstdint>

#include "fastdiv.hpp"

struct basp_plan;

namespace basp {

constexpr int kBlock = 256;               // threads per work-group unless tuned (4 waves)
constexpr uint64_t kI31Max = 0x7fffffffull;
// Buffer descriptors span at most kI31Max bytes and every real offset is
// below that, so a lane given kOutside touches nothing: its load returns zero
// and its store is dropped.
constexpr uint32_t kOutside = 0x80000000u;

// One tensor of a tile launch.
struct TileSeg {
    uint64_t seq, head;            // buffer addresses
    uint64_t bytes;                // bytes of the tensor (the same on both sides)
    uint32_t seq_tok;              // byte stride of a token, sequence-sharded
    uint32_t head_tok;             // byte stride of a token, head-sharded
    uint32_t head_head_lane;       // head stride inside a tile (0 when Th == 1)
    uint32_t Hl;                   // heads per rank
    FastDiv Ts, Th;                // tile extent in tokens and heads
    FastDiv fast;                  // blocks along the fast axis: token blocks per
                                   // member chunk, or head blocks per rank
    FastDiv mid;                   // extent of x's middle digit: P, or head
                                   // blocks per rank (tile order 3)
    uint32_t tile_begin;           // this tensor's first tile in the plane (0 for
                                   // the first, which one-tensor launches rely on)
};

// Launch-wide fields first: a kernel reads them in one batch of scalar
// loads, then the one TileSeg its tile belongs to in a second batch.
struct TileDesc {
    uint32_t plane;                // tiles per (y, z) plane
    uint32_t seg_end0, seg_end1;   // ends of the first and second tensor's tiles
    uint32_t St;
    uint32_t S;
    uint32_t token_major;          // head-sharded side is [Bl][S][Hl][d] (else [Bl][Hl][S][d])
    uint32_t row;                  // bytes per (token, head) row
    uint32_t s_fast;               // lanes along tokens (1) or heads (0)
    uint32_t load_s_fast;          // staged kernel: lane order of the loads
    uint32_t store_s_fast;         //   and of the stores
    uint32_t order;                // tile order 1, 2 or 3 (see above)
    uint32_t xcd_span;             // tiles per XCD when remapped, else 0
    uint32_t Bl;                   // sequences per group
    uint32_t gstride;              // (P - 1) * Bl (see tile_origin)
    FastDiv Blf;                   // Bl, for the group of a batch index
    FastDiv P, A;                  // group size, vectors per row
    uint32_t batch_x;              // batch index folded into x (else blockIdx.z)
    uint32_t xbound;               // tiles along x: plane, or plane * B with batch_x
    FastDiv nb;                    // B
    TileSeg seg[3];
};

// A work-group's tile of the plane and its batch index.  Either the grid's z
// coordinate is the batch index, or (batch_x) x runs over (tile, batch
// index) with the batch index fastest, so neighbouring work-groups take the
// same tile of consecutive sequences.
BASP_HD inline void tile_and_batch(const TileDesc &D, uint32_t x, uint32_t z, uint32_t &tile, uint32_t &b)
{
    if (D.batch_x) {
        tile = fastdiv(x, D.nb);
        b = x - tile * D.nb.d;
    } else {
        tile = x;
        b = z;
    }
}

// Work-groups are dispatched round-robin over the 8 XCDs.  With
// xcd_span = plane/8 > 0 the i-th tile of a plane is renumbered so that
// consecutive work-groups of one XCD walk one contiguous eighth of the first
// 8*xcd_span tiles; the remaining tiles keep their number.  A bijection.
constexpr uint32_t kXcds = 8;

BASP_HD inline uint32_t xcd_tile(uint32_t x, uint32_t span)
{
    return x < kXcds * span ? (x % kXcds) * span + x / kXcds : x;
}

// Where a tile starts and how much of it is real.
struct TileOrigin {
    uint64_t seq_off, head_off;    // byte offsets of the tile base
    uint32_t ns, nh;               // tokens and heads present (ragged tail)
};

// The tensor a (remapped) tile of the plane belongs to.
BASP_HD inline uint32_t tile_segment(const TileDesc &D, uint32_t tile)
{
    return tile < D.seg_end0 ? 0u : (tile < D.seg_end1 ? 1u : 2u);
}

// Tile `local` of tensor sg (its tile of the plane, after xcd_tile, less
// sg.tile_begin), in the plane of group member y and batch index b.
BASP_HD inline TileOrigin tile_origin(const TileDesc &D, const TileSeg &sg, uint32_t local, uint32_t y,
                                      uint32_t b)
{
    TileOrigin o;
    const uint32_t P = D.P.d;
    // x = (slow, m, f): order 1 (hb, js, tb), 2 (tb, jh, hb), 3 (jh, hb, tb)
    const uint32_t q = fastdiv(local, sg.fast), f = local - q * sg.fast.d;
    const uint32_t slow = fastdiv(q, sg.mid), m = q - slow * sg.mid.d;
    const bool o1 = D.order == 1, o2 = D.order == 2;
    const uint32_t tb = o2 ? slow : f;
    const uint32_t hb = o2 ? f : (o1 ? slow : m);
    const uint32_t js = o1 ? m : y;
    const uint32_t jh = o1 ? y : (o2 ? m : slow);
    const uint32_t Ts = sg.Ts.d, Th = sg.Th.d, Hl = sg.Hl;
    const uint32_t t0 = tb * Ts, hl0 = hb * Th;
    o.ns = D.St - t0 < Ts ? D.St - t0 : Ts;
    o.nh = Hl - hl0 < Th ? Hl - hl0 : Th;
    // Row indices of the tile base in 32 bits (a tensor holds fewer than 2^32
    // rows; the host checks), then one widening multiply by the row size.
    // Rank r = g*P + j holds local sequence bl of batch index b = g*Bl + bl,
    // so r*Bl + bl = b + g*(P-1)*Bl + j*Bl with g = b / Bl.  (Ulysses has
    // g = 0; BASP has Bl = 1, which gives b*P + j; the data-parallel fallback
    // has P = 1, which gives b.)
    // Sequence-sharded: ((r*Bl + bl)*St + t)*H + h with j = js and
    // h = jh*Hl + hl; head-sharded: ((r*Bl + bl)*Hl + hl)*S + s, or
    // ((r*Bl + bl)*S + s)*Hl + hl, with j = jh and s = js*St + t.
    const uint32_t rb = b + fastdiv(b, D.Blf) * D.gstride;
    const uint32_t pre_s = rb + js * D.Bl, pre_h = rb + jh * D.Bl;
    const uint32_t seq_row = (pre_s * D.St + t0) * (P * Hl) + jh * Hl + hl0;
    const uint32_t s0 = js * D.St + t0;
    const uint32_t head_row = D.token_major ? (pre_h * D.S + s0) * Hl + hl0 : (pre_h * Hl + hl0) * D.S + s0;
    o.seq_off = uint64_t(seq_row) * D.row;
    o.head_off = uint64_t(head_row) * D.row;
    return o;
}

// The vw-byte vector v of a tile, with lanes along tokens first (s_fast) or
// heads first: its byte offsets from the tile base in the sequence-sharded
// (so) and head-sharded (ho) buffers, and its slot in the tile's
// [token][head][vector] staging order (st).  Returns false for a vector
// outside the tile's present rows.
BASP_HD inline bool tile_vector(const TileDesc &D, const TileSeg &sg, uint32_t ns, uint32_t nh,
                                uint32_t v, uint32_t vw, bool s_fast, uint32_t &so, uint32_t &ho,
                                uint32_t &st)
{
    const uint32_t A = D.A.d, Ts = sg.Ts.d, Th = sg.Th.d;
    const uint32_t r = fastdiv(v, D.A), vi = v - r * A;
    const FastDiv fast = s_fast ? sg.Ts : sg.Th;
    const uint32_t slow = fastdiv(r, fast), fst = r - slow * fast.d;
    const uint32_t sl = s_fast ? fst : slow, hl = s_fast ? slow : fst;
    so = sl * sg.seq_tok + hl * D.row + vi * vw;
    ho = sl * sg.head_tok + hl * sg.head_head_lane + vi * vw;
    st = (sl * Th + hl) * A + vi;
    return (v < Ts * Th * A) & (sl < ns) & (hl < nh);
}

// Offsets of vector v in the direct kernel's lane order.
BASP_HD inline bool lane_offsets(const TileDesc &D, const TileSeg &sg, uint32_t ns, uint32_t nh,
                                 uint32_t v, uint32_t vw, uint32_t &so, uint32_t &ho)
{
    uint32_t st;
    return tile_vector(D, sg, ns, nh, v, vw, D.s_fast, so, ho, st);
}

struct PermSeg {
    uint64_t src, dst;
    uint64_t src_bytes, dst_bytes;
    FastDiv ext[4];        // extents of d1..d4
    uint32_t sstride[5];   // source strides in rows
    uint32_t nvec;         // vectors in this tensor
    uint32_t chunk_begin, chunk_end;
};

struct PermDesc {
    PermSeg seg[3];
    uint32_t nchunks;
    uint32_t row;
    FastDiv A;
};

constexpr int kPermVpt = 4;   // vectors per lane in the perm kernel

BASP_HD inline uint32_t perm_segment(const PermDesc &D, uint32_t chunk)
{
    return (chunk >= D.seg[0].chunk_end) + (chunk >= D.seg[1].chunk_end);
}

// Source byte offset of the vw-byte destination vector v of a tensor.
BASP_HD inline uint32_t perm_source(const PermDesc &D, const PermSeg &sg, uint32_t v, uint32_t vw)
{
    const uint32_t r = fastdiv(v, D.A), vi = v - r * D.A.d;
    uint32_t q = r, src_row = 0;
    for (int j = 3; j >= 0; --j) {
        const uint32_t qn = fastdiv(q, sg.ext[j]);
        src_row += (q - qn * sg.ext[j].d) * sg.sstride[j + 1];
        q = qn;
    }
    src_row += q * sg.sstride[0];
    return src_row * D.row + vi * vw;
}

// ------------------------------------------------------------ host side --

// A tile launch ready to go: descriptor, template parameters, grid.
struct TileLaunch {
    TileDesc D;
    int nseg;                 // tensors in the launch: 1 or 3
    int vw, vpt, policy;
    int block;                // threads per work-group: 64, 128 or 256
    bool s2h;                 // read sequence-sharded, write head-sharded
    bool staged;              // tiles pass through LDS (one pass per tile)
    uint32_t grid;            // work-groups along x (tiles loop beyond it); 0: nothing to launch
    uint32_t grid_y, grid_z;  // P group members, B batch indices
};

struct PermLaunch {
    PermDesc D;
    int vw;
    uint32_t grid;
};

// Checks and descriptors of each entry point (basp.h).  They return the
// status the entry point reports; on BASP_OK the launch(es) are filled.
int prepare_seq_to_head(const basp_plan &p, const void *q, const void *k, const void *v, void *out,
                        TileLaunch &L);
int prepare_head_to_seq(const basp_plan &p, const void *o, void *out, TileLaunch &L);
int prepare_seq_to_head_o(const basp_plan &p, const void *dout, void *out, TileLaunch &L);
int prepare_head_to_seq_qkv(const basp_plan &p, const void *in, void *dq, void *dk, void *dv,
                            TileLaunch &L);
int prepare_seq_to_head_unfused(const basp_plan &p, const void *q, const void *k, const void *v,
                                void *out, void *ws, PermLaunch L[3]);
// NULL, alignment and overlap checks of the six buffers of basp_plan_autotune
// taken together (each output against all four inputs and the other output).
int check_autotune_buffers(const basp_plan &p, const void *q, const void *k, const void *v,
                           void *qkv, const void *o, void *o_out);

}  // namespace basp
