// relayout.hip -- gfx950 kernels of libbasp and the C-ABI entry points that
// launch them (include/basp.h).  Launch planning and the per-lane index
// arithmetic are in launch.hpp / launch.cpp.
//
// Each kernel moves (token, head) rows whole with 16-byte vector accesses
// (8/4/2 bytes when the row size is not a multiple of 16 bytes; pointers
// need only their element alignment) and never interprets values.  A lane first issues all of its VPT loads, then its
// stores, with no branch in between, so the loads of a wave overlap.
//
// Every access is a raw buffer instruction through a descriptor that covers
// only what is left of the buffer being accessed: an index error can at worst
// read zeros or drop a store; it cannot reach memory outside the caller's
// buffers.  Lanes past a ragged tile edge use an offset outside the
// descriptor, so they need no branch either.
#include <hip/hip_runtime.h>

#include <hip/hip_ext.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#define BASP_HD __host__ __device__
#include "launch.hpp"
#include "plan_internal.hpp"

namespace basp {
namespace {

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor word 3: raw access, 32-bit format

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int VW> struct Vec;
template <> struct Vec<16> { typedef u32x4 type; };
template <> struct Vec<8> { typedef u32x2 type; };
template <> struct Vec<4> { typedef uint32_t type; };
template <> struct Vec<2> { typedef uint16_t type; };

// Cache-policy bits of gfx940-family memory instructions: SC0 (bit 0) and
// SC1 (bit 4) give the coherence scope, NT (bit 1) marks a line that is not
// expected to be reused.
constexpr int kSC0 = 1, kNT = 2, kSC1 = 16;
template <int POL> struct Policy;
template <> struct Policy<1> { static constexpr int load = 0, store = 0; };
template <> struct Policy<2> { static constexpr int load = 0, store = kNT; };
template <> struct Policy<3> { static constexpr int load = kNT, store = kNT; };
template <> struct Policy<4> { static constexpr int load = kNT, store = kNT | kSC1; };
template <> struct Policy<5> { static constexpr int load = kNT | kSC0 | kSC1, store = kNT | kSC0 | kSC1; };

// Bytes of a buffer of `bytes` bytes from offset `off` on (0 past the end).
__device__ inline uint64_t rest(uint64_t bytes, uint64_t off) { return off < bytes ? bytes - off : 0; }

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, uint64_t bytes)
{
    const uint32_t n = static_cast<uint32_t>(bytes > kI31Max ? kI31Max : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0,
                                             static_cast<int>(n), kRsrcWord3);
}

template <int VW, int AUX>
__device__ inline typename Vec<VW>::type vload(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (VW == 16)
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    else if constexpr (VW == 8)
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    else if constexpr (VW == 4)
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
    else
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
}

template <int VW, int AUX>
__device__ inline void vstore(__amdgpu_buffer_rsrc_t r, uint32_t off, typename Vec<VW>::type x)
{
    if constexpr (VW == 16)
        __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, AUX);
    else if constexpr (VW == 8)
        __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, AUX);
    else if constexpr (VW == 4)
        __builtin_amdgcn_raw_buffer_store_b32(x, r, off, 0, AUX);
    else
        __builtin_amdgcn_raw_buffer_store_b16(x, r, off, 0, AUX);
}

// The tensor a tile belongs to.  A launch of one tensor (ONE) reads it at a
// fixed offset of the descriptor, so a work-group's scalar loads go out in
// one batch before its first vector load; selecting it by the tile's index
// makes the work-group wait for the launch-wide fields first, a second round
// of scalar loads that cost small one-tensor calls about 0.2 us of start-up
// (measured: 3.16 against 2.95 us for a 4 MiB head->seq).
template <bool ONE>
__device__ inline uint32_t segment_of(const TileDesc &D, uint32_t t)
{
    return ONE ? 0u : tile_segment(D, t);
}

// A fused launch reads the launch-wide fields, then its tile's tensor record
// at an offset that depends on them: a later round of scalar loads, which
// on a CU's first work-groups misses in the scalar cache again.  Loading
// one word of every cache line the records occupy in the first round
// (values discarded) makes the later rounds hits.  Lines 0x00 and 0x40 hold
// the launch-wide fields, which every work-group loads anyway.
static_assert(offsetof(TileDesc, seg) < 0x80 && sizeof(TileDesc) > 0x180 && sizeof(TileDesc) <= 0x1c0,
              "touch_records() covers the descriptor's lines from 0x80 on");

struct Touched {
    uint32_t w[5];
};

__device__ inline Touched touch_records()
{
    Touched t{};
#if defined(__HIP_DEVICE_COMPILE__)
    const auto k = __builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("s_load_dword %0, %5, 0x80\n\t"
                 "s_load_dword %1, %5, 0xc0\n\t"
                 "s_load_dword %2, %5, 0x100\n\t"
                 "s_load_dword %3, %5, 0x140\n\t"
                 "s_load_dword %4, %5, 0x180"
                 : "=s"(t.w[0]), "=s"(t.w[1]), "=s"(t.w[2]), "=s"(t.w[3]), "=s"(t.w[4])
                 : "s"(k));
#endif
    return t;
}

// The touched registers stay allocated until here.  `after` is a field of
// the tile's record: the compiler waits for the scalar loads (all of them:
// they return out of order) before it reads it, so none of the touches is
// still in flight once the registers are released.
__device__ inline void release(const Touched &t, uint64_t after)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::"s"(t.w[0]), "s"(t.w[1]), "s"(t.w[2]), "s"(t.w[3]), "s"(t.w[4]), "s"(after));
#endif
}

// Fused re-layout of up to three tensors: S2H reads the sequence-sharded
// side and writes the head-sharded side, !S2H the reverse.  ONE: a launch of
// one tensor.
template <int BS, int VW, int VPT, int POL, bool S2H, bool ONE>
__global__ __launch_bounds__(BS) void tile_kernel(const TileDesc D)
{
    using V = typename Vec<VW>::type;
    // a launch has at most D.xbound work-groups along x, so each has a tile;
    // testing only after the first lets the first tile's scalar loads go
    // out in one batch
    uint32_t x = blockIdx.x;
    Touched touched;
    if constexpr (!ONE)
        touched = touch_records();
    do {
        uint32_t tile, bz;
        tile_and_batch(D, x, blockIdx.z, tile, bz);
        const uint32_t t = xcd_tile(tile, D.xcd_span);
        const TileSeg sg = D.seg[segment_of<ONE>(D, t)];   // one batch of scalar loads
        if constexpr (!ONE)
            release(touched, sg.seq);
        const TileOrigin o = tile_origin(D, sg, ONE ? t : t - sg.tile_begin, blockIdx.y, bz);
        const __amdgpu_buffer_rsrc_t rseq = make_rsrc(sg.seq + o.seq_off, rest(sg.bytes, o.seq_off));
        const __amdgpu_buffer_rsrc_t rhead =
            make_rsrc(sg.head + o.head_off, rest(sg.bytes, o.head_off));
        const uint32_t nvec = sg.Ts.d * sg.Th.d * D.A.d;
        for (uint32_t v0 = 0; v0 < nvec; v0 += BS * VPT) {
            uint32_t src[VPT], dst[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                uint32_t so, ho;
                const bool ok = lane_offsets(D, sg, o.ns, o.nh, v0 + threadIdx.x + k * BS, VW, so, ho);
                src[k] = ok ? (S2H ? so : ho) : kOutside;
                dst[k] = ok ? (S2H ? ho : so) : kOutside;
            }
            V buf[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                buf[k] = vload<VW, Policy<POL>::load>(S2H ? rseq : rhead, src[k]);
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                vstore<VW, Policy<POL>::store>(S2H ? rhead : rseq, dst[k], buf[k]);
        }
    } while ((x += gridDim.x) < D.xbound);
}

// The same re-layout with each tile staged through LDS: the loads run along
// the source layout's contiguous axis, the stores along the destination's, so
// both sides of every wave instruction are contiguous.  A tile is one pass of
// the work-group (the host sizes it to at most BS*VPT vectors).
template <int BS, int VPT, int POL, bool S2H, bool ONE>
__global__ __launch_bounds__(BS) void tile_kernel_staged(const TileDesc D)
{
    using V = typename Vec<16>::type;
    __shared__ V stage[BS * VPT];
    // a launch has at most D.xbound work-groups along x, so each has a tile;
    // testing only after the first lets the first tile's scalar loads go
    // out in one batch
    uint32_t x = blockIdx.x;
    Touched touched;
    if constexpr (!ONE)
        touched = touch_records();
    do {
        uint32_t tile, bz;
        tile_and_batch(D, x, blockIdx.z, tile, bz);
        const uint32_t t = xcd_tile(tile, D.xcd_span);
        const TileSeg sg = D.seg[segment_of<ONE>(D, t)];   // one batch of scalar loads
        if constexpr (!ONE)
            release(touched, sg.seq);
        const TileOrigin o = tile_origin(D, sg, ONE ? t : t - sg.tile_begin, blockIdx.y, bz);
        const __amdgpu_buffer_rsrc_t rseq = make_rsrc(sg.seq + o.seq_off, rest(sg.bytes, o.seq_off));
        const __amdgpu_buffer_rsrc_t rhead =
            make_rsrc(sg.head + o.head_off, rest(sg.bytes, o.head_off));
        uint32_t off[VPT], slot[VPT];
        bool ok[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            uint32_t so, ho;
            ok[k] = tile_vector(D, sg, o.ns, o.nh, threadIdx.x + k * BS, 16, D.load_s_fast, so,
                                ho, slot[k]);
            off[k] = ok[k] ? (S2H ? so : ho) : kOutside;
        }
        V buf[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            buf[k] = vload<16, Policy<POL>::load>(S2H ? rseq : rhead, off[k]);
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            if (ok[k])
                stage[slot[k]] = buf[k];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            uint32_t so, ho;
            ok[k] = tile_vector(D, sg, o.ns, o.nh, threadIdx.x + k * BS, 16, D.store_s_fast, so,
                                ho, slot[k]);
            off[k] = ok[k] ? (S2H ? ho : so) : kOutside;
            buf[k] = stage[ok[k] ? slot[k] : 0];
        }
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            vstore<16, Policy<POL>::store>(S2H ? rhead : rseq, off[k], buf[k]);
        __syncthreads();   // the next tile reuses the staging area
    } while ((x += gridDim.x) < D.xbound);
}

// One pass of the unfused baseline: linear destination, permuted source.
template <int VW>
__global__ __launch_bounds__(kBlock) void perm_kernel(const PermDesc D)
{
    using V = typename Vec<VW>::type;
    for (uint32_t chunk = blockIdx.x; chunk < D.nchunks; chunk += gridDim.x) {
        const PermSeg &sg = D.seg[perm_segment(D, chunk)];
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sg.src, sg.src_bytes);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(sg.dst, sg.dst_bytes);
        const uint32_t base = (chunk - sg.chunk_begin) * (kBlock * kPermVpt);
        uint32_t src[kPermVpt], dst[kPermVpt];
#pragma unroll
        for (int k = 0; k < kPermVpt; ++k) {
            const uint32_t v = base + threadIdx.x + k * kBlock;
            const bool ok = v < sg.nvec;
            src[k] = ok ? perm_source(D, sg, v, VW) : kOutside;
            dst[k] = ok ? v * VW : kOutside;
        }
        V buf[kPermVpt];
#pragma unroll
        for (int k = 0; k < kPermVpt; ++k)
            buf[k] = vload<VW, 0>(rs, src[k]);
#pragma unroll
        for (int k = 0; k < kPermVpt; ++k)
            vstore<VW, kNT>(rd, dst[k], buf[k]);
    }
}

// Plain copy with the same access rules, the ceiling the re-layout kernels
// are measured against: chunk c is bytes [c*kCopyWg, (c+1)*kCopyWg), one
// 16-byte vector per lane, read and written through descriptors that cover
// only the rest of each buffer, so lanes past the end read zeros and drop
// the store.  Work-groups loop over chunks beyond the grid cap.
constexpr int kCopyBlock = 64;
constexpr uint32_t kCopyWg = kCopyBlock * 16;
constexpr uint32_t kCopyGridCap = 1u << 22;

struct CopyDesc {
    uint64_t src, dst, bytes, chunks;
};

__global__ __launch_bounds__(kCopyBlock) void stream_copy_kernel(const CopyDesc D)
{
    for (uint64_t c = blockIdx.x; c < D.chunks; c += gridDim.x) {
        const uint64_t base = c * kCopyWg;   // < D.bytes
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(D.src + base, D.bytes - base);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(D.dst + base, D.bytes - base);
        const uint32_t off = threadIdx.x * 16;
        const u32x4 x = vload<16, Policy<4>::load>(rs, off);
        vstore<16, Policy<4>::store>(rd, off, x);
    }
}

typedef void (*TileFn)(const TileDesc);

// Kernel instances: 16-byte vectors with every work-group size, vectors per
// lane, cache policy and direction, direct or staged; narrower vectors direct
// with 256 threads and 4 vectors per lane.
template <int BS, int VW, int VPT, int POL>
TileFn direct_fn(bool s2h, bool one)
{
    if (one)
        return s2h ? tile_kernel<BS, VW, VPT, POL, true, true> : tile_kernel<BS, VW, VPT, POL, false, true>;
    return s2h ? tile_kernel<BS, VW, VPT, POL, true, false> : tile_kernel<BS, VW, VPT, POL, false, false>;
}

template <int BS, int VPT, int POL>
TileFn staged_fn(bool s2h, bool one)
{
    if (one)
        return s2h ? tile_kernel_staged<BS, VPT, POL, true, true> : tile_kernel_staged<BS, VPT, POL, false, true>;
    return s2h ? tile_kernel_staged<BS, VPT, POL, true, false> : tile_kernel_staged<BS, VPT, POL, false, false>;
}

template <int BS, int VW, int VPT>
TileFn by_policy(int pol, bool s2h, bool staged, bool one)
{
    switch (pol) {
    case 1: return staged ? staged_fn<BS, VPT, 1>(s2h, one) : direct_fn<BS, VW, VPT, 1>(s2h, one);
    case 2: return staged ? staged_fn<BS, VPT, 2>(s2h, one) : direct_fn<BS, VW, VPT, 2>(s2h, one);
    case 4: return staged ? staged_fn<BS, VPT, 4>(s2h, one) : direct_fn<BS, VW, VPT, 4>(s2h, one);
    case 5: return staged ? staged_fn<BS, VPT, 5>(s2h, one) : direct_fn<BS, VW, VPT, 5>(s2h, one);
    default: return staged ? staged_fn<BS, VPT, 3>(s2h, one) : direct_fn<BS, VW, VPT, 3>(s2h, one);
    }
}

template <int BS>
TileFn by_vpt(int vpt, int pol, bool s2h, bool staged, bool one)
{
    switch (vpt) {
    case 1: return by_policy<BS, 16, 1>(pol, s2h, staged, one);
    case 2: return by_policy<BS, 16, 2>(pol, s2h, staged, one);
    case 8: return by_policy<BS, 16, 8>(pol, s2h, staged, one);
    default: return by_policy<BS, 16, 4>(pol, s2h, staged, one);
    }
}

template <int VW>
TileFn narrow_fn(int pol, bool s2h, bool one)
{
    switch (pol) {
    case 1: return direct_fn<kBlock, VW, 4, 1>(s2h, one);
    case 2: return direct_fn<kBlock, VW, 4, 2>(s2h, one);
    case 4: return direct_fn<kBlock, VW, 4, 4>(s2h, one);
    case 5: return direct_fn<kBlock, VW, 4, 5>(s2h, one);
    default: return direct_fn<kBlock, VW, 4, 3>(s2h, one);
    }
}

// Kernel instance of a launch: one tensor or up to three, vector width, work-
// group size, vectors per lane, cache policy, direction, direct or staged.
TileFn tile_fn(const TileLaunch &L)
{
    const bool one = L.nseg == 1;
    if (L.vw == 16) {
        switch (L.block) {
        case 64: return by_vpt<64>(L.vpt, L.policy, L.s2h, L.staged, one);
        case 128: return by_vpt<128>(L.vpt, L.policy, L.s2h, L.staged, one);
        default: return by_vpt<256>(L.vpt, L.policy, L.s2h, L.staged, one);
        }
    }
    switch (L.vw) {
    case 8: return narrow_fn<8>(L.policy, L.s2h, one);
    case 4: return narrow_fn<4>(L.policy, L.s2h, one);
    default: return narrow_fn<2>(L.policy, L.s2h, one);
    }
}

// Events set by basp_time_next_call for the next call of this thread.
struct Timing {
    hipEvent_t start = nullptr, stop = nullptr;
};
thread_local Timing t_timing;

// The launch's own status (not the thread's sticky last error, which other
// code in the process may have left set).  first/last: this launch opens or
// closes the current entry-point call, for the timing events.
template <typename Desc>
basp_status launch_kernel(const void *fn, dim3 grid, int block, const Desc &D, void *stream,
                          bool first, bool last)
{
    void *args[] = {const_cast<Desc *>(&D)};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (t_timing.start || t_timing.stop)
        e = hipExtLaunchKernel(fn, grid, dim3(block), args, 0, st,
                               first ? t_timing.start : nullptr, last ? t_timing.stop : nullptr, 0);
    else
        e = hipLaunchKernel(fn, grid, dim3(block), args, 0, st);
    return e == hipSuccess ? BASP_OK : BASP_ERR_HIP;
}

basp_status launch(const TileLaunch &L, void *stream)
{
    if (L.grid == 0)
        return BASP_OK;
    return launch_kernel(reinterpret_cast<const void *>(tile_fn(L)), dim3(L.grid, L.grid_y, L.grid_z),
                         L.block, L.D, stream,
                         true, true);
}

basp_status launch(const PermLaunch &L, void *stream, bool first, bool last)
{
    if (L.grid == 0)
        return BASP_OK;
    const void *fn;
    switch (L.vw) {
    case 16: fn = reinterpret_cast<const void *>(perm_kernel<16>); break;
    case 8: fn = reinterpret_cast<const void *>(perm_kernel<8>); break;
    case 4: fn = reinterpret_cast<const void *>(perm_kernel<4>); break;
    default: fn = reinterpret_cast<const void *>(perm_kernel<2>); break;
    }
    return launch_kernel(fn, dim3(L.grid), kBlock, L.D, stream, first, last);
}

// Runs f, the body of an entry point, and clears the timing request after it.
template <typename F>
basp_status timed_call(F f)
{
    const basp_status s = f();
    t_timing = Timing();
    return record(s);
}

// ---------------------------------------------------------------- autotune --

// Launch shapes a plan is measured with, all with non-temporal loads and
// non-temporal device-scope stores (the policy the sweeps preferred), over
// batch order x work-group size (64, 128, 256) x tile order x vectors per
// lane x heads per tile x XCD order, each direct with both lane orders and
// LDS-staged.  Vectors per lane: 1 and 2, and also 4 and 8 when the fused
// seq->head call moves at most kWideVectorBytes: only such small calls ran
// faster with the larger tiles (fewer work-groups to dispatch), and their
// launches are short, so measuring the extra shapes costs little.
constexpr int64_t kWideVectorBytes = int64_t{64} << 20;

std::vector<basp_tuning> autotune_candidates(const basp_plan &p)
{
    std::vector<basp_tuning> c;
    const int blocks[] = {64, 128, 256}, heads[] = {1, 2, 4, 8}, vpts[] = {1, 2, 4, 8};
    const int nvpt = 2 * (p.q_elems + 2 * p.kv_elems) * p.es <= kWideVectorBytes ? 4 : 2;
    for (int bo = 1; bo <= 2; ++bo)
        for (int block : blocks)
            for (int to = 1; to <= 3; ++to)
                for (int iv = 0; iv < nvpt; ++iv)
                    for (int th : heads)
                        for (int xcd = 1; xcd <= 2; ++xcd) {
                            basp_tuning t = {};
                            t.batch_order = bo;
                            t.block_size = block;
                            t.tile_order = to;
                            t.vectors_per_thread = vpts[iv];
                            t.tile_heads = th;
                            t.xcd_remap = xcd;
                            t.cache_policy = 4;
                            t.stage = 2;
                            c.push_back(t);
                            t.stage = 1;
                            for (int lo = 1; lo <= 2; ++lo) {
                                t.lane_order = lo;
                                c.push_back(t);
                            }
                        }
    return c;
}

// One timed launch of the autotuner: a direction and a candidate shape.
struct Job {
    int dir, cand;
    float ms;
};

// The six buffers of one autotuner step: seq->head reads q, k, v and writes
// qkv; head->seq reads o and writes o_out.
struct TuneBufs {
    const void *q, *k, *v;
    void *qkv;
    const void *o;
    void *o_out;
};

// Buffers the autotuner times on.  When the six buffers together fit well
// inside the device's caches (4 MB of L2 per XCD and the 256 MB Infinity
// Cache), timed launches on them read from the caches, and a shape that is
// fastest there can be slower in a loop of calls that streams from HBM
// (measured on the tiny workload's 16 MiB).  Below kRotateBelow the timed
// launches therefore rotate over copies of the buffers' sizes in a temporary
// pool of about kRotationBytes, so that every launch finds its inputs in
// HBM, and the pairs are ranked from HIP graph replays.  Larger calls are
// timed on the caller's own buffers: some shapes run up to 16% faster or
// slower depending on where their buffers lie relative to each other, so the
// caller's placement is the one to measure.  On the pool's placement the
// picks for 56 MB and 335 MB working sets were worse than on the caller's
// buffers.  The pool holds no meaningful values (the kernels copy bits and
// every shape computes the same permutation); it is freed when the
// autotuner returns.  If it cannot be allocated, the caller's buffers are
// used alone.
constexpr uint64_t kRotateBelow = uint64_t{32} << 20;
constexpr uint64_t kRotationBytes = uint64_t{1} << 30;
constexpr uint64_t kMaxRotation = 256;

class TuneSets {
public:
    TuneSets(const basp_plan &p, const TuneBufs &caller, hipStream_t st) : st_(st)
    {
        const uint64_t qb = round_up(uint64_t(p.q_elems) * p.es);
        const uint64_t kb = round_up(uint64_t(p.kv_elems) * p.es);
        const uint64_t tb = round_up(uint64_t(p.q_elems + 2 * p.kv_elems) * p.es);
        const uint64_t set = 3 * qb + 2 * kb + tb;   // q, k, v, qkv, o, o_out
        if (set < kRotateBelow) {
            const uint64_t r = std::min(kMaxRotation, std::max<uint64_t>(2, (kRotationBytes + set - 1) / set));
            if (hipMalloc(&pool_, r * set) == hipSuccess) {
                char *base = static_cast<char *>(pool_);
                for (uint64_t i = 0; i < r; ++i) {
                    char *b = base + i * set;
                    sets_.push_back({b, b + qb, b + qb + kb, b + qb + 2 * kb, b + qb + 2 * kb + tb,
                                     b + 2 * qb + 2 * kb + tb});
                }
            } else {
                pool_ = nullptr;
                (void)hipGetLastError();   // the caller's buffers serve alone
            }
        }
        if (sets_.empty())
            sets_.push_back(caller);
    }
    ~TuneSets()
    {
        if (pool_) {   // nothing may still use the pool when it is freed
            (void)hipStreamSynchronize(st_);
            (void)hipFree(pool_);
        }
    }
    TuneSets(const TuneSets &) = delete;
    TuneSets &operator=(const TuneSets &) = delete;

    // The buffers of the next timed step, in turn.
    const TuneBufs &take()
    {
        const TuneBufs &b = sets_[next_];
        next_ = (next_ + 1) % sets_.size();
        return b;
    }
    size_t count() const { return sets_.size(); }
    bool pooled() const { return pool_ != nullptr; }

private:
    static uint64_t round_up(uint64_t n) { return (n + 255) & ~uint64_t{255}; }
    hipStream_t st_;
    void *pool_ = nullptr;
    std::vector<TuneBufs> sets_;
    size_t next_ = 0;
};

// A direction's launch on one set of buffers with the plan's current tuning.
int prepare_dir(const basp_plan &p, int dir, const TuneBufs &b, TileLaunch &L)
{
    return dir == BASP_SEQ_TO_HEAD ? prepare_seq_to_head(p, b.q, b.k, b.v, b.qkv, L)
                                   : prepare_head_to_seq(p, b.o, b.o_out, L);
}

// Launch every job once, each timed from its own dispatch timestamps, in
// batches of kPool launches that share a pool of events.  Each timed launch
// comes right after an untimed launch of the other direction (partner, with
// the plan's shape on entry) on the same buffers, as in a step that runs the
// two back to back: a launch timed alone starts on a drained memory system,
// and launch shapes ranked that way did not keep their order back to back.
// False on a HIP error; a job whose shape the plan rejects gets a time < 0.
constexpr int kPool = 64;

bool run_jobs(basp_plan &p, const std::vector<basp_tuning> &cands, std::vector<Job> &jobs,
              const basp_tuning (&entry)[2], TuneSets &ts, void *stream, hipEvent_t *ev)
{
    for (size_t first = 0; first < jobs.size(); first += kPool) {
        const size_t last = std::min(jobs.size(), first + kPool);
        for (size_t j = first; j < last; ++j) {
            Job &job = jobs[j];
            const TuneBufs &b = ts.take();
            TileLaunch partner, L;
            p.tuning[1 - job.dir] = entry[1 - job.dir];
            p.tuning[job.dir] = cands[job.cand];
            job.ms = -1.f;
            if (prepare_dir(p, 1 - job.dir, b, partner) != BASP_OK)
                return false;   // the entry shapes were accepted on the caller's buffers
            if (prepare_dir(p, job.dir, b, L) != BASP_OK)
                continue;
            if (launch(partner, stream) != BASP_OK)
                return false;
            t_timing.start = ev[2 * (j - first)];
            t_timing.stop = ev[2 * (j - first) + 1];
            const basp_status ls = launch(L, stream);
            t_timing = Timing();
            if (ls != BASP_OK)
                return false;
            job.ms = 0.f;
        }
        if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
            return false;
        for (size_t j = first; j < last; ++j)
            if (jobs[j].ms == 0.f &&
                hipEventElapsedTime(&jobs[j].ms, ev[2 * (j - first)], ev[2 * (j - first) + 1]) != hipSuccess)
                return false;
    }
    return true;
}

// Median time of each (direction, candidate) over `rounds` rounds in which
// every pair is launched once, seq->head and head->seq alternating, so that
// slow drifts of the device affect all candidates alike.
bool measure_rounds(basp_plan &p, const std::vector<basp_tuning> &cands,
                    const std::vector<int> (&pick)[2], int rounds, std::vector<float> (&med)[2],
                    const basp_tuning (&entry)[2], TuneSets &ts, void *stream, hipEvent_t *ev)
{
    const size_t n = std::max(pick[0].size(), pick[1].size());
    std::vector<std::vector<float>> times[2];
    times[0].assign(pick[0].size(), {});
    times[1].assign(pick[1].size(), {});
    for (int r = 0; r < rounds; ++r) {
        std::vector<Job> jobs;
        for (size_t i = 0; i < n; ++i)
            for (int dir = 0; dir < 2; ++dir)
                if (i < pick[dir].size())
                    jobs.push_back({dir, pick[dir][i], 0.f});
        if (!run_jobs(p, cands, jobs, entry, ts, stream, ev))
            return false;
        size_t idx[2] = {0, 0};
        for (const Job &job : jobs)
            times[job.dir][idx[job.dir]++].push_back(job.ms);
    }
    for (int dir = 0; dir < 2; ++dir) {
        med[dir].clear();
        for (std::vector<float> &t : times[dir]) {
            std::nth_element(t.begin(), t.begin() + t.size() / 2, t.end());
            med[dir].push_back(t[t.size() / 2]);
        }
    }
    return true;
}

// Median seconds per step, over `rounds` rounds, of each pair (seq->head
// shape, head->seq shape): kSteps steps run back to back, each on the next
// set of buffers, timed by events recorded only before the first and after
// the last launch (the launches are prepared before the first event).  False
// on a HIP error; a pair whose shapes the plan rejects gets a time < 0.
bool measure_pairs(basp_plan &p, const std::vector<basp_tuning> &cands,
                   const std::vector<std::pair<int, int>> &pairs, int rounds, std::vector<float> &med,
                   TuneSets &ts, void *stream, hipEvent_t *ev)
{
    constexpr int kSteps = 6;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<std::vector<float>> times(pairs.size());
    for (int r = 0; r < rounds; ++r)
        for (size_t first = 0; first < pairs.size(); first += kPool) {
            const size_t last = std::min(pairs.size(), first + kPool);
            std::vector<bool> ran(last - first, false);
            for (size_t i = first; i < last; ++i) {
                p.tuning[BASP_SEQ_TO_HEAD] = cands[pairs[i].first];
                p.tuning[BASP_HEAD_TO_SEQ] = cands[pairs[i].second];
                TileLaunch ls[kSteps], lh[kSteps];
                bool fits = true;
                for (int n = 0; n < kSteps && fits; ++n) {
                    const TuneBufs &b = ts.take();
                    fits = prepare_dir(p, BASP_SEQ_TO_HEAD, b, ls[n]) == BASP_OK &&
                           prepare_dir(p, BASP_HEAD_TO_SEQ, b, lh[n]) == BASP_OK;
                }
                if (!fits)
                    continue;
                if (hipEventRecord(ev[2 * (i - first)], st) != hipSuccess)
                    return false;
                for (int n = 0; n < kSteps; ++n)
                    if (launch(ls[n], stream) != BASP_OK || launch(lh[n], stream) != BASP_OK)
                        return false;
                if (hipEventRecord(ev[2 * (i - first) + 1], st) != hipSuccess)
                    return false;
                ran[i - first] = true;
            }
            if (hipStreamSynchronize(st) != hipSuccess)
                return false;
            for (size_t i = first; i < last; ++i) {
                float ms = -1.f;
                if (ran[i - first] &&
                    hipEventElapsedTime(&ms, ev[2 * (i - first)], ev[2 * (i - first) + 1]) != hipSuccess)
                    return false;
                times[i].push_back(ms / kSteps);
            }
        }
    med.clear();
    for (std::vector<float> &t : times) {
        std::nth_element(t.begin(), t.begin() + t.size() / 2, t.end());
        med.push_back(t[t.size() / 2]);
    }
    return true;
}

// Seconds per step of each pair (seq->head shape, head->seq shape) from HIP
// graphs, for calls timed on the pool: each pair's `steps` back-to-back steps,
// each on the next set of pool buffers, are captured once on a private
// stream and the graphs are replayed in `rounds` interleaved rounds, so no
// host launch time enters a step (a small call's step is about as short as
// the host's launch of it) and slow drift of the device affects every pair
// alike.  The graphs touch only the pool, so the private stream needs no
// ordering with the caller's.  False on a HIP error (the caller then times
// the pairs eagerly); a pair whose shapes the plan rejects gets a time < 0.
bool measure_pairs_graphs(basp_plan &p, const std::vector<basp_tuning> &cands,
                          const std::vector<std::pair<int, int>> &pairs, int rounds, int steps,
                          std::vector<float> &med, TuneSets &ts, hipEvent_t *ev)
{
    hipStream_t cs;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess)
        return false;
    std::vector<hipGraphExec_t> exec(pairs.size(), nullptr);
    std::vector<TileLaunch> ls(steps), lh(steps);
    bool ok = true;
    for (size_t i = 0; i < pairs.size() && ok; ++i) {
        p.tuning[BASP_SEQ_TO_HEAD] = cands[pairs[i].first];
        p.tuning[BASP_HEAD_TO_SEQ] = cands[pairs[i].second];
        bool fits = true;
        for (int n = 0; n < steps && fits; ++n) {
            const TuneBufs &b = ts.take();
            fits = prepare_dir(p, BASP_SEQ_TO_HEAD, b, ls[n]) == BASP_OK &&
                   prepare_dir(p, BASP_HEAD_TO_SEQ, b, lh[n]) == BASP_OK;
        }
        if (!fits)
            continue;
        if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
            ok = false;
            break;
        }
        bool captured = true;
        for (int n = 0; n < steps && captured; ++n)
            captured = launch(ls[n], cs) == BASP_OK && launch(lh[n], cs) == BASP_OK;
        hipGraph_t g = nullptr;
        ok = hipStreamEndCapture(cs, &g) == hipSuccess && captured && g;
        ok = ok && hipGraphInstantiate(&exec[i], g, nullptr, nullptr, 0) == hipSuccess;
        if (g)
            (void)hipGraphDestroy(g);
        ok = ok && hipGraphLaunch(exec[i], cs) == hipSuccess;   // untimed first replay
    }
    ok = ok && hipStreamSynchronize(cs) == hipSuccess;
    std::vector<std::vector<float>> times(pairs.size());
    for (int r = 0; r < rounds && ok; ++r)
        for (size_t i = 0; i < pairs.size() && ok; ++i) {
            float ms = -1.f;
            if (exec[i]) {
                ok = hipEventRecord(ev[0], cs) == hipSuccess && hipGraphLaunch(exec[i], cs) == hipSuccess &&
                     hipEventRecord(ev[1], cs) == hipSuccess && hipStreamSynchronize(cs) == hipSuccess &&
                     hipEventElapsedTime(&ms, ev[0], ev[1]) == hipSuccess;
                ms /= steps;
            }
            times[i].push_back(ms);
        }
    for (hipGraphExec_t e : exec)
        if (e)
            (void)hipGraphExecDestroy(e);
    (void)hipStreamSynchronize(cs);
    (void)hipStreamDestroy(cs);
    if (!ok) {
        (void)hipGetLastError();
        return false;
    }
    med.clear();
    for (std::vector<float> &t : times) {
        std::nth_element(t.begin(), t.begin() + t.size() / 2, t.end());
        med.push_back(t[t.size() / 2]);
    }
    return true;
}

}  // namespace
}  // namespace basp

using basp::record;

extern "C" basp_status basp_plan_autotune(basp_plan *p, const void *q, const void *k,
                                          const void *v, void *qkv, const void *o, void *o_out,
                                          void *stream)
{
    basp::t_timing = basp::Timing();
    if (!p)
        return record(BASP_ERR_INVALID);
    // both directions must launch on the caller's buffers with the shapes on
    // entry (the partner launches of the timed rounds use those shapes)
    basp::TileLaunch entry_launch[2];
    const basp::TuneBufs caller = {q, k, v, qkv, o, o_out};
    int s = basp::check_autotune_buffers(*p, q, k, v, qkv, o, o_out);
    for (int dir = 0; dir < 2 && s == BASP_OK; ++dir)
        s = basp::prepare_dir(*p, dir, caller, entry_launch[dir]);
    if (s != BASP_OK || p->S == 0)
        return record(basp_status(s));

    constexpr int kCoarse = 3, kFine = 7, kKeep = 6, kPairRounds = 5;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t ev[2 * basp::kPool];
    int made = 0;
    // timing-only events: without the system-scope fence an event otherwise
    // performs when it completes (a cache writeback the launches of a plain
    // back-to-back step do not pay)
    for (; made < 2 * basp::kPool; ++made)
        if (hipEventCreateWithFlags(&ev[made], hipEventDisableSystemFence) != hipSuccess)
            break;
    const basp_tuning saved[2] = {p->tuning[0], p->tuning[1]};
    bool ok = made == 2 * basp::kPool;
    basp::TuneSets ts(*p, caller, st);
    // calls timed on the pool rank their pairs from HIP graph replays, which
    // time a step as a loop of calls runs it, so more pairs are worth timing
    const int kPairs = ts.pooled() ? 6 : 3;
    const std::vector<basp_tuning> cands = basp::autotune_candidates(*p);
    std::vector<int> pick[2];
    for (int dir = 0; dir < 2; ++dir)
        for (int i = 0; i < int(cands.size()); ++i)
            if (basp::check_launch_limits(*p, cands[i]) == BASP_OK)
                pick[dir].push_back(i);
    std::vector<float> med[2];
    // coarse pass over every candidate, then a longer one over the best few;
    // a direction without any measured candidate keeps its tuning
    ok = ok && basp::measure_rounds(*p, cands, pick, kCoarse, med, saved, ts, stream, ev);
    for (int dir = 0; dir < 2 && ok; ++dir) {
        std::vector<std::pair<float, int>> order;
        for (size_t i = 0; i < pick[dir].size(); ++i)
            if (med[dir][i] > 0.f)
                order.push_back({med[dir][i], pick[dir][i]});
        std::sort(order.begin(), order.end());
        pick[dir].clear();
        for (size_t i = 0; i < order.size() && int(i) < kKeep; ++i)
            pick[dir].push_back(order[i].second);
    }
    ok = ok && basp::measure_rounds(*p, cands, pick, kFine, med, saved, ts, stream, ev);
    // the best few of each direction, then every pair of them timed as whole
    // back-to-back steps: the shapes of the two directions affect each other
    std::vector<int> top[2];
    for (int dir = 0; dir < 2 && ok; ++dir) {
        std::vector<std::pair<float, int>> order;
        for (size_t i = 0; i < pick[dir].size(); ++i)
            if (med[dir][i] > 0.f)
                order.push_back({med[dir][i], pick[dir][i]});
        std::sort(order.begin(), order.end());
        for (size_t i = 0; i < order.size() && int(i) < kPairs; ++i)
            top[dir].push_back(order[i].second);
    }
    // the plan's shapes on entry compete as one more pair, so that a pick
    // which the single-launch rounds misjudged cannot replace a faster pair
    std::vector<basp_tuning> shapes = cands;
    shapes.push_back(saved[BASP_SEQ_TO_HEAD]);
    shapes.push_back(saved[BASP_HEAD_TO_SEQ]);
    const int entry = int(cands.size());
    std::vector<std::pair<int, int>> pairs;
    for (int a : top[0])
        for (int c : top[1])
            pairs.push_back({a, c});
    pairs.push_back({entry, entry + 1});
    std::vector<float> step;
    bool graphed = false;
    if (ok && ts.pooled()) {
        // steps per graph: about 0.4 ms of device time per replay
        const double step_s = double(p->q_elems * 2 + p->kv_elems * 2) * 2 * p->es / 5e12 + 5e-6;
        const int steps = std::max(6, std::min(100, int(4e-4 / step_s)));
        graphed = basp::measure_pairs_graphs(*p, shapes, pairs, kPairRounds, steps, step, ts, ev);
    }
    if (!graphed)
        ok = ok && basp::measure_pairs(*p, shapes, pairs, kPairRounds, step, ts, stream, ev);
    basp_tuning chosen[2] = {saved[0], saved[1]};
    int best = -1;
    for (size_t i = 0; ok && i < pairs.size(); ++i)
        if (step[i] > 0.f && (best < 0 || step[i] < step[best]))
            best = int(i);
    if (best >= 0) {
        chosen[BASP_SEQ_TO_HEAD] = shapes[pairs[best].first];
        chosen[BASP_HEAD_TO_SEQ] = shapes[pairs[best].second];
    } else {   // no pair measured: each direction's own best, where it has one
        for (int dir = 0; dir < 2; ++dir)
            if (!top[dir].empty())
                chosen[dir] = cands[top[dir][0]];
    }
    p->tuning[0] = chosen[0];
    p->tuning[1] = chosen[1];
    // the two calls once more on the caller's buffers, with the chosen
    // shapes: their outputs then hold the results whichever buffers the
    // timed launches used
    for (int dir = 0; dir < 2 && ok; ++dir) {
        basp::TileLaunch L;
        ok = basp::prepare_dir(*p, dir, caller, L) == BASP_OK && basp::launch(L, stream) == BASP_OK;
    }
    ok = ok && hipStreamSynchronize(st) == hipSuccess;
    for (int i = 0; i < made; ++i)
        (void)hipEventDestroy(ev[i]);
    if (!ok) {
        p->tuning[0] = saved[0];
        p->tuning[1] = saved[1];
        return record(BASP_ERR_HIP);
    }
    return record(BASP_OK);
}

extern "C" basp_status basp_time_next_call(void *start_event, void *stop_event)
{
    basp::t_timing.start = static_cast<hipEvent_t>(start_event);
    basp::t_timing.stop = static_cast<hipEvent_t>(stop_event);
    return record(BASP_OK);
}

extern "C" basp_status basp_seq_to_head(const basp_plan *p, const void *q, const void *k,
                                        const void *v, void *out, void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (!p)
            return BASP_ERR_INVALID;
        basp::TileLaunch L;
        const int s = basp::prepare_seq_to_head(*p, q, k, v, out, L);
        return s != BASP_OK ? basp_status(s) : basp::launch(L, stream);
    });
}

extern "C" basp_status basp_head_to_seq(const basp_plan *p, const void *o, void *out, void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (!p)
            return BASP_ERR_INVALID;
        basp::TileLaunch L;
        const int s = basp::prepare_head_to_seq(*p, o, out, L);
        return s != BASP_OK ? basp_status(s) : basp::launch(L, stream);
    });
}

extern "C" basp_status basp_seq_to_head_o(const basp_plan *p, const void *dout, void *out,
                                          void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (!p)
            return BASP_ERR_INVALID;
        basp::TileLaunch L;
        const int s = basp::prepare_seq_to_head_o(*p, dout, out, L);
        return s != BASP_OK ? basp_status(s) : basp::launch(L, stream);
    });
}

extern "C" basp_status basp_head_to_seq_qkv(const basp_plan *p, const void *in, void *dq,
                                            void *dk, void *dv, void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (!p)
            return BASP_ERR_INVALID;
        basp::TileLaunch L;
        const int s = basp::prepare_head_to_seq_qkv(*p, in, dq, dk, dv, L);
        return s != BASP_OK ? basp_status(s) : basp::launch(L, stream);
    });
}

extern "C" basp_status basp_stream_copy(void *dst, const void *src, uint64_t bytes, void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (bytes == 0)
            return BASP_OK;
        if (!dst || !src)
            return BASP_ERR_INVALID;
        const uint64_t d = reinterpret_cast<uint64_t>(dst), s = reinterpret_cast<uint64_t>(src);
        if ((d | s | bytes) % 16 != 0)
            return BASP_ERR_ALIGN;
        if (bytes > (uint64_t(1) << 56))
            return BASP_ERR_UNSUPPORTED;
        if (d < s + bytes && s < d + bytes)
            return BASP_ERR_ALIAS;
        const uint64_t chunks = (bytes + basp::kCopyWg - 1) / basp::kCopyWg;
        const basp::CopyDesc D = {s, d, bytes, chunks};
        const uint32_t grid = static_cast<uint32_t>(std::min<uint64_t>(chunks, basp::kCopyGridCap));
        return basp::launch_kernel(reinterpret_cast<const void *>(basp::stream_copy_kernel), dim3(grid),
                                   basp::kCopyBlock, D, stream, true, true);
    });
}

// ------------------------------------------------- allocation-free variant --

namespace basp {
namespace {

// The workspace of basp_seq_to_head_unfused_noalloc: a device array of the
// library's own, one copy per device, which the device keeps until the
// process ends.  Host code never passes this name to a kernel or a copy (on
// the host it is only a stand-in for the symbol): it uses the device address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[BASP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device (with that device current), or nullptr on an error.
void *scratch_address(basp_status &st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        st = BASP_ERR_HIP;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        st = BASP_ERR_UNSUPPORTED;
        return nullptr;
    }
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot]() {
        slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
        if (slot.err != hipSuccess)
            slot.ptr = nullptr;
    });
    if (slot.err != hipSuccess || !slot.ptr) {
        st = BASP_ERR_HIP;
        return nullptr;
    }
    return slot.ptr;
}

}  // namespace
}  // namespace basp

extern "C" basp_status basp_seq_to_head_unfused_noalloc(const basp_plan *p, const void *q,
                                                        const void *k, const void *v, void *out,
                                                        void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (!p)
            return BASP_ERR_INVALID;
        // the size limit is checked before any device call
        if (basp_unfused_workspace_bytes(p) > BASP_NOALLOC_SCRATCH_BYTES)
            return BASP_ERR_UNSUPPORTED;
        // an empty plan touches no memory and needs no workspace
        void *ws = nullptr;
        if (p->S != 0) {
            basp_status st = BASP_OK;
            ws = basp::scratch_address(st);
            if (!ws)
                return st;
        }
        basp::PermLaunch L[3];
        int s = basp::prepare_seq_to_head_unfused(*p, q, k, v, out, ws, L);
        for (int i = 0; i < 3 && s == BASP_OK; ++i)
            s = basp::launch(L[i], stream, i == 0, i == 2);
        return basp_status(s);
    });
}

extern "C" size_t basp_unfused_workspace_bytes(const basp_plan *p)
{
    if (!p)
        return 0;
    // packed and exchanged copies of all three tensors
    return size_t(2) * uint64_t(p->q_elems + 2 * p->kv_elems) * p->es;
}

extern "C" basp_status basp_seq_to_head_unfused(const basp_plan *p, const void *q, const void *k,
                                                const void *v, void *out, void *ws, void *stream)
{
    return basp::timed_call([&]() -> basp_status {
        if (!p)
            return BASP_ERR_INVALID;
        basp::PermLaunch L[3];
        int s = basp::prepare_seq_to_head_unfused(*p, q, k, v, out, ws, L);
        for (int i = 0; i < 3 && s == BASP_OK; ++i)
            s = basp::launch(L[i], stream, i == 0, i == 2);
        return basp_status(s);
    });
}
