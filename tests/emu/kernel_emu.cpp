// CPU emulation of libbasp's kernels, for tests without a GPU.
//
// It compiles the library's own launch planning (launch.cpp), plan code
// (plan.cpp) and per-lane index arithmetic (launch.hpp) with g++, then runs
// every launch on the host: each work-group's tile loop, each lane's vector
// offsets (of the masked lanes past a tile's last vector, the first and the
// last), and each vector access as a memcpy under the rule of the raw
// buffer descriptors (an access is performed only when it lies inside the
// descriptor's range).  A lane that the kernel treats as present but whose
// access falls outside its descriptor is counted in *bad: a correct plan
// never has one.
#include <cstdint>
#include <cstring>
#include <vector>

#include "launch.hpp"
#include "plan_internal.hpp"

using namespace basp;

namespace {

uint64_t rest(uint64_t bytes, uint64_t off) { return off < bytes ? bytes - off : 0; }
uint64_t range(uint64_t bytes) { return bytes > kI31Max ? kI31Max : bytes; }
bool inside(uint32_t off, uint32_t vw, uint64_t n) { return uint64_t(off) + vw <= n; }

void copy(uint64_t dst, uint64_t src, uint32_t vw)
{
    std::memcpy(reinterpret_cast<void *>(dst), reinterpret_cast<const void *>(src), vw);
}

void run(const TileLaunch &L, uint64_t *bad)
{
    const TileDesc &D = L.D;
    std::vector<unsigned char> lds(size_t(L.block) * L.vpt * 16);
    // the launch grid: x work-groups looping over a plane's tiles, y group
    // members, z batch indices
    const uint64_t groups = uint64_t(L.grid) * L.grid_y * L.grid_z;
    for (uint64_t w = 0; w < groups; ++w) {
        const uint32_t block = uint32_t(w % L.grid), by = uint32_t(w / L.grid % L.grid_y);
        const uint32_t bz = uint32_t(w / L.grid / L.grid_y);
        for (uint32_t x = block; x < D.xbound; x += L.grid) {
            uint32_t tile, b;
            tile_and_batch(D, x, bz, tile, b);
            const uint32_t t = xcd_tile(tile, D.xcd_span);
            // a one-tensor launch's kernel takes every tile as the first
            // tensor's: every tile must be
            if (L.nseg == 1 && tile_segment(D, t) != 0)
                ++*bad;
            const TileSeg &sg = D.seg[L.nseg == 1 ? 0 : tile_segment(D, t)];
            // a one-tensor launch's kernel takes its tensor's first tile as 0
            if (L.nseg == 1 && sg.tile_begin != 0)
                ++*bad;
            const TileOrigin o = tile_origin(D, sg, t - sg.tile_begin, by, b);
            const uint64_t seq = sg.seq + o.seq_off, head = sg.head + o.head_off;
            const uint64_t nseq = range(rest(sg.bytes, o.seq_off));
            const uint64_t nhead = range(rest(sg.bytes, o.head_off));
            const uint64_t src = L.s2h ? seq : head, dst = L.s2h ? head : seq;
            const uint64_t nsrc = L.s2h ? nseq : nhead, ndst = L.s2h ? nhead : nseq;
            if (L.staged) {
                // one pass: every vector of the tile, loads in the load order
                // into the staging slots, then stores in the store order
                const uint32_t nv = uint32_t(L.block) * L.vpt;
                if (sg.Ts.d * sg.Th.d * D.A.d > nv) {
                    ++*bad;
                    continue;
                }
                for (int phase = 0; phase < 2; ++phase)
                    for (uint32_t v = 0; v < nv; ++v) {
                        uint32_t so, ho, st;
                        if (!tile_vector(D, sg, o.ns, o.nh, v, L.vw, phase ? D.store_s_fast : D.load_s_fast,
                                         so, ho, st))
                            continue;
                        const uint32_t off = (phase == 0) == L.s2h ? so : ho;
                        if (!inside(off, L.vw, phase ? ndst : nsrc) || uint64_t(st + 1) * L.vw > lds.size()) {
                            ++*bad;
                            continue;
                        }
                        if (phase == 0)
                            std::memcpy(&lds[size_t(st) * L.vw], reinterpret_cast<const void *>(src + off), L.vw);
                        else
                            std::memcpy(reinterpret_cast<void *>(dst + off), &lds[size_t(st) * L.vw], L.vw);
                    }
                continue;
            }
            const uint32_t nvec = sg.Ts.d * sg.Th.d * D.A.d;
            const uint32_t step = L.block * L.vpt;
            const uint32_t vend = (nvec + step - 1) / step * step;
            // lanes of the last pass past the tile's vectors must be masked;
            // the mask's first term (v < Ts*Th*A) is monotonic in v, so the
            // first and the last such lane stand for all of them
            for (uint32_t v : {nvec, vend - 1}) {
                uint32_t so, ho;
                if (v >= nvec && v < vend && lane_offsets(D, sg, o.ns, o.nh, v, L.vw, so, ho))
                    ++*bad;
            }
            for (uint32_t v = 0; v < nvec; ++v) {
                uint32_t so, ho;
                if (!lane_offsets(D, sg, o.ns, o.nh, v, L.vw, so, ho))
                    continue;
                if (!inside(so, L.vw, nseq) || !inside(ho, L.vw, nhead)) {
                    ++*bad;
                    continue;
                }
                if (L.s2h)
                    copy(head + ho, seq + so, L.vw);
                else
                    copy(seq + so, head + ho, L.vw);
            }
        }
    }
}

void run(const PermLaunch &L, uint64_t *bad)
{
    const PermDesc &D = L.D;
    for (uint32_t block = 0; block < L.grid; ++block) {
        for (uint32_t chunk = block; chunk < D.nchunks; chunk += L.grid) {
            const PermSeg &sg = D.seg[perm_segment(D, chunk)];
            const uint32_t base = (chunk - sg.chunk_begin) * (kBlock * kPermVpt);
            for (uint32_t i = 0; i < uint32_t(kBlock * kPermVpt); ++i) {
                const uint32_t v = base + i;
                if (v >= sg.nvec)
                    continue;
                const uint32_t src = perm_source(D, sg, v, L.vw), dst = v * L.vw;
                if (!inside(src, L.vw, range(sg.src_bytes)) || !inside(dst, L.vw, range(sg.dst_bytes))) {
                    ++*bad;
                    continue;
                }
                copy(sg.dst + dst, sg.src + src, L.vw);
            }
        }
    }
}

}  // namespace

extern "C" {

// Whether the last emulated tile launch of this process used LDS staging.
static int g_staged = 0;
int emu_last_staged(void) { return g_staged; }

int emu_seq_to_head(const basp_plan *p, const void *q, const void *k, const void *v, void *out,
                    uint64_t *bad, int *vw)
{
    TileLaunch L;
    const int s = prepare_seq_to_head(*p, q, k, v, out, L);
    *vw = L.vw;
    g_staged = L.staged;
    if (s == BASP_OK)
        run(L, bad);
    return s;
}

int emu_head_to_seq(const basp_plan *p, const void *o, void *out, uint64_t *bad, int *vw)
{
    TileLaunch L;
    const int s = prepare_head_to_seq(*p, o, out, L);
    *vw = L.vw;
    g_staged = L.staged;
    if (s == BASP_OK)
        run(L, bad);
    return s;
}

int emu_seq_to_head_o(const basp_plan *p, const void *dout, void *out, uint64_t *bad, int *vw)
{
    TileLaunch L;
    const int s = prepare_seq_to_head_o(*p, dout, out, L);
    *vw = L.vw;
    if (s == BASP_OK)
        run(L, bad);
    return s;
}

int emu_head_to_seq_qkv(const basp_plan *p, const void *in, void *dq, void *dk, void *dv,
                        uint64_t *bad, int *vw)
{
    TileLaunch L;
    const int s = prepare_head_to_seq_qkv(*p, in, dq, dk, dv, L);
    *vw = L.vw;
    if (s == BASP_OK)
        run(L, bad);
    return s;
}

int emu_seq_to_head_unfused(const basp_plan *p, const void *q, const void *k, const void *v,
                            void *out, void *ws, uint64_t *bad, int *vw)
{
    PermLaunch L[3];
    const int s = prepare_seq_to_head_unfused(*p, q, k, v, out, ws, L);
    *vw = L[0].vw;
    if (s == BASP_OK)
        for (int i = 0; i < 3; ++i)
            run(L[i], bad);
    return s;
}

}  // extern "C"
