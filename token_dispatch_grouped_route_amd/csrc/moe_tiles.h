// The persistent tile schedule shared by the grouped GEMMs (bf16 and MX): the list of (expert,
// N tile, M tile) tiles of one launch, built on the device from the routing counts, cut into one
// chunk per XCD and handed out largest first ("Mega MoE" page, Pipeline: the grouped GEMMs over
// the experts' row segments; "How Mega MoE Overlaps ..." page, Block-M Alignment for Irregular
// Token Counts: segments padded to block_m, tiles over real 32-row groups).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kXcds = 8;
constexpr int kMaxEL = 1024;

// ---------------------------------------------------------------------------------------------
// Tile list and schedule
// ---------------------------------------------------------------------------------------------
// Groups of real rows of expert e and its number of M tiles.
__device__ __forceinline__ int real_groups(const Ws& ws, int e) {
    const int c = ws.counts[e];
    return c > 0 ? (c + 31) >> 5 : 0;
}
// M tiles of an expert of `groups` 32-row groups.  Nine-group tiles cost a few percent more per
// group than eight-group ones (three ring slots, rolling fragments), which pays where they save a
// weight-panel stream on an expert of at most two tiles (9, 17 or 18 groups); larger experts keep
// tiles of at most eight groups.
template <int MAXMI>
__device__ __forceinline__ int m_tiles_of(int groups) {
    if constexpr (MAXMI == 9) return groups <= 18 ? (groups + 8) / 9 : (groups + 7) / 8;
    return (groups + MAXMI - 1) / MAXMI;
}

// s_pref[e] = M tiles of experts [0, e), e in [0, EL]; s_q[e] = groups per M tile of expert e
// (0: no rows); returns the total.
template <int NT, int MAXMI>
__device__ int m_tile_prefix(const Ws& ws, int EL, int* s_pref, int* s_q, int* s_part) {
    static_assert(4 * NT >= kMaxEL, "four experts per thread");
    const int tid = threadIdx.x;
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        const int g = e < EL ? real_groups(ws, e) : 0;
        v[q] = m_tiles_of<MAXMI>(g);
        if (e < EL) s_q[e] = v[q] > 0 ? (g + v[q] - 1) / v[q] : 0;
        sum += v[q];
    }
    s_part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        const int t = tid >= off ? s_part[tid - off] : 0;
        __syncthreads();
        s_part[tid] += t;
        __syncthreads();
    }
    int run = s_part[tid] - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        if (e <= EL) s_pref[e] = run;
        run += v[q];
    }
    // with EL == 4 * NT no thread holds index EL above: the last thread writes the total there
    if (tid == NT - 1 && EL == 4 * NT) s_pref[EL] = run;
    __syncthreads();
    return s_part[NT - 1];
}

struct TileRef {
    int e, nt, row0, groups, real_rows, last;   // groups (each holds real rows; the expert's last may
                                                // end in padding rows), 32 x groups; last: holds the
                                                // expert's last group
};

// Expert owning list position pos: expert e owns positions [n_tiles * s_pref[e],
// n_tiles * s_pref[e+1]) (their order inside: decode).
__device__ __forceinline__ int expert_of(int EL, int n_tiles, int pos, const int* s_pref) {
    int lo = 0, hi = EL;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] * n_tiles <= pos) lo = mid;
        else hi = mid;
    }
    return lo;
}

// List position -> tile.  An expert's tiles are ordered in blocks of kMBlock M tiles (the last
// block may be shorter), N tile major inside a block, so the tiles that run at the same time on
// one XCD (its ~32 workgroups) share both operands' K slices in its L2: eight M tiles the slices
// of one weight panel, four N tiles those of one row block.  With every M tile of a large expert
// adjacent instead, its row slices were each used once per N tile (Zipf-skewed share, 253-group
// expert: forward 0.917 -> 0.906 ms).
constexpr int kMBlock = 8;
__device__ __forceinline__ TileRef decode(const Ws& ws, int EL, int n_tiles, int pos, const int* s_pref) {
    const int lo = expert_of(EL, n_tiles, pos, s_pref);
    TileRef t;
    t.e = lo;
    const int mt_e = s_pref[lo + 1] - s_pref[lo];
    const int local = pos - s_pref[lo] * n_tiles;
    // blocks of kMBlock M tiles (the last may be shorter), N tile major inside a block
    const int blk = local / (kMBlock * n_tiles);
    const int m0 = blk * kMBlock, mb = min(kMBlock, mt_e - m0);
    const int in = local - m0 * n_tiles;
    t.nt = in / mb;
    const int mt = m0 + (in - t.nt * mb);
    // the expert's g groups cut as evenly as possible: the first g % mt_e tiles take one more
    const int g = real_groups(ws, lo), base = g / mt_e, rem = g - base * mt_e;
    const int q = base + (mt < rem ? 1 : 0);
    t.groups = q;
    t.row0 = ws.offsets[lo] + 32 * (mt * base + min(mt, rem));
    t.real_rows = 32 * q;
    t.last = mt == mt_e - 1;
    return t;
}

// The list is cut into one contiguous chunk per XCD (workgroup b runs on XCD b mod 8).
__device__ __forceinline__ int schedule_chunks() { return gridDim.x % kXcds == 0 ? kXcds : 1; }
__device__ __forceinline__ int chunk_size(int total) {
    const int nx = schedule_chunks();
    return (total + nx - 1) / nx;
}

// Counters in ws.tile_sync: [0, 8) one per chunk, [8] finished workgroups; all zero between
// launches (the last workgroup resets them).  A workgroup first takes ranks of its own XCD's
// chunk, then helps the others.
__device__ __forceinline__ int own_chunk() { return schedule_chunks() == kXcds ? blockIdx.x % kXcds : 0; }

// Rank p (returned by the atomic on the own chunk's counter) -> slot lo + p, or, once the own chunk
// is used up, a slot taken from another chunk, or -1.
__device__ int settle_grab(int32_t* cnt, int total, int p) {
    const int nx = schedule_chunks(), x = own_chunk(), chunk = chunk_size(total);
    const int lo = x * chunk, hi = min(total, lo + chunk);
    if (lo + p < hi) return lo + p;
    for (int k = 1; k < nx; ++k) {
        const int xx = x + k < nx ? x + k : x + k - nx;
        const int l2 = xx * chunk, h2 = min(total, l2 + chunk);
        if (l2 >= h2) continue;
        const int q = atomicAdd(&cnt[xx], 1);
        if (l2 + q < h2) return l2 + q;
    }
    return -1;
}

__device__ void finish_schedule(int32_t* cnt) {
    if (threadIdx.x == 0 && atomicAdd(&cnt[kXcds], 1) == static_cast<int>(gridDim.x) - 1)
        for (int k = 0; k <= kXcds; ++k) atomicExch(&cnt[k], 0);
}

// Inside a chunk, tiles are handed out largest first (longest-processing-time order, so the last
// tiles to start are the short ones and the workgroups finish close together): the chunk's
// experts by decreasing groups per M tile, each expert's positions in list order.  The table
// holds, per chunk, the segments of that order (first rank, first list position); a chunk that
// spans more experts than the table holds keeps list order.
constexpr int kLptMaxSeg = 64;
struct LptTable {
    int start[kXcds][kLptMaxSeg];
    int pos[kXcds][kLptMaxSeg];
    int n[kXcds];   // segments, or 0: list order
};

template <int MAXMI>
__device__ void build_lpt(int EL, int n_tiles, int total, const int* s_pref, const int* s_q, LptTable& tb) {
    const int nx = schedule_chunks(), x = threadIdx.x;
    if (x < nx) {
        const int chunk = chunk_size(total);
        const int lo = x * chunk, hi = min(total, lo + chunk);
        int n = 0;
        if (lo < hi) {
            const int e0 = expert_of(EL, n_tiles, lo, s_pref), e1 = expert_of(EL, n_tiles, hi - 1, s_pref);
            if (e1 - e0 < kLptMaxSeg) {
                int rank = 0;
                for (int q = MAXMI; q >= 1; --q)
                    for (int e = e0; e <= e1; ++e) {
                        if (s_q[e] != q) continue;
                        const int a = max(lo, s_pref[e] * n_tiles), b = min(hi, s_pref[e + 1] * n_tiles);
                        if (b <= a) continue;
                        tb.start[x][n] = rank;
                        tb.pos[x][n] = a;
                        ++n;
                        rank += b - a;
                    }
            }
        }
        tb.n[x] = n;
    }
    __syncthreads();
}

// Slot (chunk lo + rank) -> list position.
__device__ __forceinline__ int lpt_position(int total, int slot, const LptTable& tb) {
    const int chunk = chunk_size(total);
    const int x = slot / chunk, p = slot - x * chunk;
    const int n = tb.n[x];
    if (n == 0) return slot;
    int i = 0;
    while (i + 1 < n && tb.start[x][i + 1] <= p) ++i;
    return tb.pos[x][i] + (p - tb.start[x][i]);
}

// Runs the tile list: body.run<MA>(tile) for each tile this workgroup takes.  (The next tile is
// claimed only once the current one is done: a claim made earlier would hold a tile that an idle
// workgroup could start, which at the end of the list lengthens the tail.)
template <class C, class Body>
__device__ __forceinline__ void run_tiles(const Dims& d, const Ws& ws, int n_tiles, Body& body) {
    __shared__ int s_pref[kMaxEL + 1];
    __shared__ int s_q[kMaxEL];
    __shared__ int s_part[C::NT];
    __shared__ LptTable s_lpt;
    __shared__ int s_pos[2];   // alternate per tile: written for tile i + 1 while tile i's is read
    const int EL = d.EL;
    const int total = m_tile_prefix<C::NT, C::MAXMI>(ws, EL, s_pref, s_q, s_part) * n_tiles;
    build_lpt<C::MAXMI>(EL, n_tiles, total, s_pref, s_q, s_lpt);
    int32_t* const cnt = ws.tile_sync;
    if (threadIdx.x == 0) {
        const int slot = settle_grab(cnt, total, atomicAdd(&cnt[own_chunk()], 1));
        s_pos[0] = slot < 0 ? -1 : lpt_position(total, slot, s_lpt);
    }
    for (int it = 0;; ++it) {
        lds_barrier();   // publishes s_pos[it & 1]; the previous tile's LDS reads are done
        const int pos = s_pos[it & 1];
        if (pos < 0) break;
        const TileRef t = decode(ws, EL, n_tiles, pos, s_pref);
        if (t.row0 >= 0 && t.row0 + t.real_rows <= ws.rows_cap) {   // else tables not from one prologue
            switch (t.groups) {
                case 1: body.template run<1>(t); break;
                case 2: if constexpr (C::MAXMI >= 2) body.template run<2>(t); break;
                case 3: if constexpr (C::MAXMI >= 3) body.template run<3>(t); break;
                case 4: if constexpr (C::MAXMI >= 4) body.template run<4>(t); break;
                case 5: if constexpr (C::MAXMI >= 5) body.template run<5>(t); break;
                case 6: if constexpr (C::MAXMI >= 6) body.template run<6>(t); break;
                case 7: if constexpr (C::MAXMI >= 7) body.template run<7>(t); break;
                case 8: if constexpr (C::MAXMI >= 8) body.template run<8>(t); break;
                case 9: if constexpr (C::MAXMI >= 9) body.template run<9>(t); break;
                default: break;
            }
        }
        if (threadIdx.x == 0) {
            const int slot = settle_grab(cnt, total, atomicAdd(&cnt[own_chunk()], 1));
            s_pos[(it + 1) & 1] = slot < 0 ? -1 : lpt_position(total, slot, s_lpt);
        }
    }
    finish_schedule(cnt);
}

// ---------------------------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------------------------
template <class K>
int persistent_grid(K kernel, int threads, size_t lds) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    int64_t g = static_cast<int64_t>(per_cu) * device_cu_count();
    if (g > kMaxGrid) g = kMaxGrid;
    if (g >= kXcds) g -= g % kXcds;   // the same number of workgroups on every XCD
    return static_cast<int>(g < 1 ? 1 : g);
}

// Workgroups of a tile-list launch: persistent_grid, but no more than the tiles the launch can
// hold (rounded up to a multiple of the XCD count), so a launch with few tiles does not start
// workgroups that only look for work (each spends a round trip per chunk counter before it exits,
// which set the duration of launches with a few tiles).  The local pairs (at most T * k) fill at
// most ceil(T * k / 32) + EL groups of 32 rows, and tiles of up to m groups cut them into at most
// ceil(groups / m) + EL M tiles (m = min(maxmi, 8): nine-group tiles are used only where they
// replace tiles of eight).
template <class K>
int tile_grid(K kernel, int threads, size_t lds, const Dims& d, int maxmi, int n_tiles) {
    const int g = persistent_grid(kernel, threads, lds);
    const int m = maxmi < 8 ? maxmi : 8;
    const int64_t groups = (static_cast<int64_t>(d.T) * d.k + 31) / 32 + d.EL;
    const int64_t tiles = ((groups + m - 1) / m + d.EL) * n_tiles;
    int64_t cap = (tiles + kXcds - 1) / kXcds * kXcds;
    if (cap < kXcds) cap = kXcds;
    return static_cast<int>(cap < g ? cap : g);
}

template <class K>
void allow_lds(K kernel, size_t bytes) {
    static bool done[64] = {};   // per instantiation and device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    if (bytes > 64 * 1024 && (dev < 0 || !done[dev])) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
        if (dev >= 0) done[dev] = true;
    }
}

}  // namespace
}  // namespace moe
