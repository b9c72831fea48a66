// Dispatch prologue: routing tables from external top-k routing ("Mega MoE" page,
// Implementation Map: dispatch prologue (routing tables); block-M padding from the
// "How Mega MoE Overlaps ..." page, Block-M Alignment).
//
// Two launches with fixed grids, none waiting on the host:
//   1. count: each block histograms the experts of one chunk of pairs (LDS
//      counters) and counts the local pairs of a slice of tokens.
//   2. scan + place: every block stages all chunk histograms in LDS and derives what it needs
//      itself: per expert the total, the padded segment offsets (a block-wide scan) and its own
//      chunk's base inside each segment (the sum over earlier chunks).  Block 0 also writes the
//      counts, offsets and meta counters, and the blocks share the block -> expert map and the
//      -1 fill of rows no pair takes.  Then each block re-reads its chunk in pair order, 256
//      pairs at a time.  Inside a wavefront, pairs with the same expert are grouped with ballots
//      (the wave-level histogram), giving each pair its rank among earlier lanes; the per-wave
//      counts are prefix-summed across the block's waves in LDS.  So a pair's row is
//      offset[e] + (pairs of e in earlier chunks) + (in earlier sub-steps) + (in earlier waves)
//      + (in earlier lanes): ascending pair order inside every segment, no atomics on the row
//      positions, the same tables on every run.
// Shapes whose histograms do not fit in LDS (chunks x local experts > kFusedHist) run the scan
// as a one-block launch of its own between the two.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ int local_slot(int32_t id, const Dims& d) {
    if (id < 0 || id >= d.E) return -1;
    const int e = id - d.e_lo;
    return (e >= 0 && e < d.EL) ? e : -1;
}

__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* __restrict__ idx,
                                                                     Dims d, Ws ws) {
    extern __shared__ int32_t hist[];   // [EL]
    __shared__ int32_t s_drop;
    const int tid = threadIdx.x;
    for (int e = tid; e < d.EL; e += blockDim.x) hist[e] = 0;
    if (tid == 0) s_drop = 0;
    __syncthreads();

    const int64_t npairs = static_cast<int64_t>(d.T) * d.k;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * ws.route_chunk;
    const int64_t p1 = min(npairs, p0 + ws.route_chunk);
    int drop = 0;
    for (int64_t p = p0 + tid; p < p1; p += blockDim.x) {
        const int32_t id = idx[p];
        drop += (id < 0 || id >= d.E);
        const int e = local_slot(id, d);
        if (e >= 0) atomicAdd(&hist[e], 1);
    }
    if (drop) atomicAdd(&s_drop, drop);
    if (blockIdx.x == 0) {   // the zero row read by the GEMMs for padding rows; K-split counters
        for (int i = tid; i < ws.zero_len / 8; i += blockDim.x)
            reinterpret_cast<uint4*>(ws.zeros)[i] = make_uint4(0, 0, 0, 0);
        for (int i = tid; i < kMaxGrid; i += blockDim.x) ws.tile_sync[i] = 0;
    }
    __syncthreads();
    for (int e = tid; e < d.EL; e += blockDim.x)
        ws.chunk_hist[static_cast<int64_t>(blockIdx.x) * d.EL + e] = hist[e];
    if (tid == 0) ws.chunk_dropped[blockIdx.x] = s_drop;

    // local pairs per token, over an even slice of the tokens
    const int per = (d.T + gridDim.x - 1) / gridDim.x;
    const int t0 = blockIdx.x * per, t1 = min(d.T, t0 + per);
    for (int t = t0 + tid; t < t1; t += blockDim.x) {
        int n = 0;
        for (int j = 0; j < d.k; ++j) n += local_slot(idx[static_cast<int64_t>(t) * d.k + j], d) >= 0;
        ws.tok_nloc[t] = n;
    }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(Dims d, Ws ws) {
    __shared__ int32_t s_val[kScanThreads];
    __shared__ int32_t s_off[kScanThreads + 1];
    __shared__ int32_t s_drop;
    const int tid = threadIdx.x;
    const int nch = ws.num_chunks;

    // per-expert exclusive scan over chunks (in place), total count and padded count
    int padded = 0;
    if (tid < d.EL) {
        int run = 0;
        for (int c = 0; c < nch; ++c) {
            int32_t* h = ws.chunk_hist + static_cast<int64_t>(c) * d.EL + tid;
            const int v = *h;
            *h = run;
            run += v;
        }
        ws.counts[tid] = run;
        padded = (run + d.BM - 1) / d.BM * d.BM;
    }
    // inclusive Hillis-Steele scan of the padded counts
    s_val[tid] = padded;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int v = tid >= off ? s_val[tid - off] : 0;
        __syncthreads();
        s_val[tid] += v;
        __syncthreads();
    }
    s_off[tid + 1] = s_val[tid];
    if (tid == 0) {
        s_off[0] = 0;
        int dr = 0;
        for (int c = 0; c < nch; ++c) dr += ws.chunk_dropped[c];
        s_drop = dr;
    }
    __syncthreads();
    if (tid < d.EL) ws.offsets[tid] = s_off[tid];
    if (tid == 0) ws.offsets[d.EL] = s_off[d.EL];
    const int R = s_off[d.EL];
    if (tid == 0) {
        ws.meta[0] = R;
        ws.meta[1] = s_drop;
    }
    // block -> expert map: the last expert whose segment starts at or before the block
    for (int m = tid; m < ws.num_blocks; m += blockDim.x) {
        const int r0 = m * d.BM;
        int e = -1;
        if (r0 < R) {
            int lo = 0, hi = d.EL - 1;   // largest e with s_off[e] <= r0
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= r0) lo = mid; else hi = mid - 1;
            }
            e = lo;
        }
        ws.tile_expert[m] = e;
    }
}

constexpr int kPlaceWaves = kRouteThreads / 64;

__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(const int32_t* __restrict__ idx,
                                                                     Dims d, Ws ws) {
    extern __shared__ int32_t sm[];
    int32_t* base = sm;                   // [EL]
    int32_t* wcnt = sm + d.EL;            // [kPlaceWaves][EL]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t npairs = static_cast<int64_t>(d.T) * d.k;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * ws.route_chunk;
    const int64_t p1 = min(npairs, p0 + ws.route_chunk);

    for (int e = tid; e < d.EL; e += blockDim.x)
        base[e] = ws.offsets[e] + ws.chunk_hist[static_cast<int64_t>(blockIdx.x) * d.EL + e];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    for (int64_t s0 = p0; s0 < p1; s0 += kRouteThreads) {
        for (int e = lane; e < d.EL; e += 64) wcnt[wave * d.EL + e] = 0;
        __syncthreads();
        const int64_t p = s0 + tid;
        const int e = (p < p1) ? local_slot(idx[p], d) : -1;
        // group the lanes of this wave by expert; each lane learns its rank in its group
        int rank = 0;
        uint64_t todo = __ballot(e >= 0);
        while (todo) {
            const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
            const int le = __shfl(e, leader);
            const uint64_t grp = __ballot(e == le);
            if (e == le) rank = __popcll(grp & lt_mask);
            if (lane == leader) wcnt[wave * d.EL + le] = __popcll(grp);
            todo &= ~grp;
        }
        __syncthreads();
        if (e >= 0) {
            int row = base[e] + rank;
            for (int w = 0; w < wave; ++w) row += wcnt[w * d.EL + e];
            ws.row_pair[row] = static_cast<int32_t>(p);
            ws.pair_row[p] = row;
        } else if (p < p1) {
            ws.pair_row[p] = -1;
        }
        __syncthreads();
        for (int x = tid; x < d.EL; x += blockDim.x) {
            int add = 0;
            for (int w = 0; w < kPlaceWaves; ++w) add += wcnt[w * d.EL + x];
            base[x] += add;
        }
        // the next sub-step's zeroing of wcnt is ordered after these reads by its barrier
        __syncthreads();
    }

    // -1 in every row that no pair fills: padding inside segments and rows past R
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + tid; r < ws.rows_cap; r += stride) {
        const int e = ws.tile_expert[r / d.BM];
        if (e < 0 || r >= ws.offsets[e] + ws.counts[e]) ws.row_pair[r] = -1;
    }
}


// Scan + place in one launch (see the top of the file).  LDS: hist [nch * EL], tot, mine, off
// [EL + 1], base, wcnt [kPlaceWaves * EL], scan [kRouteThreads].
__global__ __launch_bounds__(kRouteThreads) void route_scan_place_kernel(const int32_t* __restrict__ idx,
                                                                         Dims d, Ws ws) {
    extern __shared__ int32_t sm[];
    const int EL = d.EL, nch = ws.num_chunks;
    int32_t* hist = sm;
    int32_t* tot = hist + nch * EL;
    int32_t* mine = tot + EL;
    int32_t* off = mine + EL;   // [EL + 1]
    int32_t* base = off + EL + 1;
    int32_t* wcnt = base + EL;
    int32_t* scan = wcnt + kPlaceWaves * EL;
    __shared__ int32_t s_drop;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int i = tid; i < nch * EL; i += blockDim.x) hist[i] = ws.chunk_hist[i];
    if (tid == 0) s_drop = 0;
    __syncthreads();
    for (int e = tid; e < EL; e += blockDim.x) {
        int t = 0, m = 0;
        for (int c = 0; c < nch; ++c) {
            const int v = hist[c * EL + e];
            m += c < static_cast<int>(blockIdx.x) ? v : 0;
            t += v;
        }
        tot[e] = t;
        mine[e] = m;
    }
    __syncthreads();
    // offsets: exclusive scan of the padded counts, kRouteThreads experts per round
    int carry = 0;
    for (int e0 = 0; e0 < EL; e0 += kRouteThreads) {
        const int e = e0 + tid;
        const int v = e < EL ? (tot[e] + d.BM - 1) / d.BM * d.BM : 0;
        scan[tid] = v;
        __syncthreads();
        for (int o = 1; o < kRouteThreads; o <<= 1) {
            const int u = tid >= o ? scan[tid - o] : 0;
            __syncthreads();
            scan[tid] += u;
            __syncthreads();
        }
        if (e < EL) off[e] = carry + scan[tid] - v;
        carry += scan[kRouteThreads - 1];
        __syncthreads();
    }
    if (tid == 0) off[EL] = carry;
    if (blockIdx.x == 0) {
        int dr = 0;
        for (int c = tid; c < nch; c += blockDim.x) dr += ws.chunk_dropped[c];
        if (dr) atomicAdd(&s_drop, dr);
    }
    __syncthreads();
    const int R = off[EL];
    if (blockIdx.x == 0) {
        for (int e = tid; e < EL; e += blockDim.x) {
            ws.counts[e] = tot[e];
            ws.offsets[e] = off[e];
        }
        if (tid == 0) {
            ws.offsets[EL] = R;
            ws.meta[0] = R;
            ws.meta[1] = s_drop;
        }
    }
    // block -> expert map (the last expert whose segment starts at or before the block), and -1 in
    // every row no pair takes: padding inside segments and rows past R; a slice per block
    const int64_t gstride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t gtid = static_cast<int64_t>(blockIdx.x) * blockDim.x + tid;
    auto expert_at = [&](int64_t r) {   // largest e with off[e] <= r < R
        int lo = 0, hi = EL - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= r) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    for (int64_t m = gtid; m < ws.num_blocks; m += gstride) {
        const int64_t r0 = m * d.BM;
        ws.tile_expert[m] = r0 < R ? expert_at(r0) : -1;
    }
    for (int64_t r = gtid; r < ws.rows_cap; r += gstride) {
        if (r >= R) {
            ws.row_pair[r] = -1;
        } else {
            const int e = expert_at(r);
            if (r >= off[e] + tot[e]) ws.row_pair[r] = -1;
        }
    }

    // placement
    const int64_t npairs = static_cast<int64_t>(d.T) * d.k;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * ws.route_chunk;
    const int64_t p1 = min(npairs, p0 + ws.route_chunk);
    for (int e = tid; e < EL; e += blockDim.x) base[e] = off[e] + mine[e];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t s0 = p0; s0 < p1; s0 += kRouteThreads) {
        for (int e = lane; e < EL; e += 64) wcnt[wave * EL + e] = 0;
        __syncthreads();
        const int64_t p = s0 + tid;
        const int e = (p < p1) ? local_slot(idx[p], d) : -1;
        int rank = 0;
        uint64_t todo = __ballot(e >= 0);
        while (todo) {
            const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
            const int le = __shfl(e, leader);
            const uint64_t grp = __ballot(e == le);
            if (e == le) rank = __popcll(grp & lt_mask);
            if (lane == leader) wcnt[wave * EL + le] = __popcll(grp);
            todo &= ~grp;
        }
        __syncthreads();
        if (e >= 0) {
            int row = base[e] + rank;
            for (int w = 0; w < wave; ++w) row += wcnt[w * EL + e];
            ws.row_pair[row] = static_cast<int32_t>(p);
            ws.pair_row[p] = row;
        } else if (p < p1) {
            ws.pair_row[p] = -1;
        }
        __syncthreads();
        for (int x = tid; x < EL; x += blockDim.x) {
            int add = 0;
            for (int w = 0; w < kPlaceWaves; ++w) add += wcnt[w * EL + x];
            base[x] += add;
        }
        __syncthreads();
    }
}

hipError_t launch_route(const Dims& d, const int32_t* topk_idx, const Ws& ws, hipStream_t s) {
    const int nch = ws.num_chunks;
    route_count_kernel<<<nch, kRouteThreads, sizeof(int32_t) * d.EL, s>>>(topk_idx, d, ws);
    const size_t lds = sizeof(int32_t) * (static_cast<size_t>(nch) * d.EL + (4 + kPlaceWaves) * d.EL + 1 +
                                          kRouteThreads);
    if (static_cast<int64_t>(nch) * d.EL <= kFusedHist && lds <= 64 * 1024) {
        route_scan_place_kernel<<<nch, kRouteThreads, lds, s>>>(topk_idx, d, ws);
    } else {
        route_scan_kernel<<<1, kScanThreads, 0, s>>>(d, ws);
        route_place_kernel<<<nch, kRouteThreads, sizeof(int32_t) * d.EL * (1 + kPlaceWaves), s>>>(
            topk_idx, d, ws);
    }
    return hipGetLastError();
}

}  // namespace moe
