// Weight gradients of the MoE expert layer on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulation), the row transforms and weight repacks they and the many-rows dgrads use, and the
// dispatch of the backward GEMMs ("Mega MoE" page, Pipeline, backward).  The dgrads and the
// many-rows weight gradients run on the forward's pipeline in moe_grouped.hip.
//
// Kernels:
//   wgrad_frag  dW2 = (w act)^T dy and dW1 = dHgu^T X (X re-gathered from x) of experts with few
//               rows: K is one expert's rows; the streamed operand (w act, or dHgu) comes as
//               hi/lo MFMA fragments prepared by rows_to_k_major, the token rows through LDS
//   wgrad2, wgrad1  the same products with both operand tiles in LDS, for shapes the fragment
//               kernel does not fit (I > H)
//   rows_to_k_major, repack_t  operand transforms of the weight gradients and of the many-rows
//               dgrads
//
// Precision of the intermediate operands.  The saved pre-activation is fp32, so the row gradients
// (dHgu) and the weighted activation (w * act) are formed in fp32 and stored as two bf16 arrays,
// hi = bf16(v) and lo = bf16(v - hi), which together carry about 16 significant bits.  The weight
// gradients of experts with few rows sum few products, so one bf16 rounding of an operand shows in
// their largest elements; their streamed operand is that split pair, multiplied by the other
// operand twice (hi, then lo) into the same accumulators.  x and dy enter unrounded (they are
// bf16 inputs), and the routing weight rides on the activation, so dW1 and dW2 carry only the
// fp32 accumulation and the output rounding.
// Weight gradients are written in the packed layout of the weights they belong to, whole 1 KB
// blocks per store instruction (the tile's M index runs along the packed reduction index).
//
// The LDS tiles of wgrad2 / wgrad1 are K-contiguous (128 bytes per row, 16-byte chunks
// XOR-swizzled by row so a wave's fragment reads spread over the banks); their operands are stored
// with M (or N) contiguous in runs of 8 and K strided, so the TRows loader moves 4 K-rows x 8
// elements per thread and transposes them in registers into 8 rows x 4 K before the LDS store.
#include <type_traits>

#include "moe_internal.h"

namespace moe {

constexpr int BK = 64;
constexpr int kXcds = 8;   // the hardware places workgroup b on XCD b mod 8, each with its own L2

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes of staged operand

// 16-byte chunk c of row r sits at position c ^ ((r >> 1) & 7): with 64 banks of 4 bytes a row
// covers half of the banks, so rows r and r + 1 fill the two halves and the 16 rows read by a
// 16-lane group of a fragment load hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <int BM_, int BN_, int WM_, int WN_, int PF_ = 1>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    // 0: one LDS buffer (launches of many short-K tiles, where occupancy matters more than
    // overlap); else two
    static constexpr int PF = PF_;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int MI = TM / 32, NI = TN / 32;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = (PF == 0 ? 1 : 2) * STAGE_BYTES;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
    static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "K-row chunks must split evenly");
};

// ---------------------------------------------------------------------------------------------
// Operand loaders
// ---------------------------------------------------------------------------------------------
// Operand tile of ROWS rows (the M or N index) x BK, stored in memory with the tile's index
// contiguous in runs of 8: elements (m .. m+7, k) = Src::chunk(k, m_base + m) for m a multiple of
// 8.  Every chunk is a valid address (absent rows point at the workspace's
// zero row), so the loads carry no branch and the compiler's wait counts stay exact: a load under
// a branch makes it wait for every load in flight before the next one.
// Unit u moves K rows 4*kq..4*kq+3 of the 16-byte column mc; kq varies fastest across lanes so
// the transposed 8-byte LDS writes of a wave fill whole rows without bank conflicts.
template <int ROWS, int NT, class Src>
struct TRows {
    static constexpr int MCH = ROWS / 8;
    static constexpr int UNITS = MCH * (BK / 4);
    static constexpr int PER = (UNITS + NT - 1) / NT;
    Src src;
    int m_base;
    u32x4 v[2][PER][4];

    template <int S>
    __device__ __forceinline__ void load(int kt, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < UNITS) {
                const int kq = u % (BK / 4), mc = u / (BK / 4);
                const uint16_t* p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = src.chunk(kt * BK + 4 * kq + r, m_base + 8 * mc);
#pragma unroll
                for (int r = 0; r < 4; ++r) v[S][i][r] = *reinterpret_cast<const u32x4*>(p[r]);
            }
        }
    }
    template <int S>
    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < UNITS) {
                const int kq = u % (BK / 4), mc = u / (BK / 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int dw = j >> 1, sh = (j & 1) * 16;
                    const uint32_t k0 = (v[S][i][0][dw] >> sh) & 0xffffu, k1 = (v[S][i][1][dw] >> sh) & 0xffffu;
                    const uint32_t k2 = (v[S][i][2][dw] >> sh) & 0xffffu, k3 = (v[S][i][3][dw] >> sh) & 0xffffu;
                    uint2 out = make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
                    *reinterpret_cast<uint2*>(lds + lds_off(8 * mc + j, kq >> 1) + (kq & 1) * 8) = out;
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------------------------
// MFMA core
// ---------------------------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void read_frags(const char* lA, const char* lB, bf16x8_t (&a)[C::MI],
                                           bf16x8_t (&b)[C::NI], int s, int wm0, int wn0, int lane) {
    const int ch = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(lA + lds_off(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(lB + lds_off(wn0 + j * 32 + (lane & 31), ch));
}

// mma_step with one operand given as hi + lo bf16 tiles (the lo tile at lX, laid out like the
// operand it completes): acc += A * B + X * B (SPLIT_A) or A * B + A * X.  Each 16-deep substep
// issues the hi products of every accumulator first, then the lo ones, so no MFMA waits on the
// one just before it; the lo fragments are read at the start of their substep (the hi MFMAs cover
// that latency), one buffer instead of two.
template <class C, bool SPLIT_A>
__device__ __forceinline__ void mma_step_split(const char* lA, const char* lB, const char* lX,
                                               f32x16_t (&acc)[C::MI][C::NI], int wm0, int wn0, int lane) {
    constexpr int KS = BK / 16;
    constexpr int NX = SPLIT_A ? C::MI : C::NI;
    bf16x8_t a[2][C::MI], b[2][C::NI], x[NX];
    read_frags<C>(lA, lB, a[0], b[0], 0, wm0, wn0, lane);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        {
            const int ch = 2 * s + (lane >> 5);
            const int w0 = SPLIT_A ? wm0 : wn0;
#pragma unroll
            for (int i = 0; i < NX; ++i)
                x[i] = *reinterpret_cast<const bf16x8_t*>(lX + lds_off(w0 + i * 32 + (lane & 31), ch));
        }
        if (s + 1 < KS) read_frags<C>(lA, lB, a[(s + 1) & 1], b[(s + 1) & 1], s + 1, wm0, wn0, lane);
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], b[s & 1][j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j) {
                if constexpr (SPLIT_A)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[i], b[s & 1][j], acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], x[j], acc[i][j], 0, 0, 0);
            }
    }
}

// ---------------------------------------------------------------------------------------------
// Weight gradients (TN, variable K = rows of the expert)
// ---------------------------------------------------------------------------------------------
// K index k is row seg0 + k of the expert's segment; k >= count reads the zero row, so the K tail
// and an expert without rows contribute nothing (an empty expert's tile stores exact zeros).
struct GatherTokenSrc {   // row k -> token row of x or dy through row_pair, optionally weighted
    const uint16_t* base;
    const uint16_t* zeros;   // ws.zeros: a zero row at least H long
    const int32_t* row_pair;
    int64_t seg0;
    int count, k, H, npairs;
    __device__ __forceinline__ int pair(int kk) const { return kk < count ? row_pair[seg0 + kk] : -1; }
    __device__ __forceinline__ const uint16_t* chunk(int kk, int m) const {
        const int p = pair(kk);
        return (p >= 0 && p < npairs) ? base + static_cast<int64_t>(p / k) * H + m : zeros + m;
    }
};
struct DirectRowSrc {   // row k -> ws row seg0 + k of a [R_max, width] buffer
    const uint16_t* base;
    const uint16_t* zeros;   // ws.zeros: a zero row at least width long
    int64_t seg0;
    int count, width;
    __device__ __forceinline__ const uint16_t* chunk(int kk, int m) const {
        return kk < count ? base + (seg0 + kk) * width + m : zeros + m;
    }
};

// The accumulator of a 32x32 MFMA block stored as one packed 1 KB block: store_packed_block in
// moe_internal.h.
__device__ __forceinline__ void store_grad_block(uint16_t* out, int64_t K, int64_t n0, int64_t k0,
                                                 const f32x16_t& acc, int lane) {
    store_packed_block(out, K, n0, k0, acc, lane);
}

constexpr int kWgradChunk = 8;   // output tiles per weight-gradient workgroup

// Full K loop of one weight-gradient tile whose operand A (SPLIT_A) or B comes as hi (la / lb)
// plus lo (lx) tiles; one LDS buffer: A | B | X.
template <class C, bool SPLIT_A, class LA, class LB, class LX>
__device__ __forceinline__ void gemm_tile_split(LA& la, LB& lb, LX& lx, int nk, char* smem,
                                                f32x16_t (&acc)[C::MI][C::NI], int tid, int wm0, int wn0, int lane) {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    if (nk <= 0) return;
    char* lA = smem;
    char* lB = smem + C::A_BYTES;
    char* lX = lB + C::B_BYTES;
    la.template load<0>(0, tid);
    lb.template load<0>(0, tid);
    lx.template load<0>(0, tid);
    la.template store<0>(lA, tid);
    lb.template store<0>(lB, tid);
    lx.template store<0>(lX, tid);
    lds_barrier();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) {
            la.template load<0>(kt + 1, tid);
            lb.template load<0>(kt + 1, tid);
            lx.template load<0>(kt + 1, tid);
        }
        mma_step_split<C, SPLIT_A>(lA, lB, lX, acc, wm0, wn0, lane);
        if (more) {
            lds_barrier();   // every wave's fragment reads of step kt are done
            la.template store<0>(lA, tid);
            lb.template store<0>(lB, tid);
            lx.template store<0>(lX, tid);
            lds_barrier();
        }
    }
}

// A run of output tiles of one expert's weight gradient that share one operand tile: with
// STREAM_A the M tiles [t0, t1) of N tile `fixed` (the N operand lb is shared), else the N tiles
// [t0, t1) of M tile `fixed` (la is shared).  The streamed operand is the one given as a hi/lo
// pair (lx loads its lo part into the third LDS tile).  When the expert has at most one K step of
// rows (the common case: K is the expert's row count), the shared tile is loaded into LDS once and
// the streamed one's loads for tile t + 1 go out before the MFMAs and stores of tile t, so the
// launch streams its output.  With more rows every tile runs the full K loop.  n_col(nt, ni) gives
// the packed column of block ni of the wave in N tile nt; K_out is the packed reduction length.
template <class C, bool STREAM_A, class LA, class LB, class LX, class NCol>
__device__ __forceinline__ void wgrad_tiles(LA& la, LB& lb, LX& lx, int count, int fixed, int t0, int t1,
                                            uint16_t* out, int64_t K_out, NCol n_col, char* smem, int tid, int wm0,
                                            int wn0, int lane) {
    const int nk = (count + BK - 1) / BK;
    f32x16_t acc[C::MI][C::NI];
    auto store = [&](int t) {
        const int mt = STREAM_A ? t : fixed, nt = STREAM_A ? fixed : t;
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                store_grad_block(out, K_out, n_col(nt, ni), mt * C::BM + wm0 + mi * 32, acc[mi][ni], lane);
    };
    auto aim = [&](int t) {   // point the streamed operand (both parts) at tile t
        if constexpr (STREAM_A) la.m_base = t * C::BM;
        else lb.m_base = t * C::BN;
        lx.m_base = t * (STREAM_A ? C::BM : C::BN);
    };
    if constexpr (STREAM_A) lb.m_base = fixed * C::BN;
    else la.m_base = fixed * C::BM;
    if (nk <= 1) {
        // Two tiles of the streamed operand are in flight (register slots 0 and 1) while tile t
        // multiplies and stores: with one, every tile waited a whole memory latency for its
        // operand.  The loads are unconditional (past the end they re-read the last tile, never
        // stored to LDS), so the compiler's wait counts stay exact.
        char* lA = smem;
        char* lB = smem + C::A_BYTES;
        char* lX = lB + C::B_BYTES;
        auto stream_load = [&](int t, auto slot) {
            aim(min(t, t1 - 1));
            if constexpr (STREAM_A) la.template load<decltype(slot)::value>(0, tid);
            else lb.template load<decltype(slot)::value>(0, tid);
            lx.template load<decltype(slot)::value>(0, tid);
        };
        auto stream_store = [&](auto slot) {
            lds_barrier();   // every wave's fragment reads of the previous tile are done
            if constexpr (STREAM_A) la.template store<decltype(slot)::value>(lA, tid);
            else lb.template store<decltype(slot)::value>(lB, tid);
            lx.template store<decltype(slot)::value>(lX, tid);
            lds_barrier();
        };
        auto compute = [&](int t) {
#pragma unroll
            for (int i = 0; i < C::MI; ++i)
#pragma unroll
                for (int j = 0; j < C::NI; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
            if (nk == 1) mma_step_split<C, STREAM_A>(lA, lB, lX, acc, wm0, wn0, lane);
            store(t);
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        aim(t0);
        la.template load<0>(0, tid);
        lb.template load<0>(0, tid);
        lx.template load<0>(0, tid);
        stream_load(t0 + 1, S1{});
        la.template store<0>(lA, tid);
        lb.template store<0>(lB, tid);
        lx.template store<0>(lX, tid);
        lds_barrier();
        for (int t = t0; t < t1; t += 2) {
            // slot 1 holds tile t + 1, slot 0 is free
            stream_load(t + 2, S0{});
            compute(t);
            if (t + 1 >= t1) break;
            stream_store(S1{});
            // slot 0 holds tile t + 2, slot 1 is free
            stream_load(t + 3, S1{});
            compute(t + 1);
            if (t + 2 >= t1) break;
            stream_store(S0{});
        }
    } else {
        for (int t = t0; t < t1; ++t) {
            aim(t);
            gemm_tile_split<C, STREAM_A>(la, lb, lx, nk, smem, acc, tid, wm0, wn0, lane);
            store(t);
            lds_barrier();   // the next tile's first LDS stores follow every wave's last reads
        }
    }
}

// Workgroup b of a weight-gradient launch: expert, the fixed tile index and its chunk [t0, t1) of
// streamed tiles; the row count of the expert, kept inside the row tables.
struct WgradWork {
    int e, fixed, t0, t1, count;
    int64_t seg0;
    __device__ WgradWork(const Ws& ws, int n_fixed, int n_stream, int chunk = kWgradChunk) {
        const int chunks = (n_stream + chunk - 1) / chunk;
        e = blockIdx.x / (n_fixed * chunks);
        const int rem = blockIdx.x - e * (n_fixed * chunks);
        fixed = rem / chunks;
        t0 = (rem - fixed * chunks) * chunk;
        t1 = min(n_stream, t0 + chunk);
        seg0 = ws.offsets[e];
        count = ws.counts[e];
        if (seg0 < 0 || seg0 > ws.rows_cap || count < 0) count = 0;
        if (count > ws.rows_cap - seg0) count = static_cast<int>(ws.rows_cap - seg0);
    }
};

// dW2[e] (packed like W2: column h, reduction index i) = sum_k (w act)[k][i] * dy[t_k][h]:
// M = I (the packed reduction index), N = H (the packed column).  The dy gather is the shared
// operand; the weighted activation tiles (hi and lo, from the dgrad's epilogue) stream.
// Two waves per SIMD: the lo tile's loads and fragments need more than the 168 registers of three.
template <class C>
__global__ __launch_bounds__(C::NT, 2) void wgrad2_kernel(const uint16_t* __restrict__ dy, Dims d, Ws ws,
                                                          uint16_t* __restrict__ dw2p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn0 = (wave % C::WN) * C::TN;
    const int H = d.H, I = d.I;
    const WgradWork wk(ws, H / C::BN, I / C::BM);

    TRows<C::BM, C::NT, DirectRowSrc> la, lx;
    la.src.base = ws.wact;
    la.src.zeros = ws.zeros;
    la.src.seg0 = wk.seg0;
    la.src.count = wk.count;
    la.src.width = I;
    lx.src = la.src;
    lx.src.base = ws.wact_lo;
    TRows<C::BN, C::NT, GatherTokenSrc> lb;
    lb.src.base = dy;
    lb.src.zeros = ws.zeros;
    lb.src.row_pair = ws.row_pair;
    lb.src.seg0 = wk.seg0;
    lb.src.count = wk.count;
    lb.src.k = d.k;
    lb.src.H = H;
    lb.src.npairs = d.T * d.k;
    uint16_t* out = dw2p + static_cast<int64_t>(wk.e) * H * I;
    wgrad_tiles<C, true>(la, lb, lx, wk.count, wk.fixed, wk.t0, wk.t1, out, I,
                         [&](int nt, int ni) { return static_cast<int64_t>(nt * C::BN + wn0 + ni * 32); }, smem,
                         tid, wm0, wn0, lane);
}

// dW1[e] (packed like W1: L1 column n, reduction index h) = sum_k x[t_k][h] * dhgu[k][n]:
// M = H (the packed reduction index), N = 2I (logical L1 columns; 32-column groups map to packed
// column groups whole).  The x gather is the shared operand; dhgu tiles (hi and lo) stream.
template <class C>
__global__ __launch_bounds__(C::NT, 2) void wgrad1_kernel(const uint16_t* __restrict__ x, Dims d, Ws ws,
                                                          uint16_t* __restrict__ dw1p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn0 = (wave % C::WN) * C::TN;
    const int H = d.H, N2 = 2 * d.I;
    const WgradWork wk(ws, H / C::BM, N2 / C::BN);

    TRows<C::BM, C::NT, GatherTokenSrc> la;
    la.src.base = x;
    la.src.zeros = ws.zeros;
    la.src.row_pair = ws.row_pair;
    la.src.seg0 = wk.seg0;
    la.src.count = wk.count;
    la.src.k = d.k;
    la.src.H = H;
    la.src.npairs = d.T * d.k;
    TRows<C::BN, C::NT, DirectRowSrc> lb, lx;
    lb.src.base = ws.dhgu;
    lb.src.zeros = ws.zeros;
    lb.src.seg0 = wk.seg0;
    lb.src.count = wk.count;
    lb.src.width = N2;
    lx.src = lb.src;
    lx.src.base = ws.dhgu_lo;
    uint16_t* out = dw1p + static_cast<int64_t>(wk.e) * N2 * H;
    const int I = d.I;
    wgrad_tiles<C, false>(la, lb, lx, wk.count, wk.fixed, wk.t0, wk.t1, out, H,
                          [&](int nt, int ni) { return l1_packed_col(nt * C::BN + wn0 + ni * 32, I); }, smem, tid,
                          wm0, wn0, lane);
}

// ---------------------------------------------------------------------------------------------
// Weight gradients of experts with few rows, the intermediate operand streamed as fragments
// ---------------------------------------------------------------------------------------------
// The intermediate operand (w * act for dW2, dhgu for dW1), split into hi and lo parts, is first
// rewritten (rows_to_k_major, PACKED) so that each 1 KB block is one MFMA operand: column group
// n / 32 and 16 rows, lane L holding the 8 consecutive rows from 8 * (L / 32) of column n % 32.
// The kernel then loads those fragments straight into registers, 16 bytes per lane, with no
// LDS and no transposes; only the shared token-row operand (dy or x rows gathered through
// row_pair) goes through LDS, once per workgroup.  A 128 x 128 output tile: with STREAM_A (dW2,
// A = w act) the four waves split its M rows (each 32 rows x 128 columns), else (dW1, B = dhgu)
// its N columns (each 128 rows x 32 columns), so every wave streams fragments no other wave
// needs.  Each 16-deep substep issues the hi products, then the lo ones.  The fragments of tile
// t + 1 are in flight while tile t multiplies and stores; with one K step of rows (the common
// case) nothing synchronises the waves after the shared tile is loaded.
template <bool STREAM_A>
struct WgFrag {
    static constexpr int FIX = 4;   // 32-wide blocks of the shared (non-streamed) tile dimension
    static constexpr int BM = STREAM_A ? 128 : 32 * FIX, BN = STREAM_A ? 32 * FIX : 128, NT = 256;
    static constexpr int MI = STREAM_A ? 1 : FIX, NI = STREAM_A ? FIX : 1;
    static constexpr int SHARED_ROWS = STREAM_A ? BN : BM;   // rows (M or N index) of the LDS tile
    static constexpr int LDS_BYTES = SHARED_ROWS * BK * 2;
    static constexpr int NFRAG = 2 * (BK / 16);              // hi and lo fragment of each substep
    static constexpr int CHUNK = 8;                           // output tiles per workgroup
};

template <bool STREAM_A>
__global__ __launch_bounds__(256, 3) void wgrad_frag_kernel(const uint16_t* __restrict__ tok,
                                                            const uint16_t* __restrict__ p_hi,
                                                            const uint16_t* __restrict__ p_lo, Dims d, Ws ws,
                                                            uint16_t* __restrict__ out) {
    using W = WgFrag<STREAM_A>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = d.H, I = d.I;
    const int M = STREAM_A ? I : H, N = STREAM_A ? H : 2 * I;   // packed reduction index, packed column
    const WgradWork wk(ws, STREAM_A ? N / W::BN : M / W::BM, STREAM_A ? M / W::BM : N / W::BN, W::CHUNK);
    // rows of the expert inside its segment (the tables keep count within it; clamped for safety)
    int count = wk.count;
    {
        const int64_t seg1 = ws.offsets[wk.e + 1];
        if (seg1 - wk.seg0 < count) count = static_cast<int>(max(seg1 - wk.seg0, static_cast<int64_t>(0)));
    }
    const int nk = (count + BK - 1) / BK;
    const int64_t Rq = ws.rows_cap / 16;                        // fragment blocks per column group
    uint16_t* o = out + static_cast<int64_t>(wk.e) * M * N;

    TRows<W::SHARED_ROWS, W::NT, GatherTokenSrc> ls;
    ls.src.base = tok;
    ls.src.zeros = ws.zeros;
    ls.src.row_pair = ws.row_pair;
    ls.src.seg0 = wk.seg0;
    ls.src.count = count;
    ls.src.k = d.k;
    ls.src.H = H;
    ls.src.npairs = d.T * d.k;
    ls.m_base = wk.fixed * W::SHARED_ROWS;

    // fragment f = 2 * substep + part of K step kt of streamed tile t: the wave's column group of
    // the streamed index (STREAM_A: M rows, else N columns); a substep past the expert's rows
    // reads the zero row instead (its rows are not the expert's)
    auto frag_addr = [&](int t, int kt, int f) -> const uint16_t* {
        const int s16 = kt * BK + 16 * (f >> 1);
        if (s16 >= count) return ws.zeros + (lane & 31) * 8;
        const int64_t g = (static_cast<int64_t>(t) * (STREAM_A ? W::BM : W::BN) + 32 * wave) >> 5;
        const int64_t blk = g * Rq + ((wk.seg0 + s16) >> 4);
        return ((f & 1) ? p_lo : p_hi) + (blk * 64 + lane) * 8;
    };
    bf16x8_t fr[2][W::NFRAG];
    auto load_frags = [&](int slot, int t, int kt) {
#pragma unroll
        for (int f = 0; f < W::NFRAG; ++f) fr[slot][f] = *reinterpret_cast<const bf16x8_t*>(frag_addr(t, kt, f));
    };
    f32x16_t acc[W::MI * W::NI];
    auto compute = [&](int slot) {
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            bf16x8_t sh[W::MI * W::NI];   // shared-operand fragments of this substep (LDS)
            const int ch = 2 * sub + (lane >> 5);
#pragma unroll
            for (int i = 0; i < W::MI * W::NI; ++i)
                sh[i] = *reinterpret_cast<const bf16x8_t*>(smem + lds_off(i * 32 + (lane & 31), ch));
#pragma unroll
            for (int part = 0; part < 2; ++part)
#pragma unroll
                for (int i = 0; i < W::MI * W::NI; ++i) {
                    const bf16x8_t f = fr[slot][2 * sub + part];
                    acc[i] = STREAM_A ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, sh[i], acc[i], 0, 0, 0)
                                      : __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh[i], f, acc[i], 0, 0, 0);
                }
        }
    };
    auto zero = [&]() {
#pragma unroll
        for (int i = 0; i < W::MI * W::NI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    };
    auto store = [&](int t) {
#pragma unroll
        for (int i = 0; i < W::MI * W::NI; ++i) {
            // STREAM_A: M rows 32 * wave of streamed M tile t, N block i of the fixed N tile;
            // else: M block i of the fixed M tile, N columns 32 * wave of streamed N tile t
            const int64_t m0 = STREAM_A ? static_cast<int64_t>(t) * W::BM + 32 * wave
                                        : static_cast<int64_t>(wk.fixed) * W::BM + 32 * i;
            const int64_t n0 = STREAM_A ? static_cast<int64_t>(wk.fixed) * W::BN + 32 * i
                                        : static_cast<int64_t>(t) * W::BN + 32 * wave;
            store_packed_block(o, M, n0, m0, acc[i], lane);
        }
    };

    if (nk <= 1) {
        ls.template load<0>(0, tid);
        load_frags(0, wk.t0, 0);
        ls.template store<0>(smem, tid);
        lds_barrier();
        for (int t = wk.t0; t < wk.t1; t += 2) {
            load_frags(1, min(t + 1, wk.t1 - 1), 0);   // unconditional: exact wait counts
            zero();
            if (nk == 1) compute(0);
            store(t);
            if (t + 1 >= wk.t1) break;
            load_frags(0, min(t + 2, wk.t1 - 1), 0);
            zero();
            if (nk == 1) compute(1);
            store(t + 1);
        }
    } else {
        for (int t = wk.t0; t < wk.t1; ++t) {
            zero();
            for (int kt = 0; kt < nk; ++kt) {
                ls.template load<0>(kt, tid);
                load_frags(0, t, kt);
                lds_barrier();   // every wave's reads of the previous step are done
                ls.template store<0>(smem, tid);
                lds_barrier();
                compute(0);
            }
            store(t);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------------------------
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Persistent grid for a kernel: resident workgroups on the whole device, capped by the most
// tiles the launch can have, rounded down to a multiple of the XCD count.
template <class K>
static int persistent_grid(K kernel, int threads, size_t lds, int64_t max_tiles) {
    static_assert(sizeof(K) > 0, "");
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    int64_t g = static_cast<int64_t>(per_cu) * device_cu_count();
    if (g > max_tiles) g = max_tiles;
    if (g >= kXcds) g -= g % kXcds;   // the same number of workgroups on every XCD
    return static_cast<int>(g < 1 ? 1 : g);
}

template <class K>
static void allow_lds(K kernel, size_t lds) {
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

using WG = Cfg<128, 128, 2, 2, 0>;   // weight-gradient tiles: K is an expert's rows, often one step

// Expected rows per local expert (T * k / E, uniform routing) from which the backward GEMMs of an
// expert run on the forward's pipeline instead of the streaming kernels above.
constexpr int64_t kWgradNtRows = 256;

// A packed weight read as the B operand of the other GEMM direction: element (a, b) of each expert
// (a < A, the output column; b < B, the reduction index) moves from the source's packed position
// (column src_col(b), reduction index a, reduction length A) to frag_index(a, b, B).  W1 -> (N = h,
// K = L1 column in [gate | up] order; A = H, B = 2I, src_col = l1_packed_col) for the L1 dgrad;
// W2 -> (N = i, K = h; A = I, B = H) for the L2 dgrad.  A 64 x 64 tile goes through LDS; both
// sides move whole 16-byte chunks.
template <bool L1COL>
__global__ __launch_bounds__(256) void repack_t_kernel(const uint16_t* __restrict__ src, int A, int B, int I, int EL,
                                                       uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];   // [b][a]
    const int tid = threadIdx.x;
    const int a_tiles = A / 64, b_tiles = B / 64;
    const int64_t per_e = static_cast<int64_t>(a_tiles) * b_tiles;
    const int64_t total = per_e * EL;
    for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
        const int64_t e = t / per_e, rem = t - e * per_e;
        const int ab = static_cast<int>(rem / b_tiles) * 64, bb = static_cast<int>(rem % b_tiles) * 64;
        const uint16_t* in = src + e * A * B;
        uint16_t* o = out + e * A * B;
        __syncthreads();   // the previous tile's LDS reads are done
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + 256 * i, b = q & 63, oa = q >> 6;   // 8 consecutive a of source column b
            const int64_t col = L1COL ? l1_packed_col(bb + b, I) : static_cast<int64_t>(bb + b);
            *reinterpret_cast<u32x4*>(&tile[b][8 * oa]) = *reinterpret_cast<const u32x4*>(in + frag_index(col, ab + 8 * oa, A));
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + 256 * i, a = q & 63, ob = q >> 6;   // 8 consecutive b of output column a
            u32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = static_cast<uint32_t>(tile[8 * ob + 2 * j][a]) | (static_cast<uint32_t>(tile[8 * ob + 2 * j + 1][a]) << 16);
            *reinterpret_cast<u32x4*>(o + frag_index(ab + a, bb + 8 * ob, B)) = v;
        }
    }
}

// The L2 dgrad of experts with many rows runs on the forward's L1 tile loop (dgrad_tile_kernel) with W2
// repacked to an (N = i, K = h) operand in ws stage (free during the backward's first GEMM; it
// holds EL * I * H elements when EL * I <= 2 * R_max).
static bool dgrad_nt_use(const Dims& d, const Ws& ws) {
    return static_cast<int64_t>(d.T) * d.k >= kWgradNtRows * d.E && dgrad_nt_fits(d) && ws.stage &&
           static_cast<int64_t>(d.EL) * d.I <= 2 * ws.rows_cap;
}

hipError_t launch_dgrad(const Dims& d, const uint16_t* dy, const float* topk_w, const uint16_t* w2p,
                        const Ws& ws, int fuse, bool topk_w_grad, hipStream_t s) {
    if (topk_w_grad && (!ws.dtw_part || ws.dtw_cols != d.I / 128)) return hipErrorInvalidValue;
    if (!ws.hgu || !ws.dact || !ws.dhgu || !ws.dhgu_lo || !ws.wact || !ws.wact_lo) return hipErrorInvalidValue;
    if (dgrad_nt_use(d, ws)) {
        uint16_t* w2t = reinterpret_cast<uint16_t*>(ws.stage);
        repack_t_kernel<false><<<device_cu_count() * 8, 256, 0, s>>>(w2p, d.I, d.H, d.I, d.EL, w2t);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? launch_dgrad_nt(d, dy, w2t, topk_w, ws, fuse, topk_w_grad, s) : e;
    }
    return launch_dgrad_tr(d, dy, w2p, topk_w, ws, fuse, topk_w_grad, s);
}

// The L1 dgrad of experts with many rows runs as the forward's L2 (NT, with its combine into
// token order, weight 1): K = 2I over the dhgu rows, B = W1 repacked by repack_t_kernel into
// ws dact (dead once dhgu exists; its R_max * I fp32 hold the EL * H * 2I bf16 elements when
// EL * H <= R_max).
static bool dgrad1_nt_use(const Dims& d, const Ws& ws) {
    return ws.dact && ws.dhgu && static_cast<int64_t>(d.T) * d.k >= kWgradNtRows * d.E && d.H % 256 == 0 &&
           (2 * d.I) % 64 == 0 && static_cast<int64_t>(d.EL) * d.H <= ws.rows_cap;
}

hipError_t launch_dgrad1(const Dims& d, const uint16_t* w1p, const Ws& ws, uint16_t* dx, hipStream_t s) {
    if (dgrad1_nt_use(d, ws)) {
        uint16_t* w1t = reinterpret_cast<uint16_t*>(ws.dact);
        repack_t_kernel<true><<<device_cu_count() * 8, 256, 0, s>>>(w1p, d.H, 2 * d.I, d.I, d.EL, w1t);
        hipError_t e = hipGetLastError();
        Dims d2 = d;
        d2.I = 2 * d.I;   // the GEMM's K: dhgu rows are 2I wide
        if (e == hipSuccess) e = launch_gemm2_combine(d2, ws.dhgu, w1t, nullptr, ws, dx, s);
        if (e == hipSuccess) e = launch_combine_finish(d, ws, dx, s);
        return e;
    }
    const hipError_t e = launch_dgrad1_tr(d, w1p, ws, dx, s);
    return e == hipSuccess ? launch_combine_finish(d, ws, dx, s) : e;
}

// ---------------------------------------------------------------------------------------------
// Operands of the weight gradients on the forward pipeline (experts with many rows)
// ---------------------------------------------------------------------------------------------
// A tile of 64 ws rows x 64 columns goes through LDS: read row by row (16 bytes per thread; zero
// for a row no pair holds), written column by column, either into At [W, R_max] (row c holds
// column c of every ws row; PACKED false) or into MFMA fragments along the rows (PACKED true:
// block (n / 32, r / 16) at (n / 32 * (R_max / 16) + r / 16) * 1 KB, lane n % 32 + 32 * ((r / 8) % 2)
// holding the 8 rows of r's octet, n the packed column of c).  Sources: ws wact rows (the
// weighted activation, hi part), the token rows of x or dy through row_pair, or ws dhgu rows
// (packed by L1 column), hi or lo parts.  With hundreds of rows per expert the weight gradients
// sum enough products that one bf16 rounding of the intermediate operand averages out, so the
// forward-pipeline paths take the hi parts only; the few-rows kernels (wgrad_frag_kernel) take
// both, in the PACKED layout.
enum RowsSrc { kWactRows, kWactLoRows, kTokenRows, kDhguRows, kDhguLoRows };

template <int SRC, bool PACKED>
__global__ __launch_bounds__(256) void rows_to_k_major_kernel(const uint16_t* __restrict__ tok, Dims d, Ws ws, int W,
                                                              uint16_t* __restrict__ dst) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const int tid = threadIdx.x;
    const int64_t Rcap = ws.rows_cap;
    const int64_t R = min(static_cast<int64_t>(ws.meta[0]), Rcap);
    const int npairs = d.T * d.k;
    const int col_tiles = W / 64;
    const int64_t total = (R + 63) / 64 * col_tiles;
    for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
        const int64_t r0 = t / col_tiles * 64;
        const int c0 = static_cast<int>(t % col_tiles) * 64;
        __syncthreads();   // the previous tile's LDS reads are done
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = tid + 256 * h, row = q >> 3, ch = q & 7;
            const int64_t r = r0 + row;
            u32x4 v = {0, 0, 0, 0};
            const int p = r < R ? ws.row_pair[r] : -1;
            if (p >= 0 && p < npairs) {
                const uint16_t* src;
                if constexpr (SRC == kWactRows) src = ws.wact + r * W;
                else if constexpr (SRC == kWactLoRows) src = ws.wact_lo + r * W;
                else if constexpr (SRC == kDhguRows) src = ws.dhgu + r * W;
                else if constexpr (SRC == kDhguLoRows) src = ws.dhgu_lo + r * W;
                else src = tok + static_cast<int64_t>(p / d.k) * W;
                v = *reinterpret_cast<const u32x4*>(src + c0 + 8 * ch);
            }
            *reinterpret_cast<u32x4*>(&tile[row][8 * ch]) = v;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = tid + 256 * h;
            const int m = PACKED ? (q & 63) : (q >> 3), o = PACKED ? (q >> 6) : (q & 7);
            u32x4 w4;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w4[j] = static_cast<uint32_t>(tile[8 * o + 2 * j][m]) | (static_cast<uint32_t>(tile[8 * o + 2 * j + 1][m]) << 16);
            const int64_t r = r0 + 8 * o;
            if (r >= Rcap) continue;   // block_m 32: the last 64-row tile may pass R_max by 32 rows
            uint16_t* dp;
            if constexpr (!PACKED) {
                dp = dst + static_cast<int64_t>(c0 + m) * Rcap + r;
            } else {
                const int64_t n = (SRC == kDhguRows || SRC == kDhguLoRows) ? l1_packed_col(c0 + m, d.I)
                                                                            : static_cast<int64_t>(c0 + m);
                const int64_t blk = (n >> 5) * (Rcap / 16) + (r >> 4);
                dp = dst + (blk * 64 + (n & 31) + 32 * ((r >> 3) & 1)) * 8;
            }
            *reinterpret_cast<u32x4*>(dp) = w4;
        }
    }
}

template <int SRC, bool PACKED>
static hipError_t rows_to_k_major(const Dims& d, const Ws& ws, const uint16_t* tok, int W, uint16_t* dst,
                                  hipStream_t s) {
    rows_to_k_major_kernel<SRC, PACKED><<<device_cu_count() * 8, 256, 0, s>>>(tok, d, ws, W, dst);
    return hipGetLastError();
}

// The forward-pipeline weight gradients pay off once an expert has several 64-row K slots
// (expected rows per expert T*k/E at least kWgradNtRows); they need segments in whole 64-row slots
// (block_m a multiple of 64) and both transformed operands inside ws stage (4 * H * R_max bytes).

static bool wgrad_nt_use(const Dims& d, int M, int N) {
    return d.BM % 64 == 0 && static_cast<int64_t>(d.T) * d.k >= kWgradNtRows * d.E && wgrad_nt_fits(M, N) &&
           static_cast<int64_t>(M) + N <= 2 * static_cast<int64_t>(d.H);
}

// The fragment-streaming weight gradients keep their operands in dead ws regions: dhgu hi (2I x
// R_max bf16) in ws stage and its lo part in ws dact (R_max x I fp32, the same bytes); w act hi and
// lo (2 x I x R_max bf16) in ws stage.  That needs I <= H (ws stage is R_max x H fp32) and tiles
// of 128 (H and I multiples of 128, which the shape check requires).
static bool wgrad_frag_fits(const Dims& d) {
    return d.I <= d.H && d.H % WgFrag<false>::BM == 0 && d.H % WgFrag<true>::BN == 0 && d.I % 128 == 0;
}

hipError_t launch_wgrad2(const Dims& d, const uint16_t* dy, const Ws& ws, uint16_t* dw2p, hipStream_t s) {
    if (!ws.wact || !ws.wact_lo) return hipErrorInvalidValue;
    if (wgrad_nt_use(d, d.I, d.H)) {   // dW2 packed like W2: reduction index i (M = I), column h (N = H)
        uint16_t* at = reinterpret_cast<uint16_t*>(ws.stage);
        uint16_t* bp = at + static_cast<int64_t>(d.I) * ws.rows_cap;
        hipError_t e = rows_to_k_major<kWactRows, false>(d, ws, nullptr, d.I, at, s);
        if (e == hipSuccess) e = rows_to_k_major<kTokenRows, true>(d, ws, dy, d.H, bp, s);
        if (e == hipSuccess) e = launch_wgrad_nt(d, at, bp, d.I, d.H, ws, dw2p, s);
        return e;
    }
    if (wgrad_frag_fits(d)) {   // w act (hi, lo) in fragment order: 4 * I * R_max bytes of ws stage
        uint16_t* p_hi = reinterpret_cast<uint16_t*>(ws.stage);
        uint16_t* p_lo = p_hi + static_cast<int64_t>(d.I) * ws.rows_cap;
        hipError_t e = rows_to_k_major<kWactRows, true>(d, ws, nullptr, d.I, p_hi, s);
        if (e == hipSuccess) e = rows_to_k_major<kWactLoRows, true>(d, ws, nullptr, d.I, p_lo, s);
        if (e != hipSuccess) return e;
        using W = WgFrag<true>;
        const int blocks = d.EL * (d.H / W::BN) * ((d.I / W::BM + W::CHUNK - 1) / W::CHUNK);
        if (blocks <= 0) return hipSuccess;
        wgrad_frag_kernel<true><<<blocks, W::NT, W::LDS_BYTES, s>>>(dy, p_hi, p_lo, d, ws, dw2p);
        return hipGetLastError();
    }
    const int blocks = d.EL * (d.H / WG::BN) * ((d.I / WG::BM + kWgradChunk - 1) / kWgradChunk);
    if (blocks <= 0) return hipSuccess;
    wgrad2_kernel<WG><<<blocks, WG::NT, WG::LDS_BYTES + WG::A_BYTES, s>>>(dy, d, ws, dw2p);
    return hipGetLastError();
}

template <class C>
static hipError_t wgrad1_launch(const Dims& d, const uint16_t* x, const Ws& ws, uint16_t* dw1p, hipStream_t s) {
    const int blocks = d.EL * (d.H / C::BM) * ((2 * d.I / C::BN + kWgradChunk - 1) / kWgradChunk);
    if (blocks <= 0) return hipSuccess;
    const size_t lds = C::LDS_BYTES + C::B_BYTES;   // A | B | lo part of B
    allow_lds(wgrad1_kernel<C>, lds);
    wgrad1_kernel<C><<<blocks, C::NT, lds, s>>>(x, d, ws, dw1p);
    return hipGetLastError();
}

hipError_t launch_wgrad1(const Dims& d, const uint16_t* x, const Ws& ws, uint16_t* dw1p, hipStream_t s) {
    if (!ws.dhgu || !ws.dhgu_lo) return hipErrorInvalidValue;
    if (wgrad_nt_use(d, d.H, 2 * d.I)) {   // dW1 packed like W1: reduction index h (M = H), packed column (N = 2I)
        uint16_t* at = reinterpret_cast<uint16_t*>(ws.stage);
        uint16_t* bp = at + static_cast<int64_t>(d.H) * ws.rows_cap;
        hipError_t e = rows_to_k_major<kTokenRows, false>(d, ws, x, d.H, at, s);
        if (e == hipSuccess) e = rows_to_k_major<kDhguRows, true>(d, ws, nullptr, 2 * d.I, bp, s);
        if (e == hipSuccess) e = launch_wgrad_nt(d, at, bp, d.H, 2 * d.I, ws, dw1p, s);
        return e;
    }
    if (wgrad_frag_fits(d) && ws.dact) {   // dhgu hi in fragment order in ws stage, lo in ws dact
        uint16_t* p_hi = reinterpret_cast<uint16_t*>(ws.stage);
        uint16_t* p_lo = reinterpret_cast<uint16_t*>(ws.dact);
        hipError_t e = rows_to_k_major<kDhguRows, true>(d, ws, nullptr, 2 * d.I, p_hi, s);
        if (e == hipSuccess) e = rows_to_k_major<kDhguLoRows, true>(d, ws, nullptr, 2 * d.I, p_lo, s);
        if (e != hipSuccess) return e;
        using W = WgFrag<false>;
        const int blocks = d.EL * (d.H / W::BM) * ((2 * d.I / W::BN + W::CHUNK - 1) / W::CHUNK);
        if (blocks <= 0) return hipSuccess;
        wgrad_frag_kernel<false><<<blocks, W::NT, W::LDS_BYTES, s>>>(x, p_hi, p_lo, d, ws, dw1p);
        return hipGetLastError();
    }
    return wgrad1_launch<WG>(d, x, ws, dw1p, s);
}

}  // namespace moe
