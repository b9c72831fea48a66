// Weight gradients of the MoE expert layer on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulation), the row transforms and weight repacks they and the many-rows dgrads use, and the
// dispatch of the backward GEMMs ("Mega MoE" page, Pipeline, backward).  The dgrads and the
// many-rows weight gradients run on the forward's pipeline in moe_grouped.hip.
//
// Kernels:
//   wgrad_tok  dW2 = (w act)^T dy and dW1 = dHgu^T X (X re-gathered from x) of experts with few
//              rows: K is one expert's rows; the token rows stream as MFMA fragments prepared by
//              rows_to_k_major, the hi / lo intermediate operand sits in LDS
//   rows_to_k_major, repack_t  operand transforms of the weight gradients and of the many-rows
//              dgrads
//
// Precision of the intermediate operands.  The saved pre-activation is fp32, so the row gradients
// (dHgu) and the weighted activation (w * act) are formed in fp32 and stored as two bf16 arrays,
// hi = bf16(v) and lo = bf16(v - hi), which together carry about 16 significant bits.  The weight
// gradients of experts with few rows sum few products, so one bf16 rounding of an operand shows in
// their largest elements; they multiply the other operand by that split pair twice (hi, then lo)
// into the same accumulators.  x and dy enter unrounded (they are bf16 inputs), and the routing
// weight rides on the activation, so dW1 and dW2 carry only the fp32 accumulation and the output
// rounding.  Weight gradients are written in the packed layout of the weights they belong to,
// whole 1 KB blocks per store instruction (the tile's M index runs along the packed reduction
// index).
//
// The LDS tiles are K-contiguous (128 bytes per row, 16-byte chunks XOR-swizzled by row so a
// wave's fragment reads spread over the banks); their sources are stored with M (or N) contiguous
// in runs of 8 and K strided, so the TRows loader moves 4 K-rows x 8 elements per thread and
// transposes them in registers into 8 rows x 4 K before the LDS store.
#include "moe_internal.h"

namespace moe {

constexpr int BK = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes of staged operand

// 16-byte chunk c of row r sits at position c ^ ((r >> 1) & 7): with 64 banks of 4 bytes a row
// covers half of the banks, so rows r and r + 1 fill the two halves and the 16 rows read by a
// 16-lane group of a fragment load hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// A 32-deep tile has 64-byte rows, four of which span the banks: chunk c of row r sits at position
// c ^ ((r >> 2) & 3), so the 16 rows of a 16-lane group again hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int lds_off32(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

template <int KR>
__device__ __forceinline__ int lds_off_k(int row, int chunk) {
    static_assert(KR == BK || KR == 32, "tile depth");
    if constexpr (KR == BK) return lds_off(row, chunk);
    else return lds_off32(row, chunk);
}

// ---------------------------------------------------------------------------------------------
// Operand loaders
// ---------------------------------------------------------------------------------------------
// Operand tile of ROWS rows (the M or N index) x KR (BK or 32), stored in memory with the tile's index
// contiguous in runs of 8: elements (m .. m+7, k) = Src::chunk(k, m_base + m) for m a multiple of
// 8.  Every chunk is a valid address (absent rows point at the workspace's
// zero row), so the loads carry no branch and the compiler's wait counts stay exact: a load under
// a branch makes it wait for every load in flight before the next one.
// Unit u moves K rows 4*kq..4*kq+3 of the 16-byte column mc; kq varies fastest across lanes so
// the transposed 8-byte LDS writes of a wave fill whole rows without bank conflicts.
template <int ROWS, int NT, class Src, int KR = BK>
struct TRows {
    static constexpr int MCH = ROWS / 8;
    static constexpr int UNITS = MCH * (KR / 4);
    static constexpr int PER = (UNITS + NT - 1) / NT;
    Src src;
    int m_base;
    u32x4 v[2][PER][4];

    // K rows k0 .. k0 + KR - 1
    template <int S>
    __device__ __forceinline__ void load(int k0, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < UNITS) {
                const int kq = u % (KR / 4), mc = u / (KR / 4);
                const uint16_t* p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = src.chunk(k0 + 4 * kq + r, m_base + 8 * mc);
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
                const int kq = u % (KR / 4), mc = u / (KR / 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int dw = j >> 1, sh = (j & 1) * 16;
                    const uint32_t k0 = (v[S][i][0][dw] >> sh) & 0xffffu, k1 = (v[S][i][1][dw] >> sh) & 0xffffu;
                    const uint32_t k2 = (v[S][i][2][dw] >> sh) & 0xffffu, k3 = (v[S][i][3][dw] >> sh) & 0xffffu;
                    uint2 out = make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
                    *reinterpret_cast<uint2*>(lds + lds_off_k<KR>(8 * mc + j, kq >> 1) + (kq & 1) * 8) = out;
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------------------------
// Weight gradients (TN, variable K = rows of the expert)
// ---------------------------------------------------------------------------------------------
// K index k is row seg0 + k of the expert's segment; k >= count reads the zero row, so the K tail
// and an expert without rows contribute nothing (an empty expert's tile stores exact zeros).
struct DirectRowSrc {   // row k -> ws row seg0 + k of a [R_max, width] buffer
    const uint16_t* base;
    const uint16_t* zeros;   // ws.zeros: a zero row at least width long
    int64_t seg0;
    int count, width;
    __device__ __forceinline__ const uint16_t* chunk(int kk, int m) const {
        return kk < count ? base + (seg0 + kk) * width + m : zeros + m;
    }
};

// Work item of a weight-gradient workgroup: expert e, the tile `fixed` of the operand held in LDS
// and streamed tiles [t0, t1).  Items run expert by expert, then chunk of streamed tiles, with the
// fixed tiles fastest: neighbouring workgroups stream the same fragments, which stay in L2.
struct WgradWork {
    int e, fixed, t0, t1, count;
    int64_t seg0;
    __device__ WgradWork(const Ws& ws, int n_fixed, int n_stream, int chunk) {
        const int chunks = (n_stream + chunk - 1) / chunk;
        e = blockIdx.x / (n_fixed * chunks);
        const int rem = blockIdx.x - e * (n_fixed * chunks);
        const int c = rem / n_fixed;
        fixed = rem - c * n_fixed;
        t0 = c * chunk;
        t1 = min(n_stream, t0 + chunk);
        seg0 = ws.offsets[e];
        count = ws.counts[e];
        if (seg0 < 0 || seg0 > ws.rows_cap || count < 0) count = 0;
        if (count > ws.rows_cap - seg0) count = static_cast<int>(ws.rows_cap - seg0);
    }
};

// ---------------------------------------------------------------------------------------------
// Weight gradients of experts with few rows, the token rows streamed as fragments
// ---------------------------------------------------------------------------------------------
// The token rows (x for dW1, dy for dW2), gathered once into MFMA-fragment order
// (rows_to_k_major<kTokenRows, PACKED>), stream into registers 16 bytes per lane, with no LDS and no
// transposes, and the intermediate operand (dhgu or w act, hi and lo) stays in LDS, loaded from its
// row-major ws rows once per workgroup of CHUNK output tiles.  A 128 x 128 output tile streams one
// bf16 operand tile (the other choice, streaming the hi/lo pair and keeping the token rows in LDS,
// streams twice the bytes and measured 5% slower for dW1).  The LDS holds the expert's first 64
// rows and, for an expert of 65 to 96 rows, a second 32-deep step beside them, so up to 96 rows
// (the common case) nothing synchronises the waves after the LDS tiles are loaded, and the next
// fragments are in flight while the current ones multiply and store; more rows take a loop that
// reloads the 64-deep tiles per step.  The four waves split the token dimension H (A_TOK, dW1:
// each 32 rows of M = H x 128 dhgu columns; else dW2: 128 rows of M = I x 32 columns of N = H).  The dhgu tile is in its
// logical [gate | up] column order, so dW1's stores map each 32-column group to its packed column.
template <bool A_TOK>
struct WgTok {
    static constexpr int FIX = 4;   // 32-wide blocks of the intermediate (LDS) tile dimension
    static constexpr int NT = 256;
    static constexpr int TILE_ROWS = 32 * FIX;                 // rows (M or N index) of each LDS tile
    static constexpr int TILE_BYTES = TILE_ROWS * BK * 2;      // one 64-deep K step
    static constexpr int KR1 = 32;                             // depth of the second, shallower step
    static constexpr int TILE1_BYTES = TILE_ROWS * KR1 * 2;
    static constexpr int KRES = BK + KR1;                      // expert rows the LDS holds at once
    static constexpr int LDS_BYTES = 2 * (TILE_BYTES + TILE1_BYTES);   // hi and lo of both steps
    static constexpr int NFRAG = BK / 16;                      // one streamed fragment per substep
    // output tiles per workgroup (the LDS tiles are loaded once per workgroup); measured on the
    // wide share: 4 for dW1 and 8 for dW2 (2, 6 and 8 for dW1, 4, 7 and 14 for dW2 slower)
    static constexpr int CHUNK = A_TOK ? 4 : 8;
};

template <bool A_TOK>
__global__ __launch_bounds__(256, 3) void wgrad_tok_kernel(const uint16_t* __restrict__ tp, Dims d, Ws ws,
                                                           uint16_t* __restrict__ out) {
    using W = WgTok<A_TOK>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = d.H, I = d.I;
    const int M = A_TOK ? H : I, N = A_TOK ? 2 * I : H;   // packed reduction index, packed column
    const int F = A_TOK ? 2 * I : I;                      // the intermediate operand's width
    const WgradWork wk(ws, F / W::TILE_ROWS, H / 128, W::CHUNK);
    int count = wk.count;   // rows of the expert inside its segment (clamped for safety)
    {
        const int64_t seg1 = ws.offsets[wk.e + 1];
        if (seg1 - wk.seg0 < count) count = static_cast<int>(max(seg1 - wk.seg0, static_cast<int64_t>(0)));
    }
    const int nk = (count + BK - 1) / BK;
    const int64_t Rq = ws.rows_cap / 16;   // fragment blocks per column group of the token rows
    uint16_t* o = out + static_cast<int64_t>(wk.e) * M * N;

    TRows<W::TILE_ROWS, W::NT, DirectRowSrc> lh, ll;
    lh.src.base = A_TOK ? ws.dhgu : ws.wact;
    lh.src.zeros = ws.zeros;
    lh.src.seg0 = wk.seg0;
    lh.src.count = count;
    lh.src.width = F;
    lh.m_base = wk.fixed * W::TILE_ROWS;
    ll.src = lh.src;
    ll.src.base = A_TOK ? ws.dhgu_lo : ws.wact_lo;
    ll.m_base = lh.m_base;
    char* const lH = smem;
    char* const lL = smem + W::TILE_BYTES;
    // the second step (expert rows BK .. KRES - 1) of an expert with more than BK rows
    char* const lH1 = smem + 2 * W::TILE_BYTES;
    char* const lL1 = lH1 + W::TILE1_BYTES;

    // substep f of K step kt of token tile t: the wave's 32 columns h of the tile; a substep past
    // the expert's rows reads the zero row instead
    auto frag_addr = [&](int t, int kt, int f) -> const uint16_t* {
        const int s16 = kt * BK + 16 * f;
        if (s16 >= count) return ws.zeros + (lane & 31) * 8;
        const int64_t g = (static_cast<int64_t>(t) * 128 + 32 * wave) >> 5;
        return tp + ((g * Rq + ((wk.seg0 + s16) >> 4)) * 64 + lane) * 8;
    };
    bf16x8_t fr[2][W::NFRAG];
    auto load_frags = [&](int slot, int t, int kt) {
#pragma unroll
        for (int f = 0; f < W::NFRAG; ++f) fr[slot][f] = *reinterpret_cast<const bf16x8_t*>(frag_addr(t, kt, f));
    };
    f32x16_t acc[W::FIX];
    // the products of the fragments in `slot` with the LDS tiles of step 0 (64 deep) or of step 1
    // (32 deep: its fragments past the second substep are never used)
    auto compute = [&](int slot, int step) {
        const int subs = step == 0 ? BK / 16 : W::KR1 / 16;
        const char* const tH = step == 0 ? lH : lH1;
        const char* const tL = step == 0 ? lL : lL1;
        // opaque per call: the tiles do not change inside the tile loops, and reads the compiler
        // hoists out of them would need registers for every substep at once
        int row = lane & 31;
        asm volatile("" : "+v"(row));
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            if (sub >= subs) break;
            bf16x8_t hi[W::FIX], lo[W::FIX];
            const int ch = 2 * sub + (lane >> 5);
#pragma unroll
            for (int i = 0; i < W::FIX; ++i) {
                const int r = i * 32 + row;
                const int off = step == 0 ? lds_off(r, ch) : lds_off32(r, ch);
                hi[i] = *reinterpret_cast<const bf16x8_t*>(tH + off);
                lo[i] = *reinterpret_cast<const bf16x8_t*>(tL + off);
            }
            const bf16x8_t f = fr[slot][sub];
#pragma unroll
            for (int i = 0; i < W::FIX; ++i)
                acc[i] = A_TOK ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, hi[i], acc[i], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi[i], f, acc[i], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < W::FIX; ++i)
                acc[i] = A_TOK ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, lo[i], acc[i], 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo[i], f, acc[i], 0, 0, 0);
        }
    };
    auto zero = [&]() {
#pragma unroll
        for (int i = 0; i < W::FIX; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    };
    auto store = [&](int t) {
#pragma unroll
        for (int i = 0; i < W::FIX; ++i) {
            // A_TOK: M rows h = 32 * wave of token tile t, N = the packed group of dhgu columns
            // [32 i, 32 i + 32) of the fixed tile; else M rows i of the fixed tile, N columns h
            const int64_t hcol = static_cast<int64_t>(t) * 128 + 32 * wave;
            const int fcol = wk.fixed * W::TILE_ROWS + 32 * i;
            const int64_t m0 = A_TOK ? hcol : static_cast<int64_t>(fcol);
            const int64_t n0 = A_TOK ? l1_packed_col(fcol, I) : hcol;
            store_packed_block(o, M, n0, m0, acc[i], lane);
        }
    };

    if (nk <= 1) {
        lh.template load<0>(0, tid);
        ll.template load<0>(0, tid);
        load_frags(0, wk.t0, 0);
        lh.template store<0>(lH, tid);
        ll.template store<0>(lL, tid);
        lds_barrier();
        for (int t = wk.t0; t < wk.t1; t += 2) {
            load_frags(1, min(t + 1, wk.t1 - 1), 0);   // unconditional: exact wait counts
            zero();
            if (nk == 1) compute(0, 0);
            store(t);
            if (t + 1 >= wk.t1) break;
            load_frags(0, min(t + 2, wk.t1 - 1), 0);
            zero();
            if (nk == 1) compute(1, 0);
            store(t + 1);
        }
    } else if (count <= W::KRES) {
        // both steps stay in LDS for the whole work item; a tile's second-step fragments are in
        // flight while its first step multiplies, the next tile's first step while its second does
        TRows<W::TILE_ROWS, W::NT, DirectRowSrc, W::KR1> lh1, ll1;
        lh1.src = lh.src;
        lh1.m_base = lh.m_base;
        ll1.src = ll.src;
        ll1.m_base = ll.m_base;
        lh.template load<0>(0, tid);
        ll.template load<0>(0, tid);
        lh1.template load<0>(BK, tid);
        ll1.template load<0>(BK, tid);
        load_frags(0, wk.t0, 0);
        lh.template store<0>(lH, tid);
        ll.template store<0>(lL, tid);
        lh1.template store<0>(lH1, tid);
        ll1.template store<0>(lL1, tid);
        lds_barrier();
        for (int t = wk.t0; t < wk.t1; ++t) {
            load_frags(1, t, 1);
            zero();
            compute(0, 0);
            load_frags(0, min(t + 1, wk.t1 - 1), 0);   // unconditional: exact wait counts
            compute(1, 1);
            store(t);
        }
    } else {
        for (int t = wk.t0; t < wk.t1; ++t) {
            zero();
            for (int kt = 0; kt < nk; ++kt) {
                lh.template load<0>(kt * BK, tid);
                ll.template load<0>(kt * BK, tid);
                load_frags(0, t, kt);
                lds_barrier();   // every wave's reads of the previous step are done
                lh.template store<0>(lH, tid);
                ll.template store<0>(lL, tid);
                lds_barrier();
                compute(0, 0);
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
    return e == hipSuccess ? launch_combine_finish(d, ws, dx, s, true) : e;
}

// ---------------------------------------------------------------------------------------------
// Operands of the weight gradients on the forward pipeline (experts with many rows)
// ---------------------------------------------------------------------------------------------
// A tile of 64 ws rows x 64 columns goes through LDS: read row by row (16 bytes per thread; zero
// for a row no pair holds), written column by column, either into At [W, R_max] (row c holds
// column c of every ws row; PACKED false) or into MFMA fragments along the rows (PACKED true:
// block (n / 32, r / 16) at (n / 32 * (R_max / 16) + r / 16) * 1 KB, lane n % 32 + 32 * ((r / 8) % 2)
// holding the 8 rows of r's octet, n the packed column of c).  Sources: ws wact rows (the
// weighted activation, hi part), the token rows of x or dy through row_pair (also the streamed
// operand of wgrad_tok_kernel), or ws dhgu rows (packed by L1 column), hi part.  With hundreds of
// rows per expert the weight gradients sum enough products that one bf16 rounding of the
// intermediate operand averages out, so the forward-pipeline paths take the hi parts only; the
// few-rows kernel takes both, from the ws rows.
enum RowsSrc { kWactRows, kTokenRows, kDhguRows };

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
                else if constexpr (SRC == kDhguRows) src = ws.dhgu + r * W;
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
                const int64_t n = SRC == kDhguRows ? l1_packed_col(c0 + m, d.I) : static_cast<int64_t>(c0 + m);
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

// Weight gradients of experts with few rows: the token rows (dy for dW2, x for dW1) in fragment
// order in ws stage (2 * H * R_max of its 4 * H * R_max bytes, dead after the forward's combine)
// stream through wgrad_tok_kernel; the hi / lo intermediate operand is read from its ws rows.
template <bool A_TOK>
static hipError_t wgrad_tok_launch(const Dims& d, const uint16_t* tok, const Ws& ws, uint16_t* out, hipStream_t s) {
    if (!ws.stage) return hipErrorInvalidValue;
    uint16_t* tp = reinterpret_cast<uint16_t*>(ws.stage);
    const hipError_t e = rows_to_k_major<kTokenRows, true>(d, ws, tok, d.H, tp, s);
    if (e != hipSuccess) return e;
    using W = WgTok<A_TOK>;
    const int F = A_TOK ? 2 * d.I : d.I;   // multiples of 128 (the shape check), as is H
    const int blocks = d.EL * (F / W::TILE_ROWS) * ((d.H / 128 + W::CHUNK - 1) / W::CHUNK);
    if (blocks <= 0) return hipSuccess;
    wgrad_tok_kernel<A_TOK><<<blocks, W::NT, W::LDS_BYTES, s>>>(tp, d, ws, out);
    return hipGetLastError();
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
    return wgrad_tok_launch<false>(d, dy, ws, dw2p, s);
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
    return wgrad_tok_launch<true>(d, x, ws, dw1p, s);
}

}  // namespace moe
