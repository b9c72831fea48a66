// Grouped GEMMs of the MoE expert layer on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulation).
//
// One core serves every GEMM: a workgroup computes a BM x BN tile with WM x WN wavefronts, each
// wave a (BM/WM) x (BN/WN) block of 32x32 MFMA tiles.  K advances 64 elements per step.  Both
// operand tiles live in LDS K-contiguous (128 bytes per row, 16-byte chunks XOR-swizzled by
// row so a wave's fragment reads spread over the banks), double-buffered so the global loads
// of step k+1 are in flight while the MFMAs of step k run; one barrier per step.
//
// Loaders differ per operand:
//   KRows  rows that are K-contiguous in memory (token rows, packed weights, activations);
//          16-byte vector loads, 8 lanes per 128-byte row segment.  A row may come from a
//          gather (the dispatch: x or dy rows through row_pair) or be absent (zeros).
//   TRows  operands stored with M (or N) contiguous and K strided (the NN/TN products of the
//          backward): each thread loads 4 K-rows x 8 elements and transposes them in registers
//          into 8 rows x 4 K before the LDS store.
//
// Kernels ("Mega MoE" page, Pipeline):
//   gemm1   dispatch gather fused into the A load + L1 NT + SwiGLU epilogue (dispatch_grouped_gemm)
//   gemm2   L2 NT + top-k weighted combine epilogue                     (grouped_gemm_combine)
//   dgrad   L2 dgrad NN, row weight and optional SwiGLU transpose in the epilogue
//   wgrad2  dW2 = dO^T A, K = rows of the expert (variable K), TN
//   wgrad1  dW1 = dHgu^T X with X re-gathered from x, TN
//
// Forward launches are persistent: a fixed grid (CUs x occupancy) walks the tile list whose
// length R / BM * n_tiles is read from the workspace on the device, so the host never needs R.
// Tiles are numbered M-major with N fastest and the grid is a multiple of the N-tile count
// when possible, so a workgroup keeps its weight panel (N tile) and the M tiles of one expert
// that share a panel run at the same time on the same XCD (workgroup ids congruent mod 8).
#include "moe_internal.h"

namespace moe {

constexpr int BK = 64;

__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int MI = TM / 32, NI = TN / 32;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
    static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "K-row chunks must split evenly");
};

// ---------------------------------------------------------------------------------------------
// Operand loaders
// ---------------------------------------------------------------------------------------------
template <int ROWS, int NT>
struct KRows {
    static constexpr int PER = ROWS * 8 / NT;   // 16-byte chunks per thread per K step
    const uint16_t* src[PER];                   // row start + chunk offset, nullptr = zero row
    uint4 v[PER];

    // chunk q = tid + i*NT covers row q/8, chunk q%8
    __device__ __forceinline__ static int row_of(int tid, int i) { return (tid + i * NT) >> 3; }
    __device__ __forceinline__ static int chunk_of(int tid, int i) { return (tid + i * NT) & 7; }

    __device__ __forceinline__ void load(int kt) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            v[i] = src[i] ? *reinterpret_cast<const uint4*>(src[i] + kt * BK) : make_uint4(0, 0, 0, 0);
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            *reinterpret_cast<uint4*>(lds + lds_off(row_of(tid, i), chunk_of(tid, i))) = v[i];
    }
};

__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float s) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(w[i] << 16) * s;
        const float hi = __uint_as_float(w[i] & 0xffff0000u) * s;
        w[i] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Operand tile of ROWS rows (the M or N index) x BK, stored in memory as K-indexed rows with the
// tile's index contiguous: element (m, k) = Src::row(k)[m_base + m] (times Src::scale(k)).
// Unit u moves K rows 4*kq..4*kq+3 of the 16-byte column mc; kq varies fastest across lanes so
// the transposed 8-byte LDS writes of a wave fill whole rows without bank conflicts.
template <int ROWS, int NT, class Src>
struct TRows {
    static constexpr int MCH = ROWS / 8;
    static constexpr int UNITS = MCH * (BK / 4);
    static constexpr int PER = (UNITS + NT - 1) / NT;
    Src src;
    int m_base;
    uint4 v[PER][4];

    __device__ __forceinline__ void load(int kt, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < UNITS) {
                const int kq = u % (BK / 4), mc = u / (BK / 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k = kt * BK + 4 * kq + r;
                    const uint16_t* p = src.row(k);
                    uint4 x = p ? *reinterpret_cast<const uint4*>(p + m_base + 8 * mc) : make_uint4(0, 0, 0, 0);
                    if (Src::kScaled && p) x = scale_bf16x8(x, src.scale(k));
                    v[i][r] = x;
                }
            }
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < UNITS) {
                const int kq = u % (BK / 4), mc = u / (BK / 4);
                const uint32_t w[4][4] = {{v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w},
                                          {v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w},
                                          {v[i][2].x, v[i][2].y, v[i][2].z, v[i][2].w},
                                          {v[i][3].x, v[i][3].y, v[i][3].z, v[i][3].w}};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int dw = j >> 1, sh = (j & 1) * 16;
                    const uint32_t k0 = (w[0][dw] >> sh) & 0xffffu, k1 = (w[1][dw] >> sh) & 0xffffu;
                    const uint32_t k2 = (w[2][dw] >> sh) & 0xffffu, k3 = (w[3][dw] >> sh) & 0xffffu;
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
__device__ __forceinline__ void mma_step(const char* lA, const char* lB, f32x16_t (&acc)[C::MI][C::NI],
                                         int wm0, int wn0, int lane) {
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
        const int ch = 2 * s + (lane >> 5);
        bf16x8_t a[C::MI], b[C::NI];
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t*>(lA + lds_off(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
            b[j] = *reinterpret_cast<const bf16x8_t*>(lB + lds_off(wn0 + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// Loader adapters: KRows loads by step only, TRows needs the thread id.
template <int R, int NT>
__device__ __forceinline__ void op_load(KRows<R, NT>& l, int kt, int) { l.load(kt); }
template <int R, int NT, class S>
__device__ __forceinline__ void op_load(TRows<R, NT, S>& l, int kt, int tid) { l.load(kt, tid); }

template <class C, class LA, class LB>
__device__ __forceinline__ void gemm_tile(LA& la, LB& lb, int nk, char* smem, f32x16_t (&acc)[C::MI][C::NI],
                                          int tid, int wm0, int wn0, int lane) {
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    if (nk <= 0) return;
    op_load(la, 0, tid);
    op_load(lb, 0, tid);
    la.store(smem, tid);
    lb.store(smem + C::A_BYTES, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        char* cur = smem + (kt & 1) * C::STAGE_BYTES;
        char* nxt = smem + ((kt + 1) & 1) * C::STAGE_BYTES;
        const bool more = kt + 1 < nk;
        if (more) {
            op_load(la, kt + 1, tid);
            op_load(lb, kt + 1, tid);
        }
        mma_step<C>(cur, cur + C::A_BYTES, acc, wm0, wn0, lane);
        if (more) {
            la.store(nxt, tid);
            lb.store(nxt + C::A_BYTES, tid);
        }
        __syncthreads();
    }
}

// Row (within the tile) and column (within the wave's N range) of accumulator element r of
// the 32x32 block: 4 groups of 8 rows, the lane's half picks 4 of them, lane%32 is the column.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------------------------
// gemm1: dispatch gather + L1 (NT) + SwiGLU
// ---------------------------------------------------------------------------------------------
// Each N tile holds BN/2 gate columns and the BN/2 matching up columns: wave wn's TN rows of the
// B tile are [gate cols | up cols] of the same BN/(2*WN) intermediate columns, so the lane that
// holds gate(r, c) in block j also holds up(r, c) in block j + NI/2.
template <class C>
__global__ __launch_bounds__(C::NT) void gemm1_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w1p, Dims d, Ws ws,
                                                      uint16_t* __restrict__ act_out,
                                                      uint16_t* __restrict__ hgu_out) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn = wave % C::WN, wn0 = wn * C::TN;
    const int H = d.H, I = d.I;
    const int m_tiles = min(ws.meta[0] / C::BM, ws.num_blocks);   // R / BM, clamped to the tables
    const int n_tiles = (2 * I) / C::BN;
    const int total = m_tiles * n_tiles;
    const int npairs = d.T * d.k;
    constexpr int HALF = C::TN / 2;   // intermediate columns per wave

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / n_tiles, nt = tile - mt * n_tiles;
        const int e = ws.tile_expert[mt];
        if (e < 0 || e >= d.EL) continue;   // uniform per workgroup
        const int64_t row0 = static_cast<int64_t>(mt) * C::BM;

        KRows<C::BM, C::NT> la;
#pragma unroll
        for (int i = 0; i < la.PER; ++i) {
            const int p = ws.row_pair[row0 + la.row_of(tid, i)];
            la.src[i] = (p >= 0 && p < npairs) ? x + static_cast<int64_t>(p / d.k) * H + 8 * la.chunk_of(tid, i) : nullptr;
        }
        KRows<C::BN, C::NT> lb;
#pragma unroll
        for (int i = 0; i < lb.PER; ++i) {
            const int nl = lb.row_of(tid, i);
            const int w = nl / C::TN, j = nl % C::TN;
            const int grow = (j / HALF) * I + nt * (C::BN / 2) + w * HALF + (j % HALF);
            lb.src[i] = w1p + (static_cast<int64_t>(e) * 2 * I + grow) * H + 8 * lb.chunk_of(tid, i);
        }
        f32x16_t acc[C::MI][C::NI];
        __syncthreads();   // the previous tile's LDS reads are done
        gemm_tile<C>(la, lb, H / BK, smem, acc, tid, wm0, wn0, lane);

#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int nh = 0; nh < C::NI / 2; ++nh) {
                const int c = nt * (C::BN / 2) + wn * HALF + nh * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = row0 + wm0 + mi * 32 + acc_row(r, lane);
                    const float g = acc[mi][nh][r], u = acc[mi][nh + C::NI / 2][r];
                    if (hgu_out) {
                        hgu_out[row * 2 * I + c] = f32_to_bf16(g);
                        hgu_out[row * 2 * I + I + c] = f32_to_bf16(u);
                    }
                    if (act_out) act_out[row * I + c] = f32_to_bf16(silu_f32(g) * u);
                }
            }
    }
}

// ---------------------------------------------------------------------------------------------
// gemm2: L2 (NT) + top-k weighted combine
// ---------------------------------------------------------------------------------------------
// Row r of pair p = (t, j): o = act[r] @ W2[e]^T, scaled by topk_w[p].  A token with one local
// pair owns its y row: the epilogue stores bf16(w * o) there.  A token with several local pairs
// gets fp32 rows in ws.stage, summed in slot order by combine_finish (deterministic, no atomics).
template <class C>
__global__ __launch_bounds__(C::NT) void gemm2_kernel(const uint16_t* __restrict__ act,
                                                      const uint16_t* __restrict__ w2p,
                                                      const float* __restrict__ topk_w, Dims d, Ws ws,
                                                      uint16_t* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    int* s_tok = reinterpret_cast<int*>(smem + C::LDS_BYTES);   // token, or -1 (padding)
    float* s_w = reinterpret_cast<float*>(s_tok + C::BM);
    int* s_direct = reinterpret_cast<int*>(s_w + C::BM);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn0 = (wave % C::WN) * C::TN;
    const int H = d.H, I = d.I;
    const int m_tiles = min(ws.meta[0] / C::BM, ws.num_blocks);   // R / BM, clamped to the tables
    const int n_tiles = H / C::BN;
    const int total = m_tiles * n_tiles;
    const int npairs = d.T * d.k;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / n_tiles, nt = tile - mt * n_tiles;
        const int e = ws.tile_expert[mt];
        if (e < 0 || e >= d.EL) continue;   // uniform per workgroup
        const int64_t row0 = static_cast<int64_t>(mt) * C::BM;

        KRows<C::BM, C::NT> la;
#pragma unroll
        for (int i = 0; i < la.PER; ++i)
            la.src[i] = act + (row0 + la.row_of(tid, i)) * I + 8 * la.chunk_of(tid, i);
        KRows<C::BN, C::NT> lb;
#pragma unroll
        for (int i = 0; i < lb.PER; ++i)
            lb.src[i] = w2p + (static_cast<int64_t>(e) * H + nt * C::BN + lb.row_of(tid, i)) * I +
                        8 * lb.chunk_of(tid, i);
        f32x16_t acc[C::MI][C::NI];
        __syncthreads();   // previous tile's LDS (operands and row info) no longer read
        for (int r = tid; r < C::BM; r += C::NT) {
            const int p = ws.row_pair[row0 + r];
            int t = -1, direct = 0;
            float w = 0.0f;
            if (p >= 0 && p < npairs) {
                t = p / d.k;
                w = topk_w[p];
                direct = ws.tok_nloc[t] == 1;
            }
            s_tok[r] = t;
            s_w[r] = w;
            s_direct[r] = direct;
        }
        gemm_tile<C>(la, lb, I / BK, smem, acc, tid, wm0, wn0, lane);   // its barriers publish row info

#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = wm0 + mi * 32 + acc_row(r, lane);
                const int t = s_tok[rl];
                if (t < 0) continue;
                const float w = s_w[rl];
                if (s_direct[rl]) {
                    uint16_t* yr = y + static_cast<int64_t>(t) * H + nt * C::BN + wn0 + (lane & 31);
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni) yr[ni * 32] = f32_to_bf16(w * acc[mi][ni][r]);
                } else {
                    float* sr = ws.stage + (row0 + rl) * H + nt * C::BN + wn0 + (lane & 31);
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni) sr[ni * 32] = w * acc[mi][ni][r];
                }
            }
    }
}

// ---------------------------------------------------------------------------------------------
// dgrad: L2 dgrad (NN) with the row weight and optional SwiGLU transpose in the epilogue
// ---------------------------------------------------------------------------------------------
struct W2ColSrc {   // B operand of the dgrad: row k = h of W2[e] in its packed [H, I] layout
    static constexpr bool kScaled = false;
    const uint16_t* base;   // w2p + e*H*I
    int I;
    __device__ __forceinline__ const uint16_t* row(int k) const { return base + static_cast<int64_t>(k) * I; }
    __device__ __forceinline__ float scale(int) const { return 1.0f; }
};

template <class C>
__global__ __launch_bounds__(C::NT) void dgrad_kernel(const uint16_t* __restrict__ dy,
                                                      const float* __restrict__ topk_w,
                                                      const uint16_t* __restrict__ w2p, Dims d, Ws ws,
                                                      int fuse) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float* s_w = reinterpret_cast<float*>(smem + C::LDS_BYTES);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn0 = (wave % C::WN) * C::TN;
    const int H = d.H, I = d.I;
    const int m_tiles = min(ws.meta[0] / C::BM, ws.num_blocks);   // R / BM, clamped to the tables
    const int n_tiles = I / C::BN;
    const int total = m_tiles * n_tiles;
    const int npairs = d.T * d.k;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / n_tiles, nt = tile - mt * n_tiles;
        const int e = ws.tile_expert[mt];
        if (e < 0 || e >= d.EL) continue;   // uniform per workgroup
        const int64_t row0 = static_cast<int64_t>(mt) * C::BM;

        KRows<C::BM, C::NT> la;
#pragma unroll
        for (int i = 0; i < la.PER; ++i) {
            const int p = ws.row_pair[row0 + la.row_of(tid, i)];
            la.src[i] = (p >= 0 && p < npairs) ? dy + static_cast<int64_t>(p / d.k) * H + 8 * la.chunk_of(tid, i) : nullptr;
        }
        TRows<C::BN, C::NT, W2ColSrc> lb;
        lb.src.base = w2p + static_cast<int64_t>(e) * H * I;
        lb.src.I = I;
        lb.m_base = nt * C::BN;
        f32x16_t acc[C::MI][C::NI];
        __syncthreads();
        for (int r = tid; r < C::BM; r += C::NT) {
            const int p = ws.row_pair[row0 + r];
            s_w[r] = (p >= 0 && p < npairs) ? topk_w[p] : 0.0f;
        }
        gemm_tile<C>(la, lb, H / BK, smem, acc, tid, wm0, wn0, lane);

#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = wm0 + mi * 32 + acc_row(r, lane);
                const int64_t row = row0 + rl;
                const float w = s_w[rl];
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    const int c = nt * C::BN + wn0 + ni * 32 + (lane & 31);
                    const float da = w * acc[mi][ni][r];
                    if (fuse) {
                        const float g = bf16_to_f32(ws.hgu[row * 2 * I + c]);
                        const float u = bf16_to_f32(ws.hgu[row * 2 * I + I + c]);
                        const float sg = 1.0f / (1.0f + __expf(-g));
                        ws.dhgu[row * 2 * I + c] = f32_to_bf16(da * u * sg * (1.0f + g * (1.0f - sg)));
                        ws.dhgu[row * 2 * I + I + c] = f32_to_bf16(da * g * sg);
                    } else {
                        ws.dact[row * I + c] = f32_to_bf16(da);
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------------------------
// Weight gradients (TN, variable K = rows of the expert)
// ---------------------------------------------------------------------------------------------
// K index k is row seg0 + k of the expert's segment; k >= count reads as zero, so the K tail and
// an expert without rows contribute nothing (an empty expert's tile stores exact zeros).
struct GatherTokenSrc {   // row k -> token row of x or dy through row_pair, optionally weighted
    static constexpr bool kScaled = false;
    const uint16_t* base;
    const int32_t* row_pair;
    int64_t seg0;
    int count, k, H, npairs;
    __device__ __forceinline__ const uint16_t* row(int kk) const {
        if (kk >= count) return nullptr;
        const int p = row_pair[seg0 + kk];
        return (p >= 0 && p < npairs) ? base + static_cast<int64_t>(p / k) * H : nullptr;
    }
    __device__ __forceinline__ float scale(int) const { return 1.0f; }
};
struct WeightedGatherSrc : GatherTokenSrc {   // dO rows: topk_w[p] * dy[t]
    static constexpr bool kScaled = true;
    const float* topk_w;
    __device__ __forceinline__ float scale(int kk) const { return topk_w[row_pair[seg0 + kk]]; }
};
struct DirectRowSrc {   // row k -> ws row seg0 + k of a [R_max, width] buffer
    static constexpr bool kScaled = false;
    const uint16_t* base;
    int64_t seg0;
    int count, width;
    __device__ __forceinline__ const uint16_t* row(int kk) const {
        return kk < count ? base + (seg0 + kk) * width : nullptr;
    }
    __device__ __forceinline__ float scale(int) const { return 1.0f; }
};

// dW2p[e][h][i] = sum_k (w dy)[k][h] * act[k][i]: M = H, N = I.
template <class C>
__global__ __launch_bounds__(C::NT) void wgrad2_kernel(const uint16_t* __restrict__ dy,
                                                       const float* __restrict__ topk_w, Dims d, Ws ws,
                                                       uint16_t* __restrict__ dw2p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn0 = (wave % C::WN) * C::TN;
    const int H = d.H, I = d.I;
    const int n_tiles = I / C::BN, m_tiles = H / C::BM;
    const int e = blockIdx.x / (m_tiles * n_tiles);
    const int rem = blockIdx.x - e * (m_tiles * n_tiles);
    const int mt = rem / n_tiles, nt = rem - mt * n_tiles;
    const int64_t seg0 = ws.offsets[e];
    int count = ws.counts[e];   // K of this expert; kept inside the row tables
    if (seg0 < 0 || seg0 > ws.rows_cap || count < 0) count = 0;
    if (count > ws.rows_cap - seg0) count = static_cast<int>(ws.rows_cap - seg0);

    TRows<C::BM, C::NT, WeightedGatherSrc> la;
    la.src.base = dy;
    la.src.row_pair = ws.row_pair;
    la.src.seg0 = seg0;
    la.src.count = count;
    la.src.k = d.k;
    la.src.H = H;
    la.src.npairs = d.T * d.k;
    la.src.topk_w = topk_w;
    la.m_base = mt * C::BM;
    TRows<C::BN, C::NT, DirectRowSrc> lb;
    lb.src.base = ws.act;
    lb.src.seg0 = seg0;
    lb.src.count = count;
    lb.src.width = I;
    lb.m_base = nt * C::BN;
    f32x16_t acc[C::MI][C::NI];
    gemm_tile<C>(la, lb, (count + BK - 1) / BK, smem, acc, tid, wm0, wn0, lane);

    uint16_t* out = dw2p + static_cast<int64_t>(e) * H * I;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t h = mt * C::BM + wm0 + mi * 32 + acc_row(r, lane);
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                out[h * I + nt * C::BN + wn0 + ni * 32 + (lane & 31)] = f32_to_bf16(acc[mi][ni][r]);
        }
}

// dW1p[e][n][h] = sum_k dhgu[k][n] * x[t_k][h]: M = 2I, N = H.
template <class C>
__global__ __launch_bounds__(C::NT) void wgrad1_kernel(const uint16_t* __restrict__ x, Dims d, Ws ws,
                                                       uint16_t* __restrict__ dw1p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::TM, wn0 = (wave % C::WN) * C::TN;
    const int H = d.H, N2 = 2 * d.I;
    const int n_tiles = H / C::BN, m_tiles = N2 / C::BM;
    const int e = blockIdx.x / (m_tiles * n_tiles);
    const int rem = blockIdx.x - e * (m_tiles * n_tiles);
    const int mt = rem / n_tiles, nt = rem - mt * n_tiles;
    const int64_t seg0 = ws.offsets[e];
    int count = ws.counts[e];   // K of this expert; kept inside the row tables
    if (seg0 < 0 || seg0 > ws.rows_cap || count < 0) count = 0;
    if (count > ws.rows_cap - seg0) count = static_cast<int>(ws.rows_cap - seg0);

    TRows<C::BM, C::NT, DirectRowSrc> la;
    la.src.base = ws.dhgu;
    la.src.seg0 = seg0;
    la.src.count = count;
    la.src.width = N2;
    la.m_base = mt * C::BM;
    TRows<C::BN, C::NT, GatherTokenSrc> lb;
    lb.src.base = x;
    lb.src.row_pair = ws.row_pair;
    lb.src.seg0 = seg0;
    lb.src.count = count;
    lb.src.k = d.k;
    lb.src.H = H;
    lb.src.npairs = d.T * d.k;
    lb.m_base = nt * C::BN;
    f32x16_t acc[C::MI][C::NI];
    gemm_tile<C>(la, lb, (count + BK - 1) / BK, smem, acc, tid, wm0, wn0, lane);

    uint16_t* out = dw1p + static_cast<int64_t>(e) * N2 * H;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t n = mt * C::BM + wm0 + mi * 32 + acc_row(r, lane);
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                out[n * H + nt * C::BN + wn0 + ni * 32 + (lane & 31)] = f32_to_bf16(acc[mi][ni][r]);
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

// Persistent grid for a kernel: resident workgroups on the whole device, rounded down to a
// multiple of the N-tile count when that keeps at least 3/4 of them (so a workgroup keeps one
// N tile), capped by the most tiles the launch can have.
template <class K>
static int persistent_grid(K kernel, int threads, size_t lds, int n_tiles, int64_t max_tiles) {
    static_assert(sizeof(K) > 0, "");
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    int64_t g = static_cast<int64_t>(per_cu) * device_cu_count();
    if (n_tiles > 0 && g >= n_tiles) {
        const int64_t r = g / n_tiles * n_tiles;
        if (4 * r >= 3 * g) g = r;
    }
    if (g > max_tiles) g = max_tiles;
    return static_cast<int>(g < 1 ? 1 : g);
}

template <class K>
static void allow_lds(K kernel, size_t lds) {
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

using G32 = Cfg<32, 128, 1, 2>;
using G64 = Cfg<64, 128, 2, 2>;
using G128 = Cfg<128, 128, 2, 2>;
using G256 = Cfg<256, 128, 4, 1>;
using WG = Cfg<128, 128, 2, 2>;   // weight-gradient tiles

template <class C>
static hipError_t gemm1_launch(const Dims& d, const uint16_t* x, const uint16_t* w1p, const Ws& ws,
                               uint16_t* act_out, uint16_t* hgu_out, hipStream_t s) {
    const size_t lds = C::LDS_BYTES;
    auto k = gemm1_kernel<C>;
    allow_lds(k, lds);
    const int n_tiles = 2 * d.I / C::BN;
    const int grid = persistent_grid(k, C::NT, lds, n_tiles, static_cast<int64_t>(ws.num_blocks) * n_tiles);
    k<<<grid, C::NT, lds, s>>>(x, w1p, d, ws, act_out, hgu_out);
    return hipGetLastError();
}

template <class C>
static hipError_t gemm2_launch(const Dims& d, const uint16_t* act, const uint16_t* w2p, const float* topk_w,
                               const Ws& ws, uint16_t* y, hipStream_t s) {
    const size_t lds = C::LDS_BYTES + 3 * sizeof(int) * C::BM;
    auto k = gemm2_kernel<C>;
    allow_lds(k, lds);
    const int n_tiles = d.H / C::BN;
    const int grid = persistent_grid(k, C::NT, lds, n_tiles, static_cast<int64_t>(ws.num_blocks) * n_tiles);
    k<<<grid, C::NT, lds, s>>>(act, w2p, topk_w, d, ws, y);
    return hipGetLastError();
}

template <class C>
static hipError_t dgrad_launch(const Dims& d, const uint16_t* dy, const float* topk_w, const uint16_t* w2p,
                               const Ws& ws, int fuse, hipStream_t s) {
    const size_t lds = C::LDS_BYTES + sizeof(float) * C::BM;
    auto k = dgrad_kernel<C>;
    allow_lds(k, lds);
    const int n_tiles = d.I / C::BN;
    const int grid = persistent_grid(k, C::NT, lds, n_tiles, static_cast<int64_t>(ws.num_blocks) * n_tiles);
    k<<<grid, C::NT, lds, s>>>(dy, topk_w, w2p, d, ws, fuse);
    return hipGetLastError();
}

hipError_t launch_gemm1(const Dims& d, const uint16_t* x, const uint16_t* w1p, const Ws& ws,
                        uint16_t* act_out, uint16_t* hgu_out, hipStream_t s) {
    switch (d.BM) {
        case 32: return gemm1_launch<G32>(d, x, w1p, ws, act_out, hgu_out, s);
        case 64: return gemm1_launch<G64>(d, x, w1p, ws, act_out, hgu_out, s);
        case 128: return gemm1_launch<G128>(d, x, w1p, ws, act_out, hgu_out, s);
        case 256: return gemm1_launch<G256>(d, x, w1p, ws, act_out, hgu_out, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm2_combine(const Dims& d, const uint16_t* act, const uint16_t* w2p, const float* topk_w,
                                const Ws& ws, uint16_t* y, hipStream_t s) {
    switch (d.BM) {
        case 32: return gemm2_launch<G32>(d, act, w2p, topk_w, ws, y, s);
        case 64: return gemm2_launch<G64>(d, act, w2p, topk_w, ws, y, s);
        case 128: return gemm2_launch<G128>(d, act, w2p, topk_w, ws, y, s);
        case 256: return gemm2_launch<G256>(d, act, w2p, topk_w, ws, y, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dgrad(const Dims& d, const uint16_t* dy, const float* topk_w, const uint16_t* w2p,
                        const Ws& ws, int fuse, hipStream_t s) {
    switch (d.BM) {
        case 32: return dgrad_launch<G32>(d, dy, topk_w, w2p, ws, fuse, s);
        case 64: return dgrad_launch<G64>(d, dy, topk_w, w2p, ws, fuse, s);
        case 128: return dgrad_launch<G128>(d, dy, topk_w, w2p, ws, fuse, s);
        case 256: return dgrad_launch<G256>(d, dy, topk_w, w2p, ws, fuse, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_wgrad2(const Dims& d, const uint16_t* dy, const float* topk_w, const Ws& ws,
                         uint16_t* dw2p, hipStream_t s) {
    const int blocks = d.EL * (d.H / WG::BM) * (d.I / WG::BN);
    if (blocks <= 0) return hipSuccess;
    wgrad2_kernel<WG><<<blocks, WG::NT, WG::LDS_BYTES, s>>>(dy, topk_w, d, ws, dw2p);
    return hipGetLastError();
}

hipError_t launch_wgrad1(const Dims& d, const uint16_t* x, const Ws& ws, uint16_t* dw1p, hipStream_t s) {
    const int blocks = d.EL * (2 * d.I / WG::BM) * (d.H / WG::BN);
    if (blocks <= 0) return hipSuccess;
    wgrad1_kernel<WG><<<blocks, WG::NT, WG::LDS_BYTES, s>>>(x, d, ws, dw1p);
    return hipGetLastError();
}

}  // namespace moe
