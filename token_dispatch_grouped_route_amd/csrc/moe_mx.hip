// MX variant of the forward ("How Mega MoE Overlaps ..." page, Code Example: activations cast per
// token to FP8 with power-of-two (UE8M0) scale factors over groups of 32 along K, weights
// transformed to FP4, a fused forward with an activation clamp): the FP8 cast, the FP4 weight
// pack, and the L1 / L2 grouped GEMMs on v_mfma_scale_f32_32x32x64_f8f6f4 (FP8 E4M3 A, FP4 E2M1 B,
// one scale byte per 32 K values of a row or column, fp32 accumulation).
//
// Operand layout of that MFMA (32 x 32 output, K = 64, determined on gfx950 with in-bounds
// probes against a CPU reference):
//   A (FP8): lane l holds row l % 32; byte p of its 8 registers is k = 32 (p / 16) + 16 (l / 32)
//            + p % 16, so a row's 64 bytes of one K step are split in 16-byte quarters over the
//            lanes l and l + 32.
//   B (FP4): lane l holds column l % 32 and k = 32 (l / 32) + q in nibble q (low nibble first) of
//            its first four registers.
//   Scale of (row or column x, 32-block b of the K step): the scale byte of lane x + 32 b.
//   Accumulator: as the 32 x 32 bf16 MFMA (row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32).
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

// Block exponent: the smallest E with amax <= fmax * 2^E (fmax = fm * 2^fe, fm in [1, 2)), clamped
// to [-127, 127]; 0 for amax == 0.  amax = f * 2^ea with f in [1, 2): E = ea - fe when f <= fm,
// else ea - fe + 1.
__device__ __forceinline__ int block_exponent(float amax, float fm, int fe) {
    if (!(amax > 0.0f)) return 0;
    int ea;
    const float f = 2.0f * frexpf(amax, &ea);   // frexp: amax = (f / 2) * 2^ea, f / 2 in [0.5, 1)
    ea -= 1;
    int E = f <= fm ? ea - fe : ea - fe + 1;
    return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Nearest FP8 E4M3 code of a finite v with |v| <= 448, ties to the even mantissa; the sign of a
// value that rounds to zero is kept.
__device__ __forceinline__ uint32_t fp8_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
    const float a = fabsf(v);
    uint32_t mag;
    if (a < 0.015625f) {   // below 2^-6: subnormal, spacing 2^-9 (a code of 8 is the smallest normal)
        mag = static_cast<uint32_t>(rintf(a * 512.0f));
    } else {
        int e;
        const float m = 2.0f * frexpf(a, &e);   // a = m * 2^(e - 1), m in [1, 2)
        e -= 1;
        uint32_t q = static_cast<uint32_t>(rintf((m - 1.0f) * 8.0f));
        if (q == 8) {
            q = 0;
            ++e;
        }
        mag = (static_cast<uint32_t>(e + 7) << 3) | q;
    }
    return sign | mag;
}

// Nearest FP4 E2M1 code (values 0, 0.5, 1, 1.5, 2, 3, 4, 6) of |v| <= 6, ties to the even mantissa.
__device__ __forceinline__ uint32_t fp4_code(float v) {
    const uint32_t sign = (__float_as_uint(v) >> 31) << 3;
    const float a = fabsf(v);
    uint32_t mag;
    if (a < 1.0f) {   // subnormal, spacing 0.5 (a code of 2 is 1.0)
        mag = static_cast<uint32_t>(rintf(a * 2.0f));
    } else {
        int e;
        const float m = 2.0f * frexpf(a, &e);
        e -= 1;
        uint32_t q = static_cast<uint32_t>(rintf((m - 1.0f) * 2.0f));
        if (q == 2) {
            q = 0;
            ++e;
        }
        mag = (static_cast<uint32_t>(e + 1) << 1) | q;
    }
    return sign | mag;
}

__device__ __forceinline__ float pow2f(int e) { return ldexpf(1.0f, e); }

// ---------------------------------------------------------------------------------------------
// FP8 cast of bf16 rows, one 32-value block per thread
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cast_fp8_kernel(int64_t nblocks, const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks;
         b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = src[i];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(u[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int E = block_exponent(amax, 1.75f, 8);   // FP8 E4M3 largest value 448 = 1.75 * 2^8
        const float inv = pow2f(-E);
        uint32_t out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            out[i] = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) out[i] |= fp8_code(v[4 * i + j] * inv) << (8 * j);
        }
        uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
        dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
        dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
        scales[b] = static_cast<uint8_t>(E + 127);
    }
}

// ---------------------------------------------------------------------------------------------
// FP4 pack of the weights: one (expert, output column, 32-block along K) per thread
// ---------------------------------------------------------------------------------------------
// Packed layout (per expert, N output columns, reduction length K): the data of (column group
// n / 32, K step k / 64) is a 1 KB block at ((n / 32) * (K / 64) + k / 64) * 1024 whose lane
// l = n % 32 + 32 * ((k % 64) / 32) holds the 16 bytes at l * 16, nibble q = k % 32 (low nibble
// first); the scale bytes of the same (group, step) are a 64-byte block at the same block index *
// 64, byte l.  For W1 the column is the packed L1 column (gate and up groups interleaved).
template <bool W1>
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint16_t* __restrict__ w, int EL, int N, int K, int I,
                                                       uint8_t* __restrict__ wq, uint8_t* __restrict__ ws) {
    // logical weights: W1 [EL, K = H, N = 2I], W2 [EL, K = I, N = H]: element (e, k, n) at (e * K + k) * N + n
    const int64_t total = static_cast<int64_t>(EL) * N * (K / 32);
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int n = static_cast<int>(t % N);   // consecutive threads: consecutive columns (coalesced reads)
        const int64_t r = t / N;
        const int kb = static_cast<int>(r % (K / 32));
        const int e = static_cast<int>(r / (K / 32));
        const uint16_t* col = w + (static_cast<int64_t>(e) * K + 32 * kb) * N + n;
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            v[i] = bf16_to_f32(col[static_cast<int64_t>(i) * N]);
            amax = fmaxf(amax, fabsf(v[i]));
        }
        const int E = block_exponent(amax, 1.5f, 2);   // FP4 E2M1 largest value 6 = 1.5 * 2^2
        const float inv = pow2f(-E);
        uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 32; ++i) out[i / 8] |= fp4_code(v[i] * inv) << (4 * (i % 8));
        const int64_t pc = W1 ? l1_packed_col(n, I) : n;
        const int64_t blk = static_cast<int64_t>(e) * (static_cast<int64_t>(N) / 32) * (K / 64) + (pc / 32) * (K / 64) + kb / 2;
        const int lane = static_cast<int>(pc % 32) + 32 * (kb % 2);
        *reinterpret_cast<uint4*>(wq + blk * 1024 + lane * 16) = make_uint4(out[0], out[1], out[2], out[3]);
        ws[blk * 64 + lane] = static_cast<uint8_t>(E + 127);
    }
}

// ---------------------------------------------------------------------------------------------
// Grouped GEMMs on the block-scaled MFMA
// ---------------------------------------------------------------------------------------------
// A workgroup computes a BM x 256 tile (BM = 32 * MG = the workspace's block_m, so a tile is one
// row block of one expert) with four waves, each holding MG row groups x two 32-column groups.
// K advances 128 per slot (two 64-deep MFMA steps).  A (FP8 rows, 128 bytes per row per slot) and
// its scale bytes (4 per row per slot) go through a double-buffered LDS stage, 16-byte chunks
// XOR-swizzled by row; B (FP4, one 1 KB fragment and 64 scale bytes per column group and step) is
// private to a wave and loaded straight into registers one slot ahead.
constexpr int kMxThreads = 256;
constexpr int kMxBN = 256;

__device__ __forceinline__ int mx_lds_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
__device__ __forceinline__ int mx_acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int MG>
struct MxStage {   // one slot of A (codes + scales) in registers on its way into LDS
    static constexpr int PER = MG;   // 16-byte chunks per thread: BM * 8 / 256
    uint4 v[PER];
    uint32_t sc;
};

struct MxB {   // one slot of a wave's B: two column groups x two K steps
    uint4 d[2][2];
    uint32_t s[2][2];
};

template <int MG, bool L1>
struct MxGemm {
    static constexpr int BM = 32 * MG;
    static constexpr int A_BYTES = BM * 128, S_BYTES = BM * 4;
    static constexpr int BUF = A_BYTES + S_BYTES;
    static constexpr int LDS = 2 * BUF + 16 * BM;   // two buffers + row info
};

// Row sources of a tile: for every row the byte address of its codes and its scale bytes (padding
// rows read the zero row).
template <int MG>
__device__ __forceinline__ void mx_load_a(MxStage<MG>& st, const uint8_t* const* rows, const uint8_t* const* srows,
                                          int kt, int tid) {
#pragma unroll
    for (int i = 0; i < MG; ++i) {
        const int q = tid + i * kMxThreads;
        st.v[i] = *reinterpret_cast<const uint4*>(rows[i] + kt * 128 + (q & 7) * 16);
    }
    if (tid < 32 * MG) st.sc = *reinterpret_cast<const uint32_t*>(srows[0] + kt * 4);
}

template <int MG>
__device__ __forceinline__ void mx_store_a(const MxStage<MG>& st, char* buf, int tid) {
#pragma unroll
    for (int i = 0; i < MG; ++i) {
        const int q = tid + i * kMxThreads;
        *reinterpret_cast<uint4*>(buf + mx_lds_off(q >> 3, q & 7)) = st.v[i];
    }
    if (tid < 32 * MG) *reinterpret_cast<uint32_t*>(buf + 32 * MG * 128 + tid * 4) = st.sc;
}

__device__ __forceinline__ void mx_load_b(MxB& b, const uint8_t* const (&blk)[2], const uint8_t* const (&sblk)[2], int kt,
                                          int lane) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            b.d[g][s] = *reinterpret_cast<const uint4*>(blk[g] + (2 * kt + s) * 1024 + lane * 16);
            b.s[g][s] = sblk[g][(2 * kt + s) * 64 + lane];
        }
}

template <int MG>
__device__ __forceinline__ void mx_mma(const char* buf, const MxB& b, f32x16_t (&acc)[MG][2], int lane) {
    const char* sc = buf + 32 * MG * 128;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        v8i bv[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            bv[g] = v8i{static_cast<int>(b.d[g][s].x), static_cast<int>(b.d[g][s].y), static_cast<int>(b.d[g][s].z),
                        static_cast<int>(b.d[g][s].w), 0, 0, 0, 0};
        }
#pragma unroll
        for (int mi = 0; mi < MG; ++mi) {
            const int row = 32 * mi + (lane & 31), h = lane >> 5;
            const uint4 lo = *reinterpret_cast<const uint4*>(buf + mx_lds_off(row, 4 * s + h));
            const uint4 hi = *reinterpret_cast<const uint4*>(buf + mx_lds_off(row, 4 * s + 2 + h));
            const v8i av = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                            static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
            const int as = static_cast<int>(static_cast<const uint8_t*>(static_cast<const void*>(sc))[row * 4 + 2 * s + h]);
#pragma unroll
            for (int g = 0; g < 2; ++g)
                acc[mi][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv[g], acc[mi][g], 0, 4, 0, as, 0,
                                                                             static_cast<int>(b.s[g][s]));
        }
    }
}

// L1: gather the FP8 x rows through row_pair, GEMM against the FP4 W1, clamped SwiGLU, FP8 cast of
// the activation rows (codes [R_max, I] and scale bytes [R_max, I / 32] in ws.act).
// L2: GEMM of the FP8 activation rows against the FP4 W2, then the combine of the bf16 path
// (bf16(w * o) into y for a token's only local pair, fp32 w * o into its stage row otherwise).
template <int MG, bool L1>
__global__ __launch_bounds__(kMxThreads) void mx_gemm_kernel(const uint8_t* __restrict__ a_codes,
                                                             const uint8_t* __restrict__ a_scales,
                                                             const uint8_t* __restrict__ wq,
                                                             const uint8_t* __restrict__ wsc,
                                                             const float* __restrict__ topk_w, Dims d, Ws ws,
                                                             float clamp, uint16_t* __restrict__ y) {
    using G = MxGemm<MG, L1>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    int4* s_row = reinterpret_cast<int4*>(smem + 2 * G::BUF);   // token (-1 padding), weight, single
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = L1 ? d.H : d.I, N = L1 ? 2 * d.I : d.H;
    const int nk = K / 128, n_tiles = N / kMxBN;
    const int npairs = d.T * d.k;
    const int m_tiles = min(ws.meta[0] / G::BM, ws.num_blocks);
    const int total = m_tiles * n_tiles;
    uint8_t* act_codes = reinterpret_cast<uint8_t*>(ws.act);
    uint8_t* act_scales = act_codes + ws.rows_cap * d.I;
    const uint8_t* zrow = reinterpret_cast<const uint8_t*>(ws.zeros);
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mt = tile / n_tiles, nt = tile - mt * n_tiles;   // N tiles of an M tile adjacent: its rows stay in L2
        const int e = ws.tile_expert[mt];
        if (e < 0 || e >= d.EL) continue;   // uniform per workgroup
        const int64_t row0 = static_cast<int64_t>(mt) * G::BM;
        // row sources of this thread's A chunks and scale row
        const uint8_t* rows[MG];
        const uint8_t* srows[1];
#pragma unroll
        for (int i = 0; i < MG; ++i) {
            const int r = (tid + i * kMxThreads) >> 3;
            const int p = ws.row_pair[row0 + r];
            const bool ok = p >= 0 && p < npairs;
            rows[i] = !ok ? zrow : (L1 ? a_codes + static_cast<int64_t>(p / d.k) * K : a_codes + (row0 + r) * K);
        }
        {
            const int r = tid < G::BM ? tid : 0;
            const int p = ws.row_pair[row0 + r];
            const bool ok = p >= 0 && p < npairs;
            srows[0] = !ok ? zrow
                           : (L1 ? a_scales + static_cast<int64_t>(p / d.k) * (K / 32) : a_scales + (row0 + r) * (K / 32));
        }
        // this wave's two column groups of the packed weights
        const int64_t ebase = static_cast<int64_t>(e) * (N / 32) * (K / 64);
        const uint8_t* blk[2];
        const uint8_t* sblk[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int64_t grp = ebase + static_cast<int64_t>(nt * 8 + wave * 2 + g) * (K / 64);
            blk[g] = wq + grp * 1024;
            sblk[g] = wsc + grp * 64;
        }
        f32x16_t acc[MG][2];
#pragma unroll
        for (int mi = 0; mi < MG; ++mi)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][g][r] = 0.0f;

        lds_barrier();   // the previous tile's LDS reads are done
        if (tid < G::BM) {
            const int p = ws.row_pair[row0 + tid];
            const bool ok = p >= 0 && p < npairs;
            const int t = ok ? p / d.k : -1;
            const float w = ok && !L1 ? topk_w[p] : 0.0f;
            const int single = ok && !L1 ? (ws.tok_nloc[t] == 1) : 0;
            s_row[tid] = make_int4(t, __float_as_int(w), single, 0);
        }
        MxStage<MG> st;
        MxB b[2];
        mx_load_a<MG>(st, rows, srows, 0, tid);
        mx_load_b(b[0], blk, sblk, 0, lane);
        mx_store_a<MG>(st, smem, tid);
        lds_barrier();
        for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int k = kt + u;
                if (k >= nk) break;
                const bool more = k + 1 < nk;
                if (more) {
                    mx_load_a<MG>(st, rows, srows, k + 1, tid);
                    mx_load_b(b[u ^ 1], blk, sblk, k + 1, lane);
                }
                mx_mma<MG>(smem + u * G::BUF, b[u], acc, lane);
                if (more) mx_store_a<MG>(st, smem + (u ^ 1) * G::BUF, tid);
                lds_barrier();
            }
        }

        if constexpr (L1) {
            // SwiGLU on (gate, up) = column groups (0, 1); the wave's 32 intermediate columns are one
            // FP8 block of each row: its largest magnitude comes from the 32 lanes holding the row.
            const int q = nt * 4 + wave;   // intermediate column block
            const int col = 32 * q + (lane & 31);
#pragma unroll
            for (int mi = 0; mi < MG; ++mi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rl = 32 * mi + mx_acc_row(r, lane);
                    float g = acc[mi][0][r], u = acc[mi][1][r];
                    if (clamp > 0.0f) {
                        g = fminf(g, clamp);
                        u = fminf(fmaxf(u, -clamp), clamp);
                    }
                    const float a = silu_f32(g) * u;
                    float amax = fabsf(a);
#pragma unroll
                    for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
                    const int E = block_exponent(amax, 1.75f, 8);
                    const uint32_t code = fp8_code(a * pow2f(-E));
                    if (s_row[rl].x >= 0) {
                        const int64_t row = row0 + rl;
                        act_codes[row * d.I + col] = static_cast<uint8_t>(code);
                        if ((lane & 31) == 0) act_scales[row * (d.I / 32) + q] = static_cast<uint8_t>(E + 127);
                    }
                }
        } else {
#pragma unroll
            for (int mi = 0; mi < MG; ++mi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rl = 32 * mi + mx_acc_row(r, lane);
                    const int4 ri = s_row[rl];
                    if (ri.x < 0) continue;
                    const float w = __int_as_float(ri.y);
                    const int64_t row = row0 + rl;
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const int m = nt * kMxBN + wave * 64 + g * 32 + (lane & 31);
                        const float v = w * acc[mi][g][r];
                        if (ri.z) y[static_cast<int64_t>(ri.x) * d.H + m] = f32_to_bf16(v);
                        else ws.stage[row * d.H + m] = v;
                    }
                }
        }
    }
}

template <int MG, bool L1>
hipError_t mx_gemm_launch(const Dims& d, const uint8_t* ac, const uint8_t* as, const uint8_t* wq, const uint8_t* wsc,
                          const float* topk_w, const Ws& ws, float clamp, uint16_t* y, hipStream_t s) {
    using G = MxGemm<MG, L1>;
    auto k = mx_gemm_kernel<MG, L1>;
    if (G::LDS > 64 * 1024)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kMxThreads, G::LDS) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    const int n_tiles = (L1 ? 2 * d.I : d.H) / kMxBN;
    int64_t grid = static_cast<int64_t>(per_cu) * device_cu_count();
    const int64_t tiles = static_cast<int64_t>(ws.num_blocks) * n_tiles;
    if (grid > tiles) grid = tiles;
    if (grid < 1) grid = 1;
    k<<<static_cast<int>(grid), kMxThreads, G::LDS, s>>>(ac, as, wq, wsc, topk_w, d, ws, clamp, y);
    return hipGetLastError();
}

template <bool L1>
hipError_t mx_gemm(const Dims& d, const uint8_t* ac, const uint8_t* as, const uint8_t* wq, const uint8_t* wsc,
                   const float* topk_w, const Ws& ws, float clamp, uint16_t* y, hipStream_t s) {
    switch (d.BM) {
        case 32: return mx_gemm_launch<1, L1>(d, ac, as, wq, wsc, topk_w, ws, clamp, y, s);
        case 64: return mx_gemm_launch<2, L1>(d, ac, as, wq, wsc, topk_w, ws, clamp, y, s);
        case 128: return mx_gemm_launch<4, L1>(d, ac, as, wq, wsc, topk_w, ws, clamp, y, s);
        case 256: return mx_gemm_launch<8, L1>(d, ac, as, wq, wsc, topk_w, ws, clamp, y, s);
        default: return hipErrorInvalidValue;
    }
}

int grid_for(int64_t items) {
    const int64_t want = (items + 255) / 256, cap = static_cast<int64_t>(device_cu_count()) * 16;
    return static_cast<int>(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

hipError_t launch_mx_cast_fp8(int64_t rows, int cols, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
    const int64_t nb = rows * (cols / 32);
    if (nb <= 0) return hipSuccess;
    cast_fp8_kernel<<<grid_for(nb), 256, 0, s>>>(nb, x, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_gemm1(const Dims& d, const uint8_t* xq, const uint8_t* xs, const uint8_t* w1q, const uint8_t* w1s,
                           const Ws& ws, float clamp, hipStream_t s) {
    return mx_gemm<true>(d, xq, xs, w1q, w1s, nullptr, ws, clamp, nullptr, s);
}

hipError_t launch_mx_gemm2(const Dims& d, const uint8_t* w2q, const uint8_t* w2s, const float* topk_w, const Ws& ws,
                           uint16_t* y, hipStream_t s) {
    const uint8_t* act_codes = reinterpret_cast<const uint8_t*>(ws.act);
    return mx_gemm<false>(d, act_codes, act_codes + ws.rows_cap * d.I, w2q, w2s, topk_w, ws, 0.0f, y, s);
}

hipError_t launch_mx_pack(const Dims& d, const uint16_t* w1, const uint16_t* w2, uint8_t* w1q, uint8_t* w1s,
                          uint8_t* w2q, uint8_t* w2s, hipStream_t s) {
    if (w1) {
        pack_fp4_kernel<true><<<grid_for(static_cast<int64_t>(d.EL) * 2 * d.I * (d.H / 32)), 256, 0, s>>>(
            w1, d.EL, 2 * d.I, d.H, d.I, w1q, w1s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (w2) {
        pack_fp4_kernel<false><<<grid_for(static_cast<int64_t>(d.EL) * d.H * (d.I / 32)), 256, 0, s>>>(
            w2, d.EL, d.H, d.I, d.I, w2q, w2s);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace moe
