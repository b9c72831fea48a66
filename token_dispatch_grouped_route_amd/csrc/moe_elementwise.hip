// Memory-bound kernels of the MoE expert layer: the one-time weight transform (and its inverse),
// the standalone SwiGLU forward and backward ("Mega MoE" page, Implementation Map: SwiGLU fwd/bwd), and the
// last step of the combine (top-k reduce, "Mega MoE" page, Pipeline).  All use 16-byte
// vector accesses on contiguous rows; row counts that depend on the routing are read from the
// workspace on the device.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// Weight transform: logical [EL, K, N] (x @ W layout) <-> fragment-major packed layout
// (frag_index).  One block moves one 32-column group x 128 K of one expert through LDS.
// ---------------------------------------------------------------------------------------------
// First logical column of packed column group nb (L1: gate and up groups alternate).
__device__ __forceinline__ int64_t group_col0(int nb, int I, bool l1) {
    return l1 ? static_cast<int64_t>(nb & 1) * I + 32 * (nb >> 1) : 32 * static_cast<int64_t>(nb);
}

template <bool PACK>
__global__ __launch_bounds__(256) void repack_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                     int K, int N, int I, int l1) {
    __shared__ uint16_t tile[128][32 + 2];
    const int nb = blockIdx.x, k0 = blockIdx.y * 128, e = blockIdx.z, tid = threadIdx.x;
    const int64_t ebase = static_cast<int64_t>(e) * K * N;
    const int64_t n0 = group_col0(nb, I, l1 != 0);
    const uint16_t* logical_in = in + ebase;
    uint16_t* logical_out = out + ebase;
    if (PACK) {
        for (int q = tid; q < 128 * 16; q += 256) {   // 128 rows x 16 pairs of columns
            const int r = q >> 4, c2 = q & 15;
            if (k0 + r < K) {
                const uint32_t v = *reinterpret_cast<const uint32_t*>(logical_in + static_cast<int64_t>(k0 + r) * N + n0 + 2 * c2);
                tile[r][2 * c2] = static_cast<uint16_t>(v & 0xffffu);
                tile[r][2 * c2 + 1] = static_cast<uint16_t>(v >> 16);
            }
        }
        __syncthreads();
        for (int q = tid; q < 8 * 64; q += 256) {   // 8 K steps x 64 lanes of 16 bytes
            const int kb = q >> 6, L = q & 63, c = L & 31, kk = kb * 16 + 8 * (L >> 5);
            if (k0 + kk >= K) continue;
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = static_cast<uint32_t>(tile[kk + 2 * j][c]) | (static_cast<uint32_t>(tile[kk + 2 * j + 1][c]) << 16);
            *reinterpret_cast<uint4*>(out + ebase + frag_index(32 * nb + c, k0 + kk, K)) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        for (int q = tid; q < 8 * 64; q += 256) {
            const int kb = q >> 6, L = q & 63, c = L & 31, kk = kb * 16 + 8 * (L >> 5);
            if (k0 + kk >= K) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(in + ebase + frag_index(32 * nb + c, k0 + kk, K));
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                tile[kk + 2 * j][c] = static_cast<uint16_t>(w[j] & 0xffffu);
                tile[kk + 2 * j + 1][c] = static_cast<uint16_t>(w[j] >> 16);
            }
        }
        __syncthreads();
        for (int q = tid; q < 128 * 16; q += 256) {
            const int r = q >> 4, c2 = q & 15;
            if (k0 + r < K)
                *reinterpret_cast<uint32_t*>(logical_out + static_cast<int64_t>(k0 + r) * N + n0 + 2 * c2) =
                    static_cast<uint32_t>(tile[r][2 * c2]) | (static_cast<uint32_t>(tile[r][2 * c2 + 1]) << 16);
        }
    }
}

// W1 [EL, H, 2I] (K = H, N = 2I, gate/up groups interleaved) and W2 [EL, I, H] (K = I, N = H).
hipError_t launch_pack(const Dims& d, const uint16_t* w1, const uint16_t* w2, uint16_t* w1p,
                       uint16_t* w2p, hipStream_t s) {
    if (w1 && w1p) {
        dim3 g(2 * d.I / 32, (d.H + 127) / 128, d.EL);
        repack_kernel<true><<<g, 256, 0, s>>>(w1, w1p, d.H, 2 * d.I, d.I, 1);
    }
    if (w2 && w2p) {
        dim3 g(d.H / 32, (d.I + 127) / 128, d.EL);
        repack_kernel<true><<<g, 256, 0, s>>>(w2, w2p, d.I, d.H, d.I, 0);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const Dims& d, const uint16_t* w1p, const uint16_t* w2p, uint16_t* w1,
                         uint16_t* w2, hipStream_t s) {
    if (w1 && w1p) {
        dim3 g(2 * d.I / 32, (d.H + 127) / 128, d.EL);
        repack_kernel<false><<<g, 256, 0, s>>>(w1p, w1, d.H, 2 * d.I, d.I, 1);
    }
    if (w2 && w2p) {
        dim3 g(d.H / 32, (d.I + 127) / 128, d.EL);
        repack_kernel<false><<<g, 256, 0, s>>>(w2p, w2, d.I, d.H, d.I, 0);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// SwiGLU forward / backward over rows [0, R)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

constexpr int kEwThreads = 256;

// 8 consecutive fp32 values (two 16-byte loads)
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
// 8 values as bf16 hi parts and lo parts (split_bf16), one 16-byte store each
__device__ __forceinline__ void store_split8(uint16_t* hi, uint16_t* lo, const float (&f)[8]) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) split_bf16(f[i], h[i], l[i]);
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wh[i] = h[2 * i] | (static_cast<uint32_t>(h[2 * i + 1]) << 16);
        wl[i] = l[2 * i] | (static_cast<uint32_t>(l[2 * i + 1]) << 16);
    }
    *reinterpret_cast<uint4*>(hi) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    *reinterpret_cast<uint4*>(lo) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
}

// act = silu(g) * u over fp32 [gate | up] rows (the forward's SwiGLU, on the saved pre-activation).
__global__ __launch_bounds__(kEwThreads) void swiglu_kernel(const float* __restrict__ hgu, Dims d, Ws ws,
                                                            uint16_t* __restrict__ act) {
    const int64_t R = ws.meta[0];
    const int v8 = d.I / 8;
    const int64_t n = R * v8;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < n;
         q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t r = q / v8;
        const int c = static_cast<int>(q - r * v8) * 8;
        float g[8], u[8], a[8];
        load8(hgu + r * 2 * d.I + c, g);
        load8(hgu + r * 2 * d.I + d.I + c, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = silu_f32(g[i]) * u[i];
        *reinterpret_cast<uint4*>(act + r * d.I + c) = pack8(a);
    }
}

// SwiGLU transpose from fp32 dact and the fp32 pre-activation; dhgu as hi and lo bf16 rows.
__global__ __launch_bounds__(kEwThreads) void swiglu_bwd_kernel(Dims d, Ws ws) {
    const int64_t R = ws.meta[0];
    const int v8 = d.I / 8;
    const int64_t n = R * v8;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < n;
         q += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t r = q / v8;
        const int c = static_cast<int>(q - r * v8) * 8;
        float g[8], u[8], da[8], dg[8], du[8];
        load8(ws.hgu + r * 2 * d.I + c, g);
        load8(ws.hgu + r * 2 * d.I + d.I + c, u);
        load8(ws.dact + r * d.I + c, da);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sg = 1.0f / (1.0f + __expf(-g[i]));
            dg[i] = da[i] * u[i] * sg * (1.0f + g[i] * (1.0f - sg));
            du[i] = da[i] * g[i] * sg;
        }
        store_split8(ws.dhgu + r * 2 * d.I + c, ws.dhgu_lo + r * 2 * d.I + c, dg);
        store_split8(ws.dhgu + r * 2 * d.I + d.I + c, ws.dhgu_lo + r * 2 * d.I + d.I + c, du);
    }
}

static int ew_grid(int64_t rows_cap, int per_row_vectors) {
    const int64_t want = (rows_cap * per_row_vectors + kEwThreads - 1) / kEwThreads;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
    return static_cast<int>(want < 1 ? 1 : (want > cap ? cap : want));
}

hipError_t launch_swiglu(const Dims& d, const float* hgu, const Ws& ws, uint16_t* act, hipStream_t s) {
    swiglu_kernel<<<ew_grid(ws.rows_cap, d.I / 8), kEwThreads, 0, s>>>(hgu, d, ws, act);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const Dims& d, const Ws& ws, hipStream_t s) {
    swiglu_bwd_kernel<<<ew_grid(ws.rows_cap, d.I / 8), kEwThreads, 0, s>>>(d, ws);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine finish: y rows of tokens with no local pair are zero; tokens with several local pairs
// sum their weighted fp32 L2 rows from ws.stage in slot order and store bf16.  Tokens with one
// local pair were written by the L2 epilogue and are left alone.
// ---------------------------------------------------------------------------------------------
// One wave per token: lanes [0, k) read the token's pair rows at once and a ballot lists its local
// pairs in slot order, so a token costs one dependent load before its stage rows stream.  A pass
// covers up to kFinishChunks 32-byte chunks per lane: all of one pair row's chunks are loaded
// before they are added, so a pass waits once per local pair, not once per chunk; each element is
// still summed in slot order.  With NT the staged rows are read with a nontemporal hint (the L1
// dgrad's, which its few-rows kernel also stores nontemporally).
constexpr int kFinishChunks = 4;

template <bool NT>
__global__ __launch_bounds__(kEwThreads) void combine_finish_kernel(Dims d, Ws ws, uint16_t* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * (kEwThreads / 64);
    const int v8 = d.H / 8;
    for (int t = blockIdx.x * (kEwThreads / 64) + (threadIdx.x >> 6); t < d.T; t += waves) {
        int r = -1;
        if (lane < d.k) r = ws.pair_row[static_cast<int64_t>(t) * d.k + lane];
        const uint64_t local = __ballot(r >= 0 && r < ws.rows_cap);
        if (__popcll(local) == 1) continue;   // the GEMM epilogue stored this token's only row
        for (int c0 = lane; c0 < v8; c0 += 64 * kFinishChunks) {
            float acc[kFinishChunks][8];
#pragma unroll
            for (int i = 0; i < kFinishChunks; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
            for (uint64_t m = local; m; m &= m - 1) {   // local pairs in slot order
                const int row = __shfl(r, __ffsll(static_cast<unsigned long long>(m)) - 1);
                const float4* src = reinterpret_cast<const float4*>(ws.stage + static_cast<int64_t>(row) * d.H);
                float4 lo[kFinishChunks], hi[kFinishChunks];
#pragma unroll
                for (int i = 0; i < kFinishChunks; ++i) {
                    const int c = c0 + 64 * i;
                    if (c < v8) {
                        if constexpr (NT) {
                            typedef float v4f __attribute__((ext_vector_type(4)));
                            const v4f l4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + 2 * c));
                            const v4f h4 = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + 2 * c + 1));
                            lo[i] = make_float4(l4.x, l4.y, l4.z, l4.w);
                            hi[i] = make_float4(h4.x, h4.y, h4.z, h4.w);
                        } else {
                            lo[i] = src[2 * c];
                            hi[i] = src[2 * c + 1];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < kFinishChunks; ++i) {
                    if (c0 + 64 * i < v8) {
                        acc[i][0] += lo[i].x; acc[i][1] += lo[i].y; acc[i][2] += lo[i].z; acc[i][3] += lo[i].w;
                        acc[i][4] += hi[i].x; acc[i][5] += hi[i].y; acc[i][6] += hi[i].z; acc[i][7] += hi[i].w;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < kFinishChunks; ++i) {
                const int c = c0 + 64 * i;
                if (c < v8) {   // nontemporal, as the L2 epilogue's direct rows
                    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
                    const uint4 p = pack8(acc[i]);
                    const v4u val = {p.x, p.y, p.z, p.w};
                    __builtin_nontemporal_store(val, reinterpret_cast<v4u*>(y + static_cast<int64_t>(t) * d.H + 8 * c));
                }
            }
        }
    }
}

hipError_t launch_combine_finish(const Dims& d, const Ws& ws, uint16_t* y, hipStream_t s, bool nt_rows) {
    if (d.T <= 0) return hipSuccess;
    const int cap = device_cu_count() * 8, want = (d.T + kEwThreads / 64 - 1) / (kEwThreads / 64);
    if (nt_rows) combine_finish_kernel<true><<<want < cap ? want : cap, kEwThreads, 0, s>>>(d, ws, y);
    else combine_finish_kernel<false><<<want < cap ? want : cap, kEwThreads, 0, s>>>(d, ws, y);
    return hipGetLastError();
}

// d(topk_w)[p] = sum over the N tiles of the L2 dgrad of its per-row partial, in tile order, for
// the row of a local pair; 0 for a pair this GPU does not handle.
__global__ __launch_bounds__(kEwThreads) void dtopk_w_finish_kernel(Dims d, Ws ws, float* __restrict__ dtopk_w) {
    const int64_t np = static_cast<int64_t>(d.T) * d.k;
    const int cols = ws.dtw_cols;
    for (int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; p < np;
         p += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int r = ws.pair_row[p];
        float sum = 0.0f;
        if (r >= 0 && r < ws.rows_cap)
            for (int j = 0; j < cols; ++j) sum += ws.dtw_part[static_cast<int64_t>(r) * cols + j];
        dtopk_w[p] = sum;
    }
}

hipError_t launch_dtopk_w_finish(const Dims& d, const Ws& ws, float* dtopk_w, hipStream_t s) {
    const int64_t np = static_cast<int64_t>(d.T) * d.k;
    if (np <= 0) return hipSuccess;
    const int64_t want = (np + kEwThreads - 1) / kEwThreads, cap = device_cu_count() * 8;
    dtopk_w_finish_kernel<<<static_cast<int>(want < cap ? want : cap), kEwThreads, 0, s>>>(d, ws, dtopk_w);
    return hipGetLastError();
}

}  // namespace moe
