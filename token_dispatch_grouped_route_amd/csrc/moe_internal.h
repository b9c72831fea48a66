// Internal declarations of the gfx950 MoE expert-layer library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Layer sizes as the kernels see them.
struct Dims {
    int32_t T, H, I, E, e_lo, EL, k, BM;
};

// Device addresses of the workspace regions (host-computed from moe_ws_layout).
struct Ws {
    int32_t* counts;
    int32_t* offsets;       // padded_offsets [EL + 1]
    int32_t* row_pair;      // [R_max]
    int32_t* pair_row;      // [T * k]
    int32_t* tile_expert;   // [R_max / BM]
    int32_t* tok_nloc;      // [T]
    int32_t* meta;          // [0] R (padded rows), [1] dropped ids
    int32_t* chunk_hist;    // [num_chunks, EL] per-chunk expert counts, then exclusive bases
    int32_t* chunk_dropped; // [num_chunks]
    uint16_t* act;          // bf16 [R_max, I]
    float* stage;           // fp32 [R_max, H]
    float* hgu;             // fp32 [R_max, 2I] saved pre-activation (train)
    float* dact;            // fp32 [R_max, I]  L2 dgrad rows (train)
    uint16_t* dhgu;         // bf16 [R_max, 2I] [gate | up] gradient rows, hi part (train)
    uint16_t* dhgu_lo;      // bf16 [R_max, 2I] lo part: dhgu + dhgu_lo carries the fp32 value (train)
    uint16_t* wact;         // bf16 [R_max, I]  w * act (routing weight times activation), hi part (train)
    uint16_t* wact_lo;      // bf16 [R_max, I]  its lo part (train)
    float* dtw_part;        // fp32 [R_max, I / 128] per-row partials of d(topk_w) (train)
    uint16_t* zeros;        // a zero row of max(H, 2I) bf16 (written by the prologue)
    int32_t* tile_sync;     // [kMaxGrid] tile-scheduler counters of the forward GEMMs (zero between launches)
    int64_t rows_cap;
    int32_t num_blocks;     // R_max / BM
    int32_t num_chunks;     // prologue chunks of route_chunk pairs
    int32_t route_chunk;    // pairs per prologue block (route_chunk_for)
    int32_t zero_len;       // elements of the zero row
    int32_t dtw_cols;       // I / 128: partials per row in dtw_part
};

constexpr int kRouteThreads = 256;
constexpr int kMaxGrid = 512;   // workgroups of a persistent GEMM launch, at most
constexpr int kRouteChunkMin = 512;   // pairs per prologue block, at least
constexpr int kFusedHist = 8192;      // chunks x local experts staged in LDS by the fused scan + place launch

// Pairs per prologue block: the smallest power of two >= kRouteChunkMin that cuts the pairs into at
// most 256 chunks (one block per CU) and keeps chunks x local experts within the fused launch's
// LDS staging when it can.  Small batches then get more, shorter blocks.
inline int32_t route_chunk_for(int64_t pairs, int EL) {
    int64_t c = kRouteChunkMin;
    while (c < (int64_t(1) << 30) && ((pairs + c - 1) / c > 256 || (pairs + c - 1) / c * EL > kFusedHist)) c <<= 1;
    return static_cast<int32_t>(c);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {   // round to nearest even
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }
// v as two bf16 values hi + lo: hi = bf16(v), lo = bf16(v - hi) (the difference is exact in fp32),
// about 16 significant bits together.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16(v);
    lo = f32_to_bf16(v - bf16_to_f32(hi));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, then s_barrier.
// __syncthreads() also fences global memory, which waits for every global load in flight
// (s_waitcnt vmcnt(0)) and so drains a software pipeline at each step.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Fragment-major packed weights.  An expert's matrix B[n][k] (n output column, k reduction index,
// K = reduction length) is stored as 1 KB blocks, one per (32-column group, 16-deep K step),
// column group major; inside a block lane L holds the 8 consecutive k of column 32*nb + L%32
// starting at 16*kb + 8*(L/32): the B operand of v_mfma_f32_32x32x16_bf16, one 16-byte load per
// lane.  Eight consecutive k (from a multiple of 8) of one column are 16 contiguous bytes.
__host__ __device__ __forceinline__ int64_t frag_index(int64_t n, int64_t k, int64_t K) {
    return (((n >> 5) * (K >> 4) + (k >> 4)) * 64 + ((k >> 3) & 1) * 32 + (n & 31)) * 8 + (k & 7);
}
// Packed column of L1 output column n ([gate | up], 2I wide): column groups alternate gate and
// up of the same 32 intermediate columns, so a wave holding groups 2g and 2g+1 holds both halves
// of SwiGLU's input for intermediate columns [32g, 32g + 32).
__host__ __device__ __forceinline__ int64_t l1_packed_col(int64_t n, int64_t I) {
    const int64_t t = n >= I ? 1 : 0, m = n - t * I;
    return (m >> 5) * 64 + t * 32 + (m & 31);
}

// Host launchers (each returns a hipError_t from the launch).
// A wave's 32x32 accumulator block as whole 1 KB blocks of a fragment-packed weight gradient
// (moe_pack_weights layout, reduction length K): the tile's M index is the packed reduction index
// k (a 32-row block spans two 16-deep K steps) and its N index the packed column n (a 32-column
// block is one packed column group).  Lane L holds column n0 + L%32 and k = k0 + 8*(r/4) +
// 4*(L/32) + r%4 for r = 0..15, while a packed block wants lane L to hold the 8 consecutive k from
// 8*(L/32) of each 16-deep step; so lanes L and L^32 trade four values per step (one
// v_permlane32_swap each, a VALU exchange of the two half-waves: lane L < 32 keeps a and gets the a
// of lane L + 32, lane L >= 32 gets the b of lane L - 32 and keeps b), and every lane then stores
// 16 bytes: one store instruction writes a whole 1 KB block, with a nontemporal hint.
__device__ __forceinline__ void store_packed_block(uint16_t* out, int64_t K, int64_t n0, int64_t k0,
                                                 const f32x16_t& acc, int lane) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[8 * st + q]),
                                                            __float_as_uint(acc[8 * st + 4 + q]), false, false);
            v[q] = __uint_as_float(r[0]);
            v[4 + q] = __uint_as_float(r[1]);
        }
        uint32_t pk[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            pk[q] = static_cast<uint32_t>(f32_to_bf16(v[2 * q])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * q + 1])) << 16);
        const int64_t blk = (n0 >> 5) * (K >> 4) + ((k0 >> 4) + st);
        // nontemporal: the gradient is written once and not read again in the step, so it should
        // not evict what the following kernels read
        typedef uint32_t v4u __attribute__((ext_vector_type(4)));
        const v4u val = {pk[0], pk[1], pk[2], pk[3]};
        __builtin_nontemporal_store(val, reinterpret_cast<v4u*>(out + (blk * 64 + lane) * 8));
    }
}


hipError_t launch_route(const Dims& d, const int32_t* topk_idx, const Ws& ws, hipStream_t s);
hipError_t launch_pack(const Dims& d, const uint16_t* w1, const uint16_t* w2, uint16_t* w1p,
                       uint16_t* w2p, hipStream_t s);
hipError_t launch_unpack(const Dims& d, const uint16_t* w1p, const uint16_t* w2p, uint16_t* w1,
                         uint16_t* w2, hipStream_t s);
hipError_t launch_gemm1(const Dims& d, const uint16_t* x, const uint16_t* w1p, const Ws& ws,
                        uint16_t* act_out, float* hgu_out, hipStream_t s);
hipError_t launch_swiglu(const Dims& d, const float* hgu, const Ws& ws, uint16_t* act,
                         hipStream_t s);
hipError_t launch_gemm2_combine(const Dims& d, const uint16_t* act, const uint16_t* w2p,
                                const float* topk_w, const Ws& ws, uint16_t* y, hipStream_t s);
hipError_t launch_combine_finish(const Dims& d, const Ws& ws, uint16_t* y, hipStream_t s, bool nt_rows = false);
hipError_t launch_dgrad(const Dims& d, const uint16_t* dy, const float* topk_w,
                        const uint16_t* w2p, const Ws& ws, int fuse_swiglu_bwd, bool topk_w_grad,
                        hipStream_t s);
hipError_t launch_dtopk_w_finish(const Dims& d, const Ws& ws, float* dtopk_w, hipStream_t s);
hipError_t launch_dgrad1(const Dims& d, const uint16_t* w1p, const Ws& ws, uint16_t* dx, hipStream_t s);
hipError_t launch_swiglu_bwd(const Dims& d, const Ws& ws, hipStream_t s);
hipError_t launch_wgrad2(const Dims& d, const uint16_t* dy, const Ws& ws, uint16_t* dw2p, hipStream_t s);
bool wgrad_nt_fits(int M, int N);
bool dgrad_nt_fits(const Dims& d);
hipError_t launch_dgrad_nt(const Dims& d, const uint16_t* dy, const uint16_t* w2t, const float* topk_w, const Ws& ws,
                           int fuse, bool topk_w_grad, hipStream_t s);
hipError_t launch_dgrad_tr(const Dims& d, const uint16_t* dy, const uint16_t* w2p, const float* topk_w, const Ws& ws,
                           int fuse, bool topk_w_grad, hipStream_t s);
hipError_t launch_dgrad1_tr(const Dims& d, const uint16_t* w1p, const Ws& ws, uint16_t* dx, hipStream_t s);
hipError_t launch_wgrad_nt(const Dims& d, const uint16_t* at, const uint16_t* bp, int M, int N, const Ws& ws,
                           uint16_t* out, hipStream_t s);
hipError_t launch_wgrad1(const Dims& d, const uint16_t* x, const Ws& ws, uint16_t* dw1p,
                         hipStream_t s);

hipError_t launch_mx_cast_fp8(int64_t rows, int cols, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);
hipError_t launch_mx_gemm1(const Dims& d, const uint8_t* xq, const uint8_t* xs, const uint8_t* w1q, const uint8_t* w1s,
                           const Ws& ws, float clamp, hipStream_t s);
hipError_t launch_mx_gemm2(const Dims& d, const uint8_t* w2q, const uint8_t* w2s, const float* topk_w, const Ws& ws,
                           uint16_t* y, hipStream_t s);
hipError_t launch_mx_pack(const Dims& d, const uint16_t* w1, const uint16_t* w2, uint8_t* w1q, uint8_t* w1s,
                          uint8_t* w2q, uint8_t* w2s, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe
