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
