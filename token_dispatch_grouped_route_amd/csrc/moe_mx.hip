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
#include "moe_tiles.h"

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
// x's scale bytes in dispatch-row order for L1, slot-major: [H / 256][R_max][8], row r holding the
// eight bytes (one 256-deep K slot) of its pair's token, a padding row zeros; only the rows the
// prologue laid out (meta[0]) are written, the ones the tiles read.  One slot's scales of 32
// consecutive rows are then 256 contiguous bytes, where the token rows would put each in a cache
// line of its own.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_scales_kernel(Dims d, Ws ws, const uint8_t* __restrict__ xs,
                                                            uint8_t* __restrict__ out) {
    const int64_t cap = ws.rows_cap, npairs = static_cast<int64_t>(d.T) * d.k;
    const int64_t R = min(static_cast<int64_t>(max(ws.meta[0], 0)), cap), n = R * (d.H / 256);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t j = i / R, r = i - j * R;   // consecutive threads: consecutive rows of one slot
        const int pr = ws.row_pair[r];
        uint2 v = make_uint2(0u, 0u);
        if (pr >= 0 && pr < npairs)
            v = *reinterpret_cast<const uint2*>(xs + static_cast<int64_t>(pr / d.k) * (d.H / 32) + 8 * j);
        *reinterpret_cast<uint2*>(out + (j * cap + r) * 8) = v;
    }
}

// ---------------------------------------------------------------------------------------------
// FP4 pack of the weights: one (expert, output column, 32-block along K) per thread
// ---------------------------------------------------------------------------------------------
// Packed layout (per expert, N output columns, reduction length K, K a multiple of 256): the data
// of (column group n / 32, K step j = k / 64) is a 1 KB block at ((n / 32) * (K / 64) + j) * 1024
// whose lane l = n % 32 + 32 * ((k % 64) / 32) holds the 16 bytes at l * 16, nibble q = k % 32 (low
// nibble first); the scale bytes of a column group are (K / 64) * 64 bytes at (n / 32) * (K / 64) *
// 64, the scale of lane l in step j at (j / 4) * 256 + l * 4 + j % 4, so that one dword per lane
// holds four steps.  For W1 the column is the packed L1 column (gate and up groups interleaved).
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
        const int64_t grp = static_cast<int64_t>(e) * (static_cast<int64_t>(N) / 32) + pc / 32;
        const int j = kb / 2;   // K step of 64 within the column group
        const int lane = static_cast<int>(pc % 32) + 32 * (kb % 2);
        *reinterpret_cast<uint4*>(wq + (grp * (K / 64) + j) * 1024 + lane * 16) = make_uint4(out[0], out[1], out[2], out[3]);
        ws[grp * (K / 64) * 64 + (j / 4) * 256 + lane * 4 + j % 4] = static_cast<uint8_t>(E + 127);
    }
}

// ---------------------------------------------------------------------------------------------
// Grouped GEMMs on the block-scaled MFMA
// ---------------------------------------------------------------------------------------------
// A workgroup computes a BM x 256 tile (BM = 32 * MG rows of one expert) with four waves, one per
// SIMD, each holding MG row groups x two 32-column groups; K advances 256 per slot (four 64-deep
// MFMA steps).  B, the FP4 weights, is the stream that sets the pace (a weight byte serves only
// BM rows): each wave streams its two column groups straight into registers (per slot and lane
// eight 16-byte loads and one scale dword per group).  A, the FP8 rows, is shared by the waves and
// goes through LDS, straight from memory (global_load_lds_dwordx4: each instruction fills four
// 256-byte rows, chunks XOR-swizzled so fragment reads spread over the banks); each lane loads its
// own rows' eight scale bytes per slot into registers.  All of it runs through a ring of three
// slots loaded two slots ahead, a quarter per MFMA step; per slot: wait for this wave's loads of
// the slot, one barrier, four steps.
typedef __attribute__((address_space(1))) void g_void;
typedef __attribute__((address_space(3))) void l_void;

constexpr int kMxThreads = 256;
constexpr int kMxWaves = 4;
constexpr int kMxBN = 256;
constexpr int kMxSK = 256;   // K per slot
constexpr int kMxSlots = 3;   // ring slots: loads go out kMxSlots - 1 slots ahead (four measured no faster)

// 16-byte chunk c of LDS row r (256 bytes) sits at position c ^ (r % 16).
__device__ __forceinline__ int mx_lds_off(int row, int chunk) { return row * kMxSK + ((chunk ^ (row & 15)) << 4); }
__device__ __forceinline__ int mx_acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// s_waitcnt vmcnt(n) alone (gfx9 encoding: expcnt and lgkmcnt fields at their no-wait maxima).
template <int N>
__device__ __forceinline__ void mx_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int MG>
struct MxGemm {
    static_assert(kMxSlots == 3 || kMxSlots == 4, "ring of three or four slots");
    static constexpr int BM = 32 * MG;
    static constexpr int SLOT = BM * kMxSK;                 // bytes of one A slot
    static constexpr int LDS = kMxSlots * SLOT + 16 * BM;   // ring + row info
    static constexpr int A_DMA = BM / 16;                   // DMA loads per wave per slot (4 rows each)
    static constexpr int LOADS = A_DMA + 8 + 2 + MG;        // this wave's loads of one slot
};

template <int MG>
struct MxPipe {
    const char* a_src[MxGemm<MG>::A_DMA];   // the lane's chunk of its row of DMA load i, at K 0
    const uint8_t* as_src[MG];              // scale bytes of row 32 mi + lane % 32, slot 0
    int64_t as_slot;                        // bytes from one slot's scale rows to the next's
    const uint8_t* b_src[2];                // the lane's 16 bytes of group g's block, K step 0
    const uint8_t* bs_src[2];               // the lane's scale dword of group g, slot 0
    uint4 b[kMxSlots][2][4];
    uint32_t bs[kMxSlots][2];
    uint2 as[kMxSlots][MG];
    int nslot;                              // K / 256 (loads past the end re-read the last slot)
    int wave;

    // part q (0..3) of the loads of slot j into ring entry buf: DMA loads i = q, q + 4, ...; B K step q
    // of both groups; the B scale dwords with part 0 and the A scales with part 1
    __device__ __forceinline__ void issue(int j, char* __restrict__ slot, int buf, int q) {
        const int jj = min(j, nslot - 1);
#pragma unroll
        for (int i = 0; i < MxGemm<MG>::A_DMA; ++i)
            if (i % 4 == q)
                __builtin_amdgcn_global_load_lds((g_void*)(a_src[i] + jj * kMxSK),
                                                 (l_void*)(slot + 1024 * (wave + kMxWaves * i)), 16, 0, 0);
#pragma unroll
        for (int g = 0; g < 2; ++g) b[buf][g][q] = *reinterpret_cast<const uint4*>(b_src[g] + (4 * jj + q) * 1024);
        if (q == 0) {
#pragma unroll
            for (int g = 0; g < 2; ++g) bs[buf][g] = *reinterpret_cast<const uint32_t*>(bs_src[g] + jj * 256);
        }
        if (q == 1) {
#pragma unroll
            for (int mi = 0; mi < MG; ++mi) as[buf][mi] = *reinterpret_cast<const uint2*>(as_src[mi] + jj * as_slot);
        }
    }
    static constexpr int loads(int q) {
        return (MxGemm<MG>::A_DMA + 3 - q) / 4 + 2 + (q == 0 ? 2 : 0) + (q == 1 ? MG : 0);
    }
};

template <int MG>
__device__ __forceinline__ void mx_read_a(v8i (&a)[MG], const char* __restrict__ slot, int J, int lane) {
#pragma unroll
    for (int mi = 0; mi < MG; ++mi) {
        const int row = 32 * mi + (lane & 31), h = lane >> 5;
        const uint4 lo = *reinterpret_cast<const uint4*>(slot + mx_lds_off(row, 4 * J + h));
        const uint4 hi = *reinterpret_cast<const uint4*>(slot + mx_lds_off(row, 4 * J + 2 + h));
        a[mi] = v8i{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                    static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
    }
}

// MFMA step J (0..3) of slot ring entry U: byte J of a scale dword is this step's scale (the
// instruction's scale byte select); the loads of part J of slot j + 2 go out between the MFMAs.
template <int MG, int U, int J, bool ISSUE>
__device__ __forceinline__ void mx_step(MxPipe<MG>& p, int j, char* __restrict__ far, v8i (&a)[2][MG],
                                        const uint32_t (&asel)[MG], const char* __restrict__ cur,
                                        f32x16_t (&acc)[MG][2], int lane) {
    constexpr int FAR = (U + kMxSlots - 1) % kMxSlots;
    if (ISSUE) p.issue(j + kMxSlots - 1, far, FAR, J);
    if (J < 3) mx_read_a<MG>(a[(J + 1) & 1], cur, J + 1, lane);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const uint4 bd = p.b[U][g][J];
        const v8i bv = {static_cast<int>(bd.x), static_cast<int>(bd.y), static_cast<int>(bd.z), static_cast<int>(bd.w),
                        0, 0, 0, 0};
#pragma unroll
        for (int mi = 0; mi < MG; ++mi)
            acc[mi][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[J & 1][mi], bv, acc[mi][g], 0, 4, J,
                                                                         static_cast<int>(asel[mi]), J,
                                                                         static_cast<int>(p.bs[U][g]));
    }
    const int nv = ISSUE ? MxPipe<MG>::loads(J) : 0;
#pragma unroll
    for (int i = 0; i < 2 * MG; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           // MFMA
        if (J < 3 && i < 2 * MG) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        if (i < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);               // global load
    }
    if (2 * MG < nv)
        for (int i = 2 * MG; i < nv; ++i) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Slot j held in ring entry U.  WAIT: this wave's loads issued after slot j's, which may still be
// in flight.
template <int MG, int U, bool ISSUE, int WAIT>
__device__ __forceinline__ void mx_slot(MxPipe<MG>& p, int j, char* __restrict__ s0, char* __restrict__ s1,
                                        char* __restrict__ s2, char* __restrict__ s3, f32x16_t (&acc)[MG][2],
                                        int lane) {
    char* const slots[4] = {s0, s1, s2, s3};
    char* const cur = slots[U];
    char* const far = slots[(U + kMxSlots - 1) % kMxSlots];
    mx_wait_vmcnt<WAIT>();
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's fragment reads are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // A scale of (row, step J, 32-block h = lane / 32) is the row's slot byte 2 J + h: this lane's
    // four, byte J for step J
    uint32_t asel[MG];
#pragma unroll
    for (int mi = 0; mi < MG; ++mi)
        asel[mi] = __builtin_amdgcn_perm(p.as[U][mi].y, p.as[U][mi].x, (lane >> 5) ? 0x07050301u : 0x06040200u);
    v8i a[2][MG];
    mx_read_a<MG>(a[0], cur, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
    mx_step<MG, U, 0, ISSUE>(p, j, far, a, asel, cur, acc, lane);
    mx_step<MG, U, 1, ISSUE>(p, j, far, a, asel, cur, acc, lane);
    mx_step<MG, U, 2, ISSUE>(p, j, far, a, asel, cur, acc, lane);
    mx_step<MG, U, 3, ISSUE>(p, j, far, a, asel, cur, acc, lane);
}

// Slots j + I .. j + kMxSlots - 1 of one turn of the unrolled loop.
template <int MG, int I>
__device__ __forceinline__ void mx_turn(MxPipe<MG>& p, int j, char* __restrict__ s0, char* __restrict__ s1,
                                        char* __restrict__ s2, char* __restrict__ s3, f32x16_t (&acc)[MG][2],
                                        int lane) {
    if constexpr (I < kMxSlots) {
        mx_slot<MG, I, true, (kMxSlots - 2) * MxGemm<MG>::LOADS>(p, j + I, s0, s1, s2, s3, acc, lane);
        mx_turn<MG, I + 1>(p, j, s0, s1, s2, s3, acc, lane);
    }
}

// The last nslot % kMxSlots slots (j a multiple of kMxSlots): the loop (or the prologue) issued
// through slot j + kMxSlots - 2, so kMxSlots - 2 - I slots' loads follow those of slot j + I.
template <int MG, int I>
__device__ __forceinline__ void mx_tail(MxPipe<MG>& p, int j, char* __restrict__ s0, char* __restrict__ s1,
                                        char* __restrict__ s2, char* __restrict__ s3, f32x16_t (&acc)[MG][2],
                                        int lane) {
    if constexpr (I < kMxSlots - 1) {
        if (j + I < p.nslot) {
            mx_slot<MG, I, false, (kMxSlots - 2 - I) * MxGemm<MG>::LOADS>(p, j + I, s0, s1, s2, s3, acc, lane);
            mx_tail<MG, I + 1>(p, j, s0, s1, s2, s3, acc, lane);
        }
    }
}

// Prologue: the loads of slots I .. kMxSlots - 2, all of one slot before any of the next (the
// waits count in issue order).
template <int MG, int I>
__device__ __forceinline__ void mx_prologue(MxPipe<MG>& p, char* __restrict__ s0, char* __restrict__ s1,
                                            char* __restrict__ s2) {
    if constexpr (I < kMxSlots - 1) {
        char* const slots[3] = {s0, s1, s2};
#pragma unroll
        for (int q = 0; q < 4; ++q) p.issue(I, slots[I], I, q);
        __builtin_amdgcn_sched_barrier(0);
        mx_prologue<MG, I + 1>(p, s0, s1, s2);
    }
}

// acc = A[rows, 0:K] . B[0:K, cols].  Ends with no load in flight and all waves past their last
// fragment read, so the caller may reuse the LDS.  s3 is unused with three slots.
template <int MG>
__device__ __forceinline__ void mx_k_loop(MxPipe<MG>& p, char* __restrict__ s0, char* __restrict__ s1,
                                          char* __restrict__ s2, char* __restrict__ s3, f32x16_t (&acc)[MG][2],
                                          int lane) {
#pragma unroll
    for (int mi = 0; mi < MG; ++mi)
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][g][r] = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    mx_prologue<MG, 0>(p, s0, s1, s2);
    int j = 0;
    for (; j + kMxSlots <= p.nslot; j += kMxSlots) mx_turn<MG, 0>(p, j, s0, s1, s2, s3, acc, lane);
    mx_tail<MG, 0>(p, j, s0, s1, s2, s3, acc, lane);
    mx_wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// L1: gather the FP8 x rows through row_pair, GEMM against the FP4 W1, clamped SwiGLU, FP8 cast of
// the activation rows (codes [R_max, I] and scale bytes [R_max, I / 32] in ws.act).
// L2: GEMM of the FP8 activation rows against the FP4 W2, then the combine of the bf16 path
// (bf16(w * o) into y for a token's only local pair, fp32 w * o into its stage row otherwise).
// Tiles come from the shared tile list (moe_tiles.h): up to MAXG real 32-row groups of one expert
// (BM = 32 MG rows for a tile of MG groups), so an expert of the wide share (41-76 rows) is one
// tile and its weights stream once, whatever block_m is.  The ring slots are sized for MAXG.  One
// workgroup per CU: the LDS of three-group tiles allows one (tiles of at most two groups at two
// workgroups per CU measured slower for L2, their tile loop spilling).
template <int MAXG>
struct MxSched {
    static constexpr int NT = kMxThreads;
    static constexpr int MAXMI = MAXG;
    static constexpr int SLOT = MxGemm<MAXG>::SLOT;   // ring slot stride
    static constexpr int LDS = MxGemm<MAXG>::LDS;
};

template <int MAXG, bool L1>
struct MxBody {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* wq;
    const uint8_t* wsc;
    const float* topk_w;
    Dims d;
    Ws ws;
    float clamp;
    uint16_t* y;
    char* smem;

    template <int MG>
    __device__ __forceinline__ void run(const TileRef& t) {
        using G = MxGemm<MG>;
        constexpr int SLOT = MxSched<MAXG>::SLOT;
        char* const s0 = smem;
        char* const s1 = smem + SLOT;
        char* const s2 = smem + 2 * SLOT;
        char* const s3 = smem + (kMxSlots - 1) * SLOT;   // the fourth slot (unused with three)
        int4* s_row = reinterpret_cast<int4*>(smem + kMxSlots * SLOT);   // token (-1 padding), weight, single
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int K = L1 ? d.H : d.I, N = L1 ? 2 * d.I : d.H;
        const int npairs = d.T * d.k;
        uint8_t* act_codes = reinterpret_cast<uint8_t*>(ws.act);
        uint8_t* act_scales = act_codes + ws.rows_cap * d.I;
        const uint8_t* zrow = reinterpret_cast<const uint8_t*>(ws.zeros);
        MxPipe<MG> p;
        p.nslot = K / kMxSK;
        p.wave = wave;
        const int nt = t.nt, e = t.e;
        const int64_t row0 = t.row0;
        // sources (padding rows read the zero row)
#pragma unroll
        for (int i = 0; i < G::A_DMA; ++i) {
            const int r = 4 * (wave + kMxWaves * i) + (lane >> 4);
            const int pr = ws.row_pair[row0 + r];
            const bool ok = pr >= 0 && pr < npairs;
            const uint8_t* src = !ok ? zrow : (L1 ? a_codes + static_cast<int64_t>(pr / d.k) * K : a_codes + (row0 + r) * K);
            p.a_src[i] = reinterpret_cast<const char*>(src) + 16 * ((lane & 15) ^ (r & 15));
        }
        // scale bytes by row, slot-major ([K / 256][R_max][8]: x's gathered into row order, the
        // activation's as L1 writes them), so a slot's scales of 32 rows are 256 contiguous bytes
        p.as_slot = static_cast<int64_t>(ws.rows_cap) * 8;
#pragma unroll
        for (int mi = 0; mi < MG; ++mi) p.as_src[mi] = a_scales + (row0 + 32 * mi + (lane & 31)) * 8;
        const int64_t ebase = static_cast<int64_t>(e) * (N / 32) * (K / 64);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int64_t grp = ebase + static_cast<int64_t>(nt * 8 + wave * 2 + g) * (K / 64);
            p.b_src[g] = wq + grp * 1024 + lane * 16;
            p.bs_src[g] = wsc + grp * 64 + lane * 4;
        }
        if (tid < G::BM) {   // read in the epilogue, after the K loop's barriers
            const int pr = ws.row_pair[row0 + tid];
            const bool ok = pr >= 0 && pr < npairs;
            const int tok = ok ? pr / d.k : -1;
            const float w = ok && !L1 ? topk_w[pr] : 0.0f;
            const int single = ok && !L1 ? (ws.tok_nloc[tok] == 1) : 0;
            s_row[tid] = make_int4(tok, __float_as_int(w), single, 0);
        }
        f32x16_t acc[MG][2];
        mx_k_loop<MG>(p, s0, s1, s2, s3, acc, lane);

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
                    const int64_t row = row0 + rl;
                    const bool real = s_row[rl].x >= 0;
                    if (real) act_codes[row * d.I + col] = static_cast<uint8_t>(code);
                    // slot-major like the gathered x scales; a padding row gets scale byte 0
                    // (L2 reads its codes from the zero row)
                    if ((lane & 31) == 0)
                        act_scales[((q >> 3) * static_cast<int64_t>(ws.rows_cap) + row) * 8 + (q & 7)] =
                            real ? static_cast<uint8_t>(E + 127) : static_cast<uint8_t>(0);
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
};

template <int MAXG, bool L1>
__global__ __launch_bounds__(kMxThreads, 1) void mx_gemm_kernel(const uint8_t* __restrict__ a_codes,
                                                             const uint8_t* __restrict__ a_scales,
                                                             const uint8_t* __restrict__ wq,
                                                             const uint8_t* __restrict__ wsc,
                                                             const float* __restrict__ topk_w, Dims d, Ws ws,
                                                             float clamp, uint16_t* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    MxBody<MAXG, L1> body{a_codes, a_scales, wq, wsc, topk_w, d, ws, clamp, y, smem};
    run_tiles<MxSched<MAXG>>(d, ws, (L1 ? 2 * d.I : d.H) / kMxBN, body);
}

template <int MAXG, bool L1>
hipError_t mx_gemm_launch(const Dims& d, const uint8_t* ac, const uint8_t* as, const uint8_t* wq, const uint8_t* wsc,
                          const float* topk_w, const Ws& ws, float clamp, uint16_t* y, hipStream_t s) {
    using S = MxSched<MAXG>;
    auto k = mx_gemm_kernel<MAXG, L1>;
    allow_lds(k, S::LDS);
    const int n_tiles = (L1 ? 2 * d.I : d.H) / kMxBN;
    k<<<tile_grid(k, kMxThreads, S::LDS, d, MAXG, n_tiles), kMxThreads, S::LDS, s>>>(ac, as, wq, wsc, topk_w, d, ws, clamp,
                                                                                    y);
    return hipGetLastError();
}

template <bool L1>
hipError_t mx_gemm(const Dims& d, const uint8_t* ac, const uint8_t* as, const uint8_t* wq, const uint8_t* wsc,
                   const float* topk_w, const Ws& ws, float clamp, uint16_t* y, hipStream_t s) {
    if (d.EL > kMaxEL) return hipErrorInvalidValue;
    return mx_gemm_launch<3, L1>(d, ac, as, wq, wsc, topk_w, ws, clamp, y, s);
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
    // the gathered scales (R_max * H / 32 bytes) go into ws stage (4 * R_max * H bytes), which L2's
    // combine rows reuse only after L1
    if (!ws.stage) return hipErrorInvalidValue;
    uint8_t* rs = reinterpret_cast<uint8_t*>(ws.stage);
    const int64_t n = static_cast<int64_t>(ws.rows_cap) * (d.H / 256);   // at most; the kernel reads R
    if (n > 0) {
        const int grid = std::min(grid_for(n), 2 * device_cu_count());
        gather_scales_kernel<<<grid, 256, 0, s>>>(d, ws, xs, rs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return mx_gemm<true>(d, xq, rs, w1q, w1s, nullptr, ws, clamp, nullptr, s);
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
