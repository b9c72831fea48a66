// Forward grouped GEMMs of the MoE expert layer on gfx950 (v_mfma_f32_32x32x16_bf16, fp32
// accumulation), reading fragment-packed weights ("Mega MoE" page, Pipeline: the L1 grouped
// GEMM with the dispatch gather and SwiGLU, and the L2 grouped GEMM with the top-k combine).
//
// Tiles.  An M tile is up to eight 32-row groups of one expert's segment (256 rows; nine, for
// experts of at most 18 groups, in the forward GEMMs of launches whose experts average at most
// 512 rows), covering only the groups that
// hold real rows: rows past the last real group are padding and get no MFMA work.  An expert with
// more groups is cut into M tiles whose group counts differ by at most one, so the workgroups
// that stream the same weight panel progress at nearly the same rate and the later reads of the
// panel hit L2.  An N tile is BN = 4 waves
// x 32*NI columns; every wave (one per SIMD) computes all rows of its own 32*NI columns.  So a
// weight panel (expert, N tile) is streamed by one workgroup per M tile, and an expert's token
// rows are read by the workgroups of all its N tiles at the same time, from L2.
//
// Operands
//   A  token rows (L1: x rows gathered through row_pair; L2: act rows), K-contiguous.  Shared by
//      the waves, so it goes through LDS, straight from memory (global_load_lds_dwordx4: no
//      staging registers, no LDS store instructions) into a ring of three 64-deep K slots; each
//      load instruction fills 8 rows x 128 bytes, chunks XOR-swizzled so fragment reads spread
//      over the banks.  The ring has SLOTS 64-deep K slots (four; three for 288-row tiles).
//   B  packed expert weights (moe_pack_weights): every 1 KB block is one MFMA B operand of a
//      32-column group and a 16-deep K step.  Each wave owns its column groups, so B never
//      touches LDS: a wave streams its blocks straight into registers, one contiguous 1 KB load
//      per block, through a ring of SLOTS 64-deep K stages.
// Both are loaded SLOTS - 1 slots ahead of their MFMAs.  Per slot: wait for this wave's loads of
// the slot, one barrier, then the slot's four 16-deep MFMA steps, each issuing a quarter of the
// loads of slot + SLOTS - 1 and reading the next step's fragments between its MFMAs.  The LDS slots
// are distinct noalias pointers of the K loop, so the compiler does not make fragment reads wait
// for the DMA loads into other slots.
//
// The backward GEMMs run on the same pipeline: the L2 dgrad (dgrad_tile_kernel) and the L1 dgrad
// (l2_kernel with dhgu rows as A) of experts with few rows read the packed weights themselves
// through LDS, transposed (TrPipe); with many rows the dgrads take repacked weights and the weight
// gradients transformed operands (wgrad_nt_kernel), all in registers.
//
// Schedule (moe_tiles.h): a persistent grid of one workgroup per CU, capped at the tiles the
// shape allows.  The tile list is ordered expert by expert, then in blocks of eight M tiles, N
// tile by N tile with the M tiles of that panel adjacent, and cut into one contiguous chunk per
// XCD (workgroup b runs on XCD b mod 8).  Workgroups take the next tile of their XCD's chunk from
// an atomic counter, largest tiles first, and help other XCDs once their own is done.
#include <type_traits>

#include "moe_internal.h"
#include "moe_tiles.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) void g_void;
typedef __attribute__((address_space(3))) void l_void;

constexpr int kWaves = 4;
constexpr int kEpiBatch = 4;   // L2 epilogue: LDS chunks read before their stores go out

// NI: 32-column groups per wave; MAXMI: 32-row groups per M tile, at most (nine only for the
// forward tiles, whose ninth group runs in VGPR-form MFMAs, see slot_step); OCC: workgroups per CU;
// SLOTS: LDS slots of A and register stages of B (64-deep K each), loaded SLOTS - 1 slots ahead;
// NTB: B loads with a nontemporal hint (for launches whose weight panels are read by one or two M
// tiles: the panel then does not evict the token rows that every N tile re-reads).
template <int NI_, int MAXMI_, int OCC_, int SLOTS_, bool NTB_ = false>
struct Tile {
    static constexpr int NI = NI_, MAXMI = MAXMI_, OCC = OCC_, SLOTS = SLOTS_;
    static constexpr bool kNtB = NTB_;
    static constexpr bool kNtStage = false;   // fp32 combine rows stored temporally (read back soon)
    static_assert(MAXMI >= 1 && MAXMI <= 9, "M tile of 1..9 groups");
    static_assert(SLOTS == 3 || SLOTS == 4, "ring of three or four slots");
    static constexpr int BM = 32 * MAXMI, BN = kWaves * 32 * NI;
    static constexpr int NT = 64 * kWaves;
    static constexpr bool kTrB = false;     // B straight into registers
    static constexpr int SLOT = BM * 128;   // bytes of one A slot: BM rows x 64 bf16
    static constexpr int SLOT_A = SLOT;
    static constexpr int RING_BYTES = SLOTS * SLOT;
    static constexpr int ROWINFO_BYTES = 16 * BM;   // L2: per row (token, weight, direct)
    static constexpr int LDS_BYTES = RING_BYTES + ROWINFO_BYTES;
};

// Tiles of the dgrads of experts with few rows, whose B operand is a packed weight read in the
// other GEMM direction (the packed reduction index becomes the output column).  Each slot holds
// the A rows and, per wave, the 4 NI packed 1 KB blocks its columns need for the slot's 64-deep K
// step (two packed column groups x 2 NI blocks of 16 reduction elements), moved by DMA as they
// are in memory; the MFMA B fragments are then read from them transposed (TrPipe).
template <int NI_, int MAXMI_, int SLOTS_>
struct TrTile {
    static constexpr int NI = NI_, MAXMI = MAXMI_, OCC = 1, SLOTS = SLOTS_;
    static_assert(MAXMI >= 1 && MAXMI <= 8 && (SLOTS == 3 || SLOTS == 4), "tile shape");
    static constexpr int BM = 32 * MAXMI, BN = kWaves * 32 * NI;
    static constexpr int NT = 64 * kWaves;
    static constexpr bool kTrB = true;
    static constexpr bool kNtStage = true;   // the L1 dgrad's combine rows: nontemporal (measured faster)
    static constexpr int SLOT_A = BM * 128;
    static constexpr int WAVE_B = NI * 4096;   // one wave's packed blocks of a slot
    static constexpr int SLOT = SLOT_A + kWaves * WAVE_B;
    static constexpr int RING_BYTES = SLOTS * SLOT;
    static constexpr int ROWINFO_BYTES = 16 * BM;
    static constexpr int LDS_BYTES = RING_BYTES + ROWINFO_BYTES;
};

// 16-byte chunk c of LDS row r sits at position c ^ ((r >> 1) & 7): rows r and r + 1 fill the
// two halves of the 64 banks, so the 16 rows of a fragment read hit 16 distinct bank groups.
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
    return static_cast<uint32_t>(row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4));
}

// Row of accumulator element r of a 32x32 MFMA block (lane % 32 is the column).
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// s_waitcnt vmcnt(n) alone (gfx9 encoding: expcnt and lgkmcnt fields at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Loads of one tile with MA active 32-row groups.  DMA instruction i of wave w fills rows
// 32 i + 8 w .. 32 i + 8 w + 7 of a slot: lane L lands at position L % 8 of row 32 i + 8 w + L / 8
// and fetches the logical chunk the swizzle keeps there.
template <class C, int MA>
struct Pipe {
    const char* a_src[MA];       // the lane's chunk of its row in group i, at K 0
    const char* b_src[C::NI];    // the lane's 16 bytes of block (column group, K step 0)
    bf16x8_t b[C::SLOTS][C::NI][4];
    int nslot;                   // K / 64 (loads past the end re-read the last slot)
    int wave;

    // part q (0..3) of the loads of slot j: A rows of groups i = q, q + 4, ...; B K step q
    __device__ __forceinline__ void a_issue(int j, char* __restrict__ slot, int q) const {
        const int jj = min(j, nslot - 1);
#pragma unroll
        for (int i = 0; i < MA; ++i)
            if (i % 4 == q)
                __builtin_amdgcn_global_load_lds((g_void*)(a_src[i] + jj * 128),
                                                 (l_void*)(slot + 1024 * (wave + kWaves * i)), 16, 0, 0);
    }
    __device__ __forceinline__ void b_issue(int j, int buf, int q) {
        const int jj = min(j, nslot - 1);
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
            b[buf][ni][q] = C::kNtB ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(b_src[ni] + (4 * jj + q) * 1024))
                                    : *reinterpret_cast<const bf16x8_t*>(b_src[ni] + (4 * jj + q) * 1024);
    }
    __device__ __forceinline__ void b_issue(int j, int buf, char* __restrict__, int q) { b_issue(j, buf, q); }
    static constexpr int a_loads(int q) { return (MA + 3 - q) / 4; }
    static constexpr int kBLoads = 4 * C::NI;
    static constexpr int kLoadsPerSlot = MA + kBLoads;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 l_v4i16;

// The transposed-B pipe.  A as in Pipe, except that a row's slots may be a_step bytes apart (128:
// K-contiguous rows; 64: rows in [gate | up] order whose slot j takes gate columns 32 j .. 32 j + 31
// and the same up columns, the order of the packed W1 column groups 2 j and 2 j + 1).
//
// B: the dgrad's output column n is the packed weight's reduction index and its K index the packed
// column.  A packed block (column group G, reduction block b) holds, in 16-byte chunk
// c = g % 32 + 32 * ((n % 16) / 8), the 8 reduction elements n of column g.  The MFMA B operand of
// 32 output columns x 16 K needs the transpose: lane L holds 8 consecutive K of column L % 32.
// gfx950's ds_read_b64_tr_b16 gives it: in each 16-lane group, lane i receives in slot s element
// i % 4 of the 8 bytes lane 4 s + i / 4 addresses, so if source lane j points at 4 consecutive n
// (n0 + 4 (j % 4)) of K row k0 + j / 4, lane i gets K rows k0 .. k0 + 3 of column n0 + i.  Two such
// reads make one operand.  The DMA places chunk c of a block with parity p (its reduction block's
// index mod 2) at position c ^ (4 (c / 32)) ^ (8 p): a half-wave's 32 eight-byte reads then cover
// the 64 banks once.  The swizzle is applied on the source side, since lane l of a DMA lands at
// position l.
template <class C, int MA>
struct TrPipe {
    const char* a_src[MA];
    const char* b_src[2];   // the lane's chunk of the wave's first block pair of slot 0, even / odd block
    int64_t b_grp;          // bytes of one packed column group
    int a_step;
    int nslot;
    int wave;
    uint32_t b_off;         // the lane's transposed-read offset inside a block pair

    // w_e: the expert's packed weight, kp its reduction length (the dgrad's N), n0 the wave's first
    // output column (a multiple of 32).
    __device__ __forceinline__ void b_setup(const char* w_e, int kp, int n0, int lane) {
        b_grp = static_cast<int64_t>(kp) * 64;
        const int c0 = lane ^ ((lane >> 5) << 2);
        b_src[0] = w_e + static_cast<int64_t>(n0 / 16) * 1024 + 16 * c0;
        b_src[1] = w_e + static_cast<int64_t>(n0 / 16 + 1) * 1024 + 16 * (c0 ^ 8);
        const int g = lane >> 4, j = lane & 15, q = (j & 3) >> 1;
        const int c = 8 * (g >> 1) + (j >> 2) + 32 * q;
        b_off = static_cast<uint32_t>((g & 1) * 1024 + 16 * (c ^ (q << 2) ^ ((g & 1) << 3)) + 8 * (j & 1));
    }
    __device__ __forceinline__ void a_issue(int j, char* __restrict__ slot, int q) const {
        const int jj = min(j, nslot - 1);
#pragma unroll
        for (int i = 0; i < MA; ++i)
            if (i % 4 == q)
                __builtin_amdgcn_global_load_lds((g_void*)(a_src[i] + jj * a_step),
                                                 (l_void*)(slot + 1024 * (wave + kWaves * i)), 16, 0, 0);
    }
    // part q of slot j's blocks: block u = q NI + v (K group u / (2 NI), reduction block u % (2 NI))
    __device__ __forceinline__ void b_issue(int j, int, char* __restrict__ slot, int q) const {
        const int jj = min(j, nslot - 1);
#pragma unroll
        for (int v = 0; v < C::NI; ++v) {
            const int u = q * C::NI + v, kg = u / (2 * C::NI), nb = u % (2 * C::NI);
            __builtin_amdgcn_global_load_lds(
                (g_void*)(b_src[nb & 1] + (2 * jj + kg) * b_grp + (nb >> 1) * 2048),
                (l_void*)(slot + C::SLOT_A + wave * C::WAVE_B + u * 1024), 16, 0, 2);   // nontemporal
        }
    }
    // B fragments of 16-deep step kb of a slot
    __device__ __forceinline__ void read_b(bf16x8_t (&b)[C::NI], const char* __restrict__ slot, int kb) const {
        const char* base = slot + C::SLOT_A + wave * C::WAVE_B + (kb >> 1) * (2 * C::NI * 1024) + (kb & 1) * 256;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((l_v4i16*)(base + ni * 2048 + b_off));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((l_v4i16*)(base + ni * 2048 + (b_off ^ 64u)));
            const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            b[ni] = __builtin_bit_cast(bf16x8_t, v);
        }
    }
    static constexpr int a_loads(int q) { return (MA + 3 - q) / 4; }
    static constexpr int kBLoads = 4 * C::NI;
    static constexpr int kLoadsPerSlot = MA + kBLoads;
};

template <class C, int MA>
using PipeOf = std::conditional_t<C::kTrB, TrPipe<C, MA>, Pipe<C, MA>>;

template <class C, int MA>
__device__ __forceinline__ void read_frags(bf16x8_t (&a)[MA], const char* __restrict__ slot, int kb, int lane) {
#pragma unroll
    for (int mi = 0; mi < MA; ++mi)
        a[mi] = *reinterpret_cast<const bf16x8_t*>(slot + lds_off(mi * 32 + (lane & 31), 2 * kb + (lane >> 5)));
}

// One slot of the unrolled loop (U = j % SLOTS static: LDS slot and B stage U).  The loads of
// slot j + SLOTS - 1 go out a quarter per 16-deep step, between the MFMAs (a burst would stall
// the waves on the CU's shared address unit); each step reads the next step's fragments between
// its MFMAs.
//
// ISSUE false (the slots past the unrolled loop) issues nothing: those loads would only fetch
// past the end, the compiler drops the register ones as dead, and the wait counts count loads in
// issue order, so they must match what really went out.  WAIT is the number of this wave's loads
// issued after slot j's, which may still be in flight.
template <class C, int MA, int U, bool ISSUE, int WAIT>
__device__ __forceinline__ void slot_step(PipeOf<C, MA>& p, int j, char* __restrict__ s0, char* __restrict__ s1,
                                          char* __restrict__ s2, char* __restrict__ s3,
                                          f32x16_t (&acc)[MA][C::NI], int lane) {
    char* const slots[4] = {s0, s1, s2, s3};
    constexpr int FAR = (U + C::SLOTS - 1) % C::SLOTS;   // slot of j + SLOTS - 1 = slot of j - 1
    // this wave's loads of slot j landed, then everyone's have, and slot FAR is no longer read
    wait_vmcnt<WAIT>();
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's fragment reads are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!C::kTrB && MA == 9) {
        // Nine groups: 288 accumulator registers, more than the 256 AGPRs, and the compiler keeps
        // every MFMA it emits in AGPR form (it then moves accumulators through scratch).  So
        // groups 0-7 use the builtin (AGPRs) and group 8 an inline MFMA in VGPR form; k_loop adds
        // the wait states the compiler cannot see.  Dependent accumulation into the same
        // registers needs none.  The fragments roll: group mi's fragment of step kb + 1 is read
        // as soon as its MFMAs of step kb are issued (MA + 1 fragments live, not 2 MA).
        bf16x8_t a[MA];
        read_frags<C, MA>(a, slots[U], 0, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (ISSUE) {
                p.a_issue(j + C::SLOTS - 1, slots[FAR], kb);
                p.b_issue(j + C::SLOTS - 1, FAR, slots[FAR], kb);
            }
#pragma unroll
            for (int mi = 0; mi < MA; ++mi) {
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    if (mi < 8)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], p.b[U][ni][kb], acc[mi][ni], 0, 0, 0);
                    else
                        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                                     : "+v"(acc[mi][ni])
                                     : "v"(a[mi]), "v"(p.b[U][ni][kb]));
                }
                if (kb < 3)
                    a[mi] = *reinterpret_cast<const bf16x8_t*>(slots[U] + lds_off(mi * 32 + (lane & 31), 2 * (kb + 1) + (lane >> 5)));
            }
            // the builtin MFMAs, each group's fragment read after its last one, the loads
            constexpr int NM = 8 * C::NI;
            const int nv = ISSUE ? PipeOf<C, MA>::a_loads(kb) + C::NI : 0;
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         // MFMA
                if (kb < 3 && i % C::NI == C::NI - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                if (i < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                             // global load
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    bf16x8_t a[2][MA];
    bf16x8_t bt[2][C::NI];   // transposed B fragments (kTrB)
    read_frags<C, MA>(a[0], slots[U], 0, lane);
    if constexpr (C::kTrB) p.read_b(bt[0], slots[U], 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (ISSUE) {
            p.a_issue(j + C::SLOTS - 1, slots[FAR], kb);
            p.b_issue(j + C::SLOTS - 1, FAR, slots[FAR], kb);
        }
        if (kb < 3) {
            read_frags<C, MA>(a[(kb + 1) & 1], slots[U], kb + 1, lane);
            if constexpr (C::kTrB) p.read_b(bt[(kb + 1) & 1], slots[U], kb + 1);
        }
#pragma unroll
        for (int mi = 0; mi < MA; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                if constexpr (C::kTrB)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb & 1][mi], bt[kb & 1][ni], acc[mi][ni], 0, 0, 0);
                else
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb & 1][mi], p.b[U][ni][kb], acc[mi][ni], 0, 0, 0);
            }
        // order: MFMA, fragment read, global load alternating
        constexpr int NM = MA * C::NI;
        const int nv = ISSUE ? PipeOf<C, MA>::a_loads(kb) + C::NI : 0;
        if constexpr (C::kTrB) {
            // MA + 2 NI fragment reads (two per B operand) and nv loads spread over the NM MFMAs
            constexpr int NR = MA + 2 * C::NI;
            const int nr = kb < 3 ? NR : 0;
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
#pragma unroll
                for (int x = 0; x < (NR + NM - 1) / NM; ++x)
                    if (x * NM + i < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
#pragma unroll
                for (int x = 0; x < 2; ++x)
                    if (x * NM + i < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
            }
        } else {
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // MFMA
                if (kb < 3 && i < MA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                if (i < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);            // global load
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Slots j + I .. j + SLOTS - 1 of one turn of the unrolled loop.
template <class C, int MA, int I>
__device__ __forceinline__ void loop_turn(PipeOf<C, MA>& p, int j, char* __restrict__ s0, char* __restrict__ s1,
                                          char* __restrict__ s2, char* __restrict__ s3,
                                          f32x16_t (&acc)[MA][C::NI], int lane) {
    if constexpr (I < C::SLOTS) {
        slot_step<C, MA, I, true, (C::SLOTS - 2) * PipeOf<C, MA>::kLoadsPerSlot>(p, j + I, s0, s1, s2, s3, acc, lane);
        loop_turn<C, MA, I + 1>(p, j, s0, s1, s2, s3, acc, lane);
    }
}

// The last nslot % SLOTS slots (j is a multiple of SLOTS): all their loads went out in the
// prologue or the loop, which issued through slot j + SLOTS - 2 (re-reading the last slot past
// the end), so SLOTS - 2 - I slots' loads follow those of slot j + I.
template <class C, int MA, int I>
__device__ __forceinline__ void loop_tail(PipeOf<C, MA>& p, int j, char* __restrict__ s0, char* __restrict__ s1,
                                          char* __restrict__ s2, char* __restrict__ s3,
                                          f32x16_t (&acc)[MA][C::NI], int lane) {
    if constexpr (I < C::SLOTS - 1) {
        if (j + I < p.nslot) {
            slot_step<C, MA, I, false, (C::SLOTS - 2 - I) * PipeOf<C, MA>::kLoadsPerSlot>(p, j + I, s0, s1, s2, s3, acc, lane);
            loop_tail<C, MA, I + 1>(p, j, s0, s1, s2, s3, acc, lane);
        }
    }
}

// Issues the loads of slots I .. SLOTS - 2 (prologue), all of one slot before any of the next: the
// waits count loads in issue order.
template <class C, int MA, int I>
__device__ __forceinline__ void prologue_issue(PipeOf<C, MA>& p, char* __restrict__ s0, char* __restrict__ s1,
                                               char* __restrict__ s2) {
    if constexpr (I < C::SLOTS - 1) {
        char* const slots[3] = {s0, s1, s2};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            p.a_issue(I, slots[I], q);
            p.b_issue(I, I, slots[I], q);
        }
        __builtin_amdgcn_sched_barrier(0);
        prologue_issue<C, MA, I + 1>(p, s0, s1, s2);
    }
}

// acc = A[rows, 0:K] . B[0:K, cols] (K a multiple of 128).  Ends with no load in flight and all
// waves past their last fragment read, so the caller may reuse the LDS.  s3 is unused with three
// slots.
template <class C, int MA>
__device__ __forceinline__ void k_loop(PipeOf<C, MA>& p, char* __restrict__ s0, char* __restrict__ s1,
                                       char* __restrict__ s2, char* __restrict__ s3,
                                       f32x16_t (&acc)[MA][C::NI], int lane) {
#pragma unroll
    for (int mi = 0; mi < MA; ++mi)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    if constexpr (!C::kTrB && MA == 9) {
        // VALU write -> MFMA SrcC read of the VGPR-form group: 2 wait states (the operands tie
        // the wait to those registers, so no access to them moves across it)
        static_assert(C::NI == 2, "two VGPR-form accumulators");
        asm volatile("s_nop 4" : "+v"(acc[8][0]), "+v"(acc[8][1]));
    }
    __builtin_amdgcn_sched_barrier(0);
    prologue_issue<C, MA, 0>(p, s0, s1, s2);
    int j = 0;
    for (; j + C::SLOTS <= p.nslot; j += C::SLOTS) loop_turn<C, MA, 0>(p, j, s0, s1, s2, s3, acc, lane);
    loop_tail<C, MA, 0>(p, j, s0, s1, s2, s3, acc, lane);
    // MFMA (16 passes) write -> VALU, LDS or memory read of the result: 18 wait states (19 given)
    if constexpr (!C::kTrB && MA == 9) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[8][0]), "+v"(acc[8][1]));
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------------------------
// L1: dispatch gather + grouped GEMM (NT) + SwiGLU
// ---------------------------------------------------------------------------------------------
// Packed W1 column group nb holds gate columns (nb even) or the matching up columns (nb odd) of
// intermediate columns [32 (nb/2), 32 (nb/2) + 32), so a wave's blocks 2q and 2q + 1 are the gate
// and up of the same columns, lane by lane.
template <class C>
struct L1Body {
    const uint16_t* x;
    const uint16_t* w1f;
    Dims d;
    Ws ws;
    uint16_t* act_out;
    float* hgu_out;
    char* smem;

    template <int MA>
    __device__ __forceinline__ void run(const TileRef& t) {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int H = d.H, I = d.I, npairs = d.T * d.k;
        Pipe<C, MA> p;
        p.nslot = H / 64;
        p.wave = __builtin_amdgcn_readfirstlane(wave);
        const char* zrow = reinterpret_cast<const char*>(ws.zeros);
#pragma unroll
        for (int i = 0; i < MA; ++i) {
            const int row = 32 * i + 8 * wave + (lane >> 3);
            const int pr = row < t.real_rows ? ws.row_pair[t.row0 + row] : -1;
            const int c16 = 16 * ((lane & 7) ^ ((row >> 1) & 7));
            p.a_src[i] = (pr >= 0 && pr < npairs)
                             ? reinterpret_cast<const char*>(x + static_cast<int64_t>(pr / d.k) * H) + c16
                             : zrow + c16;
        }
        const char* wb = reinterpret_cast<const char*>(w1f) + static_cast<int64_t>(t.e) * (2 * I) * H * 2;
        const int nb0 = t.nt * (C::BN / 32) + wave * C::NI;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
            p.b_src[ni] = wb + static_cast<int64_t>(nb0 + ni) * (H / 16) * 1024 + lane * 16;
        f32x16_t acc[MA][C::NI];
        k_loop<C, MA>(p, smem, smem + C::SLOT, smem + 2 * C::SLOT, smem + (C::SLOTS - 1) * C::SLOT, acc, lane);

        const int g0 = nb0 / 2;   // first intermediate column group of the wave
#pragma unroll
        for (int q = 0; q < C::NI / 2; ++q) {
            const int col = 32 * (g0 + q) + (lane & 31);
#pragma unroll
            for (int mi = 0; mi < MA; ++mi) {
                if (32 * mi >= t.real_rows) break;   // zero rows that belong to no output
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = t.row0 + mi * 32 + acc_row(r, lane);
                    const float g = acc[mi][2 * q][r], u = acc[mi][2 * q + 1][r];
                    if (hgu_out) {   // nontemporal: read back only by the backward, after L2
                        __builtin_nontemporal_store(g, hgu_out + row * 2 * I + col);
                        __builtin_nontemporal_store(u, hgu_out + row * 2 * I + I + col);
                    }
                    if (act_out) act_out[row * I + col] = f32_to_bf16(silu_f32(g) * u);
                }
            }
        }
        if (t.last) {   // padding rows after the last real group read as zero rows downstream
            const int64_t r0 = t.row0 + t.real_rows, r1 = min(static_cast<int64_t>(ws.offsets[t.e + 1]), ws.rows_cap);
            const int c0 = t.nt * (C::BN / 2);
            constexpr int CH = C::BN / 16;   // 8-column chunks of the tile's intermediate columns
            for (int64_t u = tid; u < (r1 - r0) * CH; u += C::NT) {
                const int64_t row = r0 + u / CH;
                const int c = c0 + static_cast<int>(u % CH) * 8;
                const u32x4 z = 0;
                if (act_out) *reinterpret_cast<u32x4*>(act_out + row * I + c) = z;
                if (hgu_out) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        *reinterpret_cast<u32x4*>(hgu_out + row * 2 * I + c + 4 * h) = z;
                        *reinterpret_cast<u32x4*>(hgu_out + row * 2 * I + I + c + 4 * h) = z;
                    }
                }
            }
        }
    }
};

template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void l1_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w1f,
                                                     Dims d, Ws ws, uint16_t* __restrict__ act_out,
                                                     float* __restrict__ hgu_out) {
    static_assert(C::NI % 2 == 0, "a wave holds whole gate/up pairs");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    L1Body<C> body{x, w1f, d, ws, act_out, hgu_out, smem};
    run_tiles<C>(d, ws, 2 * d.I / C::BN, body);
}

// ---------------------------------------------------------------------------------------------
// L2: grouped GEMM (NT) + top-k weighted combine
// ---------------------------------------------------------------------------------------------
// Row r of pair p = (t, j): o = act[r] @ W2[e]^T scaled by topk_w[p].  A token with one local
// pair owns its y row, so the epilogue stores bf16(w * o) there; a token with several local
// pairs gets fp32 rows in ws.stage that combine_finish sums in slot order.
//
// With a transposed-B tile (C::kTrB) the same body is the L1 dgrad of experts with few rows: A the
// dhgu rows ([gate | up], K = d.I = 2 x the intermediate size), B the packed W1 read transposed
// (its reduction index H is the output column), row weight 1.
template <class C>
struct L2Body {
    const uint16_t* act;
    const uint16_t* w2f;
    const float* topk_w;
    Dims d;
    Ws ws;
    uint16_t* y;
    char* smem;

    template <int MA>
    __device__ __forceinline__ void run(const TileRef& t) {
        int4* s_row = reinterpret_cast<int4*>(smem + C::RING_BYTES);   // token (-1: none), weight, direct
        constexpr int RPT = (C::BM + C::NT - 1) / C::NT;   // rows per thread
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int H = d.H, I = d.I, npairs = d.T * d.k;
        // the row's pair now; what depends on it is loaded after the K loop, so the loop does not
        // start behind a chain of dependent loads
        int pr[RPT];
#pragma unroll
        for (int u = 0; u < RPT; ++u) pr[u] = tid + u * C::NT < t.real_rows ? ws.row_pair[t.row0 + tid + u * C::NT] : -1;
        PipeOf<C, MA> p;
        p.nslot = I / 64;
        p.wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int i = 0; i < MA; ++i) {
            const int row = 32 * i + 8 * wave + (lane >> 3);
            const int lc = (lane & 7) ^ ((row >> 1) & 7);
            // [gate | up] rows: logical chunks 0-3 are gate columns, 4-7 the same up columns
            const int c16 = C::kTrB ? (lc < 4 ? 16 * lc : I + 16 * (lc - 4)) : 16 * lc;
            p.a_src[i] = row < t.real_rows
                             ? reinterpret_cast<const char*>(act + (t.row0 + row) * static_cast<int64_t>(I)) + c16
                             : reinterpret_cast<const char*>(ws.zeros) + c16;
        }
        const char* wb = reinterpret_cast<const char*>(w2f) + static_cast<int64_t>(t.e) * H * I * 2;
        if constexpr (C::kTrB) {
            p.a_step = 64;
            p.b_setup(wb, H, t.nt * C::BN + wave * 32 * C::NI, lane);
        } else {
            const int nb0 = t.nt * (C::BN / 32) + wave * C::NI;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                p.b_src[ni] = wb + static_cast<int64_t>(nb0 + ni) * (I / 16) * 1024 + lane * 16;
        }
        f32x16_t acc[MA][C::NI];
        k_loop<C, MA>(p, smem, smem + C::SLOT, smem + 2 * C::SLOT, smem + (C::SLOTS - 1) * C::SLOT, acc, lane);

#pragma unroll
        for (int u = 0; u < RPT; ++u)
            if (tid + u * C::NT < 32 * MA) {
                int tok = -1, direct = 0;
                float w = 0.0f;
                if (pr[u] >= 0 && pr[u] < npairs) {
                    tok = pr[u] / d.k;
                    w = topk_w ? topk_w[pr[u]] : 1.0f;   // no weights: the L1 dgrad's combine into dx
                    direct = ws.tok_nloc[tok] == 1;
                }
                s_row[tid + u * C::NT] = make_int4(tok, __float_as_int(w), direct, 0);
            }

        // Epilogue through LDS (the ring is free after the K loop), GP 32-row groups per pass: the
        // waves drop their accumulators into a row-major fp32 tile, then each wave takes whole
        // rows, scales them by the pair's weight and stores 4-column chunks (bf16 into y for a
        // token's only local pair, fp32 into the stage row otherwise), so every store instruction
        // covers a contiguous row segment.  A pass first reads all its chunks, then stores them.
        constexpr int LD = C::BN + 8;   // floats per LDS row: rows r and r + 4 fall in opposite bank halves
        constexpr int CH = C::BN / 4;   // 4-column chunks per row
        constexpr int GP = 2;
        constexpr int ITER = GP * 32 * CH / C::NT;
        static_assert(ITER % kEpiBatch == 0, "whole batches");
        static_assert(GP * 32 * LD * 4 <= C::RING_BYTES, "a pass fits in the ring");
        static_assert(C::NT % CH == 0, "a thread's chunks share their column");
        constexpr int RSTEP = C::NT / CH;   // rows between a thread's consecutive chunks
        float* tile = reinterpret_cast<float*>(smem);
        // Per-lane bases, re-derived in every tile (the empty asm hides their value), so that the
        // element addresses are a base plus a constant offset instead of dozens of precomputed
        // addresses held across the tile loop.
        int wbase = 4 * (lane >> 5) * LD + wave * 32 * C::NI + (lane & 31);   // accumulator row 0 of a group
        int rrow = tid / CH, rcol = (tid % CH) * 4;                             // first chunk of a pass
        asm volatile("" : "+v"(wbase), "+v"(rrow), "+v"(rcol));
#pragma unroll
        for (int m0 = 0; m0 < MA; m0 += GP) {
            if (m0 > 0) lds_barrier();   // the previous pass's reads are done
#pragma unroll
            for (int mm = 0; mm < GP; ++mm)
                if (m0 + mm < MA)
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            tile[wbase + (mm * 32 + 8 * (r >> 2) + (r & 3)) * LD + ni * 32] =
                                acc[m0 + mm < MA ? m0 + mm : 0][ni][r];
            lds_barrier();   // also publishes s_row (first pass)
            const int rows = (m0 + GP <= MA ? GP : MA - m0) * 32;
            // The pass's row records: lane j reads row j's (one contiguous 16-byte-per-lane LDS
            // read; the empty asm keeps the unused fourth word in it), and readlane hands each
            // row's record out, since a row is wave-uniform (half-wave-uniform on 128-column
            // tiles). Every lane reading the same 12-byte record, row by row, costs LDS bank
            // conflicts.
            static_assert(GP * 32 == 64, "one record per lane");
            int4 rin = make_int4(-1, 0, 0, 0);
            if (lane < rows) rin = s_row[m0 * 32 + lane];
            asm volatile("" : "+v"(rin.w));
            const int r_lo = __builtin_amdgcn_readfirstlane(rrow);   // the first half-wave's row
#pragma unroll
            for (int k0 = 0; k0 < ITER; k0 += kEpiBatch) {
                typedef float v4f __attribute__((ext_vector_type(4)));   // read as one ds_read_b128
                v4f v[kEpiBatch];
                int4 ri[kEpiBatch];
#pragma unroll
                for (int k = 0; k < kEpiBatch; ++k) {
                    const int rr = rrow + (k0 + k) * RSTEP;
                    if ((k0 + k) * RSTEP < rows) {   // rows is a multiple of 32 >= RSTEP
                        v[k] = *reinterpret_cast<const v4f*>(tile + rr * LD + rcol);
                        const int sl = r_lo + (k0 + k) * RSTEP;
                        if constexpr (CH == 64) {   // a wave is one row
                            ri[k] = make_int4(__builtin_amdgcn_readlane(rin.x, sl), __builtin_amdgcn_readlane(rin.y, sl),
                                              __builtin_amdgcn_readlane(rin.z, sl), 0);
                        } else {                    // the second half-wave's row is the next one
                            const int x0 = __builtin_amdgcn_readlane(rin.x, sl), x1 = __builtin_amdgcn_readlane(rin.x, sl + 1);
                            const int y0 = __builtin_amdgcn_readlane(rin.y, sl), y1 = __builtin_amdgcn_readlane(rin.y, sl + 1);
                            const int z0 = __builtin_amdgcn_readlane(rin.z, sl), z1 = __builtin_amdgcn_readlane(rin.z, sl + 1);
                            ri[k] = lane < 32 ? make_int4(x0, y0, z0, 0) : make_int4(x1, y1, z1, 0);
                        }
                    }
                }
#pragma unroll
                for (int k = 0; k < kEpiBatch; ++k) {
                    const int rr = rrow + (k0 + k) * RSTEP;
                    if ((k0 + k) * RSTEP >= rows || ri[k].x < 0) continue;
                    const float w = __int_as_float(ri[k].y);
                    const int64_t col = static_cast<int64_t>(t.nt) * C::BN + rcol;
                    if (ri[k].z) {
                        const uint32_t lo = f32_to_bf16(w * v[k].x) | (static_cast<uint32_t>(f32_to_bf16(w * v[k].y)) << 16);
                        const uint32_t hi = f32_to_bf16(w * v[k].z) | (static_cast<uint32_t>(f32_to_bf16(w * v[k].w)) << 16);
                        // nontemporal: the layer's output is not read again by this layer's kernels
                        typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                        const v2u val = {lo, hi};
                        __builtin_nontemporal_store(val, reinterpret_cast<v2u*>(y + static_cast<int64_t>(ri[k].x) * H + col));
                    } else {
                        float* dst = ws.stage + (t.row0 + m0 * 32 + rr) * static_cast<int64_t>(H) + col;
                        if constexpr (C::kNtStage) {
                            const v4f sv = {w * v[k].x, w * v[k].y, w * v[k].z, w * v[k].w};
                            __builtin_nontemporal_store(sv, reinterpret_cast<v4f*>(dst));
                        } else {
                            *reinterpret_cast<float4*>(dst) = make_float4(w * v[k].x, w * v[k].y, w * v[k].z, w * v[k].w);
                        }
                    }
                }
            }
        }
    }
};

template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void l2_kernel(const uint16_t* __restrict__ act,
                                                     const uint16_t* __restrict__ w2f,
                                                     const float* __restrict__ topk_w, Dims d, Ws ws,
                                                     uint16_t* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    L2Body<C> body{act, w2f, topk_w, d, ws, y, smem};
    run_tiles<C>(d, ws, d.H / C::BN, body);
}

// ---------------------------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------------------------
template <class C>
hipError_t l1_launch(const Dims& d, const uint16_t* x, const uint16_t* w1f, const Ws& ws, uint16_t* act_out,
                     float* hgu_out, hipStream_t s) {
    auto k = l1_kernel<C>;
    allow_lds(k, C::LDS_BYTES);
    k<<<tile_grid(k, C::NT, C::LDS_BYTES, d, C::MAXMI, 2 * d.I / C::BN), C::NT, C::LDS_BYTES, s>>>(x, w1f, d, ws, act_out,
                                                                                            hgu_out);
    return hipGetLastError();
}

template <class C>
hipError_t l2_launch(const Dims& d, const uint16_t* act, const uint16_t* w2f, const float* topk_w, const Ws& ws,
                     uint16_t* y, hipStream_t s) {
    auto k = l2_kernel<C>;
    allow_lds(k, C::LDS_BYTES);
    k<<<tile_grid(k, C::NT, C::LDS_BYTES, d, C::MAXMI, d.H / C::BN), C::NT, C::LDS_BYTES, s>>>(act, w2f, topk_w, d, ws, y);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Weight gradients of experts with many rows, on the forward's pipeline
// ---------------------------------------------------------------------------------------------
// dW[e] (packed: reduction index m, packed column n) = sum over the expert's rows r of
// At[m][r] * B[r][n].  At is the row operand transposed to K-contiguous rows ([M, R_max]: row m
// holds column m of every ws row), B the column operand packed into MFMA fragments along the rows
// (a 1 KB block per (32-column group, 16 rows) at (group * (R_max / 16) + r / 16) * 1 KB); the
// transforms of moe_gemm.hip build both, with zeros in rows no pair holds.  A 256 x 256 tile (an
// M tile and an N tile of one expert) runs the forward's K loop over the expert's rows rounded
// up to 64 (inside its segment: block_m is a multiple of 64, and the padding rows are zero) and
// stores whole packed blocks; an expert without rows gets exact zeros.
template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void wgrad_nt_kernel(const uint16_t* __restrict__ at,
                                                                 const uint16_t* __restrict__ bp, int M, int N,
                                                                 Dims d, Ws ws, uint16_t* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    constexpr int MA = C::MAXMI;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m_tiles = M / C::BM, n_tiles = N / C::BN;
    const int total = d.EL * m_tiles * n_tiles;
    const int64_t R = ws.rows_cap;   // row stride of At, K extent of B
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int e = tile / (m_tiles * n_tiles);
        const int rem = tile - e * (m_tiles * n_tiles);
        const int mt = rem / n_tiles, nt = rem - mt * n_tiles;
        const int64_t seg0 = ws.offsets[e], seg1 = ws.offsets[e + 1];
        int64_t len = (static_cast<int64_t>(ws.counts[e]) + 63) / 64 * 64;
        if (seg0 < 0 || seg1 > R || seg1 < seg0 || (seg0 & 63)) len = 0;   // tables not from one prologue
        else if (len > seg1 - seg0) len = (seg1 - seg0) / 64 * 64;
        uint16_t* o = out + static_cast<int64_t>(e) * M * N;
        if (len < 64) {   // no rows: exact zeros, tile (mt, nt) of the packed gradient
            const uint4 z = make_uint4(0, 0, 0, 0);
            for (int mi = 0; mi < MA; ++mi)
                for (int ni = 0; ni < C::NI; ++ni)
                    for (int st = 0; st < 2; ++st) {
                        const int64_t n0 = static_cast<int64_t>(nt) * C::BN + wave * 32 * C::NI + ni * 32;
                        const int64_t blk = (n0 >> 5) * (M >> 4) + ((static_cast<int64_t>(mt) * C::BM + mi * 32) >> 4) + st;
                        *reinterpret_cast<uint4*>(o + (blk * 64 + lane) * 8) = z;
                    }
            continue;
        }
        f32x16_t acc[MA][C::NI];
        Pipe<C, MA> p;
        p.nslot = static_cast<int>(len / 64);
        p.wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int i = 0; i < MA; ++i) {
            const int row = 32 * i + 8 * wave + (lane >> 3);   // M row of the tile
            const int c16 = 16 * ((lane & 7) ^ ((row >> 1) & 7));
            p.a_src[i] = reinterpret_cast<const char*>(at + (static_cast<int64_t>(mt) * C::BM + row) * R + seg0) + c16;
        }
        const int64_t g0 = static_cast<int64_t>(nt) * (C::BN / 32) + wave * C::NI;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
            p.b_src[ni] = reinterpret_cast<const char*>(bp) + ((g0 + ni) * (R / 16) + seg0 / 16) * 1024 + lane * 16;
        k_loop<C, MA>(p, smem, smem + C::SLOT, smem + 2 * C::SLOT, smem + (C::SLOTS - 1) * C::SLOT, acc, lane);
#pragma unroll
        for (int mi = 0; mi < MA; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) {
                store_packed_block(o, M, static_cast<int64_t>(nt) * C::BN + wave * 32 * C::NI + ni * 32,
                                   static_cast<int64_t>(mt) * C::BM + mi * 32, acc[mi][ni], lane);
                __builtin_amdgcn_sched_barrier(0);   // one block at a time: keeps the epilogue's registers few
            }
    }
}

// ---------------------------------------------------------------------------------------------
// L2 dgrad on the forward's pipeline
// ---------------------------------------------------------------------------------------------
// dA'[r] = dy[t] @ W2[e]^T (t the row's token) on the L1 tile loop: the dy rows gathered through
// row_pair into the A ring.  Experts with many rows (256-row tiles) take W2 repacked to an
// (N = i, K = h) operand streaming into B registers; experts with few rows (C::kTrB) read the
// packed W2 itself, transposed out of LDS, so nothing is repacked.
// The epilogue is the streaming dgrad's: the row weight (dA = w * dA'), the activation
// a = silu(g) * u recomputed in fp32 from the saved fp32 pre-activation and written as w * a (hi
// and lo bf16, the dW2 operand), the SwiGLU transpose (fuse; dhgu hi and lo) or plain fp32 dA
// rows, and the routing-weight partials: for each 128-column half of the 256-column tile (waves
// 2h and 2h + 1) the sum over its columns of dA' * a, in the [R_max, I / 128] layout of ws
// dtw_part.
template <class C>
struct DgradBody {
    const uint16_t* dy;
    const uint16_t* w2b;   // repacked W2 (register B) or the packed W2 (kTrB)
    const float* topk_w;
    Dims d;
    Ws ws;
    int fuse, tw;
    char* smem;

    template <int MA>
    __device__ __forceinline__ void run(const TileRef& t) {
        static_assert(C::BN == 256 || C::BN == 128, "whole 128-column routing-weight partials");
        float* s_w = reinterpret_cast<float*>(smem + C::RING_BYTES);   // row weight (0: no pair)
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int H = d.H, I = d.I, npairs = d.T * d.k;
        const int pr_own = tid < t.real_rows ? ws.row_pair[t.row0 + tid] : -1;
        PipeOf<C, MA> p;
        p.nslot = H / 64;
        p.wave = __builtin_amdgcn_readfirstlane(wave);
        const char* zrow = reinterpret_cast<const char*>(ws.zeros);
#pragma unroll
        for (int i = 0; i < MA; ++i) {
            const int row = 32 * i + 8 * wave + (lane >> 3);
            const int pr = row < t.real_rows ? ws.row_pair[t.row0 + row] : -1;
            const int c16 = 16 * ((lane & 7) ^ ((row >> 1) & 7));
            p.a_src[i] = (pr >= 0 && pr < npairs)
                             ? reinterpret_cast<const char*>(dy + static_cast<int64_t>(pr / d.k) * H) + c16
                             : zrow + c16;
        }
        const char* wb = reinterpret_cast<const char*>(w2b) + static_cast<int64_t>(t.e) * I * H * 2;
        if constexpr (C::kTrB) {
            p.a_step = 128;
            p.b_setup(wb, I, t.nt * C::BN + wave * 32 * C::NI, lane);
        } else {
            const int nb0 = t.nt * (C::BN / 32) + wave * C::NI;
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni)
                p.b_src[ni] = wb + static_cast<int64_t>(nb0 + ni) * (H / 16) * 1024 + lane * 16;
        }
        f32x16_t acc[MA][C::NI];
        k_loop<C, MA>(p, smem, smem + C::SLOT, smem + 2 * C::SLOT, smem + (C::SLOTS - 1) * C::SLOT, acc, lane);

        if (tid < 32 * MA) s_w[tid] = (pr_own >= 0 && pr_own < npairs) ? topk_w[pr_own] : 0.0f;
        // Epilogue through LDS, GP 32-row groups per pass: the waves drop dA' into a row-major fp32
        // tile, then each wave takes whole rows (64 lanes x 4 columns: one 256-column row, or two
        // 128-column rows), so the hgu reads and the dhgu / dact / wact writes are contiguous row
        // segments, and each 32-lane half's sum is one 128-column routing-weight partial.
        constexpr int LD = C::BN + 4;   // floats per LDS row: rows r and r + 4 fall on different banks
        constexpr int GP = 2;
        constexpr int LPR = C::BN / 4, RPI = 64 / LPR;   // lanes per row, rows per wave instruction
        static_assert(GP * 32 * LD * 4 <= C::RING_BYTES, "a pass fits in the ring");
        float* tile = reinterpret_cast<float*>(smem);
        const int cols_tw = I / 128;
        const int lrow = lane / LPR, lcol = (lane % LPR) * 4;
        const int half = C::BN == 256 ? (lane >> 5) : 0;   // the lane's 128-column partial in the tile
#pragma unroll
        for (int m0 = 0; m0 < MA; m0 += GP) {
            if (32 * m0 >= t.real_rows) break;   // groups that belong to no row
            lds_barrier();   // the previous pass's reads are done; publishes s_w on the first pass
#pragma unroll
            for (int mm = 0; mm < GP; ++mm)
                if (m0 + mm < MA)
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            tile[(mm * 32 + acc_row(r, lane)) * LD + wave * 32 * C::NI + ni * 32 + (lane & 31)] =
                                acc[m0 + mm < MA ? m0 + mm : 0][ni][r];
            lds_barrier();
            // rows is a multiple of 32, so a wave instruction's RPI rows are all valid or none is
            const int rows = min(GP * 32, t.real_rows - 32 * m0);
            // four row steps per wave at a time: their hgu loads all go out before any is used
            constexpr int RB = 4, WS = C::NT / 64;
            for (int rb = wave * RPI; rb < rows; rb += RB * WS * RPI) {
                float4 gv[RB], uv[RB];
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    const int rr = rb + b * WS * RPI + lrow;
                    gv[b] = uv[b] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    if (rr < rows) {
                        const int64_t row = t.row0 + 32 * m0 + rr;
                        const int c = t.nt * C::BN + lcol;
                        gv[b] = *reinterpret_cast<const float4*>(ws.hgu + row * 2 * I + c);
                        uv[b] = *reinterpret_cast<const float4*>(ws.hgu + row * 2 * I + I + c);
                    }
                }
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    const int rr = rb + b * WS * RPI + lrow;
                    if (rr >= rows) break;   // uniform over the wave
                    const int rl = 32 * m0 + rr;
                    const int64_t row = t.row0 + rl;
                    const float w = s_w[rl];
                    const int c = t.nt * C::BN + lcol;
                    const float4 v = *reinterpret_cast<const float4*>(tile + rr * LD + lcol);
                    const float va[4] = {v.x, v.y, v.z, v.w};
                    const float ga[4] = {gv[b].x, gv[b].y, gv[b].z, gv[b].w};
                    const float ua[4] = {uv[b].x, uv[b].y, uv[b].z, uv[b].w};
                    float part = 0.0f;
                    uint16_t wh[4], wl[4], gh[4], gl[4], uh[4], ul[4];
                    float dv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float g = ga[q], u = ua[q];
                        const float sg = 1.0f / (1.0f + __expf(-g));
                        const float a = g * sg * u;
                        const float da = w * va[q];
                        part += va[q] * a;
                        split_bf16(w * a, wh[q], wl[q]);
                        split_bf16(da * u * sg * (1.0f + g * (1.0f - sg)), gh[q], gl[q]);
                        split_bf16(da * g * sg, uh[q], ul[q]);
                        dv[q] = da;
                    }
                    auto pk = [](const uint16_t (&h)[4]) {
                        return make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16),
                                          h[2] | (static_cast<uint32_t>(h[3]) << 16));
                    };
                    *reinterpret_cast<uint2*>(ws.wact + row * I + c) = pk(wh);
                    *reinterpret_cast<uint2*>(ws.wact_lo + row * I + c) = pk(wl);
                    if (fuse) {
                        *reinterpret_cast<uint2*>(ws.dhgu + row * 2 * I + c) = pk(gh);
                        *reinterpret_cast<uint2*>(ws.dhgu_lo + row * 2 * I + c) = pk(gl);
                        *reinterpret_cast<uint2*>(ws.dhgu + row * 2 * I + I + c) = pk(uh);
                        *reinterpret_cast<uint2*>(ws.dhgu_lo + row * 2 * I + I + c) = pk(ul);
                    } else {
                        *reinterpret_cast<float4*>(ws.dact + row * I + c) = make_float4(dv[0], dv[1], dv[2], dv[3]);
                    }
                    if (tw) {   // uniform over the wave: each 32-lane half holds one 128-column partial
#pragma unroll
                        for (int off = 16; off >= 1; off >>= 1) part += __shfl_xor(part, off);
                        if ((lane & 31) == 0) ws.dtw_part[row * cols_tw + t.nt * (C::BN / 128) + half] = part;
                    }
                }
            }
        }
        if (t.last) {   // the segment's padding rows after its last real group hold zeros
            const int64_t r0 = t.row0 + t.real_rows, r1 = min(static_cast<int64_t>(ws.offsets[t.e + 1]), ws.rows_cap);
            const int c0 = t.nt * C::BN;
            constexpr int CH = C::BN / 8;   // 8-column chunks of the tile's columns
            const u32x4 z = 0;
            for (int64_t u = tid; u < (r1 - r0) * CH; u += C::NT) {
                const int64_t row = r0 + u / CH;
                const int c = c0 + static_cast<int>(u % CH) * 8;
                *reinterpret_cast<u32x4*>(ws.wact + row * I + c) = z;
                *reinterpret_cast<u32x4*>(ws.wact_lo + row * I + c) = z;
                if (fuse) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        *reinterpret_cast<u32x4*>(ws.dhgu + row * 2 * I + h * I + c) = z;
                        *reinterpret_cast<u32x4*>(ws.dhgu_lo + row * 2 * I + h * I + c) = z;
                    }
                } else {
                    *reinterpret_cast<u32x4*>(ws.dact + row * I + c) = z;
                    *reinterpret_cast<u32x4*>(ws.dact + row * I + c + 4) = z;
                }
            }
            if (tw)
                for (int64_t u = tid; u < (r1 - r0) * (C::BN / 128); u += C::NT)
                    ws.dtw_part[(r0 + u / (C::BN / 128)) * cols_tw + t.nt * (C::BN / 128) + u % (C::BN / 128)] = 0.0f;
        }
    }
};

template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void dgrad_tile_kernel(const uint16_t* __restrict__ dy,
                                                                   const uint16_t* __restrict__ w2b,
                                                                 const float* __restrict__ topk_w, Dims d, Ws ws,
                                                                 int fuse, int tw) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    DgradBody<C> body{dy, w2b, topk_w, d, ws, fuse, tw, smem};
    run_tiles<C>(d, ws, d.I / C::BN, body);
}

using L1Tile = Tile<2, 8, 1, 4>;
using L2Tile = Tile<2, 8, 1, 4>;
using L2TileNarrow = Tile<1, 8, 1, 4>;
// Nine-group forward tiles (three ring slots: 288-row slots): an expert of 257-288 rows, about
// half of them when rows per expert average 256, runs as one tile, so its weight panels stream
// once instead of twice (two tiles of five and four groups).
using L1TileNt = Tile<2, 9, 1, 3, true>;
using L2TileNt = Tile<2, 9, 1, 3, true>;
using L2TileNarrowNt = Tile<1, 8, 1, 4, true>;
using WgTile = Tile<2, 8, 1, 3>;   // three ring slots measured slightly faster than four here
// Few-rows dgrads: M tiles of up to 96 rows (an expert of the wide share in one tile, its weights
// streamed once), three ring slots of 44 KB.
using DgTrTile = TrTile<2, 3, 3>;
using DgTrTileNarrow = TrTile<1, 3, 3>;

template <class C>
hipError_t dgrad_tile_launch(const Dims& d, const uint16_t* dy, const uint16_t* w2b, const float* topk_w,
                             const Ws& ws, int fuse, bool topk_w_grad, hipStream_t s) {
    auto k = dgrad_tile_kernel<C>;
    allow_lds(k, C::LDS_BYTES);
    k<<<tile_grid(k, C::NT, C::LDS_BYTES, d, C::MAXMI, d.I / C::BN), C::NT, C::LDS_BYTES, s>>>(dy, w2b, topk_w, d, ws, fuse,
                                                                           topk_w_grad ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

bool wgrad_nt_fits(int M, int N) { return M % WgTile::BM == 0 && N % WgTile::BN == 0; }

bool dgrad_nt_fits(const Dims& d) { return d.I % L1Tile::BN == 0 && d.H % 64 == 0 && d.EL <= kMaxEL; }

hipError_t launch_dgrad_nt(const Dims& d, const uint16_t* dy, const uint16_t* w2t, const float* topk_w, const Ws& ws,
                           int fuse, bool topk_w_grad, hipStream_t s) {
    if (!dgrad_nt_fits(d)) return hipErrorInvalidValue;
    return dgrad_tile_launch<L1Tile>(d, dy, w2t, topk_w, ws, fuse, topk_w_grad, s);
}

// Few-rows dgrads (I and H are multiples of 128): 256-column tiles where the width allows.
hipError_t launch_dgrad_tr(const Dims& d, const uint16_t* dy, const uint16_t* w2p, const float* topk_w, const Ws& ws,
                           int fuse, bool topk_w_grad, hipStream_t s) {
    if (d.EL > kMaxEL || d.I % 128 != 0 || d.H % 64 != 0) return hipErrorInvalidValue;
    return d.I % 256 == 0 ? dgrad_tile_launch<DgTrTile>(d, dy, w2p, topk_w, ws, fuse, topk_w_grad, s)
                          : dgrad_tile_launch<DgTrTileNarrow>(d, dy, w2p, topk_w, ws, fuse, topk_w_grad, s);
}

// dX rows of the L1 dgrad: the dhgu rows times the packed W1 read transposed, combined into dx
// like the forward's L2 (weight 1); the caller runs combine_finish.
hipError_t launch_dgrad1_tr(const Dims& d, const uint16_t* w1p, const Ws& ws, uint16_t* dx, hipStream_t s) {
    if (d.EL > kMaxEL || d.H % 128 != 0 || d.I % 32 != 0 || !ws.dhgu) return hipErrorInvalidValue;
    Dims d2 = d;
    d2.I = 2 * d.I;   // the GEMM's K: dhgu rows are 2I wide
    return d.H % 256 == 0 ? l2_launch<DgTrTile>(d2, ws.dhgu, w1p, nullptr, ws, dx, s)
                          : l2_launch<DgTrTileNarrow>(d2, ws.dhgu, w1p, nullptr, ws, dx, s);
}

hipError_t launch_wgrad_nt(const Dims& d, const uint16_t* at, const uint16_t* bp, int M, int N, const Ws& ws,
                           uint16_t* out, hipStream_t s) {
    if (!wgrad_nt_fits(M, N) || d.EL > kMaxEL) return hipErrorInvalidValue;
    auto k = wgrad_nt_kernel<WgTile>;
    allow_lds(k, WgTile::LDS_BYTES);
    k<<<persistent_grid(k, WgTile::NT, WgTile::LDS_BYTES), WgTile::NT, WgTile::LDS_BYTES, s>>>(at, bp, M, N, d, ws, out);
    return hipGetLastError();
}

// Weight panels stream with a nontemporal hint when an expert's rows fill at most two 256-row M
// tiles (expected rows T * k / E <= 512, uniform routing): with more M tiles re-reading each panel
// from L2 the hint costs more than it saves (measured at page scale).
static bool weights_nontemporal(const Dims& d) {
    return static_cast<int64_t>(d.T) * d.k <= 512 * static_cast<int64_t>(d.E);
}

// L1 N tiles are 256 columns (2I is a multiple of 256); L2 N tiles 256 columns when H allows, else 128.
hipError_t launch_gemm1(const Dims& d, const uint16_t* x, const uint16_t* w1f, const Ws& ws, uint16_t* act_out,
                        float* hgu_out, hipStream_t s) {
    if (d.EL > kMaxEL) return hipErrorInvalidValue;
    return weights_nontemporal(d) ? l1_launch<L1TileNt>(d, x, w1f, ws, act_out, hgu_out, s)
                                  : l1_launch<L1Tile>(d, x, w1f, ws, act_out, hgu_out, s);
}

hipError_t launch_gemm2_combine(const Dims& d, const uint16_t* act, const uint16_t* w2f, const float* topk_w,
                                const Ws& ws, uint16_t* y, hipStream_t s) {
    if (d.EL > kMaxEL) return hipErrorInvalidValue;
    const bool nt = weights_nontemporal(d), wide = d.H % L2Tile::BN == 0;
    if (nt) return wide ? l2_launch<L2TileNt>(d, act, w2f, topk_w, ws, y, s)
                        : l2_launch<L2TileNarrowNt>(d, act, w2f, topk_w, ws, y, s);
    return wide ? l2_launch<L2Tile>(d, act, w2f, topk_w, ws, y, s)
                : l2_launch<L2TileNarrow>(d, act, w2f, topk_w, ws, y, s);
}

}  // namespace moe
