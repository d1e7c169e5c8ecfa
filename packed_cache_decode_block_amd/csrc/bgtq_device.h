// Device helpers shared by the HIP kernel sources of the library (gfx950, wave64): constants,
// frozen codebook tables, fp16/bf16 conversions, wave-level LDS ordering, the matrix-core tile
// helpers of the packed decode (operand assembly from staged key records, value-stream lookups,
// DPP row reductions) and the per-workgroup partial merge.  Each including source gets its own
// copy (anonymous namespace).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bgtq.h"
#include "bgtq_internal.h"
#include "generated/bgtq_codebook_data.h"

namespace bgtq {
namespace {

constexpr int TILE = 64;
constexpr int D = 128;
constexpr int PART = 132;                       // floats per partial record: o[128], m, l
constexpr int kAppendFewMax = 64;               // appends of at most this many positions per sequence take k_append
constexpr float kLog2eOverSqrtD = 0.12751743074233076f;  // log2(e) / sqrt(128)

__constant__ uint32_t c_cent32[BGTQ_CB_CENTROIDS] = BGTQ_CB_CENTROID_F32_INIT;
__constant__ uint16_t c_cent16[BGTQ_CB_CENTROIDS] = BGTQ_CB_CENTROID_F16_INIT;
__constant__ uint32_t c_thr32[BGTQ_CB_THRESHOLDS] = BGTQ_CB_THRESHOLD_F32_INIT;
// LDS image of the matrix-core decode's tables: pair tables of widths 5..1, then the fp16
// centroid tables of widths 8..1, each at a multiple of its size (offsets BGTQ_CB_MX_*_OFFSETS).
__constant__ __attribute__((aligned(16))) uint32_t c_mxtab[BGTQ_CB_MX_WORDS] = BGTQ_CB_MX_INIT;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
// Read-only global data the kernel never writes, read through the constant address space so
// uniform loads become scalar loads.
typedef __attribute__((address_space(4))) uint32_t cu32_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int cent_base(int w) { return (1 << w) - 2; }
__device__ __forceinline__ int thr_base(int w) { return (1 << w) - w - 1; }
constexpr int thr_base_c(int w) { return (1 << w) - w - 1; }
__device__ __forceinline__ float h2f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float bf2f(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

__device__ __forceinline__ float load_act(const void* p, int64_t i, int dtype) {
    if (dtype == BGTQ_F32) return ((const float*)p)[i];
    const uint32_t u = ((const uint16_t*)p)[i];
    return dtype == BGTQ_F16 ? h2f(u) : bf2f(u);
}

// Orders LDS traffic of one wave: lanes exchange data through LDS without a workgroup barrier.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// merge_waves for four waves with 16-byte accesses: thread (h, quad of dims) handles 4 dims.
template <int G>
__device__ __forceinline__ void merge_waves4(const float* red, float* sc, float* part, int n_parts, int split) {
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, red[(wv * G + h) * PART + 128]);
        float L = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
            const float m = red[(wv * G + h) * PART + 128];
            const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
            sc[wv * G + h] = f;
            L += f * red[(wv * G + h) * PART + 129];
        }
        // partials are read once, by the split merge: stream them past the caches
        float* dst = part + ((size_t)h * n_parts + split) * PART;
        dst[128] = M;
        dst[129] = L;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * 32; idx += blockDim.x) {
        const int h = idx >> 5, j = 4 * (idx & 31);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
            const float* rw = red + (wv * G + h) * PART;
            const float f = sc[wv * G + h];
            acc += f * (*(const f32x4_t*)(rw + j) + rw[130]);
        }
        *(f32x4_t*)(part + ((size_t)h * n_parts + split) * PART + j) = acc;
    }
}

// Stream order of the RoPE blocks (lane = block, w = its width): rank among the nonzero blocks by
// width descending (ties: lower block first), bit position of its 2w-bit field in the K record,
// and the number of nonzero blocks.  Nine wave ballots, one per width.
__device__ __forceinline__ void block_order(int w, int lane, int& rank, int& pos, int& nnz) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    rank = 0;
    pos = 0;
    nnz = 0;
#pragma unroll
    for (int v = 0; v <= 8; ++v) {
        const uint64_t mk = __ballot(w == v);
        const int c = __popcll(mk);
        if (v == 0) nnz = 64 - c;
        if (v > w) {
            rank += c;
            pos += 2 * v * c;
        } else if (v == w) {
            const int cl = __popcll(mk & lt);
            rank += cl;
            pos += 2 * v * cl;
        }
    }
}

// Global inputs of the preparation (lane = RoPE block), loaded raw and converted later so a kernel
// can issue them, then its tile prefetch, before anything waits on them.
template <int G> struct PrepIn {
    uint32_t r0[G], r1[G];  // fp32 bits of (q_2i, q_2i+1), or the packed 16-bit pair in r0
    float sg;
    uint32_t w4;  // the dword of the width array holding this block's width (byte lane & 3)
    int dtype;
};

template <int G, bool SORTED>
__device__ __forceinline__ PrepIn<G> prep_load(const void* q, int dtype, const uint8_t* bits, const float* sigma, int b,
                                               int h, int Hq, int lane) {
    PrepIn<G> in;
    in.dtype = dtype;
    in.w4 = 0u;
    in.sg = 0.f;
    if constexpr (SORTED) {
        in.w4 = ((const uint32_t*)(bits + h * 64))[lane >> 2];
        in.sg = sigma[h * 64 + lane];
    }
    const int64_t row0 = ((int64_t)b * Hq + (int64_t)h * G) * D + 2 * lane;
    if (dtype == BGTQ_F32) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const uint2 v = *(const uint2*)((const float*)q + row0 + (int64_t)hh * D);
            in.r0[hh] = v.x;
            in.r1[hh] = v.y;
        }
    } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            in.r0[hh] = *(const uint32_t*)((const uint16_t*)q + row0 + (int64_t)hh * D);
            in.r1[hh] = 0u;
        }
    }
    return in;
}

__device__ __forceinline__ half8_t as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(half8_t, v);
}
__device__ __forceinline__ f32x4_t mfma16(half8_t a, half8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Column descriptor of one stream slot (one dword, built in the prologue; a lane reads the four of a
// k-step with one 16-byte LDS read).  A lane
// row reads the two adjacent slots A = 2i, B = 2i + 1 of a column pair from one 64-bit window
// that starts at a stage row boundary below A's field:
//   bits 0..5   64-bit shift that moves the slot's field (pair) or first code (coordinates) to bit
//               2 (pair) or bit 1 (coordinates)
//   bits 6..11  64-bit shift that moves the second code to bit 1 (coordinate columns)
//   bits 12..16 field width: 2w for a pair column, w for a coordinate column (0: empty slot)
//   bits 17..31 byte offset of the window's first stage row (slot A's descriptor)
// posA/coordA: slot A's record position and column mode; pos/w/coord: this slot's.  Every shift
// stays below 64 and every field inside the window: A's offset is below 32 and A and B together
// span at most 32 bits.
__device__ __forceinline__ uint32_t mx_desc(int posA, bool coordA, int pos, int w, bool coord) {
    const int uA = posA - (coordA ? 1 : 2);       // >= -2
    const int rr = uA >= 0 ? uA >> 5 : -1;        // window row (-1: the spare row)
    const int base = 32 * rr;
    const int s0 = pos - (coord ? 1 : 2) - base;
    const uint32_t sh0 = (uint32_t)(s0 < 0 ? 0 : s0);  // < 0 only for empty slots
    const uint32_t sh1 = coord ? sh0 + (uint32_t)w : 0u;
    const uint32_t fw = (uint32_t)(w == 0 ? 0 : (coord ? w : 2 * w));
    return sh0 | (sh1 << 6) | (fw << 12) | ((uint32_t)(rr + 1) * BGTQ_KST_ROW_BYTES << 17);
}

// ((1 << (width & 31)) - 1) << OFF in one v_bfm_b32.
template <int OFF>
__device__ __forceinline__ uint32_t bfm(uint32_t width) {
    uint32_t r;
    asm("v_bfm_b32 %0, %1, %2" : "=v"(r) : "v"(width), "n"(OFF));
    return r;
}

// Slot of a column read as a coordinate pair: 64-bit shift, and_or into the pair table of the
// slot's width, one 4-byte read.
__device__ __forceinline__ uint32_t slot_pair(const uint8_t* lds, uint64_t win, uint32_t dsc, uint32_t mask,
                                              uint32_t base) {
    const uint32_t x = (uint32_t)(win >> (dsc & 63u));
    return *(const uint32_t*)(lds + ((x & mask) | base));
}
// Slot of a column read per coordinate (the column's first slot is wider than 5 bits): two
// shifts, two 2-byte reads from the fp16 centroid table of the slot's width.
__device__ __forceinline__ uint32_t slot_coord(const uint8_t* lds, uint64_t win, uint32_t dsc, uint32_t mask,
                                               uint32_t base) {
    const uint32_t x0 = (uint32_t)(win >> (dsc & 63u));
    const uint32_t x1 = (uint32_t)(win >> ((dsc >> 6) & 63u));
    const uint32_t c0 = *(const uint16_t*)(lds + ((x0 & mask) | base));
    const uint32_t c1 = *(const uint16_t*)(lds + ((x1 & mask) | base));
    return c0 | (c1 << 16);
}

// Both column pairs of a k-step: the eight windows (two column pairs x four token groups) as one
// batch of ds_read2, then the sixteen slot lookups, so that a k-step waits on two LDS round trips
// rather than three.  CA0/CB0, CA1/CB1: coordinate mode of columns 0..3.
template <bool CA0, bool CB0, bool CA1, bool CB1>
__device__ __forceinline__ void col_pairs_both(uint32_t (&P)[16], const uint8_t* lds, const u32x4_t dk, uint32_t lb) {
    const uint32_t ad0 = (dk[0] >> 17) + lb, ad1 = (dk[2] >> 17) + lb;
    const uint32_t m0 = CA0 ? bfm<1>(dk[0] >> 12) : bfm<2>(dk[0] >> 12);
    const uint32_t m1 = CB0 ? bfm<1>(dk[1] >> 12) : bfm<2>(dk[1] >> 12);
    const uint32_t m2 = CA1 ? bfm<1>(dk[2] >> 12) : bfm<2>(dk[2] >> 12);
    const uint32_t m3 = CB1 ? bfm<1>(dk[3] >> 12) : bfm<2>(dk[3] >> 12);
    const uint32_t b0 = m0 + (CA0 ? BGTQ_CB_MX_COORD_BIAS : BGTQ_CB_MX_PAIR_BIAS);
    const uint32_t b1 = m1 + (CB0 ? BGTQ_CB_MX_COORD_BIAS : BGTQ_CB_MX_PAIR_BIAS);
    const uint32_t b2 = m2 + (CA1 ? BGTQ_CB_MX_COORD_BIAS : BGTQ_CB_MX_PAIR_BIAS);
    const uint32_t b3 = m3 + (CB1 ? BGTQ_CB_MX_COORD_BIAS : BGTQ_CB_MX_PAIR_BIAS);
    static_assert(BGTQ_KST_ROW_BYTES == 320, "window read offsets assume 80-dword stage rows");
    uint64_t wa[4], wb[4];
    asm volatile("ds_read2_b32 %0, %8 offset1:80\n\t"
                 "ds_read2_b32 %1, %8 offset0:16 offset1:96\n\t"
                 "ds_read2_b32 %2, %8 offset0:32 offset1:112\n\t"
                 "ds_read2_b32 %3, %8 offset0:48 offset1:128\n\t"
                 "ds_read2_b32 %4, %9 offset1:80\n\t"
                 "ds_read2_b32 %5, %9 offset0:16 offset1:96\n\t"
                 "ds_read2_b32 %6, %9 offset0:32 offset1:112\n\t"
                 "ds_read2_b32 %7, %9 offset0:48 offset1:128\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(wa[0]), "=&v"(wa[1]), "=&v"(wa[2]), "=&v"(wa[3]),
                   "=&v"(wb[0]), "=&v"(wb[1]), "=&v"(wb[2]), "=&v"(wb[3])
                 : "v"((uint32_t)(uintptr_t)(lds + ad0)), "v"((uint32_t)(uintptr_t)(lds + ad1))
                 : "memory");
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        P[4 * g + 0] = CA0 ? slot_coord(lds, wa[g], dk[0], m0, b0) : slot_pair(lds, wa[g], dk[0], m0, b0);
        P[4 * g + 1] = CB0 ? slot_coord(lds, wa[g], dk[1], m1, b1) : slot_pair(lds, wa[g], dk[1], m1, b1);
        P[4 * g + 2] = CA1 ? slot_coord(lds, wb[g], dk[2], m2, b2) : slot_pair(lds, wb[g], dk[2], m2, b2);
        P[4 * g + 3] = CB1 ? slot_coord(lds, wb[g], dk[3], m3, b3) : slot_pair(lds, wb[g], dk[3], m3, b3);
    }
    // Every lookup address first, then every lookup, then the halves joined: one LDS round trip for
    // the k-step's sixteen operands instead of one per token group.
    __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
}

// k-step KS of a tile; dk = the lane row's four column descriptors of this k-step, ncc
// (wave-uniform) = number of coordinate columns of the whole record (the first ncc columns are
// read per coordinate, the rest as pairs).  The column modes only change how the operands are
// built; the products sit after the branches.
template <int KS>
__device__ __forceinline__ void mx_kstep_any(f32x4_t (&c)[4], const uint8_t* lds, const u32x4_t* qa, int lane,
                                             const u32x4_t dk, uint32_t lb, int ncc) {
    uint32_t P[16];
    const int a = ncc - 4 * KS;
    if (a <= 0) col_pairs_both<false, false, false, false>(P, lds, dk, lb);
    else if (a == 1) col_pairs_both<true, false, false, false>(P, lds, dk, lb);
    else if (a == 2) col_pairs_both<true, true, false, false>(P, lds, dk, lb);
    else if (a == 3) col_pairs_both<true, true, true, false>(P, lds, dk, lb);
    else col_pairs_both<true, true, true, true>(P, lds, dk, lb);
    const half8_t q = __builtin_bit_cast(half8_t, qa[KS * 64 + lane]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const half8_t kb = as_h8(P[4 * g], P[4 * g + 1], P[4 * g + 2], P[4 * g + 3]);
        c[g] = KS == 0 ? mfma16(q, kb, f32x4_t{0.f, 0.f, 0.f, 0.f}) : mfma16(q, kb, c[g]);
    }
}

// The matrix-core decode's value table holds interleaved copies (entry e of copy c at dword
// e * copies + c) and lane l reads copy l % copies.  With 32 copies (values of up to 3 bits, 8 KB
// at 3 bits) every lane of the 32 that the LDS serves per pass owns one of its 32 banks, so random
// entries never conflict (measured on gfx950: random reads from a table wider than 32 dwords cost
// 1.7x to 2.8x a conflict-free read); 4-bit values keep 4 copies (the 256-entry table).
template <int VB> struct VLutGeom {
    static constexpr int LOG2_COPIES = VB <= 3 ? 5 : 2;
    static constexpr int COPIES = 1 << LOG2_COPIES;
    static constexpr int BYTES = 4 * COPIES * (1 << (2 * VB));
};
// Field F of this lane's value stream scaled to a byte offset in the replicated table, OR-ed with
// the lane's copy offset (one shift, one and_or).
template <int VB, int F>
__device__ __forceinline__ uint32_t vfield_rep(const uint32_t* r, uint32_t lane_copy) {
    constexpr int bit = 2 * VB * F, w = bit / 32, sh = bit % 32, nb = 2 * VB;
    constexpr int S = 2 + VLutGeom<VB>::LOG2_COPIES;
    constexpr uint32_t m = ((1u << nb) - 1u) << S;
    uint32_t x;
    if constexpr (sh + nb > 32) x = __builtin_amdgcn_alignbit(r[w + 1], r[w], sh - S);
    else if constexpr (sh >= S) x = r[w] >> (sh - S);
    else x = r[w] << (S - sh);
    return (x & m) | lane_copy;
}

// P·V of one 32-token half S: B = W rows of this lane's head column, A = value fields (S, db, m).
template <int VB, int F>
__device__ __forceinline__ uint32_t vpair(const uint32_t* vs, const uint32_t* vlut, uint32_t lane_copy) {
    return *(const uint32_t*)((const uint8_t*)vlut + vfield_rep<VB, F>(vs, lane_copy));
}
// ZERO: the products start from zero instead of accumulating into o (a wave's first tile).
template <int VB, int S, bool ZERO = false>
__device__ __forceinline__ void mx_pv(f32x4_t (&o)[8], const uint32_t* vs, const uint32_t* vlut, const uint32_t* wx,
                                      int lane, uint32_t lc) {
    const u32x4_t wq = *(const u32x4_t*)(wx + (lane & 15) * 32 + 16 * S + 4 * (lane >> 4));
    const half8_t wb = __builtin_bit_cast(half8_t, wq);
#define BGTQ_PV(DB)                                                                                          \
    o[DB] = mfma16(as_h8(vpair<VB, (S * 8 + DB) * 4>(vs, vlut, lc), vpair<VB, (S * 8 + DB) * 4 + 1>(vs, vlut, lc), \
                         vpair<VB, (S * 8 + DB) * 4 + 2>(vs, vlut, lc), vpair<VB, (S * 8 + DB) * 4 + 3>(vs, vlut, lc)), \
                   wb, ZERO ? f32x4_t{0.f, 0.f, 0.f, 0.f} : o[DB])
    BGTQ_PV(0); BGTQ_PV(1); BGTQ_PV(2); BGTQ_PV(3); BGTQ_PV(4); BGTQ_PV(5); BGTQ_PV(6); BGTQ_PV(7);
#undef BGTQ_PV
}

// Plain v_max_f32 / v_max3_f32: the operands here are never NaN (scores, -inf for masked tokens),
// so the quieting that fmaxf adds on values of unknown origin is dead work.
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// Max over the 16 lanes of a row: four DPP row rotations fused into the max (two wait states
// before each, as a DPP source written by the previous VALU instruction requires).
__device__ __forceinline__ float row_max16(float v) {
    float r;
    asm("s_nop 1\n\t"
        "v_max_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf"
        : "=&v"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    return v;
}

constexpr int a16(int x) { return (x + 15) & ~15; }
constexpr int cmax(int x, int y) { return x > y ? x : y; }

// ---------------------------------------------------------------------------------------------
// Quantize one token (shared by the append kernels and the decode that appends).  The float32
// steps are spelled out one IEEE operation at a time (no contraction) so the codes and fp16 scales
// are reproducible bit for bit.
// Code of x among the 2^w - 1 scaled thresholds t * thr[thr_base(w) + m] (ascending): the number
// of thresholds x reaches, by binary search.
__device__ __forceinline__ uint32_t tq_code(float x, float t, int w, const float* thr) {
#pragma clang fp contract(off)
    uint32_t code = 0;
    const float* tb = thr + thr_base(w);
    for (int st = w - 1; st >= 0; --st) {
        const uint32_t cand = code + (1u << st);
        const float th = t * tb[cand - 1];
        if (x >= th) code = cand;
    }
    return code;
}


__device__ __forceinline__ float lane_f(float v, int i) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
}

// The per-token fp16 RMS scale of a row spread over the wave (lane i holds elements 2i, 2i+1 and
// the block's 1/sigma r): the same IEEE steps as rms_scale16, u = x*r, u*u, summed in element
// order, each term read across lanes so the sequential sum waits on no memory.
__device__ __forceinline__ float wave_rms16(float x0, float x1, float r, bool use_r, uint16_t* s16) {
#pragma clang fp contract(off)
    const float u0 = use_r ? x0 * r : x0, u1 = use_r ? x1 * r : x1;
    const float q0 = u0 * u0, q1 = u1 * u1;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        acc = acc + lane_f(q0, i);
        acc = acc + lane_f(q1, i);
    }
    const float ms = acc / 128.0f;
    const uint16_t h = f2h(sqrtf(ms));
    *s16 = h;
    return h2f(h);
}

// min and max of elements [j0, j0 + n) of a row spread over the wave, folded in element order
// from element j0 (the order affine_group takes); j0 and n are wave-uniform, n even.
__device__ __forceinline__ void wave_minmax(float x0, float x1, int j0, int n, float& mn, float& mx) {
    mn = mx = lane_f(x0, j0 >> 1);
    mx = fmaxf(mx, lane_f(x1, j0 >> 1));
    mn = fminf(mn, lane_f(x1, j0 >> 1));
    for (int i = (j0 >> 1) + 1; i < ((j0 + n) >> 1); ++i) {
        const float a = lane_f(x0, i), c = lane_f(x1, i);
        mn = fminf(mn, a);
        mx = fmaxf(mx, a);
        mn = fminf(mn, c);
        mx = fmaxf(mx, c);
    }
}

// Launch with the armed event pair, if any (consumed), else plainly.
template <typename K, typename A>
static hipError_t launch_main(K kernel, dim3 grid, dim3 block, hipStream_t s, const A& a) {
    if (t_ev_start) {
        hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
        t_ev_start = t_ev_stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, a);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace bgtq
