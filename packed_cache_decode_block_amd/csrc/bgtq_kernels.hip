// HIP kernels for packed-cache decode attention on CDNA4 (gfx950), wave64.
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (Block-GTQ; abstract, review
// §1/§3, Figures 1-2): keys quantized per RoPE block with greedy integer widths, values at one
// width, attention computed directly from the packed codes.  Affine K4/V2 groups follow the
// "Quantize What Counts" summary (Results: group-size sensitivity); the fp16 recent ring and the
// order-free concatenation follow the "LogQuant" summary (Method 2 and Method 4).
//
// Decode kernels here, each one workgroup = 4 waves = one split of one (batch, kv head), emitting
// one (o, m, l) partial per query head that k_combine merges across splits:
//  * k_decode (vector ALUs only; every format and head ratio): lane = token.  The tile's K records
//    are staged dword-major in LDS; each nonzero RoPE block (sorted by width) is one slot: a 64-bit
//    LDS window, alignbit, two bit-field extracts, two centroid reads from an LDS table, then 2g
//    FMAs whose query operand is broadcast from VGPRs with DPP.  P·V: the 2*v_bits-bit pair field
//    indexes an LDS table of fp16 centroid pairs and v_dot2_f32_f16 accumulates
//    w(t, t+1)·c(t, t+1) in fp32, with w = p * scale rounded to fp16 (as flash attention rounds P
//    before P·V).  The library takes it for g <= 2, and for any g when a cache asks for the
//    vector path.
//  * k_decode_mxa (affine keys, g >= 4): q·k and P·V on the matrix cores.
//  * k_decode_fp16 / k_decode_fp16_mx: fp16 rows (the unquantized comparator and the recent ring).
// Block-GTQ keys with g >= 4 take the matrix-core kernel of bgtq_decode_gtq.hip.
// Both use an online softmax in base 2 with the exact running maximum per head.
#include "bgtq_internal.h"

#include <hip/hip_ext.h>

#include "../../include/bgtq.h"
#include "bgtq_device.h"
#include "generated/bgtq_codebook_data.h"

namespace bgtq {
namespace {


// ---------------------------------------------------------------------------------------------
// acc[h] += bcast(q, lane BASE + h) * va ; acc[h] += bcast(q, lane BASE + G + h) * vb
// DPP row_newbcast reads lane n of each 16-lane row; s_nop 1 covers the VALU->DPP read hazard.
template <int G, int BASE> struct SlotFma;

#define BGTQ_F(A, L, SRC) "v_fmac_f32_dpp " A ", %[q], " SRC " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n"

template <int BASE> struct SlotFma<8, BASE> {
    static __device__ __forceinline__ void run(float* a, float q, float va, float vb) {
        static_assert(BASE == 0, "g = 8 uses whole VGPRs");
        asm volatile("s_nop 1\n"
                     BGTQ_F("%0", 0, "%[va]") BGTQ_F("%1", 1, "%[va]") BGTQ_F("%2", 2, "%[va]")
                     BGTQ_F("%3", 3, "%[va]") BGTQ_F("%4", 4, "%[va]") BGTQ_F("%5", 5, "%[va]")
                     BGTQ_F("%6", 6, "%[va]") BGTQ_F("%7", 7, "%[va]")
                     BGTQ_F("%0", 8, "%[vb]") BGTQ_F("%1", 9, "%[vb]") BGTQ_F("%2", 10, "%[vb]")
                     BGTQ_F("%3", 11, "%[vb]") BGTQ_F("%4", 12, "%[vb]") BGTQ_F("%5", 13, "%[vb]")
                     BGTQ_F("%6", 14, "%[vb]") BGTQ_F("%7", 15, "%[vb]")
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                       "+v"(a[6]), "+v"(a[7])
                     : [q] "v"(q), [va] "v"(va), [vb] "v"(vb));
    }
};

#define BGTQ_FN(A, L, SRC) "v_fmac_f32_dpp " A ", %[q], " SRC " row_newbcast:%c[" L "] row_mask:0xf bank_mask:0xf\n"

template <int BASE> struct SlotFma<4, BASE> {
    static __device__ __forceinline__ void run(float* a, float q, float va, float vb) {
        asm volatile("s_nop 1\n"
                     BGTQ_FN("%0", "l0", "%[va]") BGTQ_FN("%1", "l1", "%[va]")
                     BGTQ_FN("%2", "l2", "%[va]") BGTQ_FN("%3", "l3", "%[va]")
                     BGTQ_FN("%0", "l4", "%[vb]") BGTQ_FN("%1", "l5", "%[vb]")
                     BGTQ_FN("%2", "l6", "%[vb]") BGTQ_FN("%3", "l7", "%[vb]")
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
                     : [q] "v"(q), [va] "v"(va), [vb] "v"(vb), [l0] "n"(BASE), [l1] "n"(BASE + 1),
                       [l2] "n"(BASE + 2), [l3] "n"(BASE + 3), [l4] "n"(BASE + 4), [l5] "n"(BASE + 5),
                       [l6] "n"(BASE + 6), [l7] "n"(BASE + 7));
    }
};

template <int BASE> struct SlotFma<2, BASE> {
    static __device__ __forceinline__ void run(float* a, float q, float va, float vb) {
        asm volatile("s_nop 1\n"
                     BGTQ_FN("%0", "l0", "%[va]") BGTQ_FN("%1", "l1", "%[va]")
                     BGTQ_FN("%0", "l2", "%[vb]") BGTQ_FN("%1", "l3", "%[vb]")
                     : "+v"(a[0]), "+v"(a[1])
                     : [q] "v"(q), [va] "v"(va), [vb] "v"(vb), [l0] "n"(BASE), [l1] "n"(BASE + 1),
                       [l2] "n"(BASE + 2), [l3] "n"(BASE + 3));
    }
};

template <int BASE> struct SlotFma<1, BASE> {
    static __device__ __forceinline__ void run(float* a, float q, float va, float vb) {
        asm volatile("s_nop 1\n"
                     BGTQ_FN("%0", "l0", "%[va]") BGTQ_FN("%0", "l1", "%[vb]")
                     : "+v"(a[0])
                     : [q] "v"(q), [va] "v"(va), [vb] "v"(vb), [l0] "n"(BASE), [l1] "n"(BASE + 1));
    }
};

// slot s (RoPE block in sorted or natural order) -> (q VGPR, first DPP lane)
template <int G, int S> struct SlotPos {
    static constexpr int vgpr = (S * 2 * G) / 16;
    static constexpr int base = (S * 2 * G) % 16;
};

// ---------------------------------------------------------------------------------------------
// Per-wave softmax / P·V state.
template <int G> struct WaveState {
    float m[G];        // running max (base-2 logits), wave-uniform
    float l[G];        // per-lane partial sum of p
    float zs[G];       // per-lane partial sum of p * zero (affine values)
    float o[G][8];     // lane (quad slot, 8-dim group) accumulators
};

template <int G> __device__ __forceinline__ void state_init(WaveState<G>& st) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.m[h] = -INFINITY;
        st.l[h] = 0.f;
        st.zs[h] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) st.o[h][j] = 0.f;
    }
}

// z: base-2 logits of this lane's token (-inf if invalid).  wscale multiplies p into the fp16
// weight; zero (affine values) accumulates p * zero.  Writes the fp16 weights to wbuf, as pairs
// (2t, 2t+1) per head, [t/2][h][2] (PAIR32 false), or as pairs (t, t+32), [h][t%32][2] (PAIR32 true).
template <int G, bool PAIR32 = false>
__device__ __forceinline__ void softmax_tile(WaveState<G>& st, const float* z, bool valid, float wscale,
                                             float zero, uint16_t* wbuf, int lane) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (__ballot(z[h] > st.m[h])) {
            const float mn = fmaxf(st.m[h], wave_max(z[h]));
            const float alpha = __builtin_amdgcn_exp2f(st.m[h] - mn);
            st.m[h] = mn;
            st.l[h] *= alpha;
            st.zs[h] *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) st.o[h][j] *= alpha;
        }
        const float p = valid ? __builtin_amdgcn_exp2f(z[h] - st.m[h]) : 0.f;
        st.l[h] += p;
        st.zs[h] += p * zero;
        const int wi = PAIR32 ? (h * 32 + (lane & 31)) * 2 + (lane >> 5) : ((lane >> 1) * G + h) * 2 + (lane & 1);
        wbuf[wi] = valid ? f2h(p * wscale) : (uint16_t)0;
    }
}

// Extract the 2*VB-bit field f (static) from a VB-dword record.
template <int VB, int F>
__device__ __forceinline__ uint32_t vfield(const uint32_t* r) {
    constexpr int bit = 2 * VB * F, w = bit / 32, sh = bit % 32, nb = 2 * VB;
    if constexpr (sh + nb <= 32) {
        return (r[w] >> sh) & ((1u << nb) - 1u);
    } else {
        return __builtin_amdgcn_alignbit(r[w + 1], r[w], sh) & ((1u << nb) - 1u);
    }
}
// The same field times 4 (a byte offset into a table of dwords), one shift and one AND.
template <int VB, int F>
__device__ __forceinline__ uint32_t vfield4(const uint32_t* r) {
    constexpr int bit = 2 * VB * F, w = bit / 32, sh = bit % 32, nb = 2 * VB;
    constexpr uint32_t m4 = ((1u << nb) - 1u) << 2;
    if constexpr (sh + nb > 32) return __builtin_amdgcn_alignbit(r[w + 1], r[w], sh - 2) & m4;
    else if constexpr (sh >= 2) return (r[w] >> (sh - 2)) & m4;
    else return (r[w] << (2 - sh)) & m4;
}

// P·V of one tile for lane L = dd + 16j over its value stream (lane-stream layout): field
// (s, db, m) holds the codes of dim 16db + dd for the token pair (p, p + 32), p = 16s + 4j + m;
// the pair table turns it into two fp16 centroids and v_dot2 multiplies them by the fp16 weights
// (w_p, w_p+32) of each head.  o[h][db] accumulates dim 16db + dd.
template <int G, int VB, int SDB>
__device__ __forceinline__ void pv_block(WaveState<G>& st, const uint32_t* vs, const uint32_t* vlut,
                                         const uint32_t (&w)[G][4]) {
    constexpr int db = SDB % 8;
    const uint32_t cp[4] = {vlut[vfield<VB, 4 * SDB>(vs)], vlut[vfield<VB, 4 * SDB + 1>(vs)],
                            vlut[vfield<VB, 4 * SDB + 2>(vs)], vlut[vfield<VB, 4 * SDB + 3>(vs)]};
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int h = 0; h < G; ++h)
            st.o[h][db] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[h][m]),
                                                 __builtin_bit_cast(half2_t, cp[m]), st.o[h][db], false);
}

template <int G, int VB, int S>
__device__ __forceinline__ void pv_half(WaveState<G>& st, const uint32_t* vs, const uint32_t* vlut,
                                        const uint32_t* wb32, int j) {
    uint32_t w[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uint4 q = *(const uint4*)(wb32 + h * 32 + 16 * S + 4 * j);
        w[h][0] = q.x; w[h][1] = q.y; w[h][2] = q.z; w[h][3] = q.w;
    }
    pv_block<G, VB, S * 8 + 0>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 1>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 2>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 3>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 4>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 5>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 6>(st, vs, vlut, w);
    pv_block<G, VB, S * 8 + 7>(st, vs, vlut, w);
}

// Load the fp16 weight pairs of quad `quad` (pairs 2quad, 2quad+1) for all heads.
template <int G>
__device__ __forceinline__ void load_w(uint32_t (&w)[2][G], const uint16_t* wbuf, int quad) {
    const uint32_t* wb = (const uint32_t*)wbuf + 2 * quad * G;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int h = 0; h < G; ++h) w[p][h] = wb[p * G + h];
}

// Merge the NW waves' (o, m, l, zero term) records in red[wave][h] into one partial per head:
// part[h][split] = (sum_w e^(m_w - M) (o_w + zs_w), M, sum_w e^(m_w - M) l_w).  The scale factors
// are computed once per (wave, head) into sc (LDS, NW * G floats) before the element loop.
template <int G, int NW = 4>
__device__ __forceinline__ void merge_waves(const float* red, float* sc, float* part, int n_parts, int split) {
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, red[(wv * G + h) * PART + 128]);
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            const float m = red[(wv * G + h) * PART + 128];
            sc[wv * G + h] = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        }
        part[((size_t)h * n_parts + split) * PART + 128] = M;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * 129; idx += blockDim.x) {
        const int h = idx / 129, jj = idx % 129, j = jj < 128 ? jj : 129;
        float acc = 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            const float* rw = red + (wv * G + h) * PART;
            acc += sc[wv * G + h] * (j < 128 ? rw[j] + rw[130] : rw[129]);
        }
        part[((size_t)h * n_parts + split) * PART + j] = acc;
    }
}


// Epilogue: merge lanes and waves, write one (o[128], m, l) partial per query head.
// STRIDE16: o[h][j] holds dim 16j + lane (lanes 0..15 after the merge); else dim 8*lane + j.
template <int G, bool STRIDE16 = false>
__device__ __forceinline__ void write_partial(WaveState<G>& st, float* red /*[4][G][PART]*/, float* part,
                                              int n_parts, int split, int wave, int lane) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v = st.o[h][j];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            st.o[h][j] = v;
        }
        st.l[h] = wave_sum(st.l[h]);
        st.zs[h] = wave_sum(st.zs[h]);
    }
    float* r = red + wave * G * PART;
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) r[h * PART + (STRIDE16 ? 16 * j + lane : lane * 8 + j)] = st.o[h][j];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            r[h * PART + 128] = st.m[h];
            r[h * PART + 129] = st.l[h];
            r[h * PART + 130] = st.zs[h];
        }
    }
    __syncthreads();
    merge_waves<G>(red, red + 4 * G * PART, part, n_parts, split);
}

// ---------------------------------------------------------------------------------------------
// q·k over Block-GTQ slots, records staged dword-major in LDS.  Three stages per slot:
// window read (two dwords around the slot's bit offset), centroid reads (two table lookups),
// DPP-broadcast FMAs.  Groups of four slots are software-pipelined: the next group's window reads
// are issued before this group's FMAs so their LDS latency hides behind the arithmetic.
struct Win {
    uint32_t lo, hi;
};

__device__ __forceinline__ uint32_t dsc16(const uint32_t* dsc, int s) {
    return (dsc[s >> 1] >> (16 * (s & 1))) & 0xFFFFu;
}

__device__ __forceinline__ Win win_read(const uint32_t* stage, uint32_t li, uint32_t d16) {
    const uint32_t k = d16 & 31u;
    return Win{stage[k * TILE + li], stage[(k + 1) * TILE + li]};
}

__device__ __forceinline__ void lut_read(float& va, float& vb, const Win& wn, uint32_t d16, const float* klut) {
    const uint32_t o = (d16 >> 5) & 31u, w = d16 >> 10;
    const uint32_t x = __builtin_amdgcn_alignbit(wn.hi, wn.lo, o);
    const float* lut = klut + ((1 << w) - 2);
    va = lut[x & ((1u << w) - 1u)];
    vb = lut[__builtin_amdgcn_ubfe(x, w, w)];
}

template <int G, int GR = 0>
__device__ __forceinline__ void gtq_pipe(float* acc, const float* qv, const uint32_t* dsc, int nnz_pad,
                                         const uint32_t* stage, uint32_t li, const float* klut, Win* wn) {
    if constexpr (GR < 16) {
        if (GR * 4 < nnz_pad) {
            float va[4], vb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) lut_read(va[j], vb[j], wn[j], dsc16(dsc, 4 * GR + j), klut);
            if constexpr (GR + 1 < 16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) wn[j] = win_read(stage, li, dsc16(dsc, 4 * (GR + 1) + j));
            }
            SlotFma<G, SlotPos<G, 4 * GR + 0>::base>::run(acc, qv[SlotPos<G, 4 * GR + 0>::vgpr], va[0], vb[0]);
            SlotFma<G, SlotPos<G, 4 * GR + 1>::base>::run(acc, qv[SlotPos<G, 4 * GR + 1>::vgpr], va[1], vb[1]);
            SlotFma<G, SlotPos<G, 4 * GR + 2>::base>::run(acc, qv[SlotPos<G, 4 * GR + 2>::vgpr], va[2], vb[2]);
            SlotFma<G, SlotPos<G, 4 * GR + 3>::base>::run(acc, qv[SlotPos<G, 4 * GR + 3>::vgpr], va[3], vb[3]);
            gtq_pipe<G, GR + 1>(acc, qv, dsc, nnz_pad, stage, li, klut, wn);
        }
    }
}

// q·k over natural-order blocks of an in-register fp16 row chunk (blocks B0..B0+15).
template <int G, int B0, int I = 0>
__device__ __forceinline__ void fp16_blocks(float* acc, const float* qv, const uint32_t* row16) {
    if constexpr (I < 16) {
        const uint32_t x = row16[I];
        SlotFma<G, SlotPos<G, B0 + I>::base>::run(acc, qv[SlotPos<G, B0 + I>::vgpr], h2f(x & 0xFFFFu), h2f(x >> 16));
        fp16_blocks<G, B0, I + 1>(acc, qv, row16);
    }
}

template <int N> __device__ __forceinline__ float ubyte_f(uint32_t x) { return (float)((x >> (8 * N)) & 0xFFu); }

// q·k over affine 4-bit keys: 16 dwords of nibbles (coordinate j at bits 4j).  Dword K holds
// coordinates 8K..8K+7; masking even/odd nibbles into bytes gives blocks 4K..4K+3 as byte pairs.
// Per group of KG coordinates: z += scale * sum_j q_j code_j + zero * sum_j q_j.
template <int G, int KG, int K = 0>
__device__ __forceinline__ void affine4_run(float* acc, float* gp, const float* qv, const uint32_t* rec,
                                            const float* scl, const float* zer, const float* qs) {
    if constexpr (K < 16) {
        const uint32_t x = rec[K];
        const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
        SlotFma<G, SlotPos<G, 4 * K + 0>::base>::run(gp, qv[SlotPos<G, 4 * K + 0>::vgpr],
                                                       ubyte_f<0>(lo), ubyte_f<0>(hi));
        SlotFma<G, SlotPos<G, 4 * K + 1>::base>::run(gp, qv[SlotPos<G, 4 * K + 1>::vgpr],
                                                       ubyte_f<1>(lo), ubyte_f<1>(hi));
        SlotFma<G, SlotPos<G, 4 * K + 2>::base>::run(gp, qv[SlotPos<G, 4 * K + 2>::vgpr],
                                                       ubyte_f<2>(lo), ubyte_f<2>(hi));
        SlotFma<G, SlotPos<G, 4 * K + 3>::base>::run(gp, qv[SlotPos<G, 4 * K + 3>::vgpr],
                                                       ubyte_f<3>(lo), ubyte_f<3>(hi));
        constexpr int DPG = KG / 8;
        if constexpr ((K + 1) % DPG == 0) {
            constexpr int gi = K / DPG;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                acc[h] += scl[gi] * gp[h] + zer[gi] * qs[gi * G + h];
                gp[h] = 0.f;
            }
        }
        affine4_run<G, KG, K + 1>(acc, gp, qv, rec, scl, zer, qs);
    }
}

// fp16 tiles (recent ring or the unquantized comparator): rows [n][128] fp16 of one (b, h).
template <int G>
__device__ void fp16_tiles(WaveState<G>& st, const uint16_t* K16, const uint16_t* V16, int64_t n,
                           int64_t t_lo, int64_t t_hi, int wave, const float* qv, uint16_t* wbuf, int lane) {
    for (int64_t t = t_lo + wave; t < t_hi; t += 4) {
        const int64_t pos = t * TILE + lane;
        const bool valid = pos < n;
        float acc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = 0.f;
        const uint4* rowp = (const uint4*)(K16 + (valid ? pos : 0) * D);
        // 256-byte row in four 64-byte chunks; the next chunk is in flight while one is consumed.
        uint32_t cur[16], nxt[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint4 v = rowp[u];
            cur[4 * u] = v.x; cur[4 * u + 1] = v.y; cur[4 * u + 2] = v.z; cur[4 * u + 3] = v.w;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c < 3) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint4 v = rowp[(c + 1) * 4 + u];
                    nxt[4 * u] = v.x; nxt[4 * u + 1] = v.y; nxt[4 * u + 2] = v.z; nxt[4 * u + 3] = v.w;
                }
            }
            asm volatile("" ::: "memory");
            if (c == 0) fp16_blocks<G, 0>(acc, qv, cur);
            if (c == 1) fp16_blocks<G, 16>(acc, qv, cur);
            if (c == 2) fp16_blocks<G, 32>(acc, qv, cur);
            if (c == 3) fp16_blocks<G, 48>(acc, qv, cur);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < 16; ++u) cur[u] = nxt[u];
        }
        float z[G];
#pragma unroll
        for (int h = 0; h < G; ++h) z[h] = valid ? acc[h] : -INFINITY;
        wave_lds_fence();
        softmax_tile<G>(st, z, valid, 1.0f, 0.f, wbuf, lane);
        wave_lds_fence();
        // P·V: lane = (quad slot, 8-dim group); tokens 4quad..4quad+3, dims 8dg..8dg+7
        const int dg = lane & 15;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int quad = it * 4 + (lane >> 4);
            uint32_t w[2][G];
            load_w<G>(w, wbuf, quad);
            uint4 vr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t p = t * TILE + quad * 4 + u;
                vr[u] = p < n ? *(const uint4*)(V16 + p * D + dg * 8) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const uint32_t a4[4] = {vr[2 * pr].x, vr[2 * pr].y, vr[2 * pr].z, vr[2 * pr].w};
                const uint32_t b4[4] = {vr[2 * pr + 1].x, vr[2 * pr + 1].y, vr[2 * pr + 1].z, vr[2 * pr + 1].w};
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2) {
                    const uint32_t lo = __builtin_amdgcn_perm(b4[m2], a4[m2], 0x05040100u);  // (a.lo, b.lo)
                    const uint32_t hi = __builtin_amdgcn_perm(b4[m2], a4[m2], 0x07060302u);  // (a.hi, b.hi)
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        st.o[h][2 * m2] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[pr][h]),
                                                                 __builtin_bit_cast(half2_t, lo), st.o[h][2 * m2], false);
                        st.o[h][2 * m2 + 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[pr][h]),
                                                                     __builtin_bit_cast(half2_t, hi), st.o[h][2 * m2 + 1], false);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// ---------------------------------------------------------------------------------------------
// Per-workgroup query preparation (wave 0, lane = RoPE block i).  Writes, in LDS:
//  qp[s*2G + e*G + h]: query coordinate (block s, half e) of head h times log2(e)/sqrt(d), with
//    Block-GTQ keys in slot order (width descending, ties by block index) and sigma folded in;
//    natural block order otherwise; zero for padding slots.
//  dsc16[s]: slot descriptor (start dword | bit offset << 5 | width << 10); padding = width 1 at 0.
//  qs[g*G + h]: per-key-group sums of the natural scaled query (affine keys).
// The block order comes from nine wave ballots (one per width) instead of a sort.

// Keys stored rotated (y = H (s * k) / 16): the query goes to H (s * q) / 8, so q'.y = q.k.  A
// wave holds coordinates 2 lane + e (q0: e = 0, q1: e = 1); stage 1 pairs them inside the lane,
// stages 2..64 pair lane with lane ^ m (m = 1..32): the lower lane keeps a + b, the upper one a - b.
template <int G>
__device__ __forceinline__ void rotate_query(float (&q0)[G], float (&q1)[G], const uint8_t* rot, int lane) {
    const uint32_t sbits = (uint32_t)rot[lane >> 2] >> (2 * (lane & 3));
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        const float a0 = (sbits & 1u) ? -q0[hh] : q0[hh], a1 = (sbits & 2u) ? -q1[hh] : q1[hh];
        float u = a0 + a1, v = a0 - a1;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const float pu = __shfl_xor(u, m, 64), pv = __shfl_xor(v, m, 64);
            const bool upper = (lane & m) != 0;
            u = upper ? pu - u : u + pu;
            v = upper ? pv - v : v + pv;
        }
        q0[hh] = u * 0.125f;
        q1[hh] = v * 0.125f;
    }
}

template <int G, bool SORTED, int KG>
__device__ void prep_store(const PrepIn<G>& in, int lane, float* qp, uint16_t* dsc16, uint32_t* nnz_pad, float* qs,
                           int3* order = nullptr, const uint8_t* rot = nullptr) {
    float q0[G], q1[G];
    if (in.dtype == BGTQ_F32) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            q0[hh] = __builtin_bit_cast(float, in.r0[hh]);
            q1[hh] = __builtin_bit_cast(float, in.r1[hh]);
        }
    } else if (in.dtype == BGTQ_F16) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            q0[hh] = h2f(in.r0[hh] & 0xFFFFu);
            q1[hh] = h2f(in.r0[hh] >> 16);
        }
    } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            q0[hh] = bf2f(in.r0[hh] & 0xFFFFu);
            q1[hh] = bf2f(in.r0[hh] >> 16);
        }
    }
    if (rot) rotate_query<G>(q0, q1, rot, lane);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        q0[hh] *= kLog2eOverSqrtD;
        q1[hh] *= kLog2eOverSqrtD;
    }
    if constexpr (SORTED) {
        const int bw = (int)((in.w4 >> (8 * (lane & 3))) & 0xFFu);
        const int w = bw < 8 ? bw : 8;  // widths above 8 are invalid; clamp
        const float sg = in.sg;
        int rank, pos, nnz;
        block_order(w, lane, rank, pos, nnz);
        if (order) *order = int3{rank, pos, nnz};
        if (w > 0) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                qp[rank * 2 * G + hh] = q0[hh] * sg;
                qp[rank * 2 * G + G + hh] = q1[hh] * sg;
            }
            dsc16[rank] = (uint16_t)((pos >> 5) | ((pos & 31) << 5) | (w << 10));
        }
        if (lane >= nnz) {
#pragma unroll
            for (int hh = 0; hh < 2 * G; ++hh) qp[lane * 2 * G + hh] = 0.f;
            dsc16[lane] = (uint16_t)(1u << 10);
        }
        if (lane == 0) *nnz_pad = (uint32_t)((nnz + 3) & ~3);
    } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            qp[lane * 2 * G + hh] = q0[hh];
            qp[lane * 2 * G + G + hh] = q1[hh];
        }
        if constexpr (KG > 0) {
            wave_lds_fence();
            constexpr int NG = D / KG;
            if (lane < NG * G) {
                const int gi = lane / G, hh = lane % G;
                float acc = 0.f;
                for (int j = gi * KG; j < (gi + 1) * KG; ++j) acc += qp[(j >> 1) * 2 * G + (j & 1) * G + hh];
                qs[gi * G + hh] = acc;
            }
        }
    }
}

template <int G, bool SORTED, int KG>
__device__ void prep_wave(const void* q, int dtype, const uint8_t* bits, const float* sigma, int b, int h,
                          int Hq, int lane, float* qp, uint16_t* dsc16, uint32_t* nnz_pad, float* qs,
                          const uint8_t* rot = nullptr) {
    prep_store<G, SORTED, KG>(prep_load<G, SORTED>(q, dtype, bits, sigma, b, h, Hq, lane), lane, qp, dsc16, nnz_pad, qs,
                              nullptr, rot);
}

template <int G>
__device__ __forceinline__ void load_qv_lds(float* qv, const float* qp, int lane) {
#pragma unroll
    for (int v = 0; v < 8 * G; ++v) qv[v] = qp[v * 16 + (lane & 15)];
}

// KG == 0: Block-GTQ keys (R record dwords); KG > 0: affine 4-bit keys with groups of KG.
template <int G, int R, int VB, int KG>
__global__ __launch_bounds__(256, 2) void k_decode(const DecodeArgs a) {
    constexpr bool AFFINE_K = KG > 0;
    constexpr int NG = AFFINE_K ? D / (KG > 0 ? KG : 1) : 1;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __shared__ float s_klut[512];
    __shared__ uint32_t s_vlut[1 << (2 * VB)];
    __shared__ uint32_t s_stage[4][AFFINE_K ? 1 : (R + 1) * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t s_w[4][64 * G];
    __shared__ float s_red[4 * G * PART + 4 * G];  // wave records, then merge scale factors
    __shared__ float s_qp[128 * G];
    __shared__ uint16_t s_dsc[64];
    __shared__ uint32_t s_nnz;
    __shared__ float s_qs[AFFINE_K ? NG * G : 1];

    const size_t bh = (size_t)b * a.Hkv + h;
    constexpr int ng = NG;
    const int64_t n_packed = a.n_packed[b];
    const int64_t n_tiles_b = (n_packed + TILE - 1) / TILE;
    const int64_t t_lo = (int64_t)split * a.tiles_per_split;
    const int64_t t_hi = t_lo + a.tiles_per_split < n_tiles_b ? t_lo + a.tiles_per_split : n_tiles_b;

    const uint32_t* kc = (const uint32_t*)(a.k_codes + bh * a.n_tiles * a.k_tile_bytes);
    const uint32_t* vc = (const uint32_t*)(a.v_codes + bh * a.n_tiles * a.v_tile_bytes);
    const uint16_t* ks = a.k_scale + bh * a.n_cap * ng;
    const uint16_t* kz = AFFINE_K ? a.k_zero + bh * a.n_cap * ng : nullptr;
    const uint16_t* vs = a.v_scale + bh * a.n_cap;
    const uint16_t* vz = a.v_affine ? a.v_zero + bh * a.n_cap : nullptr;
    uint32_t* stage = s_stage[wave];
    constexpr int RK = AFFINE_K ? 16 : R;

    // Registers of the tile in flight (prefetched one tile ahead).
    uint32_t kn[RK], vn[4 * VB];
    uint16_t ksn[NG], kzn[NG], vsn, vzn;
    auto fetch = [&](int64_t t) {
        const uint32_t* kt = kc + t * (a.k_tile_bytes / 4);
        const uint32_t* vt = vc + t * (a.v_tile_bytes / 4);
#pragma unroll
        // the packed tiles are read once per step: non-temporal loads
        for (int k = 0; k < RK; ++k) kn[k] = __builtin_nontemporal_load(kt + k * TILE + lane);
#pragma unroll
        for (int c4 = 0; c4 < VB; ++c4) {
            const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)vt + c4 * 64 + lane);
            vn[4 * c4] = v[0]; vn[4 * c4 + 1] = v[1]; vn[4 * c4 + 2] = v[2]; vn[4 * c4 + 3] = v[3];
        }
        const int64_t p = t * TILE + lane < n_packed ? t * TILE + lane : 0;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            ksn[gi] = ks[p * NG + gi];
            kzn[gi] = AFFINE_K ? kz[p * NG + gi] : (uint16_t)0;
        }
        vsn = vs[p];
        vzn = vz ? vz[p] : (uint16_t)0;
    };
    if (t_lo + wave < t_hi) fetch(t_lo + wave);

    for (int i = threadIdx.x; i < BGTQ_CB_CENTROIDS; i += blockDim.x) s_klut[i] = __builtin_bit_cast(float, c_cent32[i]);
    for (int i = threadIdx.x; i < (1 << (2 * VB)); i += blockDim.x) {
        const uint32_t ca = i & ((1 << VB) - 1), cb = i >> VB;
        uint32_t ha, hb;
        if (a.v_affine) {
            ha = f2h((float)ca);
            hb = f2h((float)cb);
        } else {
            ha = c_cent16[cent_base(VB) + ca];
            hb = c_cent16[cent_base(VB) + cb];
        }
        s_vlut[i] = ha | (hb << 16);
    }
    if (wave == 0)
        prep_wave<G, !AFFINE_K, KG>(a.q, a.q_dtype, a.bits, a.sigma, b, h, a.Hq, lane, s_qp, s_dsc, &s_nnz, s_qs,
                                    AFFINE_K && a.k_rot ? a.k_rot + h * 16 : nullptr);
    __syncthreads();

    float* part = a.part + ((size_t)b * a.Hq + (size_t)h * G) * a.n_parts * PART;
    uint16_t* wbuf = s_w[wave];

    WaveState<G> st;
    state_init<G>(st);
    float qv[8 * G];
    load_qv_lds<G>(qv, s_qp, lane);
    uint32_t dsc[32];
    int nnz_pad = 0;
    float qs[NG * G];
    if constexpr (!AFFINE_K) {
        const uint32_t* d32 = (const uint32_t*)s_dsc;
#pragma unroll
        for (int i = 0; i < 32; ++i) dsc[i] = __builtin_amdgcn_readfirstlane(d32[i]);
        nnz_pad = (int)__builtin_amdgcn_readfirstlane(s_nnz);
    } else {
#pragma unroll
        for (int i = 0; i < NG * G; ++i) qs[i] = s_qs[i];
    }


    for (int64_t t = t_lo + wave; t < t_hi; t += 4) {
        const int64_t pos = t * TILE + lane;
        const bool valid = pos < n_packed;
        uint32_t kr[RK], vr[4 * VB];
#pragma unroll
        for (int k = 0; k < RK; ++k) kr[k] = kn[k];
#pragma unroll
        for (int c = 0; c < 4 * VB; ++c) vr[c] = vn[c];
        float scl[NG], zer[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            scl[gi] = h2f(ksn[gi]);
            zer[gi] = h2f(kzn[gi]);
        }
        const float vsc = h2f(vsn), vzr = h2f(vzn);
        if (t + 4 < t_hi) fetch(t + 4);

        float acc[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
        if constexpr (!AFFINE_K) {
            // Per-slot scalar values and lane addresses are recomputed each tile (not hoisted).
#pragma unroll
            for (int i = 0; i < 32; ++i) asm volatile("" : "+s"(dsc[i]));
            uint32_t li = lane;
            asm volatile("" : "+v"(li));
            wave_lds_fence();
#pragma unroll
            for (int k = 0; k < R; ++k) stage[k * TILE + li] = kr[k];
            wave_lds_fence();
            Win wn[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wn[j] = win_read(stage, li, dsc16(dsc, j));
            gtq_pipe<G>(acc, qv, dsc, nnz_pad, stage, li, s_klut, wn);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) acc[hh] *= scl[0];
        } else {
            float gp[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) gp[hh] = 0.f;
            affine4_run<G, KG>(acc, gp, qv, kr, scl, zer, qs);
        }
        float z[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) z[hh] = valid ? acc[hh] : -INFINITY;
        wave_lds_fence();
        softmax_tile<G, true>(st, z, valid, vsc, vzr, wbuf, lane);
        wave_lds_fence();
        pv_half<G, VB, 0>(st, vr, s_vlut, (const uint32_t*)wbuf, lane >> 4);
        pv_half<G, VB, 1>(st, vr, s_vlut, (const uint32_t*)wbuf, lane >> 4);
    }
    __syncthreads();
    write_partial<G, true>(st, s_red, part, a.n_parts, split, wave, lane);
}


// Matrix-core decode over affine 4-bit keys in groups of KG = 32, 64 or 128 dims (the "Quantize
// What Counts" K4V2 configuration uses 32), for 4 or 8 query heads per kv head.  A key group spans
// KG / 32 k-steps of q·k: a lane's B operand is one record dword (dims 32 ks + 8u .. 8u + 7 of
// its token, nibble i at bits 4i),
// turned into fp16 by OR-ing the nibble pairs (i, i + 4) into 1024 + n and one packed fp16
// subtraction of 1024, both exact; the A operand holds the query in the matching order (dims
// 32 ks + 8u + {0, 4, 1, 5, 2, 6, 3, 7}), split into fp16 high and low parts.  The products of a
// group's k-steps accumulate on the matrix cores, then take the group's scale and zero:
// z += scale * (q'.codes) + zero * sum(q' over the group).  Softmax, P·V (codebook or affine values)
// and the wave merge are those of the Block-GTQ matrix-core decode; keys need no windows or tables.
template <int G, int VB> struct MxaLds {
    static constexpr int VLUT = 0;
    static constexpr int WX = a16(VLUT + VLutGeom<VB>::BYTES);    // u32 [4 waves][16 heads][32 pairs]
    static constexpr int ALPHA = WX + 4 * 16 * 32 * 4;           // f32 [4 waves][16]
    static constexpr int QSUM = ALPHA + 4 * 16 * 4;              // f32 [8 heads][4 groups]
    static constexpr int QS = QSUM + 8 * 4 * 4;                  // f32 [8 heads][128]: the scaled query
    static constexpr int SST = QS + 8 * 128 * 4;                 // per wave: V scales, V zeros (fp16 [2][64])
    static constexpr int SST_W = 2 * 64 * 2;
    static constexpr int RED = a16(SST + 4 * SST_W);              // epilogue: f32 [4 G PART + 4 G]
    static constexpr int SIZE = RED + 4 * (4 * G * PART + 4 * G);
};

// Two resident workgroups per CU for every value width: the record dwords, group scales and query
// operands held per lane need the registers.
constexpr int kMxaWgsPerCu = 2;

template <int G, int VB, int KG>
__global__ __launch_bounds__(256, kMxaWgsPerCu) void k_decode_mxa(const DecodeArgs a) {
    static_assert(G == 4 || G == 8, "matrix-core decode serves 4 or 8 query heads per kv head");
    static_assert(KG == 32 || KG == 64 || KG == 128, "key groups of 32, 64 or 128 dims");
    constexpr int NG = D / KG, KPG = KG / 32;  // key groups; k-steps per group
    using LD = MxaLds<G, VB>;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int row = lane >> 4, col = lane & 15;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LD::SIZE];
    uint32_t* s_vlut = (uint32_t*)(lds + LD::VLUT);
    float* s_alpha = (float*)(lds + LD::ALPHA) + wave * 16;
    float* s_qsum = (float*)(lds + LD::QSUM);
    float* s_q = (float*)(lds + LD::QS);
    uint16_t* sst = (uint16_t*)(lds + LD::SST + wave * LD::SST_W);
    uint32_t* wx = (uint32_t*)(lds + LD::WX) + wave * 16 * 32;

    const size_t bh = (size_t)b * a.Hkv + h;
    const int64_t n_packed = a.n_packed[b];
    const int64_t n_tiles_b = (n_packed + TILE - 1) / TILE;
    const int64_t t_lo = (int64_t)split * a.tiles_per_split;
    const int64_t t_hi = t_lo + a.tiles_per_split < n_tiles_b ? t_lo + a.tiles_per_split : n_tiles_b;
    const uint32_t* kc = (const uint32_t*)(a.k_codes + bh * a.n_tiles * a.k_tile_bytes);
    const uint32_t* vc = (const uint32_t*)(a.v_codes + bh * a.n_tiles * a.v_tile_bytes);
    const uint16_t* ksc = a.k_scale + bh * a.n_cap * NG;  // the NG group scales of a token
    const uint16_t* kzr = a.k_zero + bh * a.n_cap * NG;   // and its NG group zeros
    const uint32_t* vs32 = (const uint32_t*)(a.v_scale + bh * a.n_cap);  // fp16 pairs (token 2i, 2i + 1)
    const uint32_t* vz32 = a.v_affine ? (const uint32_t*)(a.v_zero + bh * a.n_cap) : nullptr;
    const bool vaff = a.v_affine != 0;

    // Prologue: the query (wave 0), the value table and the first tile's keys go out first.
    const PrepIn<G> pin = prep_load<G, false>(a.q, a.q_dtype, nullptr, nullptr, b, h, a.Hq, lane);
    constexpr int VCOP = VLutGeom<VB>::COPIES, VENT = 1 << (2 * VB);
    constexpr int VROUNDS = (VENT * VCOP + 255) / 256;
    uint32_t vla[VROUNDS], vlb[VROUNDS];
#pragma unroll
    for (int k = 0; k < VROUNDS; ++k) {
        const uint32_t e = ((threadIdx.x + 256u * k) / VCOP) & (VENT - 1);
        vla[k] = c_cent16[cent_base(VB) + (e & ((1u << VB) - 1u))];
        vlb[k] = c_cent16[cent_base(VB) + (e >> VB)];
    }
    // Tile data per lane: the record dword of k-step ks for token group g (kd[ks][g]), the group
    // scales and zeros of its four tokens, and one dword of value scales (lanes 0..31, tokens 2l and
    // 2l + 1) or value zeros (lanes 32..63); the value streams as in the Block-GTQ matrix-core decode.
    uint32_t kd[4][4], vsd;
    float kss[4][NG], kzz[4][NG];  // [token group][key group]
    u32x4_t vn[VB], vx[VB];
    auto fetch_k = [&](int64_t t) {
        const uint32_t* kt = kc + t * (a.k_tile_bytes / 4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int g = 0; g < 4; ++g) kd[ks][g] = __builtin_nontemporal_load(kt + (4 * ks + row) * 64 + 16 * g + col);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t tok = t * TILE + 16 * g + col;
            if constexpr (NG == 4) {
                const uint2 sw = *(const uint2*)(ksc + tok * 4), zw = *(const uint2*)(kzr + tok * 4);
                kss[g][0] = h2f(sw.x & 0xFFFFu); kss[g][1] = h2f(sw.x >> 16);
                kss[g][2] = h2f(sw.y & 0xFFFFu); kss[g][3] = h2f(sw.y >> 16);
                kzz[g][0] = h2f(zw.x & 0xFFFFu); kzz[g][1] = h2f(zw.x >> 16);
                kzz[g][2] = h2f(zw.y & 0xFFFFu); kzz[g][3] = h2f(zw.y >> 16);
            } else if constexpr (NG == 2) {
                const uint32_t sw = *(const uint32_t*)(ksc + tok * 2), zw = *(const uint32_t*)(kzr + tok * 2);
                kss[g][0] = h2f(sw & 0xFFFFu); kss[g][1] = h2f(sw >> 16);
                kzz[g][0] = h2f(zw & 0xFFFFu); kzz[g][1] = h2f(zw >> 16);
            } else {
                kss[g][0] = h2f(ksc[tok]);
                kzz[g][0] = h2f(kzr[tok]);
            }
        }
        vsd = lane < 32 ? vs32[t * (TILE / 2) + lane] : (vz32 ? vz32[t * (TILE / 2) + (lane & 31)] : 0u);
    };
    auto fetch_v = [&](u32x4_t (&dst)[VB], int64_t t) {
        const u32x4_t* vt = (const u32x4_t*)(vc + t * (a.v_tile_bytes / 4));
#pragma unroll
        for (int c = 0; c < VB; ++c) dst[c] = __builtin_nontemporal_load(vt + c * 64 + lane);
    };
    const int64_t t_first = t_lo + wave < t_hi ? t_lo + wave : (t_lo < a.n_tiles ? t_lo : 0);
    fetch_k(t_first);

#pragma unroll
    for (int k = 0; k < VROUNDS; ++k) {
        const uint32_t i = threadIdx.x + 256u * k;
        const uint32_t e = (i / VCOP) & (VENT - 1);
        if (i < (uint32_t)(VENT * VCOP))
            s_vlut[i] = a.v_affine ? (uint32_t)f2h((float)(e & ((1u << VB) - 1u))) | ((uint32_t)f2h((float)(e >> VB)) << 16)
                                   : vla[k] | (vlb[k] << 16);
    }
#pragma unroll
    for (int i = threadIdx.x; i < 4 * 16 * 32 / 4; i += 256) ((u32x4_t*)(lds + LD::WX))[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (wave == 0) {
        // lane = RoPE block: q' = (rotated) q * log2(e)/sqrt(d) of heads 0..G-1 to LDS, then the
        // per-group sums of q' (lanes 0 .. 4G-1: head lane / 4, group lane % 4)
        float q0[G], q1[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            if (pin.dtype == BGTQ_F32) {
                q0[hh] = __builtin_bit_cast(float, pin.r0[hh]);
                q1[hh] = __builtin_bit_cast(float, pin.r1[hh]);
            } else if (pin.dtype == BGTQ_F16) {
                q0[hh] = h2f(pin.r0[hh] & 0xFFFFu);
                q1[hh] = h2f(pin.r0[hh] >> 16);
            } else {
                q0[hh] = bf2f(pin.r0[hh] & 0xFFFFu);
                q1[hh] = bf2f(pin.r0[hh] >> 16);
            }
        }
        if (a.k_rot) rotate_query<G>(q0, q1, a.k_rot + h * 16, lane);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            s_q[hh * 128 + 2 * lane] = q0[hh] * kLog2eOverSqrtD;
            s_q[hh * 128 + 2 * lane + 1] = q1[hh] * kLog2eOverSqrtD;
        }
        wave_lds_fence();
        if (lane < NG * G) {
            const float* qg = s_q + (lane / NG) * 128 + KG * (lane % NG);
            float acc = 0.f;
            for (int j = 0; j < KG; ++j) acc += qg[j];
            s_qsum[lane] = acc;
        }
    }
    __syncthreads();
    // A operands: lane = A row col (head 2 (col / 4) + (col / 2) % 2; fp16 high part for col even,
    // low part for col odd), lane row u = row: dims 32 ks + 8 row + {j, j + 4} in dword j
    u32x4_t qa[4];
    float qsg[2][NG];
    {
        const int qh = 2 * (col >> 2) + ((col >> 1) & 1), lo_part = col & 1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint32_t hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t e2[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float qv = qh < G ? s_q[qh * 128 + 32 * ks + 8 * row + j + 4 * c] : 0.f;
                    const _Float16 hi = (_Float16)qv;
                    const _Float16 lo = (_Float16)(qv - (float)hi);
                    e2[c] = (uint32_t)__builtin_bit_cast(uint16_t, lo_part ? lo : hi);
                }
                hv[j] = e2[0] | (e2[1] << 16);
            }
            qa[ks] = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) qsg[hh][gi] = 2 * row + hh < G ? s_qsum[(2 * row + hh) * NG + gi] : 0.f;
    }
    fetch_v(vn, t_first);

    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f}, zs[2] = {0.f, 0.f};
    f32x4_t o[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t lcopy = 4u * ((uint32_t)lane & (VLutGeom<VB>::COPIES - 1));
    const half2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};

    constexpr bool VDB = VB <= 3;
    auto tile = [&](const int64_t t, u32x4_t (&vcur)[VB], u32x4_t (&vnext)[VB]) __attribute__((always_inline)) {
        // value scales / zeros to LDS (transposed: token u at (u % 16) * 4 + u / 16)
        wave_lds_fence();
        {
            const int u0 = 2 * (lane & 31), reg = lane < 32 ? 0 : 64;
            sst[reg + (u0 & 15) * 4 + (u0 >> 4)] = (uint16_t)(vsd & 0xFFFFu);
            sst[reg + ((u0 + 1) & 15) * 4 + ((u0 + 1) >> 4)] = (uint16_t)(vsd >> 16);
        }
        // q·k on the matrix cores: the k-steps of a key group accumulate, then the group's scale
        // and zero apply
        float z[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) z[g][0] = z[g][1] = 0.f;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KPG; ++kk) {
                    const int ks = gi * KPG + kk;
                    const uint32_t x = kd[ks][g];
                    uint32_t e[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t pair = ((x >> (4 * j)) & 0x000F000Fu) | 0x64006400u;  // (1024 + n_j, 1024 + n_j+4)
                        e[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pair) - k1024);
                    }
                    d = mfma16(__builtin_bit_cast(half8_t, qa[ks]), as_h8(e[0], e[1], e[2], e[3]), d);
                }
                z[g][0] += kss[g][gi] * (d[0] + d[1]) + kzz[g][gi] * qsg[0][gi];
                z[g][1] += kss[g][gi] * (d[2] + d[3]) + kzz[g][gi] * qsg[1][gi];
            }
        }
        {
            // the keys of this tile are consumed: the next tile's go out (a wave's last tile
            // requests itself again, so that no branch joins the wait counts)
            const int64_t tn = t + 4 < t_hi ? t + 4 : t;
            fetch_k(tn);
            if constexpr (VDB) fetch_v(vnext, tn);
        }
        wave_lds_fence();
        float sv[4], sz[4] = {0.f, 0.f, 0.f, 0.f};
        {
            const uint2 v2 = *(const uint2*)(sst + col * 4);
            sv[0] = h2f(v2.x & 0xFFFFu); sv[1] = h2f(v2.x >> 16); sv[2] = h2f(v2.y & 0xFFFFu); sv[3] = h2f(v2.y >> 16);
            if (vaff) {
                const uint2 z2 = *(const uint2*)(sst + 64 + col * 4);
                sz[0] = h2f(z2.x & 0xFFFFu); sz[1] = h2f(z2.x >> 16); sz[2] = h2f(z2.y & 0xFFFFu); sz[3] = h2f(z2.y >> 16);
            }
        }
        if ((t + 1) * TILE > n_packed) {  // the sequence ends inside this tile
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (t * TILE + 16 * g + col >= n_packed) {
                    sv[g] = 0.f;
                    sz[g] = 0.f;
                    z[g][0] = z[g][1] = -INFINITY;
                }
            }
        }
        float tmax[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) tmax[hh] = vmax(vmax3(z[0][hh], z[1][hh], z[2][hh]), z[3][hh]);
        if (t == t_lo + wave) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) m[hh] = row_max16(tmax[hh]);
        } else if (__ballot(tmax[0] > m[0] || tmax[1] > m[1])) {
            float alpha[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float mn = vmax(m[hh], row_max16(tmax[hh]));
                alpha[hh] = __builtin_amdgcn_exp2f(m[hh] - mn);
                m[hh] = mn;
                l[hh] *= alpha[hh];
                zs[hh] *= alpha[hh];
            }
            wave_lds_fence();
            if (col == 0) {
                s_alpha[2 * row] = alpha[0];
                s_alpha[2 * row + 1] = alpha[1];
            }
            wave_lds_fence();
            const float al = s_alpha[col];
#pragma unroll
            for (int db = 0; db < 8; ++db) o[db] *= al;
        }
        uint16_t wh[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float p = __builtin_amdgcn_exp2f(z[g][hh] - m[hh]);
                l[hh] += p;
                if (vaff) zs[hh] += p * sz[g];
                wh[g][hh] = f2h(p * sv[g]);
            }
        }
        wave_lds_fence();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint32_t* wr = wx + (2 * row + hh) * 32 + col;
            wr[0] = (uint32_t)wh[0][hh] | ((uint32_t)wh[2][hh] << 16);
            wr[16] = (uint32_t)wh[1][hh] | ((uint32_t)wh[3][hh] << 16);
        }
        wave_lds_fence();
        uint32_t vs[4 * VB];
#pragma unroll
        for (int c = 0; c < VB; ++c) {
            vs[4 * c] = vcur[c][0]; vs[4 * c + 1] = vcur[c][1]; vs[4 * c + 2] = vcur[c][2]; vs[4 * c + 3] = vcur[c][3];
        }
        mx_pv<VB, 0>(o, vs, s_vlut, wx, lane, lcopy);
        mx_pv<VB, 1>(o, vs, s_vlut, wx, lane, lcopy);
        if constexpr (!VDB) {
            if (t + 4 < t_hi) fetch_v(vcur, t + 4);
        }
    };
    if constexpr (VDB) {
        for (int64_t t = t_lo + wave; t < t_hi; t += 8) {
            tile(t, vn, vx);
            if (t + 4 < t_hi) tile(t + 4, vx, vn);
        }
    } else {
        for (int64_t t = t_lo + wave; t < t_hi; t += 4) tile(t, vn, vn);
    }

    // Epilogue: row sums of l and the zero term, O^T to LDS, merge the waves.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        l[hh] = row_sum16(l[hh]);
        zs[hh] = row_sum16(zs[hh]);
    }
    __syncthreads();
    float* s_red = (float*)(lds + LD::RED);
    float* r = s_red + wave * G * PART;
    if (col < G) {
#pragma unroll
        for (int db = 0; db < 8; ++db) *(f32x4_t*)(r + col * PART + 16 * db + 4 * row) = o[db];
    }
    if (col == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int hd = 2 * row + hh;
            if (hd < G) {
                r[hd * PART + 128] = m[hh];
                r[hd * PART + 129] = l[hh];
                r[hd * PART + 130] = zs[hh];
            }
        }
    }
    __syncthreads();
    float* part = a.part + ((size_t)b * a.Hq + (size_t)h * G) * a.n_parts * PART;
    merge_waves4<G>(s_red, s_red + 4 * G * PART, part, a.n_parts, split);
}

// fp16 tiles: the unquantized comparator over [B][Hkv][N][128], and the fp16 recent ring of a packed
// cache (one split, concatenated order-free with the packed tokens).
template <int G>
__global__ __launch_bounds__(256, 2) void k_decode_fp16(const Fp16Args a) {
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __shared__ uint16_t s_w[4][64 * G];
    __shared__ float s_red[4 * G * PART + 4 * G];  // wave records, then merge scale factors
    const size_t bh = (size_t)b * a.Hkv + h;
    __shared__ float s_qp[128 * G];
    if (wave == 0)
        prep_wave<G, false, 0>(a.q, a.q_dtype, nullptr, nullptr, b, h, a.Hq, lane, s_qp, nullptr, nullptr, nullptr);
    __syncthreads();
    float qv[8 * G];
    load_qv_lds<G>(qv, s_qp, lane);
    WaveState<G> st;
    state_init<G>(st);
    const int64_t n = a.n_valid[b];
    const int64_t n_tiles = (n + TILE - 1) / TILE;
    const int64_t t_lo = (int64_t)split * a.tiles_per_split;
    const int64_t t_hi = t_lo + a.tiles_per_split < n_tiles ? t_lo + a.tiles_per_split : n_tiles;
    fp16_tiles<G>(st, a.k16 + bh * a.rows * D, a.v16 + bh * a.rows * D, n, t_lo, t_hi, wave, qv, s_w[wave], lane);
    __syncthreads();
    float* part = a.part + ((size_t)b * a.Hq + (size_t)h * G) * a.n_parts * PART;
    write_partial<G>(st, s_red, part, a.n_parts, a.split0 + split, wave, lane);
}

// Matrix-core decode over fp16 rows [n][128] of one (b, h), for 4 or 8 query heads per kv head
// (the unquantized comparator, and the fp16 recent ring of a packed cache).  Same split-K
// structure, softmax and wave merge as the packed matrix-core kernel; only the operands differ:
//  * q·k: A = Q' (row 4u + e: head 2u + e/2, the fp16 high part of q * log2(e)/sqrt(d) for e
//    even, the low part for e odd), built per lane in registers; B = K^T straight from HBM: lane
//    (token column n, lane row u) of k-step ks loads the 16 bytes of dims 32 ks + 8u .. 8u + 7 of
//    its token, which is exactly its B operand (one instruction reads 16 whole 64-byte segments).
//  * P·V: A = V^T from the tile staged in LDS.  A 4-byte read gives two adjacent dims of one
//    token; the even dims feed one product and the odd dims another, so lane (i, u) of dim block
//    j reads dims 32 j + 2i, 32 j + 2i + 1 of the tokens (p, p + 32), p = 16 S + 4u + e.  The
//    tile is staged 32 tokens at a time (the two halves S), rows of 272 bytes: the 32 lanes of a
//    read then hit 32 distinct banks.  B = W through LDS in (p, p + 32) pair order.
constexpr int F16MX_VROW = 272;  // bytes per staged value row (256 + 16)
template <int G> struct F16MxLds {
    static constexpr int VST = 0;                               // per wave: 32 rows
    static constexpr int VST_W = 32 * F16MX_VROW;
    static constexpr int WX = VST + 4 * VST_W;                  // u32 [4 waves][16 heads][32 pairs]
    static constexpr int ALPHA = WX + 4 * 16 * 32 * 4;          // f32 [4 waves][16]
    static constexpr int RED = VST;                             // epilogue: f32 [4 G PART + 4 G]
    static constexpr int SIZE = cmax(ALPHA + 4 * 16 * 4, RED + 4 * (4 * G * PART + 4 * G));
};

template <int G>
__global__ __launch_bounds__(256, 2) void k_decode_fp16_mx(const Fp16Args a) {
    static_assert(G == 4 || G == 8, "matrix-core fp16 decode serves 4 or 8 query heads per kv head");
    using LD = F16MxLds<G>;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int row = lane >> 4, col = lane & 15;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LD::SIZE];
    uint8_t* vst = lds + LD::VST + wave * LD::VST_W;
    uint32_t* wx = (uint32_t*)(lds + LD::WX) + wave * 16 * 32;
    float* s_alpha = (float*)(lds + LD::ALPHA) + wave * 16;

    const size_t bh = (size_t)b * a.Hkv + h;
    const int64_t n = a.n_valid[b];
    const int64_t n_tiles = (n + TILE - 1) / TILE;
    const int64_t t_lo = (int64_t)split * a.tiles_per_split;
    const int64_t t_hi = t_lo + a.tiles_per_split < n_tiles ? t_lo + a.tiles_per_split : n_tiles;
    const uint16_t* K16 = a.k16 + bh * a.rows * D;
    const uint16_t* V16 = a.v16 + bh * a.rows * D;
    const int64_t last = n > 0 ? n - 1 : 0;  // rows past the end are never read: loads clamp to it

    // Tile loads (non-temporal: the rows are read once per step): kk[g][ks] is the B operand of
    // token group g, k-step ks; vv[k] is the 16 bytes at tile offset 1024 k + 16 lane (token
    // 4k + lane / 16, dims 8 (lane % 16) ..).
    u32x4_t kk[4][4], vv[16];
    // idle = true (a wave's prefetch past its last tile): every lane reads row 0, one cached row,
    // instead of a whole tile; the loads stay unconditional so that no branch joins the wait counts.
    auto fetch_k = [&](int64_t t, bool idle) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t tok = idle ? 0 : t * TILE + 16 * g + col;
            const u32x4_t* r = (const u32x4_t*)(K16 + (tok < last ? tok : last) * D);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kk[g][ks] = __builtin_nontemporal_load(r + 4 * ks + row);
        }
    };
    auto fetch_v = [&](int64_t t, bool idle) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t tok = idle ? 0 : t * TILE + 4 * k + row;
            vv[k] = __builtin_nontemporal_load((const u32x4_t*)(V16 + (tok < last ? tok : last) * D) + col);
        }
    };
    const int64_t t_first = t_lo + wave < t_hi ? t_lo + wave : (t_lo < n_tiles ? t_lo : 0);
    fetch_k(t_first, false);
    fetch_v(t_first, false);

    // Query operands (lane = A row col, lane row u = row): dims 32 ks + 8 row .. of head qh.
    u32x4_t qa[4];
    {
        const int qh = 2 * (col >> 2) + ((col >> 1) & 1), lo_part = col & 1;
        const int64_t qrow = ((int64_t)b * a.Hq + (int64_t)h * G + (qh < G ? qh : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float x[8];
            const int d0 = 32 * ks + 8 * row;
            if (a.q_dtype == BGTQ_F32) {
                const f32x4_t v0 = *(const f32x4_t*)((const float*)a.q + qrow + d0);
                const f32x4_t v1 = *(const f32x4_t*)((const float*)a.q + qrow + d0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) { x[j] = v0[j]; x[4 + j] = v1[j]; }
            } else {
                const u32x4_t v = *(const u32x4_t*)((const uint16_t*)a.q + qrow + d0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[2 * j] = a.q_dtype == BGTQ_F16 ? h2f(v[j] & 0xFFFFu) : bf2f(v[j] & 0xFFFFu);
                    x[2 * j + 1] = a.q_dtype == BGTQ_F16 ? h2f(v[j] >> 16) : bf2f(v[j] >> 16);
                }
            }
            uint32_t hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t e2[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const float qs = x[2 * j + c] * kLog2eOverSqrtD;
                    const _Float16 hi = (_Float16)qs;
                    const _Float16 lo = (_Float16)(qs - (float)hi);
                    e2[c] = qh < G ? (uint32_t)__builtin_bit_cast(uint16_t, lo_part ? lo : hi) : 0u;
                }
                hv[j] = e2[0] | (e2[1] << 16);
            }
            qa[ks] = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
        }
    }
    // W rows of absent heads stay zero
#pragma unroll
    for (int i = threadIdx.x; i < 4 * 16 * 32 / 4; i += 256) ((u32x4_t*)(lds + LD::WX))[i] = u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();

    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    f32x4_t o[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j][0] = o[j][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // value rows of half S: instruction k holds tokens 4k .. 4k + 3; half S holds tokens
    // 16 S .. 16 S + 15 (stage rows 0..15) and 32 + 16 S .. 47 + 16 S (rows 16..31)
    auto stage_half = [&](int S) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int tok = 4 * k + row;
            if (((tok >> 4) & 1) != S) continue;  // compile-time per k (row varies only inside a group of 4)
            const int srow = (tok & 15) + 16 * (tok >> 5);
            *(u32x4_t*)(vst + srow * F16MX_VROW + 16 * col) = vv[k];
        }
    };
    auto pv_half = [&](int S) __attribute__((always_inline)) {
        const u32x4_t wq = *(const u32x4_t*)(wx + col * 32 + 16 * S + 4 * row);
        const half8_t wb = __builtin_bit_cast(half8_t, wq);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t d0 = *(const uint32_t*)(vst + (4 * row + e) * F16MX_VROW + 4 * (16 * j + col));
                const uint32_t d1 = *(const uint32_t*)(vst + (16 + 4 * row + e) * F16MX_VROW + 4 * (16 * j + col));
                lo[e] = __builtin_amdgcn_perm(d1, d0, 0x05040100u);  // (V[p][2i], V[p+32][2i])
                hi[e] = __builtin_amdgcn_perm(d1, d0, 0x07060302u);  // (V[p][2i+1], V[p+32][2i+1])
            }
            o[j][0] = mfma16(as_h8(lo[0], lo[1], lo[2], lo[3]), wb, o[j][0]);
            o[j][1] = mfma16(as_h8(hi[0], hi[1], hi[2], hi[3]), wb, o[j][1]);
        }
    };

    for (int64_t t = t_lo + wave; t < t_hi; t += 4) {
        // q·k on the matrix cores
        f32x4_t c[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            c[g] = mfma16(__builtin_bit_cast(half8_t, qa[0]), __builtin_bit_cast(half8_t, kk[g][0]), f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int ks = 1; ks < 4; ++ks)
                c[g] = mfma16(__builtin_bit_cast(half8_t, qa[ks]), __builtin_bit_cast(half8_t, kk[g][ks]), c[g]);
        }
        // the keys of this tile are consumed: the next tile's go out
        const bool last_tile = t + 4 >= t_hi;
        const int64_t tn = last_tile ? t : t + 4;
        fetch_k(tn, last_tile);
        // first value half to LDS; the second stays in registers until the first is consumed
        wave_lds_fence();
        stage_half(0);

        // softmax over the tile: lane holds tokens 16g + col, heads 2row, 2row + 1
        float z[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const bool valid = t * TILE + 16 * g + col < n;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) z[g][hh] = valid ? c[g][2 * hh] + c[g][2 * hh + 1] : -INFINITY;
        }
        float tmax[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) tmax[hh] = vmax(vmax3(z[0][hh], z[1][hh], z[2][hh]), z[3][hh]);
        if (t == t_lo + wave) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) m[hh] = row_max16(tmax[hh]);
        } else if (__ballot(tmax[0] > m[0] || tmax[1] > m[1])) {
            float alpha[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float mn = vmax(m[hh], row_max16(tmax[hh]));
                alpha[hh] = __builtin_amdgcn_exp2f(m[hh] - mn);
                m[hh] = mn;
                l[hh] *= alpha[hh];
            }
            wave_lds_fence();
            if (col == 0) {
                s_alpha[2 * row] = alpha[0];
                s_alpha[2 * row + 1] = alpha[1];
            }
            wave_lds_fence();
            const float al = s_alpha[col];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o[j][0] *= al;
                o[j][1] *= al;
            }
        }
        uint16_t wh[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float p = __builtin_amdgcn_exp2f(z[g][hh] - m[hh]);
                l[hh] += p;
                wh[g][hh] = f2h(p);
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint32_t* wr = wx + (2 * row + hh) * 32 + col;
            wr[0] = (uint32_t)wh[0][hh] | ((uint32_t)wh[2][hh] << 16);
            wr[16] = (uint32_t)wh[1][hh] | ((uint32_t)wh[3][hh] << 16);
        }
        wave_lds_fence();
        pv_half(0);
        wave_lds_fence();
        stage_half(1);
        wave_lds_fence();
        fetch_v(tn, last_tile);  // the values of this tile are all staged
        pv_half(1);
    }

    // Epilogue: row sums of l, O^T to LDS (over the stages), merge the waves.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) l[hh] = row_sum16(l[hh]);
    __syncthreads();  // every wave is done with its stage
    float* s_red = (float*)(lds + LD::RED);
    float* r = s_red + wave * G * PART;
    if (col < G) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r[col * PART + 32 * j + 2 * (4 * row + e)] = o[j][0][e];
                r[col * PART + 32 * j + 2 * (4 * row + e) + 1] = o[j][1][e];
            }
    }
    if (col == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int hd = 2 * row + hh;
            if (hd < G) {
                r[hd * PART + 128] = m[hh];
                r[hd * PART + 129] = l[hh];
                r[hd * PART + 130] = 0.f;
            }
        }
    }
    __syncthreads();
    float* part = a.part + ((size_t)b * a.Hq + (size_t)h * G) * a.n_parts * PART;
    merge_waves4<G>(s_red, s_red + 4 * G * PART, part, a.n_parts, a.split0 + split);
}

// Sum / max over all 64 lanes, returned wave-uniform: DPP rotations within each row of 16, then
// row_bcast:15 and row_bcast:31 fold the rows into the last row, and lane 63 is read out.
__device__ __forceinline__ float wave_total_sum(float v) {
    v = row_sum16(v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_total_max(float v) {
    constexpr int NEG_INF = (int)0xFF800000u;
    v = row_max16(v);
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(NEG_INF, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(NEG_INF, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false)));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Split merge by log-sum-exp, one workgroup of four waves per (batch, query head) row; lane l holds
// dims 2l and 2l + 1.  Wave w folds chunks of CMB_CHUNK consecutive partials (chunks w, w + 4, ...):
// lanes 0..CMB_CHUNK-1 load the chunk's maxima and sums, and every lane loads the chunk's o rows
// (one coalesced 512-byte read per partial), all issued together; lane j computes the weight
// e^(m_j - M) of partial j and readlane broadcasts it to the products.  A split without tokens
// holds m = -inf, l = 0, o = 0 and weighs 0.  The four wave states merge through LDS.
//
// With WIN the merge also attends to the row's fp16 window (the packed cache's recent rows), wave
// w taking tokens 64 w .. 64 w + 63, then 256 further on, so the window costs no launch of its own:
// - q.k: lane (u, c) = (lane / 16, lane % 16) loads dims 32 ks + 8 u .. + 7 (ks = 0..3) of tokens
//   16 g + c (g = 0..3), so one instruction reads 64-byte row segments of 16 tokens; the lane's 32
//   query values are fp32 registers, and it sums its 32 dims for its 4 tokens in fp32.  Two
//   butterfly exchanges (lane ^ 32, then lane ^ 16) leave lane l with token l's whole product.
// - softmax over the block in the base-2 domain of the partials (q.k times log2(e)/sqrt(d));
// - P.V: lane l loads dims 2l, 2l + 1 of each token's value row (one coalesced 256-byte row per
//   instruction); the weights, fp32, are broadcast by readlane.
// The block's (m, l, o) folds into the wave's state as one more partial would.  A wave's first
// window block and its first chunk of partials are loaded together, before either is used.
constexpr int CMB_CHUNK = 32;
template <bool WIN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, WIN ? 2 : 4))) void k_combine(const CombineArgs a) {
    const int row = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: addresses stay scalar
    const float* pr = a.part + (size_t)row * a.n_parts * PART;
    float M = -INFINITY, L = 0.f, ox = 0.f, oy = 0.f;
    float2 ml, ov[CMB_CHUNK];
    // one chunk of partials from bs on (fewer than CMB_CHUNK at the end; none past it: every read
    // is then partial 0's, and weighs 0)
    auto chunk_count = [&](int bs) { return a.n_parts - bs < CMB_CHUNK ? a.n_parts - bs : CMB_CHUNK; };
    auto chunk_load = [&](int bs) {
        const int cnt = chunk_count(bs);
        const int b0 = cnt > 0 ? bs : 0;
        ml = *(const float2*)(pr + (size_t)(b0 + (lane < cnt ? lane : 0)) * PART + 128);
#pragma unroll
        for (int j = 0; j < CMB_CHUNK; ++j)
            ov[j] = *(const float2*)(pr + (size_t)(b0 + (j < cnt ? j : 0)) * PART + 2 * lane);
    };
    auto chunk_fold = [&](int bs) {
        const int cnt = chunk_count(bs);
        const float mj = lane < cnt ? ml.x : -INFINITY;
        const float mn = fmaxf(M, wave_total_max(mj));  // -inf while every split so far is empty
        const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
        const float f = mj == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mj - mn);
        L = L * fo + wave_total_sum(f * ml.y);
        ox *= fo;
        oy *= fo;
#pragma unroll
        for (int j = 0; j < CMB_CHUNK; ++j) {  // past cnt, f is 0 and ov[j] repeats the chunk's first row
            const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
            ox = fmaf(fj, ov[j].x, ox);
            oy = fmaf(fj, ov[j].y, oy);
        }
        M = mn;
    };
    if constexpr (!WIN) {
        for (int base = wave * CMB_CHUNK; base < a.n_parts; base += 4 * CMB_CHUNK) {
            chunk_load(base);
            chunk_fold(base);
        }
    } else {
        const int u = lane >> 4, c = lane & 15;
        const int b = row / a.Hq, h = (row % a.Hq) / a.G;
        const int wn = a.n_valid[b];
        const uint16_t* WK = a.k16 + ((size_t)b * a.Hkv + h) * a.rows * D;
        const uint16_t* WV = a.v16 + ((size_t)b * a.Hkv + h) * a.rows * D;
        u32x4_t wk[4][4];  // [g][ks]: dims 32 ks + 8 u .. of token 16 g + c
        uint32_t wv[64];   // dims 2 lane, 2 lane + 1 of token j
        // rows past the valid ones are never read: every index clamps to the last valid row (row 0
        // of the window, always allocated, when none is valid)
        auto win_load = [&](int t0) {
            const int last = wn > 0 ? wn - 1 : 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int tok = t0 + 16 * g + c < last ? t0 + 16 * g + c : last;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) wk[g][ks] = ((const u32x4_t*)(WK + (size_t)tok * D))[4 * ks + u];
            }
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                const int tok = t0 + j < last ? t0 + j : last;
                wv[j] = ((const uint32_t*)(WV + (size_t)tok * D))[lane];
            }
        };
        // the window block and the chunk of partials go out first, the query's raw bits last
        // (fp32: two 16-byte pieces per k-step; fp16/bf16: one); one wait then covers them all
        int base = wave * CMB_CHUNK;
        win_load(64 * wave);
        chunk_load(base);
        float wq[32];  // query dims 32 ks + 8 u + e at [8 ks + e]
        const size_t q0 = (size_t)row * D;
        if (a.q_dtype == BGTQ_F32) {
            // (loaded as float vectors and read by element: a bit cast of a vector element would
            // take the vector's first element)
            f32x4_t qf[8];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                qf[2 * ks] = *(const f32x4_t*)((const float*)a.q + q0 + 32 * ks + 8 * u);
                qf[2 * ks + 1] = *(const f32x4_t*)((const float*)a.q + q0 + 32 * ks + 8 * u + 4);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wq[8 * ks + e] = qf[2 * ks][e];
                    wq[8 * ks + 4 + e] = qf[2 * ks + 1][e];
                }
        } else {
            u32x4_t qr[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qr[ks] = *(const u32x4_t*)((const uint16_t*)a.q + q0 + 32 * ks + 8 * u);
            if (a.q_dtype == BGTQ_F16) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wq[8 * ks + 2 * e] = h2f(qr[ks][e] & 0xFFFFu);
                        wq[8 * ks + 2 * e + 1] = h2f(qr[ks][e] >> 16);
                    }
            } else {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wq[8 * ks + 2 * e] = bf2f(qr[ks][e] & 0xFFFFu);
                        wq[8 * ks + 2 * e + 1] = bf2f(qr[ks][e] >> 16);
                    }
            }
        }
        auto win_fold = [&](int t0) {
            float s[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float acc = 0.f;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc = fmaf(wq[8 * ks + 2 * e], h2f(wk[g][ks][e] & 0xFFFFu), acc);
                        acc = fmaf(wq[8 * ks + 2 * e + 1], h2f(wk[g][ks][e] >> 16), acc);
                    }
                s[g] = acc;
            }
            // lanes u and u ^ 2 sum groups {0, 1} (kept where u < 2) and {2, 3}; then lanes u and
            // u ^ 1 sum the group each keeps, u
            const bool hi = u >= 2, odd = u & 1;
            float t[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float send = hi ? s[i] : s[2 + i];
                t[i] = (hi ? s[2 + i] : s[i]) + __shfl_xor(send, 32, 64);
            }
            const float zs = (odd ? t[1] : t[0]) + __shfl_xor(odd ? t[0] : t[1], 16, 64);
            const float z = t0 + lane < wn ? zs * kLog2eOverSqrtD : -INFINITY;
            const float mw = wave_total_max(z);
            const float p = z == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z - mw);
            const float lw = wave_total_sum(p);
            float wx = 0.f, wy = 0.f;
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), j));
                wx = fmaf(pj, h2f(wv[j] & 0xFFFFu), wx);
                wy = fmaf(pj, h2f(wv[j] >> 16), wy);
            }
            const float mn = fmaxf(M, mw);
            const float fo = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mn);
            const float fw = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mn);
            L = L * fo + lw * fw;
            ox = ox * fo + wx * fw;
            oy = oy * fo + wy * fw;
            M = mn;
        };
        chunk_fold(base);
        for (base += 4 * CMB_CHUNK; base < a.n_parts; base += 4 * CMB_CHUNK) {
            chunk_load(base);
            chunk_fold(base);
        }
        win_fold(64 * wave);
        for (int t0 = 64 * wave + 256; t0 < wn; t0 += 256) {
            win_load(t0);
            win_fold(t0);
        }
    }
    __shared__ float s_m[4], s_l[4];
    __shared__ float2 s_o[4][64];
    if (lane == 0) {
        s_m[wave] = M;
        s_l[wave] = L;
    }
    s_o[wave][lane] = float2{ox, oy};
    __syncthreads();
    if (wave == 0) {
        const float Mt = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
        float Lt = 0.f, rx = 0.f, ry = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = s_m[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w] - Mt);
            Lt += f * s_l[w];
            rx += f * s_o[w][lane].x;
            ry += f * s_o[w][lane].y;
        }
        const float inv = 1.f / Lt;
        float o0 = rx * inv, o1 = ry * inv;
        if (a.v_rot) {
            // values stored as H (s * v) / 16: the output is rotated back once, o = s * (H o') / 8
            // (lane holds dims 2 lane and 2 lane + 1: stage 1 inside the lane, stages 2..64 with
            // lane ^ m, the lower lane keeping a + b, the upper one a - b)
            const int hq = row % a.Hq;
            const uint32_t sb = (uint32_t)a.v_rot[(hq / a.G) * 16 + (lane >> 2)] >> (2 * (lane & 3));
            float u = o0 + o1, v = o0 - o1;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float pu = __shfl_xor(u, m, 64), pv = __shfl_xor(v, m, 64);
                const bool upper = (lane & m) != 0;
                u = upper ? pu - u : u + pu;
                v = upper ? pv - v : v + pv;
            }
            o0 = (sb & 1u) ? -(u * 0.125f) : u * 0.125f;
            o1 = (sb & 2u) ? -(v * 0.125f) : v * 0.125f;
        }
        *(float2*)(a.out + (size_t)row * D + 2 * lane) = float2{o0, o1};
    }
}

// Calibration energy sums in fp64: out[h][i] = (sum_t |k_t,blk i|^2, sum_{t,g} |q_t,g,blk i|^2).
// Grid (kv head, token chunk): chunk c sums tokens [c*tc, (c+1)*tc) into out[c][h][i] (fp64);
// the host adds the chunks in order, so the sums are deterministic for a given chunk count.
__global__ __launch_bounds__(256) void k_energy(const EnergyArgs a) {
    const int h = blockIdx.x, chunk = blockIdx.y, blk = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int Hq = a.Hkv * a.G;
    const int64_t t0 = (int64_t)chunk * a.tc, t1 = t0 + a.tc < a.T ? t0 + a.tc : a.T;
    double ek = 0.0, eq = 0.0;
    for (int64_t t = t0 + part; t < t1; t += 4) {
        const int64_t kb = (t * a.Hkv + h) * D + 2 * blk;
        const double k0 = load_act(a.k, kb, a.dtype), k1 = load_act(a.k, kb + 1, a.dtype);
        ek += k0 * k0 + k1 * k1;
        for (int g = 0; g < a.G; ++g) {
            const int64_t qb = (t * Hq + (int64_t)h * a.G + g) * D + 2 * blk;
            const double q0 = load_act(a.q, qb, a.dtype), q1 = load_act(a.q, qb + 1, a.dtype);
            eq += q0 * q0 + q1 * q1;
        }
    }
    __shared__ double s_e[4][64][2];
    s_e[part][blk][0] = ek;
    s_e[part][blk][1] = eq;
    __syncthreads();
    if (part == 0) {
        double sk = 0.0, sq = 0.0;
        for (int p = 0; p < 4; ++p) {
            sk += s_e[p][blk][0];
            sq += s_e[p][blk][1];
        }
        double* o = a.out + (((size_t)chunk * a.Hkv + h) * 64 + blk) * 2;
        o[0] = sk;
        o[1] = sq;
    }
}


// ---------------------------------------------------------------------------------------------
// Quantize-append.  The float32 steps are spelled out one IEEE operation at a time (no
// contraction) so the codes and fp16 scales are reproducible bit for bit (tq_code and the
// wave-wide row helpers are in bgtq_device.h).
// One token's row in LDS, in the activation's own format (fp32, or the fp16 / bf16 bits, which
// convert to fp32 exactly).
template <typename XT> struct XRow {
    const XT* p;
    int dtype;
    __device__ __forceinline__ float operator[](int j) const {
        if constexpr (sizeof(XT) == 4) return p[j];
        else return dtype == BGTQ_F16 ? h2f(p[j]) : bf2f(p[j]);
    }
    __device__ __forceinline__ XRow operator+(int j) const { return XRow{p + j, dtype}; }
};

template <typename X>
__device__ __forceinline__ float rms_scale16(const X& x /*one token's row*/, const float* r /*per block or null*/,
                                             uint16_t* s16) {
#pragma clang fp contract(off)
    float acc = 0.f;
    for (int j = 0; j < D; ++j) {
        const float u = r ? x[j] * r[j >> 1] : x[j];
        acc = acc + u * u;
    }
    const float ms = acc / 128.0f;
    const uint16_t h = f2h(sqrtf(ms));
    *s16 = h;
    return h2f(h);
}

// Value codes of one token (codebook width VB): the thresholds scaled by the token's scale are
// formed once (the same fp32 products the search forms), and each code is the number of them at
// or below the coordinate, which is the search's result since the products ascend (S >= 0).  The
// 128 codes collect in registers, one byte each, and are stored after every element is read.
template <int VB, typename X>
__device__ __forceinline__ void v_codes_row(const X& x, float S, bool active, uint8_t* cr, const float* thr) {
    constexpr int NT = (1 << VB) - 1;
    float th[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma clang fp contract(off)
        th[m] = S * thr[thr_base(VB) + m];
    }
    uint32_t pk[D / 4];
#pragma unroll
    for (int k = 0; k < D / 4; ++k) pk[k] = 0u;
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const float v = x[j];
        uint32_t c = 0;
#pragma unroll
        for (int m = 0; m < NT; ++m) c += v >= th[m] ? 1u : 0u;
        pk[j >> 2] |= c << (8 * (j & 3));
    }
    uint32_t* dst = (uint32_t*)cr;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) dst[k] = active ? pk[k] : 0u;
}

template <typename X>
__device__ __forceinline__ void affine_group(const X& x, int n, int bits, uint16_t* sc16, uint16_t* z16,
                                             uint32_t* codes) {
#pragma clang fp contract(off)
    float mn = x[0], mx = x[0];
    for (int j = 1; j < n; ++j) {
        mn = fminf(mn, x[j]);
        mx = fmaxf(mx, x[j]);
    }
    const float range = mx - mn;
    const float scale = range / (float)((1 << bits) - 1);
    const uint16_t s16 = f2h(scale), zz = f2h(mn);
    *sc16 = s16;
    *z16 = zz;
    const float s32 = h2f(s16), z32 = h2f(zz);
    const float top = (float)((1 << bits) - 1);
    for (int j = 0; j < n; ++j) {
        float c = 0.f;
        if (s32 != 0.f) {
            const float q = (x[j] - z32) / s32;
            c = fminf(fmaxf(rintf(q), 0.f), top);
        }
        codes[j] = (uint32_t)c;
    }
}

// One workgroup = one tile of 64 positions of one (b, h); lane = token for the per-token steps.
// The tile's rows are first staged in LDS by the whole wave: with 16-byte aligned rows
// (QuantArgs::vec16) each instruction moves whole 64-byte row segments, otherwise one element
// per lane and instruction.  Rows are kept in the activation's format (XT = float for fp32,
// uint16_t bits for fp16 / bf16), padded to an odd number of dwords so that the per-lane row
// reads of the quantizer hit distinct banks.  Value codes overwrite their own row in place (code
// j lands in bytes the row's elements 0..j already vacated).
// ROT: affine keys and / or values stored rotated, y = H (s * x) / 16 (s from QuantArgs::k_rot,
// v_rot): the row is rotated in registers by the fast transform (stages 1, 2, ..., 64, one fp32
// addition or subtraction per output, the final 1/16 exact) and staged as fp32 for the quantizer.
template <typename XT, bool ROT>
__global__ __launch_bounds__(64) void k_quant(const QuantArgs a) {
    constexpr int XS = sizeof(XT) == 4 ? D + 1 : D + 2;  // row stride in elements (129 dwords / 65 dwords)
    constexpr int EPC = 16 / sizeof(XT);                 // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                         // chunks per row
    const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int64_t tile = a.tile0[b] + blockIdx.x;
    if (tile * TILE >= a.pos_hi[b]) return;  // whole workgroup beyond this sequence's range
    const int64_t pos = tile * TILE + lane;
    const bool active = pos >= a.pos_lo[b] && pos < a.pos_hi[b];
    __shared__ float s_thr[BGTQ_CB_THRESHOLDS];
    __shared__ __attribute__((aligned(16))) XT s_x[64 * XS];
    __shared__ float s_y[ROT ? 64 * (D + 1) : 1];  // rotated rows (ROT only)
    __shared__ int s_order[64];
    __shared__ int s_wid[64];
    __shared__ float s_r[64], s_sig[64];
    for (int i = lane; i < BGTQ_CB_THRESHOLDS; i += 64) s_thr[i] = __builtin_bit_cast(float, c_thr32[i]);
    const size_t bh = (size_t)b * a.Hkv + h;
    const bool do_k = a.which & 1, do_v = (a.which >> 1) & 1;
    int nnz = 0;
    if (do_k && a.k_mode == BGTQ_K_BLOCKGTQ) {
        const int w = a.bits[h * 64 + lane] < 8 ? a.bits[h * 64 + lane] : 8;  // widths above 8 are invalid; clamp
        s_wid[lane] = w;
        s_r[lane] = a.inv_sigma[h * 64 + lane];
        s_sig[lane] = a.sigma[h * 64 + lane];
        __syncthreads();
        int rank = 0;
        for (int j = 0; j < 64; ++j) {
            const int wj = s_wid[j];
            rank += wj > w || (wj == w && j < lane);
            nnz += wj > 0;
        }
        if (w > 0) s_order[rank] = lane;
    }
    __syncthreads();
    // source element offset of the row of tile position u (inactive positions read nothing)
    auto row_base = [&](int u, bool& act) -> int64_t {
        const int64_t p = tile * TILE + u;
        act = p >= a.pos_lo[b] && p < a.pos_hi[b];
        int64_t row = 0;
        if (act) {
            if (a.gather) {
                row = a.gather[b * a.gather_stride + (p - a.pos_lo[b])];
            } else {
                row = p - a.off[b];
                if (a.mod_n) row %= a.mod_n;
            }
        }
        return (int64_t)b * a.sB + row * a.sT + (int64_t)h * a.sH;
    };
    for (int pass = 0; pass < 2; ++pass) {
        if ((pass == 0 && !do_k) || (pass == 1 && !do_v)) continue;
        const void* src = pass == 0 ? a.src_k : a.src_v;
        __syncthreads();  // the previous pass is done with the rows
        if (a.vec16) {
            // 16-byte chunks: instruction k covers rows (64 / CPR) * k + lane / CPR; every load of
            // the pass is issued before the first LDS write, one round trip for the tile's rows
            // (non-temporal, as the key records below: each is touched once here)
            u32x4_t ld[CPR];
#pragma unroll
            for (int k = 0; k < CPR; ++k) {
                const int u = (64 / CPR) * k + lane / CPR, c = lane % CPR;
                bool act;
                const int64_t off = row_base(u, act);
                ld[k] = u32x4_t{0u, 0u, 0u, 0u};
                if (act) ld[k] = __builtin_nontemporal_load((const u32x4_t*)((const XT*)src + off + EPC * c));
            }
#pragma unroll
            for (int k = 0; k < CPR; ++k) {
                const int u = (64 / CPR) * k + lane / CPR, c = lane % CPR;
                const u32x4_t v = ld[k];
                uint32_t* dst = (uint32_t*)(s_x + u * XS + EPC * c);
                dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
            }
        } else {
            // one element per lane: instruction j covers element j of every row
            bool act;
            const int64_t off = row_base(lane, act);
            for (int j = 0; j < D; ++j) {
                XT v = 0;
                if (act) v = ((const XT*)src)[off + j];
                s_x[lane * XS + j] = v;
            }
        }
        int xdt = a.dtype;
        if (a.round16) {
            // rows as the fp16 store holds them: each lane rounds its own row in place
            __syncthreads();
            XT* r = s_x + lane * XS;
            for (int j = 0; j < D; ++j) {
                if constexpr (sizeof(XT) == 4) {
                    r[j] = h2f(f2h(r[j]));
                } else {
                    const float f = a.dtype == BGTQ_F16 ? h2f(r[j]) : bf2f(r[j]);
                    r[j] = f2h(f);
                }
            }
            if constexpr (sizeof(XT) == 2) xdt = BGTQ_F16;
        }
        __syncthreads();
        const XRow<XT> x{s_x + lane * XS, xdt};
        // The row rotated to y = H (s * x) / 16 (fast transform: stages 1, 2, ..., 64, one fp32
        // addition or subtraction per output, the 1/16 exact), staged as fp32 in this lane's row of
        // s_y; sg: the (layer, kv head)'s sign bits.
        auto rotate_row = [&](const uint8_t* sg) -> const float* {
            float y[D];
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const float v = x[j];
                y[j] = ((sg[j >> 3] >> (j & 7)) & 1u) ? -v : v;
            }
#pragma unroll
            for (int hs = 1; hs < D; hs <<= 1) {
#pragma unroll
                for (int i0 = 0; i0 < D; i0 += 2 * hs) {
#pragma unroll
                    for (int j = i0; j < i0 + hs; ++j) {
#pragma clang fp contract(off)
                        const float p = y[j], r = y[j + hs];
                        y[j] = p + r;
                        y[j + hs] = p - r;
                    }
                }
            }
            float* yr = s_y + lane * (D + 1);
#pragma unroll
            for (int j = 0; j < D; ++j) yr[j] = y[j] * 0.0625f;
            return yr;
        };
        if (pass == 0) {
            // ---- keys
            uint32_t* kt = (uint32_t*)(a.k_codes + (bh * a.n_tiles + tile) * a.k_tile_bytes);
            if (a.k_mode == BGTQ_K_BLOCKGTQ) {
                uint16_t s16;
                const float S = rms_scale16(x, s_r, &s16);
                uint64_t buf = 0;
                int nb = 0, k = 0;
                // the slots' threshold searches are independent: unrolled so that they interleave
#pragma unroll 4
                for (int s = 0; s < nnz; ++s) {
                    const int i = s_order[s], w = s_wid[i];
                    float t;
                    {
#pragma clang fp contract(off)
                        t = S * s_sig[i];
                    }
                    const uint32_t ca = tq_code(x[2 * i], t, w, s_thr);
                    const uint32_t cb = tq_code(x[2 * i + 1], t, w, s_thr);
                    buf |= (uint64_t)(ca | (cb << w)) << nb;
                    nb += 2 * w;
                    if (nb >= 32) {
                        // widths summing past the budget (invalid metadata) never write past the record
                        if (active && k < a.R) __builtin_nontemporal_store((uint32_t)buf, kt + k * TILE + lane);
                        buf >>= 32;
                        nb -= 32;
                        ++k;
                    }
                }
                if (active) a.k_scale[bh * a.n_cap + pos] = s16;
            } else {
                const int ng = D / a.k_group;
                uint32_t codes[D];
                auto groups = [&](const auto& xr) {
                    for (int gi = 0; gi < ng; ++gi) {
                        uint16_t sc, zz;
                        affine_group(xr + gi * a.k_group, a.k_group, a.k_bits, &sc, &zz, codes + gi * a.k_group);
                        if (active) {
                            a.k_scale[(bh * a.n_cap + pos) * ng + gi] = sc;
                            a.k_zero[(bh * a.n_cap + pos) * ng + gi] = zz;
                        }
                    }
                };
                if constexpr (ROT) {
                    if (a.k_rot) groups(XRow<float>{rotate_row(a.k_rot + h * 16), BGTQ_F32});
                    else groups(x);
                } else {
                    groups(x);
                }
                const int per = 32 / a.k_bits;
                for (int k = 0; k < a.R; ++k) {
                    uint32_t wv = 0;
                    for (int u = 0; u < per; ++u) wv |= codes[k * per + u] << (u * a.k_bits);
                    if (active) kt[k * TILE + lane] = wv;
                }
            }
        } else {
            // ---- values: lane-stream layout.  Codes of the 64 tokens go through LDS (over their own
            // rows); thread L then assembles stream L (4*vb dwords).  Bits of tokens before pos_lo
            // are kept (read-modify-write); tokens at or past pos_hi get zero codes (never written
            // before, appends are in order).
            const int vb = a.v_bits;
            uint16_t s16 = 0, z16 = 0;
            uint8_t* cr = (uint8_t*)(s_x + lane * XS);
            auto vquant = [&](const auto& xr) {
                if (a.v_mode == BGTQ_V_CODEBOOK) {
                    const float S = rms_scale16(xr, nullptr, &s16);
                    switch (vb) {
                        case 1: v_codes_row<1>(xr, S, active, cr, s_thr); break;
                        case 2: v_codes_row<2>(xr, S, active, cr, s_thr); break;
                        case 3: v_codes_row<3>(xr, S, active, cr, s_thr); break;
                        default: v_codes_row<4>(xr, S, active, cr, s_thr); break;
                    }
                } else {
                    uint32_t codes[D];
                    affine_group(xr, D, vb, &s16, &z16, codes);
                    for (int j = 0; j < D; ++j) cr[j] = active ? (uint8_t)codes[j] : (uint8_t)0;
                }
            };
            if constexpr (ROT) {
                if (a.v_rot) vquant(XRow<float>{rotate_row(a.v_rot + h * 16), BGTQ_F32});
                else vquant(x);
            } else {
                vquant(x);
            }
            if (active) {
                a.v_scale[bh * a.n_cap + pos] = s16;
                if (a.v_mode == BGTQ_V_AFFINE) a.v_zero[bh * a.n_cap + pos] = z16;
            }
            __syncthreads();
            auto code_at = [&](int p, int dim) -> uint32_t { return ((const uint8_t*)(s_x + p * XS))[dim]; };
            const int64_t t0 = tile * TILE;
            const int lo = a.pos_lo[b] > t0 ? (int)(a.pos_lo[b] - t0) : 0;
            const int dd = lane & 15, jj = lane >> 4;
            const uint32_t cm = (1u << vb) - 1u;
            uint32_t* vt = (uint32_t*)(a.v_codes + (bh * a.n_tiles + tile) * a.v_tile_bytes);
            for (int c = 0; c < 4 * vb; ++c) {
                uint64_t val = 0, msk = 0;
                const int phi0 = (32 * c) / (2 * vb), phi1 = (32 * c + 31) / (2 * vb);
                for (int phi = phi0; phi <= phi1 && phi < 64; ++phi) {
                    const int m = phi & 3, db = (phi >> 2) & 7, sh = phi >> 5;
                    const int p = 16 * sh + 4 * jj + m, dim = 16 * db + dd;
                    const uint64_t f = (uint64_t)(code_at(p, dim) | (code_at(p + 32, dim) << vb));
                    const uint64_t fm = (uint64_t)((p >= lo ? cm : 0u) | (p + 32 >= lo ? cm << vb : 0u));
                    const int bit = 2 * vb * phi - 32 * c;   // field position relative to dword c
                    if (bit >= 0) {
                        val |= f << bit;
                        msk |= fm << bit;
                    } else {
                        val |= f >> -bit;
                        msk |= fm >> -bit;
                    }
                }
                const uint32_t v32 = (uint32_t)val, m32 = (uint32_t)msk;
                uint32_t* dst = vt + ((c >> 2) * 64 + lane) * 4 + (c & 3);
                if (m32 == 0xFFFFFFFFu) *dst = v32;
                else if (m32) *dst = (*dst & ~m32) | (v32 & m32);
            }
        }
    }
}

// Quantize-append of a few tokens: one workgroup of NW waves per (tile, kv head, sequence); wave w
// takes the tile's new tokens w, w + NW, ... one after another, the whole wave on each token
// (lane i holds RoPE block i, dims 2i and 2i+1), so one new token costs a few short chains instead
// of one lane's full sequential pass, and NW tokens run at once.  Every float step is the one k_quant takes (rows convert to fp32 exactly from
// all three activation formats): the same scale sum in the same order, the same threshold
// products and searches, the same affine min/max order.  Key records and value streams
// are assembled in LDS (atomicOr of each lane's fields: a record per wave, the tile's value streams
// shared) and written once; value dwords keep the bits of other positions (read-modify-write by
// wave 0 at the end; the tile belongs to this workgroup alone).
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_append(const QuantArgs a) {
    const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile = a.tile0[b] + blockIdx.x;
    const int64_t t0 = tile * TILE;
    if (t0 >= a.pos_hi[b]) return;  // whole workgroup beyond this sequence's range
    const int u_lo = a.pos_lo[b] > t0 ? (int)(a.pos_lo[b] - t0) : 0;
    const int u_hi = a.pos_hi[b] - t0 < TILE ? (int)(a.pos_hi[b] - t0) : TILE;
    const size_t bh = (size_t)b * a.Hkv + h;
    const bool do_k = a.which & 1, do_v = (a.which >> 1) & 1;
    const int vb = a.v_bits;
    // Every load the first token needs is issued here, before the first barrier, so that one
    // memory round trip covers the rows, this lane's value-stream dwords, the metadata and the
    // thresholds (the tile's value dwords are this workgroup's alone until it ends).
    auto row_src = [&](int u) -> int64_t {
        int64_t row;
        if (a.gather) {
            row = a.gather[b * a.gather_stride + (t0 + u - a.pos_lo[b])];
        } else {
            row = t0 + u - a.off[b];
            if (a.mod_n) row %= a.mod_n;
        }
        return (int64_t)b * a.sB + row * a.sT + (int64_t)h * a.sH + 2 * lane;
    };
    float kx0 = 0.f, kx1 = 0.f, vx0 = 0.f, vx1 = 0.f;
    auto r16 = [&](float x) { return a.round16 ? h2f(f2h(x)) : x; };  // as the fp16 store holds it
    auto load_rows = [&](int u) {
        const int64_t src = row_src(u);
        if (do_k) {
            kx0 = r16(load_act(a.src_k, src, a.dtype));
            kx1 = r16(load_act(a.src_k, src + 1, a.dtype));
        }
        if (do_v) {
            vx0 = r16(load_act(a.src_v, src, a.dtype));
            vx1 = r16(load_act(a.src_v, src + 1, a.dtype));
        }
    };
    if (u_lo + wave < u_hi) load_rows(u_lo + wave);
    uint32_t* vt = (uint32_t*)(a.v_codes + (bh * a.n_tiles + tile) * a.v_tile_bytes);
    uint32_t old[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
        old[c] = (wave == 0 && do_v && c < 4 * vb) ? vt[((c >> 2) * 64 + lane) * 4 + (c & 3)] : 0u;
    __shared__ float s_thr[BGTQ_CB_THRESHOLDS];
    __shared__ uint32_t s_recs[NW][32];
    __shared__ uint32_t s_vv[64 * 16], s_vm[64 * 16];  // value streams of the tile: bits and written mask
    uint32_t* s_rec = s_recs[wave];
    for (int i = threadIdx.x; i < BGTQ_CB_THRESHOLDS; i += 64 * NW) s_thr[i] = __builtin_bit_cast(float, c_thr32[i]);
    for (int i = threadIdx.x; i < 64 * 16; i += 64 * NW) s_vv[i] = s_vm[i] = 0u;
    if (lane < 32) s_rec[lane] = 0u;
    const bool gtq = a.k_mode == BGTQ_K_BLOCKGTQ;
    int w = 0, off = 0;  // this lane's block: width and bit offset in the key record
    float r_blk = 1.f, sig_blk = 1.f;
    if (do_k && gtq) {
        w = a.bits[h * 64 + lane] < 8 ? a.bits[h * 64 + lane] : 8;  // widths above 8 are invalid; clamp
        r_blk = a.inv_sigma[h * 64 + lane];
        sig_blk = a.sigma[h * 64 + lane];
        // slots in descending width, ties by block index: the fields stored before this one
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            const int wj = __builtin_amdgcn_readlane(w, j);
            off += (wj > w || (wj == w && j < lane)) ? 2 * wj : 0;
        }
    }
    __syncthreads();
    for (int u = u_lo + wave; u < u_hi; u += NW) {
        const int64_t pos = t0 + u;
        if (u > u_lo + wave) load_rows(u);
        for (int pass = 0; pass < 2; ++pass) {
            if ((pass == 0 && !do_k) || (pass == 1 && !do_v)) continue;
            const float x0 = pass == 0 ? kx0 : vx0, x1 = pass == 0 ? kx1 : vx1;
            wave_lds_fence();  // the wave's previous token or pass is done with its record
            if (pass == 0) {
                uint32_t* kt = (uint32_t*)(a.k_codes + (bh * a.n_tiles + tile) * a.k_tile_bytes);
                if (gtq) {
                    uint16_t s16;
                    const float S = wave_rms16(x0, x1, r_blk, true, &s16);
                    if (w > 0) {
                        float t;
                        {
#pragma clang fp contract(off)
                            t = S * sig_blk;
                        }
                        const uint32_t f = tq_code(x0, t, w, s_thr) | (tq_code(x1, t, w, s_thr) << w);
                        const int k = off >> 5, sh = off & 31;
                        if (k < a.R) atomicOr(&s_rec[k], f << sh);
                        if (sh + 2 * w > 32 && k + 1 < a.R) atomicOr(&s_rec[k + 1], f >> (32 - sh));
                    }
                    if (lane == 0) a.k_scale[bh * a.n_cap + pos] = s16;
                } else {
#pragma clang fp contract(off)
                    const int kg = a.k_group, gi = (2 * lane) / kg, ng = D / kg;
                    float mn = 0.f, mx = 0.f;
                    for (int g2 = 0; g2 < ng; ++g2) {  // every group on every lane; keep this lane's
                        float gmn, gmx;
                        wave_minmax(x0, x1, g2 * kg, kg, gmn, gmx);
                        if (g2 == gi) {
                            mn = gmn;
                            mx = gmx;
                        }
                    }
                    const float scale = (mx - mn) / (float)((1 << a.k_bits) - 1);
                    const uint16_t sc16 = f2h(scale), zz16 = f2h(mn);
                    const float s32 = h2f(sc16), z32 = h2f(zz16), top = (float)((1 << a.k_bits) - 1);
                    float c0 = 0.f, c1 = 0.f;
                    if (s32 != 0.f) {
                        c0 = fminf(fmaxf(rintf((x0 - z32) / s32), 0.f), top);
                        c1 = fminf(fmaxf(rintf((x1 - z32) / s32), 0.f), top);
                    }
                    const int per = 32 / a.k_bits, sh = ((2 * lane) % per) * a.k_bits;
                    atomicOr(&s_rec[(2 * lane) / per], ((uint32_t)c0 << sh) | ((uint32_t)c1 << (sh + a.k_bits)));
                    if ((2 * lane) % kg == 0) {
                        a.k_scale[(bh * a.n_cap + pos) * ng + gi] = sc16;
                        a.k_zero[(bh * a.n_cap + pos) * ng + gi] = zz16;
                    }
                }
                wave_lds_fence();
                if (lane < a.R) {
                    kt[lane * TILE + u] = s_rec[lane];
                    s_rec[lane] = 0u;
                }
            } else {
                uint32_t c0, c1;
                uint16_t s16 = 0, z16 = 0;
                if (a.v_mode == BGTQ_V_CODEBOOK) {
                    const float S = wave_rms16(x0, x1, 1.f, false, &s16);
                    c0 = c1 = 0u;
                    for (int m = 0; m < (1 << vb) - 1; ++m) {
                        float th;
                        {
#pragma clang fp contract(off)
                            th = S * s_thr[thr_base(vb) + m];
                        }
                        c0 += x0 >= th ? 1u : 0u;
                        c1 += x1 >= th ? 1u : 0u;
                    }
                } else {
#pragma clang fp contract(off)
                    float mn, mx;
                    wave_minmax(x0, x1, 0, D, mn, mx);
                    const float scale = (mx - mn) / (float)((1 << vb) - 1);
                    s16 = f2h(scale);
                    z16 = f2h(mn);
                    const float s32 = h2f(s16), z32 = h2f(z16), top = (float)((1 << vb) - 1);
                    float f0 = 0.f, f1 = 0.f;
                    if (s32 != 0.f) {
                        f0 = fminf(fmaxf(rintf((x0 - z32) / s32), 0.f), top);
                        f1 = fminf(fmaxf(rintf((x1 - z32) / s32), 0.f), top);
                    }
                    c0 = (uint32_t)f0;
                    c1 = (uint32_t)f1;
                }
                if (lane == 0) {
                    a.v_scale[bh * a.n_cap + pos] = s16;
                    if (a.v_mode == BGTQ_V_AFFINE) a.v_zero[bh * a.n_cap + pos] = z16;
                }
                // lane-stream position of (token u, dim): stream dd + 16*jj, pair field phi, the
                // token's half of it chosen by u >= 32 (the layout k_quant assembles per stream)
                const int p = u & 31, hi = u >> 5;
                const int sh = p >> 4, jj = (p >> 2) & 3, m = p & 3;
                const uint32_t cm = (1u << vb) - 1u;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int dim = 2 * lane + e;
                    const int L = (dim & 15) + 16 * jj, phi = m + 4 * (dim >> 4) + 32 * sh;
                    const int bit = 2 * vb * phi + vb * hi, c = bit >> 5, o = bit & 31;
                    const uint32_t code = e ? c1 : c0;
                    atomicOr(&s_vv[L * 16 + c], code << o);
                    atomicOr(&s_vm[L * 16 + c], cm << o);
                    if (o + vb > 32) {
                        atomicOr(&s_vv[L * 16 + c + 1], code >> (32 - o));
                        atomicOr(&s_vm[L * 16 + c + 1], cm >> (32 - o));
                    }
                }
            }
        }
    }
    if (!do_v) return;
    __syncthreads();
    if (wave != 0) return;
    // this lane's stream: the written fields merged into the dwords read at the start
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const uint32_t m32 = c < 4 * vb ? s_vm[lane * 16 + c] : 0u, v32 = s_vv[lane * 16 + c];
        if (m32) vt[((c >> 2) * 64 + lane) * 4 + (c & 3)] = (old[c] & ~m32) | (v32 & m32);
    }
}

// Copy rows into the fp16 ring (slot = position % n_recent).
__global__ __launch_bounds__(128) void k_ring(const RingArgs a) {
    const int h = blockIdx.y, b = blockIdx.z, j = threadIdx.x;
    const int64_t pos = a.pos_lo[b] + blockIdx.x;
    if (pos >= a.pos_hi[b]) return;
    const int64_t row = a.gather ? (int64_t)a.gather[b * a.gather_stride + (pos - a.pos_lo[b])] : pos - a.off[b];
    const int64_t src = (int64_t)b * a.sB + row * a.sT + (int64_t)h * a.sH + j;
    const size_t dst = (((size_t)b * a.Hkv + h) * a.n_recent + (size_t)(pos % a.n_recent)) * D + j;
    a.ring_k[dst] = f2h(load_act(a.k, src, a.dtype));
    a.ring_v[dst] = f2h(load_act(a.v, src, a.dtype));
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Launchers
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

hipError_t copy_to_device(void* dst, const void* src, size_t bytes, hipStream_t s) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s);
}

hipError_t launch_combine(const CombineArgs& a, int rows, hipStream_t s) {
    if (!a.part || !a.out || a.n_parts < 1 || a.n_parts > BGTQ_MAX_PARTS) return hipErrorInvalidValue;
    if (a.k16) {
        if (!a.v16 || !a.q || a.rows < 1 || a.Hkv < 1 || a.G < 1 || a.Hq != a.Hkv * a.G) return hipErrorInvalidValue;
        for (int b = 0; b < rows / a.Hq; ++b)
            if (a.n_valid[b] < 0 || a.n_valid[b] > a.rows || a.n_valid[b] > kMergeWindowMax) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_combine<true>, dim3(rows), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(k_combine<false>, dim3(rows), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_energy(const EnergyArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_energy, dim3(a.Hkv, a.n_chunks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    if ((a.which & 1) && a.k_mode == BGTQ_K_BLOCKGTQ && (!a.bits || !a.sigma || !a.inv_sigma))
        return hipErrorInvalidValue;
    QuantArgs q = a;
    const int es = a.dtype == BGTQ_F32 ? 4 : 2;
    q.vec16 = ((uintptr_t)a.src_k % 16 == 0) && ((uintptr_t)a.src_v % 16 == 0) && (a.sB * es) % 16 == 0 &&
              (a.sT * es) % 16 == 0 && (a.sH * es) % 16 == 0;
    const dim3 grid((unsigned)max_tiles, a.Hkv, B);
    const bool rot = (a.k_rot && a.k_mode == BGTQ_K_AFFINE && (a.which & 1)) || (a.v_rot && (a.which & 2));
    int64_t most = 0;  // the most positions any sequence appends
    for (int b = 0; b < B; ++b) most = std::max<int64_t>(most, a.pos_hi[b] - a.pos_lo[b]);
    // one wave per token beats a tile launch for short appends; the register-row bulk kernel takes
    // over sooner (a 64-row append: 16 us against 40 us for one wave per token)
    constexpr int kAppendFewRows = 16;
    if (!rot && most <= (quant_rows_supported(q) ? kAppendFewRows : kAppendFewMax)) {
        // one wave per token in flight, up to 16 (each wave takes every NW-th token of its tile)
        const int per_tile = most < TILE ? (int)most : TILE;
        if (per_tile <= 1) return launch_main(k_append<1>, grid, dim3(64), s, q);
        if (per_tile <= 4) return launch_main(k_append<4>, grid, dim3(256), s, q);
        return launch_main(k_append<16>, grid, dim3(1024), s, q);
    }
    if (!rot && quant_rows_supported(q)) return launch_quant_rows(q, B, max_tiles, s);
    if (rot) {
        if (a.dtype == BGTQ_F32) return launch_main(k_quant<float, true>, grid, dim3(64), s, q);
        return launch_main(k_quant<uint16_t, true>, grid, dim3(64), s, q);
    }
    if (a.dtype == BGTQ_F32) return launch_main(k_quant<float, false>, grid, dim3(64), s, q);
    return launch_main(k_quant<uint16_t, false>, grid, dim3(64), s, q);
}

hipError_t launch_ring(const RingArgs& a, int B, int64_t max_rows, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_ring, dim3((unsigned)max_rows, a.Hkv, B), dim3(D), 0, s, a);
    return hipGetLastError();
}

template <int G>
static hipError_t launch_fp16_g(const Fp16Args& a, int B, hipStream_t s) {
    if constexpr (G >= 4) return launch_main(k_decode_fp16_mx<G>, dim3(a.n_splits, a.Hkv, B), dim3(256), s, a);
    else return launch_main(k_decode_fp16<G>, dim3(a.n_splits, a.Hkv, B), dim3(256), s, a);
}

hipError_t launch_fp16(const Fp16Args& a, int B, hipStream_t s) {
    if (!a.k16 || !a.v16 || !a.q || !a.part || B < 1 || B > BGTQ_MAXB) return hipErrorInvalidValue;
    switch (a.G) {
        case 1: return launch_fp16_g<1>(a, B, s);
        case 2: return launch_fp16_g<2>(a, B, s);
        case 4: return launch_fp16_g<4>(a, B, s);
        case 8: return launch_fp16_g<8>(a, B, s);
    }
    return hipErrorInvalidValue;
}

template <int G, int R, int VB, int KG>
static hipError_t launch_dec(const DecodeArgs& a, int B, hipStream_t s) {
    return launch_main(k_decode<G, R, VB, KG>, dim3(a.n_splits, a.Hkv, B), dim3(256), s, a);
}

template <int G, int VB>
static hipError_t launch_dec_gv(const DecodeArgs& a, int B, int k_mode, int R, bool vector_only, hipStream_t s) {
    if (k_mode == BGTQ_K_AFFINE) {
        if constexpr (G >= 4) if (!vector_only) {
            const dim3 grid(a.n_splits, a.Hkv, B);
            switch (a.k_group) {
                case 32: return launch_main(k_decode_mxa<G, VB, 32>, grid, dim3(256), s, a);
                case 64: return launch_main(k_decode_mxa<G, VB, 64>, grid, dim3(256), s, a);
                case 128: return launch_main(k_decode_mxa<G, VB, 128>, grid, dim3(256), s, a);
            }
        }
        switch (a.k_group) {
            case 32: return launch_dec<G, 16, VB, 32>(a, B, s);
            case 64: return launch_dec<G, 16, VB, 64>(a, B, s);
            case 128: return launch_dec<G, 16, VB, 128>(a, B, s);
        }
        return hipErrorInvalidValue;
    }
    switch (R) {
        case 8: return launch_dec<G, 8, VB, 0>(a, B, s);
        case 12: return launch_dec<G, 12, VB, 0>(a, B, s);
        case 16: return launch_dec<G, 16, VB, 0>(a, B, s);
    }
    return hipErrorInvalidValue;
}

template <int G>
static hipError_t launch_dec_g(const DecodeArgs& a, int B, int k_mode, int R, int v_bits, bool vector_only,
                               hipStream_t s) {
    switch (v_bits) {
        case 2: return launch_dec_gv<G, 2>(a, B, k_mode, R, vector_only, s);
        case 3: return launch_dec_gv<G, 3>(a, B, k_mode, R, vector_only, s);
        case 4: return launch_dec_gv<G, 4>(a, B, k_mode, R, vector_only, s);
    }
    return hipErrorInvalidValue;
}

// Vector-ALU decode (k_decode) for every format, or the affine matrix-core kernel for affine keys at
// g >= 4 unless vector_only.  Block-GTQ keys at g >= 4 come here only on the vector path.
hipError_t launch_decode(const DecodeArgs& a, int B, int k_mode, int R, int v_bits, bool vector_only, hipStream_t s) {
    if (!a.k_codes || !a.v_codes || !a.k_scale || !a.v_scale || !a.q || !a.part || B < 1 || B > BGTQ_MAXB)
        return hipErrorInvalidValue;
    if (k_mode == BGTQ_K_BLOCKGTQ && (!a.bits || !a.sigma)) return hipErrorInvalidValue;
    if (k_mode == BGTQ_K_AFFINE && !a.k_zero) return hipErrorInvalidValue;
    if (a.v_affine && !a.v_zero) return hipErrorInvalidValue;
    switch (a.G) {
        case 1: return launch_dec_g<1>(a, B, k_mode, R, v_bits, vector_only, s);
        case 2: return launch_dec_g<2>(a, B, k_mode, R, v_bits, vector_only, s);
        case 4: return launch_dec_g<4>(a, B, k_mode, R, v_bits, vector_only, s);
        case 8: return launch_dec_g<8>(a, B, k_mode, R, v_bits, vector_only, s);
    }
    return hipErrorInvalidValue;
}

void arm_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_ev_start = start;
    t_ev_stop = stop;
}
void disarm_launch_events() { t_ev_start = t_ev_stop = nullptr; }

int decode_wgs_per_cu(int k_mode, int G, int v_bits, int k_group, bool vector_only) {
    if (!vector_only && G >= 4 && k_mode == BGTQ_K_AFFINE && (k_group == 32 || k_group == 64 || k_group == 128)) return kMxaWgsPerCu;
    return 2;
}

bool decode_supported(int k_mode, int R, int k_bits, int k_group, int v_bits, int G) {
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return false;
    if (v_bits < 2 || v_bits > 4) return false;
    if (k_mode == BGTQ_K_AFFINE) return k_bits == 4 && (k_group == 32 || k_group == 64 || k_group == 128);
    return R == 8 || R == 12 || R == 16;
}

}  // namespace bgtq
