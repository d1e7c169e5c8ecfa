// Packed-cache decode over Block-GTQ keys on the matrix cores, one workgroup per compute unit
// ("RoPE-Aware Bit Allocation for KV-Cache Quantization": abstract; review §1 Packed-Cache,
// Figure 2: attention computed straight from the packed codes).
//
// The g query heads of a kv head share every dequantized key and value, so per 64-token tile q·K^T
// is a (g x 128) x (128 x 64) product and P·V a (g x 64) x (64 x 128) product, both on
// v_mfma_f32_16x16x32_f16; the vector ALUs unpack codes and run the online softmax.
//  * A = Q' (16 rows x 32 K): row 4u + e is head 2u + e/2, with e even the fp16 high part and e odd
//    the fp16 low part of q' = q * sigma * log2(e)/sqrt(d) (hi + lo carries ~22 bits).  Centroids
//    are fp16 values exactly, so the products lose nothing and the matrix cores sum in fp32.
//  * B = K^ (32 K x 16 tokens): lane (token j, row u) builds its own operand: K index 8u + e is
//    coordinate e % 2 of stream slot 16 ks + 8 (e / 4) + 2u + (e / 2) % 2, so a lane row reads two
//    adjacent slots of the record from one 64-bit window of the staged record (per token group),
//    shifts it and ANDs/ORs the field into a table address (pair tables for widths <= 5, fp16
//    coordinate tables for wider columns).  No transposes.
//  * C (16 x 16 tokens): lane (token 16g + r, row group u) holds heads 2u, 2u + 1 as (hi, lo).
//  * P·V: A = V^T (16 dims x 32 tokens) straight from the lane-stream value fields through a
//    replicated pair table, B = W (32 tokens x 16 heads) through LDS in pair order (t, t + 32);
//    O^T accumulates per 16-dim block.
//  * Online softmax with the exact running max per head (a wave-uniform branch raises it), so the
//    largest weight of a split is fp16(scale) exactly, whatever the split boundaries.
//
// What depends only on the widths of a (layer, kv head) — the block order, the column descriptors
// of the operand assembly and the per-block operand position of the query — is computed once by
// k_plan into a small plan record; every workgroup of every decode loads it instead of rebuilding
// it.  One workgroup per compute unit (sixteen waves with one tile each, or eight waves looping over
// their tiles) merges its waves into one (o, m, l) partial per query head, so a split-K launch
// writes one partial per compute unit and kv head.
#include <hip/hip_ext.h>

#include "bgtq_device.h"

namespace bgtq {
namespace {


// Plan record of one (layer, kv head): u32 desc[64] (column descriptors, index kq*16 + 4ks + 2mp +
// odd as mx_desc builds them), u8 rank[64] (stream slot of block i, 0xFF for width 0), u32 nnz_pad
// (nonzero slots rounded up to 4), ncc (coordinate columns), nnz, then u16 off[64] (bit offset of
// block i's field in the key record).
constexpr int kPlanDesc = 0, kPlanRank = 256, kPlanCounts = 320, kPlanOff = 336;
static_assert(kPlanOff + 128 <= BGTQ_PLAN_BYTES, "plan record size");

// One wave per kv head, lane = RoPE block.
__global__ __launch_bounds__(64) void k_plan(const uint8_t* bits, uint8_t* plan) {
    const int h = blockIdx.x, lane = threadIdx.x;
    const int bw = bits[h * 64 + lane];
    const int w = bw < 8 ? bw : 8;  // widths above 8 are invalid; clamp
    int rank, pos, nnz;
    block_order(w, lane, rank, pos, nnz);
    const int n_wide = __popcll(__ballot(w > 5));
    __shared__ int s_sw[64], s_sp[64];
    if (w > 0) {
        s_sw[rank] = w;
        s_sp[rank] = pos;
    }
    if (lane >= nnz) {
        s_sw[lane] = 0;
        s_sp[lane] = 0;
    }
    __syncthreads();
    uint8_t* p = plan + (size_t)h * BGTQ_PLAN_BYTES;
    // stream slot r is k-step r / 16, column pair (r % 16) / 8, lane row (r % 8) / 2, second of its
    // pair if odd; a column is read per coordinate when its first slot is wider than 5 bits
    const int r = lane, ks = r >> 4, mp = (r >> 3) & 1, kq = (r >> 1) & 3, odd = r & 1;
    auto coord_of = [&](int first) { return first < n_wide; };
    const bool ca = coord_of(16 * ks + 8 * mp), cs = coord_of(16 * ks + 8 * mp + odd);
    ((uint32_t*)(p + kPlanDesc))[kq * 16 + 4 * ks + 2 * mp + odd] = mx_desc(s_sp[r & ~1], ca, s_sp[r], s_sw[r], cs);
    p[kPlanRank + lane] = (uint8_t)(w > 0 ? rank : 0xFF);
    ((uint16_t*)(p + kPlanOff))[lane] = (uint16_t)pos;
    if (lane == 0) {
        int nc = 0;
        for (int c = 0; c < 16; ++c) nc += coord_of(16 * (c >> 2) + 8 * ((c >> 1) & 1) + (c & 1)) ? 1 : 0;
        uint32_t* cnt = (uint32_t*)(p + kPlanCounts);
        cnt[0] = (uint32_t)((nnz + 3) & ~3);
        cnt[1] = (uint32_t)nc;
        cnt[2] = (uint32_t)nnz;
    }
}

// Query operand image (LDS, u32x4 [4 k-steps][64 lanes]): q' = q * sigma * log2(e)/sqrt(d) of the
// block in stream slot r (its rank), split into an fp16 high part and an fp16 low part, sits at
// k-step r / 16, lane row (r % 8) / 2, element pair 2 ((r % 16) / 8) + r % 2 of the operand lanes
// of its head (column 2h: high part, 2h + 1: low part).  Slots past the nonzero blocks, and the
// columns of absent heads, hold zeros.
//
// Query operands from the plan, one (head, block) item per thread (threads 0 .. 511: head hh =
// thread / 64, block = thread % 64).  The item's coordinates go to stream slot rank of the image as
// fp16 high and low parts (rows 2hh and 2hh + 1); the item also clears its head's rows of slot
// `block` when that slot is past the nonzero blocks, and heads beyond G clear their rows of every
// slot.
struct QItem {
    uint32_t r0, r1;  // the item's two coordinates (fp32 bits, or the packed 16-bit pair in r0)
    float sg;         // sigma of the block
    int rank;         // stream slot of the block (0xFF: width 0)
};

template <int G>
__device__ __forceinline__ QItem gtq_q_item_load(const void* q, int dtype, const float* sigma, const uint8_t* plan_rank,
                                                 int b, int h, int Hq) {
    const int i = threadIdx.x < 512 ? threadIdx.x : 0;
    const int hh = i >> 6, blk = i & 63;
    const int64_t at = ((int64_t)b * Hq + (int64_t)h * G + (hh < G ? hh : 0)) * D + 2 * blk;
    QItem it;
    if (dtype == BGTQ_F32) {
        const uint2 v = *(const uint2*)((const float*)q + at);
        it.r0 = v.x;
        it.r1 = v.y;
    } else {
        it.r0 = *(const uint32_t*)((const uint16_t*)q + at);
        it.r1 = 0u;
    }
    it.sg = sigma[h * 64 + blk];
    it.rank = plan_rank[blk];
    return it;
}

template <int G>
__device__ void gtq_q_item_store(const QItem& it, int dtype, int nnz, uint8_t* qa) {
    const int i = threadIdx.x;
    if (i >= 512) return;
    const int hh = i >> 6, blk = i & 63;
    auto slot_base = [&](int r) {
        const int ks = r >> 4, rr = r & 15, urow = (rr >> 1) & 3, mpair = 2 * (rr >> 3) + (rr & 1);
        return qa + (size_t)(ks * 64 + 16 * urow) * 16 + 4 * mpair;
    };
    if (hh < G && it.rank != 0xFF) {
        float q0, q1;
        if (dtype == BGTQ_F32) {
            q0 = __builtin_bit_cast(float, it.r0);
            q1 = __builtin_bit_cast(float, it.r1);
        } else {
            q0 = dtype == BGTQ_F16 ? h2f(it.r0 & 0xFFFFu) : bf2f(it.r0 & 0xFFFFu);
            q1 = dtype == BGTQ_F16 ? h2f(it.r0 >> 16) : bf2f(it.r0 >> 16);
        }
        const float sg = it.sg * kLog2eOverSqrtD;
        q0 *= sg;
        q1 *= sg;
        const _Float16 h0 = (_Float16)q0, h1 = (_Float16)q1;
        const _Float16 l0 = (_Float16)(q0 - (float)h0), l1 = (_Float16)(q1 - (float)h1);
        uint8_t* base = slot_base(it.rank);
        *(uint32_t*)(base + (2 * hh) * 16) =
            (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        *(uint32_t*)(base + (2 * hh + 1) * 16) =
            (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    if (hh >= G || blk >= nnz) {
        uint8_t* base = slot_base(blk);
        *(uint32_t*)(base + (2 * hh) * 16) = 0u;
        *(uint32_t*)(base + (2 * hh + 1) * 16) = 0u;
    }
}

// Query operands from the plan (wave 0, lane = RoPE block): q' = q * sigma * log2(e)/sqrt(d) of
// block i goes to stream slot rank_i of the operand image (layout above); slots past the
// nonzero blocks get zeros.
template <int G>
__device__ void gtq_prep_q(const PrepIn<G>& in, int rank, int nnz, int lane, uint8_t* qa) {
    float q0[G], q1[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        if (in.dtype == BGTQ_F32) {
            q0[hh] = __builtin_bit_cast(float, in.r0[hh]);
            q1[hh] = __builtin_bit_cast(float, in.r1[hh]);
        } else if (in.dtype == BGTQ_F16) {
            q0[hh] = h2f(in.r0[hh] & 0xFFFFu);
            q1[hh] = h2f(in.r0[hh] >> 16);
        } else {
            q0[hh] = bf2f(in.r0[hh] & 0xFFFFu);
            q1[hh] = bf2f(in.r0[hh] >> 16);
        }
        q0[hh] = q0[hh] * kLog2eOverSqrtD * in.sg;
        q1[hh] = q1[hh] * kLog2eOverSqrtD * in.sg;
    }
    auto put = [&](int r, bool zero) {
        const int ks = r >> 4, rr = r & 15, urow = (rr >> 1) & 3, mpair = 2 * (rr >> 3) + (rr & 1);
        uint8_t* base = qa + (size_t)(ks * 64 + 16 * urow) * 16 + 4 * mpair;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            uint32_t hi2 = 0u, lo2 = 0u;
            if (hh < G && !zero) {
                const _Float16 h0 = (_Float16)q0[hh], h1 = (_Float16)q1[hh];
                const _Float16 l0 = (_Float16)(q0[hh] - (float)h0), l1 = (_Float16)(q1[hh] - (float)h1);
                hi2 = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
                lo2 = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
            }
            *(uint32_t*)(base + (2 * hh) * 16) = hi2;
            *(uint32_t*)(base + (2 * hh + 1) * 16) = lo2;
        }
    };
    if (rank != 0xFF) put(rank, false);
    if (lane >= nnz) put(lane, true);
}

// Workgroup barrier that orders LDS only: the waves' LDS writes complete first, global loads still
// in flight stay in flight (__syncthreads also waits for every outstanding global access).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Merge the NW waves' (o, m, l, zero term) records in red[wave][h] into one partial per head:
// thread (h, quad of dims) reads the NW maxima of its head (broadcast reads), forms its own scale
// factors and folds 4 dims of the NW records; the first of a head's threads also writes M and L.
// No LDS writes between the reads (no serial chain), and the global stores come after the last
// barrier.
template <int G, int NW>
__device__ __forceinline__ void merge_waves_n(const float* red, float* part, int n_parts, int split) {
    for (int idx = threadIdx.x; idx < G * 32; idx += blockDim.x) {
        const int h = idx >> 5, j = 4 * (idx & 31);
        float mw[NW];
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            mw[wv] = red[(wv * G + h) * PART + 128];
            M = fmaxf(M, mw[wv]);
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            const float* rw = red + (wv * G + h) * PART;
            const float f = mw[wv] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[wv] - M);
            acc += f * (*(const f32x4_t*)(rw + j) + rw[130]);
            L += f * rw[129];
        }
        // plain stores: the split merge that follows reads the partials from the caches
        // (non-temporal stores, which stream past them, made the decode-plus-merge step 4% slower)
        float* dst = part + ((size_t)h * n_parts + split) * PART;
        *(f32x4_t*)(dst + j) = acc;
        if (j == 0) {
            dst[128] = M;
            dst[129] = L;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// One-token append inside the decode (bgtq_decode_step on this kernel; LogQuant summary,
// Conclusion: fusing the write into the attention launch).  In the workgroup whose splits hold the
// appended token (the last packed one of its sequence), wave 0 quantizes it in the prologue, before
// the barrier that releases the tiles, with the steps of the append kernels (one wave, lane i =
// RoPE block i with dims 2i and 2i + 1): the key record, fp16 scales and value codes go to the cache
// and to LDS; the wave that stages the token's tile patches its record column, scales and value
// fields in, so the token is attended with the rest of its tile.

// The token's key record (R dwords), scales (key, value, value zero), the squares summed for the
// scales, and its value fields as they go into the streams of lanes 16 jj .. 16 jj + 15 (bits and
// mask per stream dword; jj from the token's tile position).
struct AppLds {  // 16-byte aligned (read 16 bytes at a time): the arrays come first
    float sq[256];  // squares of the scaled key row, then of the value row
    uint32_t vval[16][16];
    uint32_t vmsk[16][16];
    uint32_t rec[16];
    uint16_t sc[4];
};
static_assert(offsetof(AppLds, vval) % 16 == 0 && offsetof(AppLds, vmsk) % 16 == 0, "16-byte rows");

struct AppRow {
    float kx0, kx1, vx0, vx1;  // the lane's two elements of the key and value rows
    int w, off;                // width of the lane's block and its bit offset in the record
    float r, sg;               // 1/sigma and sigma of the lane's block
    uint32_t thr[(BGTQ_CB_THRESHOLDS + 63) / 64];  // thresholds lane + 64 k
};

__device__ __forceinline__ AppRow app_load(const DecodeArgs& a, const uint8_t* plan, int b, int h, int lane) {
    const int64_t src = (int64_t)b * a.app_sB + (int64_t)h * a.app_sH + 2 * lane;
    AppRow r;
    r.kx0 = load_act(a.app_k, src, a.app_dtype);
    r.kx1 = load_act(a.app_k, src + 1, a.app_dtype);
    r.vx0 = load_act(a.app_v, src, a.app_dtype);
    r.vx1 = load_act(a.app_v, src + 1, a.app_dtype);
    const int bw = a.bits[h * 64 + lane];
    r.w = bw < 8 ? bw : 8;
    r.off = ((const uint16_t*)(plan + kPlanOff))[lane];
    r.r = a.inv_sigma[h * 64 + lane];
    r.sg = a.sigma[h * 64 + lane];
#pragma unroll
    for (int k = 0; k < (BGTQ_CB_THRESHOLDS + 63) / 64; ++k)
        r.thr[k] = c_thr32[lane + 64 * k < BGTQ_CB_THRESHOLDS ? lane + 64 * k : 0];
    return r;
}

// Quantize the token at position pos of (batch, kv head) bh and write it to the cache; leave the
// record, scales and value codes in ap.  thr: LDS for the scalar thresholds.
template <int R, int VB>
__device__ void app_quantize(const DecodeArgs& a, const AppRow& in, int lane, size_t bh, int64_t pos, bool vaff,
                             float* thr, AppLds* ap) {
#pragma unroll
    for (int k = 0; k < (BGTQ_CB_THRESHOLDS + 63) / 64; ++k)
        if (lane + 64 * k < BGTQ_CB_THRESHOLDS) thr[lane + 64 * k] = __builtin_bit_cast(float, in.thr[k]);
    if (lane < R) ap->rec[lane] = 0u;
    {
#pragma clang fp contract(off)
        const float u0 = in.kx0 * in.r, u1 = in.kx1 * in.r;
        ap->sq[2 * lane] = u0 * u0;
        ap->sq[2 * lane + 1] = u1 * u1;
        ap->sq[128 + 2 * lane] = in.vx0 * in.vx0;
        ap->sq[128 + 2 * lane + 1] = in.vx1 * in.vx1;
    }
    wave_lds_fence();
    // The per-token scales: squares summed in element order (lane 0: keys, lane 32: values; the
    // steps of the append kernels), mean, square root, fp16.
    float acc = 0.f;
    {
        const f32x4_t* sq4 = (const f32x4_t*)(ap->sq + (lane >= 32 ? 128 : 0));
#pragma unroll
        for (int i0 = 0; i0 < 32; i0 += 8) {  // eight reads in flight, then their 32 additions
            f32x4_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = sq4[i0 + i];
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                acc = acc + v[i][0];
                acc = acc + v[i][1];
                acc = acc + v[i][2];
                acc = acc + v[i][3];
            }
        }
    }
    const uint16_t ks16 = f2h(sqrtf(lane_f(acc, 0) / 128.0f));
    const float S = h2f(ks16);
    if (in.w > 0) {
        float t;
        {
#pragma clang fp contract(off)
            t = S * in.sg;
        }
        // both coordinates' binary searches (tq_code) in one loop, so their reads overlap
        uint32_t q0 = 0u, q1 = 0u;
        const float* tb = thr + thr_base(in.w);
        for (int st = in.w - 1; st >= 0; --st) {
#pragma clang fp contract(off)
            const uint32_t a0 = q0 + (1u << st), a1 = q1 + (1u << st);
            const float th0 = t * tb[a0 - 1], th1 = t * tb[a1 - 1];
            if (in.kx0 >= th0) q0 = a0;
            if (in.kx1 >= th1) q1 = a1;
        }
        const uint32_t f = q0 | (q1 << in.w);
        const int k = in.off >> 5, sh = in.off & 31;
        if (k < R) atomicOr(&ap->rec[k], f << sh);
        if (sh + 2 * in.w > 32 && k + 1 < R) atomicOr(&ap->rec[k + 1], f >> (32 - sh));
    }
    uint32_t c0 = 0u, c1 = 0u;
    uint16_t vs16 = 0, vz16 = 0;
    if (!vaff) {
        vs16 = f2h(sqrtf(lane_f(acc, 32) / 128.0f));
        const float Sv = h2f(vs16);
        static_assert(thr_base_c(VB) + (1 << VB) - 1 <= 64, "value thresholds in the first register");
#pragma unroll
        for (int m = 0; m < (1 << VB) - 1; ++m) {
            float th;
            {
#pragma clang fp contract(off)
                th = Sv * __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)in.thr[0], thr_base_c(VB) + m));
            }
            c0 += in.vx0 >= th ? 1u : 0u;
            c1 += in.vx1 >= th ? 1u : 0u;
        }
    } else {
#pragma clang fp contract(off)
        float mn, mx;
        wave_minmax(in.vx0, in.vx1, 0, D, mn, mx);
        const float scale = (mx - mn) / (float)((1 << VB) - 1);
        vs16 = f2h(scale);
        vz16 = f2h(mn);
        const float s32 = h2f(vs16), z32 = h2f(vz16), top = (float)((1 << VB) - 1);
        float f0 = 0.f, f1 = 0.f;
        if (s32 != 0.f) {
            f0 = fminf(fmaxf(rintf((in.vx0 - z32) / s32), 0.f), top);
            f1 = fminf(fmaxf(rintf((in.vx1 - z32) / s32), 0.f), top);
        }
        c0 = (uint32_t)f0;
        c1 = (uint32_t)f1;
    }
    // Value fields: dim 16 db + dd of the token goes to stream dd + 16 jj, field (s * 8 + db) * 4 + m
    // (p = u % 32 = 16 s + 4 jj + m, the token's half chosen by u >= 32); lane i places dims 2i and
    // 2i + 1 into the bits and masks of their streams' dwords (rows dd of vval / vmsk).
    ap->vval[lane >> 2][4 * (lane & 3)] = 0u;  // 64 lanes x 4 = the 256 dwords of each table
    ap->vval[lane >> 2][4 * (lane & 3) + 1] = 0u;
    ap->vval[lane >> 2][4 * (lane & 3) + 2] = 0u;
    ap->vval[lane >> 2][4 * (lane & 3) + 3] = 0u;
    ap->vmsk[lane >> 2][4 * (lane & 3)] = 0u;
    ap->vmsk[lane >> 2][4 * (lane & 3) + 1] = 0u;
    ap->vmsk[lane >> 2][4 * (lane & 3) + 2] = 0u;
    ap->vmsk[lane >> 2][4 * (lane & 3) + 3] = 0u;
    wave_lds_fence();
    {
        const int u = (int)(pos % TILE), p = u & 31, hi = u >> 5, s = p >> 4, m = p & 3;
        constexpr uint32_t cm = (1u << VB) - 1u;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int dim = 2 * lane + e, dd = dim & 15, db = dim >> 4;
            const uint32_t code = e ? c1 : c0;
            const int bit = 2 * VB * (m + 4 * db + 32 * s) + VB * hi, c = bit >> 5, o = bit & 31;
            atomicOr(&ap->vval[dd][c], code << o);
            atomicOr(&ap->vmsk[dd][c], cm << o);
            if (o + VB > 32) {
                atomicOr(&ap->vval[dd][c + 1], code >> (32 - o));
                atomicOr(&ap->vmsk[dd][c + 1], cm >> (32 - o));
            }
        }
    }
    if (lane == 0) {
        ap->sc[0] = ks16;
        ap->sc[1] = vs16;
        ap->sc[2] = vz16;
        a.app_k_scale[bh * a.n_cap + pos] = ks16;
        a.app_v_scale[bh * a.n_cap + pos] = vs16;
        if (vaff) a.app_v_zero[bh * a.n_cap + pos] = vz16;
    }
    wave_lds_fence();
    if (lane < R) {
        uint32_t* kt = (uint32_t*)(a.app_k_codes + (bh * a.n_tiles + pos / TILE) * a.k_tile_bytes);
        kt[lane * TILE + pos % TILE] = ap->rec[lane];
    }
}

// Patch the appended token (tile position u) into the staged tile: its record column and scales
// in LDS, its value fields in the stream registers of lanes 16 jj .. 16 jj + 15; the stream dwords
// that change are written to the cache (the rest of each dword is as the tile loaded it).
template <int R, int VB>
__device__ __forceinline__ void app_patch(const DecodeArgs& a, const AppLds* ap, int lane, int u, size_t bh,
                                          int64_t tile, uint8_t* kst, uint16_t* sst, bool vaff, u32x4_t (&vcur)[VB]) {
    if (lane < R) *(uint32_t*)(kst + (lane + 1) * BGTQ_KST_ROW_BYTES + 4 * u) = ap->rec[lane];
    if (lane == 0) {
        const int si = (u & 15) * 4 + (u >> 4);
        sst[si] = ap->sc[0];
        sst[64 + si] = ap->sc[1];
        if (vaff) sst[128 + si] = ap->sc[2];
    }
    if ((lane >> 4) != ((u >> 2) & 3)) return;
    uint32_t* vt = (uint32_t*)(a.app_v_codes + (bh * a.n_tiles + tile) * a.v_tile_bytes);
#pragma unroll
    for (int c4 = 0; c4 < VB; ++c4) {
        const u32x4_t mk = *(const u32x4_t*)&ap->vmsk[lane & 15][4 * c4];
        const u32x4_t vv = *(const u32x4_t*)&ap->vval[lane & 15][4 * c4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (mk[e]) {
                const uint32_t nv = (vcur[c4][e] & ~mk[e]) | vv[e];
                vcur[c4][e] = nv;
                vt[(c4 * 64 + lane) * 4 + e] = nv;
            }
        }
    }
}

// LDS arena (byte offsets): tables at offset 0 (the arena is 8192-aligned, so table offsets are
// LDS addresses), column descriptors, value pair table, query operands, weight exchange, softmax
// rescale factors, counts, the append's thresholds and token, then per wave the stage of the tile in flight (K record rows -1 .. R at
// BGTQ_KST_ROW_BYTES stride, then its scales).  The epilogue records alias the stages.
template <int G, int R, int VB, int NW> struct GtqLds {
    static constexpr int TAB = 0;
    static constexpr int DESC = a16(TAB + BGTQ_CB_MX_BYTES);          // u32 [4 lane rows][16 columns]
    static constexpr int VLUT = DESC + 64 * 4;                        // u32 [4^VB][copies]
    static constexpr int QA = a16(VLUT + VLutGeom<VB>::BYTES);        // u32x4 [4 k-steps][64 lanes]
    static constexpr int WX = QA + 4 * 64 * 16;                       // u32 [NW waves][16 heads][32 pairs]
    static constexpr int ALPHA = WX + NW * 16 * 32 * 4;               // f32 [NW waves][16]
    static constexpr int NNZ = ALPHA + NW * 16 * 4;                   // u32 [4]: nnz_pad, ncc, nnz
    static constexpr int THR = a16(NNZ + 16);                         // f32 [BGTQ_CB_THRESHOLDS] (append)
    static constexpr int APP = a16(THR + 4 * BGTQ_CB_THRESHOLDS);     // AppLds (append), 16-byte aligned
    static constexpr int KST = a16(APP + (int)sizeof(AppLds));        // per wave: R + 2 rows
    static constexpr int KST_W = (R + 2) * BGTQ_KST_ROW_BYTES;
    static constexpr int SST = KST + NW * KST_W;                      // per wave: K scales, V scales, V zeros
    static constexpr int SST_W = 3 * 64 * 2;
    static constexpr int RED = KST;                                   // epilogue: f32 [NW G PART + NW G]
    static constexpr int SIZE = cmax(SST + NW * SST_W, RED + 4 * NW * G * PART);
};

template <int G, int R, int VB, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_decode_gtq(const DecodeArgs a) {
    static_assert(G == 4 || G == 8, "matrix-core decode serves 4 or 8 query heads per kv head");
    static_assert(R % 4 == 0, "K records are staged in 16-byte chunks");
    using LD = GtqLds<G, R, VB, NW>;
    static_assert(LD::SIZE <= 160 * 1024, "LDS budget");
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int row = lane >> 4, col = lane & 15;
    __shared__ __attribute__((aligned(8192))) uint8_t lds[LD::SIZE];
    uint32_t* s_vlut = (uint32_t*)(lds + LD::VLUT);
    u32x4_t* s_qa = (u32x4_t*)(lds + LD::QA);
    float* s_alpha = (float*)(lds + LD::ALPHA) + wave * 16;
    uint32_t* s_nnz = (uint32_t*)(lds + LD::NNZ);
    uint8_t* kst = lds + LD::KST + wave * LD::KST_W;
    uint16_t* sst = (uint16_t*)(lds + LD::SST + wave * LD::SST_W);
    uint32_t* wx = (uint32_t*)(lds + LD::WX) + wave * 16 * 32;

    const size_t bh = (size_t)b * a.Hkv + h;
    const int64_t n_packed = a.n_packed[b];
    const int64_t n_tiles_b = (n_packed + TILE - 1) / TILE;
    const int64_t t_lo = (int64_t)split * a.tiles_per_split;
    const int64_t t_hi = t_lo + a.tiles_per_split < n_tiles_b ? t_lo + a.tiles_per_split : n_tiles_b;
    const uint32_t* kc = (const uint32_t*)(a.k_codes + bh * a.n_tiles * a.k_tile_bytes);
    const uint32_t* vc = (const uint32_t*)(a.v_codes + bh * a.n_tiles * a.v_tile_bytes);
    const uint32_t* ks32 = (const uint32_t*)(a.k_scale + bh * a.n_cap);  // fp16 pairs (token 2i, 2i + 1)
    const uint32_t* vs32 = (const uint32_t*)(a.v_scale + bh * a.n_cap);
    const uint32_t* vz32 = a.v_affine ? (const uint32_t*)(a.v_zero + bh * a.n_cap) : nullptr;
    const bool vaff = a.v_affine != 0;
    const uint8_t* plan = a.plan + (size_t)h * BGTQ_PLAN_BYTES;
    // Append in this launch: the sequence's last packed token, at tile t_app, position u_app; the
    // wave that will stage that tile quantizes it (t_app is -1 without an append).
    const bool app = a.app_k != nullptr;
    const int64_t t_app = app ? (n_packed - 1) / TILE : -1;
    const int u_app = app ? (int)((n_packed - 1) % TILE) : 0;
    const bool app_here = t_app >= t_lo && t_app < t_hi;  // this workgroup's splits hold the token
    float* s_thr = (float*)(lds + LD::THR);
    AppLds* s_app = (AppLds*)(lds + LD::APP);

    // Prologue.  Global loads first: the query and this lane's block of the plan (wave 0), the
    // plan's descriptors and counts, the table image and the value centroids, then the first tile's
    // keys; loads retire in order, so the LDS writes below do not wait for HBM.  Loads are
    // unconditional (clamped indices) so that no branch forces an early wait.
    PrepIn<G> pin;
    int prank = 0;
    QItem qit;
    if constexpr (NW > 8) {
        qit = gtq_q_item_load<G>(a.q, a.q_dtype, a.sigma, plan + kPlanRank, b, h, a.Hq);
    } else {
        pin = prep_load<G, true>(a.q, a.q_dtype, a.bits, a.sigma, b, h, a.Hq, lane);
        prank = plan[kPlanRank + lane];
    }
    AppRow arow{};
    if (app_here && wave == 0) arow = app_load(a, plan, b, h, lane);
    const uint32_t pdesc = threadIdx.x < 64 ? ((const uint32_t*)(plan + kPlanDesc))[threadIdx.x] : 0u;
    const uint32_t pcnt = threadIdx.x < 3 ? ((const uint32_t*)(plan + kPlanCounts))[threadIdx.x] : 0u;
    constexpr int TAB4 = BGTQ_CB_MX_WORDS / 4;
    const u32x4_t* tab4 = (const u32x4_t*)c_mxtab;
    constexpr int NT = 64 * NW;
    u32x4_t tv[(TAB4 + NT - 1) / NT];
#pragma unroll
    for (int k = 0; k < (TAB4 + NT - 1) / NT; ++k)
        tv[k] = tab4[threadIdx.x + NT * k < TAB4 ? threadIdx.x + NT * k : 0];
    constexpr int VCOP = VLutGeom<VB>::COPIES, VENT = 1 << (2 * VB);
    constexpr int VROUNDS = (VENT * VCOP + NT - 1) / NT;
    uint32_t vla[VROUNDS], vlb[VROUNDS];
#pragma unroll
    for (int k = 0; k < VROUNDS; ++k) {
        const uint32_t e = ((threadIdx.x + (uint32_t)NT * k) / VCOP) & (VENT - 1);
        vla[k] = c_cent16[cent_base(VB) + (e & ((1u << VB) - 1u))];
        vlb[k] = c_cent16[cent_base(VB) + (e >> VB)];
    }

    // Tile data: K chunks and one dword of scales per lane (lanes 0..31: K scales of tokens 2l,
    // 2l+1; lanes 32..63: V scales; V zeros in a second dword for affine values) are prefetched one
    // tile ahead and staged to LDS when their tile starts; the value streams stay in registers
    // (each lane reads its own stream).
    u32x4_t kn[R / 4], vn[VB], vx[VB];
    uint32_t sn, zn;
    // The packed tiles and their scales are read once per step: non-temporal loads keep them from
    // displacing what is reused (tables, plan, the partials the merge reads), 2-5% per step in
    // same-box A/B runs.
    auto fetch_k = [&](int64_t t) {
        const u32x4_t* kt = (const u32x4_t*)(kc + t * (a.k_tile_bytes / 4));
#pragma unroll
        for (int c = 0; c < R / 4; ++c) kn[c] = __builtin_nontemporal_load(kt + c * 64 + lane);
        sn = __builtin_nontemporal_load((lane < 32 ? ks32 : vs32) + t * (TILE / 2) + (lane & 31));
        zn = vz32 ? __builtin_nontemporal_load(vz32 + t * (TILE / 2) + (lane & 31)) : 0u;
    };
    auto fetch_v = [&](u32x4_t (&dst)[VB], int64_t t) {
        const u32x4_t* vt = (const u32x4_t*)(vc + t * (a.v_tile_bytes / 4));
#pragma unroll
        for (int c = 0; c < VB; ++c) dst[c] = __builtin_nontemporal_load(vt + c * 64 + lane);
    };
    // Unconditional (branch-free prologue); a wave without tiles reads a tile inside the allocation
    // and never uses it.  With eight waves the first keys go out right behind the small loads above
    // (the scheduling fence keeps them behind); with sixteen they wait for the barrier below.
    const int64_t t_first = t_lo + wave < t_hi ? t_lo + wave : (t_lo < a.n_tiles ? t_lo : 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NW <= 8) fetch_k(t_first);

#pragma unroll
    for (int k = 0; k < (TAB4 + NT - 1) / NT; ++k)
        if (threadIdx.x + NT * k < TAB4) ((u32x4_t*)(lds + LD::TAB))[threadIdx.x + NT * k] = tv[k];
#pragma unroll
    for (int k = 0; k < VROUNDS; ++k) {
        const uint32_t i = threadIdx.x + (uint32_t)NT * k;
        const uint32_t e = (i / VCOP) & (VENT - 1);
        if (i < (uint32_t)(VENT * VCOP))
            s_vlut[i] = a.v_affine ? (uint32_t)f2h((float)(e & ((1u << VB) - 1u))) | ((uint32_t)f2h((float)(e >> VB)) << 16)
                                   : vla[k] | (vlb[k] << 16);
    }
#pragma unroll
    for (int i = threadIdx.x; i < NW * 16 * 32 / 4; i += NT) ((u32x4_t*)(lds + LD::WX))[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (threadIdx.x < 64) ((uint32_t*)(lds + LD::DESC))[threadIdx.x] = pdesc;
    if (threadIdx.x < 3) s_nnz[threadIdx.x] = pcnt;
    if constexpr (NW > 8) {
        const int nnz = (int)__builtin_amdgcn_readfirstlane(((const uint32_t*)(plan + kPlanCounts))[2]);
        gtq_q_item_store<G>(qit, a.q_dtype, nnz, lds + LD::QA);
    } else if (wave == 0) {
        const int nnz = (int)__builtin_amdgcn_readfirstlane(((const uint32_t*)(plan + kPlanCounts))[2]);
        gtq_prep_q<G>(pin, prank, nnz, lane, lds + LD::QA);
    }
    if (app_here && wave == 0) {  // ahead of every tile of this workgroup, at raised issue priority
        __builtin_amdgcn_s_setprio(3);
        app_quantize<R, VB>(a, arow, lane, bh, n_packed - 1, vaff, s_thr, s_app);
        __builtin_amdgcn_s_setprio(0);
    }
    lds_barrier();  // tables, descriptors and query operands are in place
    if constexpr (NW > 8) {
        // One tile per wave, every wave's tile issued right after the barrier.  The small loads
        // were waited for before it, so no wave's prologue queues behind the tile bursts of the
        // chip.  (Issuing the waves in groups with a barrier between groups, so that the first
        // group's tiles land first, measured slower: 4 groups 2-3% and 8 groups 4% slower per step,
        // 2 groups no faster.)
        fetch_k(t_first);
        fetch_v(vn, t_first);
    }

    const int nnz_pad = (int)__builtin_amdgcn_readfirstlane(s_nnz[0]);  // nonzero slots rounded up to 4
    const int nks = (nnz_pad + 15) >> 4;
    const int ncc = (int)__builtin_amdgcn_readfirstlane(s_nnz[1]);      // coordinate columns
    // This lane row's column descriptors of the four k-steps, read while the tile data is in flight.
    u32x4_t dks[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) dks[ks] = ((const u32x4_t*)(lds + LD::DESC))[4 * row + ks];
    if constexpr (NW <= 8) fetch_v(vn, t_first);

    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f}, zs[2] = {0.f, 0.f};
    f32x4_t o[8];
    if constexpr (NW <= 8) {
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    uint32_t lb = (uint32_t)(LD::KST + wave * LD::KST_W) + 4u * (uint32_t)col;
    asm volatile("" : "+v"(lb));  // keep the stage base inside lb: one add per column address
    const uint32_t lcopy = 4u * ((uint32_t)lane & (VLutGeom<VB>::COPIES - 1));  // this lane's value-table copy

    // With eight waves, two tiles per iteration: the value streams of the next tile load into the
    // other buffer (4-bit values: one buffer, reloaded after P·V).  With sixteen waves one buffer: the
    // other waves of the SIMD cover the reload.
    constexpr bool VDB = VB <= 3 && NW <= 8;
    auto tile = [&](const int64_t t, u32x4_t (&vcur)[VB], u32x4_t (&vnext)[VB]) __attribute__((always_inline)) {
        // Stage the tile: K rows (row rho of the record at stage row rho + 1), scales (transposed:
        // token u at (u%16)*4 + u/16).
        wave_lds_fence();
#pragma unroll
        for (int c = 0; c < R / 4; ++c)
            *(u32x4_t*)(kst + (4 * c + row + 1) * BGTQ_KST_ROW_BYTES + 16 * col) = kn[c];
        {
            const int u0 = 2 * (lane & 31), reg = lane < 32 ? 0 : 64;
            sst[reg + (u0 & 15) * 4 + (u0 >> 4)] = (uint16_t)(sn & 0xFFFFu);
            sst[reg + ((u0 + 1) & 15) * 4 + ((u0 + 1) >> 4)] = (uint16_t)(sn >> 16);
            if (lane < 32) {
                sst[128 + (u0 & 15) * 4 + (u0 >> 4)] = (uint16_t)(zn & 0xFFFFu);
                sst[128 + ((u0 + 1) & 15) * 4 + ((u0 + 1) >> 4)] = (uint16_t)(zn >> 16);
            }
        }
        wave_lds_fence();
        if (t == t_app) {
            app_patch<R, VB>(a, s_app, lane, u_app, bh, t, kst, sst, vaff, vcur);
            wave_lds_fence();
        }
        asm volatile("" ::: "memory");
        if constexpr (NW <= 8) {
            // unconditional, so that no branch merges the wait counts (the last tile re-reads itself)
            const int64_t tn = t + NW < t_hi ? t + NW : t;
            fetch_k(tn);
            if constexpr (VDB) fetch_v(vnext, tn);
        }

        // q·k on the matrix cores
        f32x4_t c[4];
        if (nks == 0) {
#pragma unroll
            for (int g = 0; g < 4; ++g) c[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (nks > 0) mx_kstep_any<0>(c, lds, s_qa, lane, dks[0], lb, ncc);
        if (nks > 1) mx_kstep_any<1>(c, lds, s_qa, lane, dks[1], lb, ncc);
        if (nks > 2) mx_kstep_any<2>(c, lds, s_qa, lane, dks[2], lb, ncc);
        if (nks > 3) mx_kstep_any<3>(c, lds, s_qa, lane, dks[3], lb, ncc);

        // softmax over the tile: lane holds tokens 16g + col, heads 2row, 2row + 1
        float sk[4], sv[4], sz[4] = {0.f, 0.f, 0.f, 0.f};
        {
            const uint2 k2 = *(const uint2*)(sst + col * 4), v2 = *(const uint2*)(sst + 64 + col * 4);
            sk[0] = h2f(k2.x & 0xFFFFu); sk[1] = h2f(k2.x >> 16); sk[2] = h2f(k2.y & 0xFFFFu); sk[3] = h2f(k2.y >> 16);
            sv[0] = h2f(v2.x & 0xFFFFu); sv[1] = h2f(v2.x >> 16); sv[2] = h2f(v2.y & 0xFFFFu); sv[3] = h2f(v2.y >> 16);
            if (vaff) {
                const uint2 z2 = *(const uint2*)(sst + 128 + col * 4);
                sz[0] = h2f(z2.x & 0xFFFFu); sz[1] = h2f(z2.x >> 16); sz[2] = h2f(z2.y & 0xFFFFu); sz[3] = h2f(z2.y >> 16);
            }
        }
        float z[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) z[g][hh] = sk[g] * (c[g][2 * hh] + c[g][2 * hh + 1]);
        if ((t + 1) * TILE > n_packed) {  // the sequence ends inside this tile
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // scales of tokens past the end are never written: keep them out of the arithmetic
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
            // the wave's first tile: nothing accumulated yet, so no rescale
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

        // P·V on the matrix cores from this lane's value stream
        uint32_t vs[4 * VB];
#pragma unroll
        for (int cc = 0; cc < VB; ++cc) {
            vs[4 * cc] = vcur[cc][0]; vs[4 * cc + 1] = vcur[cc][1]; vs[4 * cc + 2] = vcur[cc][2]; vs[4 * cc + 3] = vcur[cc][3];
        }
        if constexpr (NW > 8) {
            mx_pv<VB, 0, true>(o, vs, s_vlut, wx, lane, lcopy);  // the wave's only tile: start from zero
        } else {
            mx_pv<VB, 0>(o, vs, s_vlut, wx, lane, lcopy);
        }
        mx_pv<VB, 1>(o, vs, s_vlut, wx, lane, lcopy);
        if constexpr (NW <= 8 && !VDB) {
            if (t + NW < t_hi) fetch_v(vcur, t + NW);
        }
    };
    if constexpr (VDB) {
        for (int64_t t = t_lo + wave; t < t_hi; t += 2 * NW) {
            tile(t, vn, vx);
            if (t + NW < t_hi) tile(t + NW, vx, vn);
        }
    } else if constexpr (NW > 8) {
        // one tile per wave (the host sizes the splits so): straight-line code, its loads issued in
        // the prologue; its P·V starts the accumulators, a wave without a tile clears them
        if (t_lo + wave < t_hi) {
            tile(t_lo + wave, vn, vn);
        } else {
#pragma unroll
            for (int db = 0; db < 8; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    } else {
        for (int64_t t = t_lo + wave; t < t_hi; t += NW) tile(t, vn, vn);
    }

    // Epilogue: row sums of l and the zero term, O^T to LDS (over the stages), merge the waves.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        l[hh] = row_sum16(l[hh]);
        zs[hh] = row_sum16(zs[hh]);
    }
    lds_barrier();  // every wave is done with its stages
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
    lds_barrier();
    float* part = a.part + ((size_t)b * a.Hq + (size_t)h * G) * a.n_parts * PART;
    merge_waves_n<G, NW>(s_red, part, a.n_parts, split);
}

template <int G, int VB, int NW>
hipError_t launch_gtq_gvw(const DecodeArgs& a, int B, int R, hipStream_t s) {
    const dim3 grid(a.n_splits, a.Hkv, B), block(64 * NW);
    switch (R) {
        case 8: return launch_main(k_decode_gtq<G, 8, VB, NW>, grid, block, s, a);
        case 12: return launch_main(k_decode_gtq<G, 12, VB, NW>, grid, block, s, a);
        case 16: return launch_main(k_decode_gtq<G, 16, VB, NW>, grid, block, s, a);
    }
    return hipErrorInvalidValue;
}

// Splits of at most kGtqWavesOneTile tiles take the sixteen-wave kernel (one tile per wave,
// straight-line), longer splits the eight-wave kernel that loops over its tiles.
template <int G, int VB>
hipError_t launch_gtq_gv(const DecodeArgs& a, int B, int R, hipStream_t s) {
    if (a.tiles_per_split <= kGtqWavesOneTile) return launch_gtq_gvw<G, VB, kGtqWavesOneTile>(a, B, R, s);
    return launch_gtq_gvw<G, VB, kGtqWavesLoop>(a, B, R, s);
}

template <int G>
hipError_t launch_gtq_g(const DecodeArgs& a, int B, int R, int v_bits, hipStream_t s) {
    switch (v_bits) {
        case 2: return launch_gtq_gv<G, 2>(a, B, R, s);
        case 3: return launch_gtq_gv<G, 3>(a, B, R, s);
        case 4: return launch_gtq_gv<G, 4>(a, B, R, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_plan(const uint8_t* bits, uint8_t* plan, int Hkv, hipStream_t s) {
    if (!bits || !plan || Hkv < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_plan, dim3(Hkv), dim3(64), 0, s, bits, plan);
    return hipGetLastError();
}

hipError_t launch_decode_gtq(const DecodeArgs& a, int B, int R, int v_bits, hipStream_t s) {
    if (!a.plan || B < 1 || B > BGTQ_MAXB) return hipErrorInvalidValue;
    switch (a.G) {
        case 4: return launch_gtq_g<4>(a, B, R, v_bits, s);
        case 8: return launch_gtq_g<8>(a, B, R, v_bits, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace bgtq
