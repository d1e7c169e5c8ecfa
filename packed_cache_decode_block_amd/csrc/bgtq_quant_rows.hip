// Bulk quantize-append with each token's row held in registers (gfx950, wave64).
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (Block-GTQ; abstract, review
// §1/§3): each key is scaled per token, every RoPE block i is coded against the scalar quantizer's
// thresholds at its own width w_i, and the blocks' code pairs are packed widest first; values are
// coded at one width against the same quantizer.  The arithmetic is the one the tile quantizer
// k_quant spells out (fp32, one IEEE operation at a time, the per-token sum in element order), so
// codes and fp16 scales are the same bits.
//
// One kernel, k_quant_rows: a workgroup of two waves codes either the keys or the values of one
// tile of 64 positions of one (sequence, kv head) (the role is fixed per workgroup, so each wave
// runs one of the two paths), lane = token; wave hw takes elements 64 hw .. 64 hw + 63
// of every row.  A wave reads its 64 half rows with 16-byte loads (eight half rows per
// instruction) and turns them through LDS in four rounds of 16, so that lane t ends with its
// token's 64 elements in 32 registers (element pairs, as stored): the per-token chains read
// registers, not LDS, and each wave carries half of the tile's chains.  The RMS sum keeps its
// element order across the two waves: wave 0 sums its half, wave 1 continues from that partial
// sum and returns the scale.
//  * keys: the blocks of the wave's half in index order, each block's two binary searches over
//    its scaled thresholds, the pair OR-ed into the token's record (in LDS, shared by the two
//    waves) at the bit position the width order gives it;
//  * values: the codes by counting the scaled thresholds each element reaches, exchanged through
//    the wave's LDS in the order the lane streams read them, then each lane assembles the fields
//    of the wave's half of its stream (whole dwords: fields of dims 64 hw .. 64 hw + 63 fill
//    dwords VB (2 sh + hw) .. VB (2 sh + hw + 1) - 1 for token halves sh) with shifts known at
//    compile time.
// Rows that are not 16-byte aligned, fp32 rows, affine formats, the rotations and width or sigma
// arrays off a 4-byte boundary take k_quant.
#include "bgtq_internal.h"

#include <hip/hip_ext.h>

#include "../../include/bgtq.h"
#include "bgtq_device.h"
#include "generated/bgtq_codebook_data.h"

namespace bgtq {
namespace {

constexpr int QR_HALF = 32;                    // element pairs per wave (half a row)
constexpr int QR_ROWS = 16;                    // half rows per LDS round
constexpr int QR_STRIDE = 36;                  // dwords per staged half row: 16-byte reads of 16 lanes hit distinct banks
constexpr int QR_STAGE = QR_ROWS * QR_STRIDE;  // dwords of one round's half rows
constexpr int QR_VSTR = 10;                    // dwords per token in the value-code exchange (conflict-free reads)
constexpr int QR_VAREA = cmax(QR_STAGE, TILE * QR_VSTR);
constexpr int QR_THR = (BGTQ_CB_THRESHOLDS + 3) & ~3;  // threshold words at the start of the key kernel's LDS
constexpr int QR_RMAX = 32;                    // key record dwords at most (budget 512 units)

// LDS words of the key kernel for R-dword records: thresholds, each wave's staging, the records
// (an odd stride of R | 1 dwords per token), the partial sums and the scales.
constexpr int qr_key_words(int R) { return QR_THR + 2 * QR_STAGE + TILE * (R | 1) + 2 * TILE; }
// LDS words of the value role: each wave's staging and code exchange, the partial sums, the scales.
constexpr int qr_value_words = 2 * QR_VAREA + 2 * TILE;

// Element formats: bf16 bits, fp16 bits, and bf16 rows first rounded to fp16 (rows that passed
// an fp16 store).
enum { QR_BF16 = 0, QR_F16 = 1, QR_BF16_TO_F16 = 2 };

template <int MODE> __device__ __forceinline__ float qr_e0(uint32_t p) {
    if constexpr (MODE == QR_BF16) return __builtin_bit_cast(float, p << 16);
    else return h2f(p & 0xFFFFu);
}
template <int MODE> __device__ __forceinline__ float qr_e1(uint32_t p) {
    if constexpr (MODE == QR_BF16) return __builtin_bit_cast(float, p & 0xFFFF0000u);
    else return h2f(p >> 16);
}

// Source element offset of tile position u's row (0 and act = false outside [pos_lo, pos_hi)).
__device__ __forceinline__ int64_t qr_row(const QuantArgs& a, int64_t tile, int b, int h, int u, bool& act) {
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
}

// Lane t receives elements 64 hw .. 64 hw + 63 of token t's row: x[i] = elements 64 hw + 2i (low
// half) and 64 hw + 2i + 1 (high half).  Rows outside the append's range are zero.  stage:
// QR_STAGE dwords of this wave's LDS.
template <int MODE>
__device__ __forceinline__ void qr_load_half(const QuantArgs& a, const uint16_t* src, int64_t tile, int b, int h,
                                             int lane, int hw, uint32_t* stage, uint32_t (&x)[QR_HALF]) {
    // each lane finds its own token's row once; load instruction k reads half rows 8k .. 8k + 7
    // (lane 8 * (row - 8k) + 16-byte chunk) at the offsets their lanes found
    // (rows out of range read the first row in range, or lane 0's row 0 of the sequence when it
    // appends nothing inside a tile another sequence needs, and are zeroed, so that every load is
    // issued unconditionally)
    bool act_mine;
    int64_t off_mine = qr_row(a, tile, b, h, lane, act_mine) + 64 * hw;
    const uint64_t am = __ballot(act_mine);
    const int first = am ? (int)__builtin_ctzll(am) : 0;
    const int64_t off_first = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(off_mine >> 32), first) << 32) |
                                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)off_mine, first));
    if (!act_mine) off_mine = off_first;
    const int32_t off_lo = (int32_t)(uint32_t)off_mine, off_hi = (int32_t)(off_mine >> 32);
    u32x4_t ld[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int u = 8 * k + (lane >> 3);
        const int64_t off =
            (int64_t)(((uint64_t)(uint32_t)__shfl(off_hi, u, 64) << 32) | (uint32_t)__shfl(off_lo, u, 64));
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(src + off + 8 * (lane & 7)));
        ld[k] = ((am >> u) & 1u) ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            *(u32x4_t*)(stage + (8 * k + (lane >> 3)) * QR_STRIDE + 4 * (lane & 7)) = ld[2 * r + k];
        wave_lds_fence();
        if ((lane >> 4) == r) {
            const uint32_t* row = stage + (lane & 15) * QR_STRIDE;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const u32x4_t v = *(const u32x4_t*)(row + 4 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (MODE == QR_BF16_TO_F16)
                        x[4 * c + e] = (uint32_t)f2h(qr_e0<QR_BF16>(v[e])) | ((uint32_t)f2h(qr_e1<QR_BF16>(v[e])) << 16);
                    else
                        x[4 * c + e] = v[e];
                }
            }
        }
        wave_lds_fence();  // the next round overwrites the rows this one read
    }
}

// Hides the row's values from the optimizer between phases, so that each phase converts the
// element pairs it reads again instead of keeping the fp32 elements live from the one before.
// `done`, the previous phase's result, passes first: that phase cannot sink below this point
// (which would keep the row twice).
__device__ __forceinline__ void qr_opaque(uint32_t (&x)[QR_HALF], float& done) {
    asm volatile("" : "+v"(done));
#pragma unroll
    for (int i = 0; i < QR_HALF; ++i) asm volatile("" : "+v"(x[i]));
}

// The per-token RMS sum over the wave's 64 elements, continued from acc: u = x_j * r_(j/2)
// (keys; r: the blocks' 1/sigma, 32 of them from the wave's first block) or x_j (values),
// acc = acc + u*u in element order.
template <int MODE, bool KEYS>
__device__ __forceinline__ float qr_sumsq(const uint32_t (&x)[QR_HALF], float acc, const cu32_t* r) {
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < QR_HALF; ++i) {
        float u0 = qr_e0<MODE>(x[i]), u1 = qr_e1<MODE>(x[i]);
        if constexpr (KEYS) {
            const float ri = __builtin_bit_cast(float, r[i]);
            u0 = u0 * ri;
            u1 = u1 * ri;
        }
        acc = acc + u0 * u0;
        acc = acc + u1 * u1;
    }
    return acc;
}

// The fp16 scale of the row, both waves of the tile: wave 0 sums its half from zero and passes
// the partial sum through s_acc, wave 1 continues it (the sum in element order), forms the mean
// over 128, its square root rounded to fp16, and passes the scale back through s_S.  Contains the
// workgroup's two barriers.
template <int MODE, bool KEYS>
__device__ __forceinline__ float qr_scale16(const uint32_t (&x)[QR_HALF], int hw, int lane, const cu32_t* r,
                                            float* s_acc, float* s_S, uint16_t* s16) {
    float S = 0.f;
    if (hw == 0) s_acc[lane] = qr_sumsq<MODE, KEYS>(x, 0.f, r);
    __syncthreads();
    if (hw == 1) {
        const float acc = qr_sumsq<MODE, KEYS>(x, s_acc[lane], r);
        const float ms = acc / 128.0f;
        *s16 = f2h(sqrtf(ms));
        S = h2f(*s16);
        s_S[lane] = S;
    }
    __syncthreads();
    if (hw == 0) S = s_S[lane];
    return S;
}

// Codes of x0 and x1 among the 2^w - 1 thresholds t * thr[thr_base(w) + m]: the two binary
// searches side by side, each the number of thresholds its coordinate reaches.  q0 and q1 point at
// the table entry of the code found so far; step st (unrolled, taken for st < w) reads the
// threshold 2^st - 1 entries further (an immediate offset) and moves by 2^st if the coordinate
// reaches it.
typedef __attribute__((address_space(3))) const float lds_cf;
__device__ __forceinline__ uint32_t qr_pair(float x0, float x1, float t, int w, lds_cf* thr) {
#pragma clang fp contract(off)
    lds_cf* tb = thr + thr_base(w);
    lds_cf *q0 = tb, *q1 = tb;
#pragma unroll
    for (int st = 7; st >= 0; --st) {
        if (st < w) {
            const float th0 = t * q0[(1 << st) - 1], th1 = t * q1[(1 << st) - 1];
            if (x0 >= th0) q0 += 1 << st;
            if (x1 >= th1) q1 += 1 << st;
        }
    }
    // LDS addresses are 32-bit: the codes are the byte distances over 4
    const uint32_t a0 = (uint32_t)(uintptr_t)tb;
    return (((uint32_t)(uintptr_t)q0 - a0) >> 2) | ((((uint32_t)(uintptr_t)q1 - a0) >> 2) << w);
}

// Keys: Block-GTQ records and fp16 scales of tile tile0[b] + tx.  LDS: qr_key_words(R) words.
template <int MODE>
__device__ __forceinline__ void qr_keys_tile(const QuantArgs& a, int64_t tx, uint32_t* s_dyn) {
    const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
    const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile = a.tile0[b] + tx;
    if (tile * TILE >= a.pos_hi[b]) return;  // whole workgroup beyond this sequence's range
    const int R = a.R;
    float* s_thr = (float*)s_dyn;
    uint32_t* stage = s_dyn + QR_THR + hw * QR_STAGE;
    uint32_t* recs = s_dyn + QR_THR + 2 * QR_STAGE;
    float* s_acc = (float*)(recs + TILE * (R | 1));
    float* s_S = s_acc + TILE;
    // block `lane`'s width (above 8 is invalid metadata: clamped), requested ahead of the rows;
    // the blocks' widths, sigmas and 1/sigmas are read again below as scalars
    int w = a.bits[h * 64 + lane];
    for (int i = threadIdx.x; i < BGTQ_CB_THRESHOLDS; i += 128) s_thr[i] = __builtin_bit_cast(float, c_thr32[i]);
    uint32_t* rec = recs + lane * (R | 1);  // odd stride: one bank per token
    if (hw == 0)
        for (int k = 0; k < R; ++k) rec[k] = 0u;
    uint32_t x[QR_HALF];
    qr_load_half<MODE>(a, (const uint16_t*)a.src_k, tile, b, h, lane, hw, stage, x);
    w = w < 8 ? w : 8;
    // bit position of block lane's pair in the record: the pairs of wider blocks, and of equally
    // wide blocks of lower index, come first (one ballot per width, widest first)
    int bp = 0, wider = 0;
#pragma unroll
    for (int v = 8; v >= 1; --v) {
        const uint64_t m = __ballot(w == v);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (w == v) bp = wider + 2 * v * below;
        wider += 2 * v * __popcll(m);
    }
    const int i0 = QR_HALF * hw;  // the wave's first block
    uint16_t s16 = 0;
    float S = qr_scale16<MODE, true>(x, hw, lane, (const cu32_t*)(a.inv_sigma + h * 64 + i0), s_acc, s_S, &s16);
    qr_opaque(x, S);
    const cu32_t* wbytes = (const cu32_t*)(a.bits + h * 64 + i0);  // four widths per dword
    const cu32_t* sgw = (const cu32_t*)(a.sigma + h * 64 + i0);
#pragma unroll
    for (int i = 0; i < QR_HALF; ++i) {
        int wi = (int)((wbytes[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        wi = wi < 8 ? wi : 8;
        if (wi == 0) continue;
        float t;
        {
#pragma clang fp contract(off)
            t = S * __builtin_bit_cast(float, sgw[i]);
        }
        const uint32_t pr = qr_pair(qr_e0<MODE>(x[i]), qr_e1<MODE>(x[i]), t, wi, (lds_cf*)s_thr);
        const int bpi = __builtin_amdgcn_readlane(bp, i0 + i), d = bpi >> 5, sh = bpi & 31;
        // widths summing past the budget (invalid metadata) never write past the record
        if (d < R) __hip_atomic_fetch_or(rec + d, pr << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (sh + 2 * wi > 32 && d + 1 < R)
            __hip_atomic_fetch_or(rec + d + 1, pr >> (32 - sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();  // both halves of every record are in
    const int64_t pos = tile * TILE + lane;
    if (pos >= a.pos_lo[b] && pos < a.pos_hi[b]) {
        const size_t bh = (size_t)b * a.Hkv + h;
        uint32_t* kt = (uint32_t*)(a.k_codes + (bh * a.n_tiles + tile) * a.k_tile_bytes);
        for (int k = hw; k < R; k += 2) __builtin_nontemporal_store(rec[k], kt + k * TILE + lane);
        if (hw == 1) a.k_scale[bh * a.n_cap + pos] = s16;
    }
}

// Values (tile tile0[b] + tx; LDS: qr_value_words words): codes at width VB, fp16 scales and the tile's lane streams (stream L = dd + 16 jj holds,
// at field phi = 32 sh + 4 db + m, the codes of dim 16 db + dd for tokens p = 16 sh + 4 jj + m and
// p + 32).  Wave hw holds dims 64 hw .. 64 hw + 63, i.e. db = 4 hw + dbl (dbl 0..3).
template <int MODE, int VB>
__device__ __forceinline__ void qr_values_tile(const QuantArgs& a, int64_t tx, uint32_t* s_dyn) {
    const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
    const int hw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile = a.tile0[b] + tx;
    if (tile * TILE >= a.pos_hi[b]) return;  // whole workgroup beyond this sequence's range
    uint32_t* area = s_dyn + hw * QR_VAREA;
    float* s_acc = (float*)(s_dyn + 2 * QR_VAREA);
    float* s_S = s_acc + TILE;
    const int64_t pos = tile * TILE + lane;
    const bool active = pos >= a.pos_lo[b] && pos < a.pos_hi[b];
    uint32_t x[QR_HALF];
    qr_load_half<MODE>(a, (const uint16_t*)a.src_v, tile, b, h, lane, hw, area, x);
    uint16_t s16 = 0;
    float S = qr_scale16<MODE, false>(x, hw, lane, nullptr, s_acc, s_S, &s16);
    qr_opaque(x, S);
    constexpr int NT = (1 << VB) - 1;
    float th[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma clang fp contract(off)
        th[m] = S * __builtin_bit_cast(float, c_thr32[thr_base_c(VB) + m]);
    }
    // exchange word q of the token: the codes of dims dd = 2q (bits 4 dbl) and 2q + 1 (bits
    // 16 + 4 dbl) of the wave's four 16-dim groups, i.e. of x[8 dbl + q]'s two halves
    uint32_t* mine = area + lane * QR_VSTR;
#pragma unroll
    for (int q = 0; q < 8; q += 2) {
        uint32_t wd[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            wd[e] = 0u;
#pragma unroll
            for (int dbl = 0; dbl < 4; ++dbl) {
                const uint32_t p = x[8 * dbl + q + e];
                const float v0 = qr_e0<MODE>(p), v1 = qr_e1<MODE>(p);
                uint32_t c0 = 0, c1 = 0;
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    c0 += v0 >= th[m] ? 1u : 0u;
                    c1 += v1 >= th[m] ? 1u : 0u;
                }
                wd[e] |= (c0 << (4 * dbl)) | (c1 << (16 + 4 * dbl));
            }
        }
        *(uint2*)(mine + q) = active ? make_uint2(wd[0], wd[1]) : make_uint2(0u, 0u);
    }
    wave_lds_fence();
    const int dd = lane & 15, jj = lane >> 4;
    const int sel = 16 * (dd & 1);
    uint32_t cw[2][4][2];  // [sh][m][+32]: the exchange word holding this lane's dim column for each token
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
                cw[sh][m][t2] = area[(16 * sh + 4 * jj + m + 32 * t2) * QR_VSTR + (dd >> 1)] >> sel;
    constexpr uint32_t CM = (1u << VB) - 1u;
    // st[sh][k]: stream dword VB (2 sh + hw) + k, fields 32 sh + 16 hw + 4 dbl + m at local bit
    // 2 VB (4 dbl + m)
    uint32_t st[2][VB];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
        for (int k = 0; k < VB; ++k) st[sh][k] = 0u;
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            const int dbl = f >> 2, m = f & 3;
            const uint32_t v = ((cw[sh][m][0] >> (4 * dbl)) & CM) | (((cw[sh][m][1] >> (4 * dbl)) & CM) << VB);
            const int bit = 2 * VB * f;
            st[sh][bit >> 5] |= v << (bit & 31);
            if ((bit & 31) + 2 * VB > 32) st[sh][(bit >> 5) + 1] |= v >> (32 - (bit & 31));
        }
    }
    const size_t bh = (size_t)b * a.Hkv + h;
    uint32_t* vt = (uint32_t*)(a.v_codes + (bh * a.n_tiles + tile) * a.v_tile_bytes);
    const int64_t t0 = tile * TILE;
    const int lo = a.pos_lo[b] > t0 ? (int)(a.pos_lo[b] - t0) : 0;
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
        // the tile's first lo tokens were appended before: their fields keep their bits
        uint32_t mk[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k) mk[k] = 0u;
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            const int p = 16 * sh + 4 * jj + (f & 3);
            const uint32_t v = (p >= lo ? CM : 0u) | (p + 32 >= lo ? CM << VB : 0u);
            const int bit = 2 * VB * f;
            mk[bit >> 5] |= v << (bit & 31);
            if ((bit & 31) + 2 * VB > 32) mk[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
        }
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            const int c = VB * (2 * sh + hw) + k;
            uint32_t* dst = vt + ((c >> 2) * 64 + lane) * 4 + (c & 3);
            if (mk[k] == 0xFFFFFFFFu) __builtin_nontemporal_store(st[sh][k], dst);
            else if (mk[k]) *dst = (*dst & ~mk[k]) | (st[sh][k] & mk[k]);
        }
    }
    if (hw == 1 && active) a.v_scale[bh * a.n_cap + pos] = s16;
}

// One launch for a layer's bulk append: workgroup x codes the keys (even x) or the values (odd x)
// of tile x / 2 when both are appended, else the one half of tile x.  The two roles interleave in
// launch order, so the rows of workgroups that start later load while earlier ones code theirs.
template <int MODE, int VB>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(MODE == QR_BF16 ? 6 : 4))) void k_quant_rows(const QuantArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];
    const bool both = (a.which & 3) == 3;
    const int64_t tx = both ? (int64_t)(blockIdx.x >> 1) : (int64_t)blockIdx.x;
    const bool keys = both ? (blockIdx.x & 1) == 0 : (a.which & 1) != 0;
    if (keys) qr_keys_tile<MODE>(a, tx, s_dyn);
    else qr_values_tile<MODE, VB>(a, tx, s_dyn);
}

template <int MODE>
hipError_t launch_rows(const QuantArgs& a, int64_t max_tiles, int Hkv, int B, hipStream_t s) {
    const bool keys = a.which & 1, values = (a.which >> 1) & 1;
    const dim3 grid((unsigned)(max_tiles * (keys && values ? 2 : 1)), Hkv, B);
    const int words = cmax(keys ? qr_key_words(a.R) : 0, values ? qr_value_words : 0);
    auto k = a.v_bits == 1 ? k_quant_rows<MODE, 1>
           : a.v_bits == 2 ? k_quant_rows<MODE, 2>
           : a.v_bits == 3 ? k_quant_rows<MODE, 3>
                           : k_quant_rows<MODE, 4>;
    if (t_ev_start) {
        hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
        t_ev_start = t_ev_stop = nullptr;
        hipExtLaunchKernelGGL(k, grid, dim3(128), (size_t)(4 * words), s, e0, e1, 0, a);
    } else {
        hipLaunchKernelGGL(k, grid, dim3(128), (size_t)(4 * words), s, a);
    }
    return hipGetLastError();
}

}  // namespace

bool quant_rows_supported(const QuantArgs& a) {
    // the key kernel reads the widths, sigmas and 1/sigmas as scalar dwords: 4-byte aligned arrays
    const bool meta4 = (uintptr_t)a.bits % 4 == 0 && (uintptr_t)a.sigma % 4 == 0 && (uintptr_t)a.inv_sigma % 4 == 0;
    return a.dtype != BGTQ_F32 && a.vec16 && a.R >= 1 && a.R <= QR_RMAX && a.v_bits >= 1 && a.v_bits <= 4 &&
           (!(a.which & 1) || (a.k_mode == BGTQ_K_BLOCKGTQ && meta4)) && (!(a.which & 2) || a.v_mode == BGTQ_V_CODEBOOK);
}

hipError_t launch_quant_rows(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t s) {
    if (!quant_rows_supported(a)) return hipErrorInvalidValue;
    if (a.dtype == BGTQ_F16) return launch_rows<QR_F16>(a, max_tiles, a.Hkv, B, s);
    if (a.round16) return launch_rows<QR_BF16_TO_F16>(a, max_tiles, a.Hkv, B, s);
    return launch_rows<QR_BF16>(a, max_tiles, a.Hkv, B, s);
}

}  // namespace bgtq
