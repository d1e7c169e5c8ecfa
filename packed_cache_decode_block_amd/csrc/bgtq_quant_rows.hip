// Bulk quantize-append with each token's row held in registers (gfx950, wave64).
//
// Method: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (Block-GTQ; abstract, review
// §1/§3): each key is scaled per token, every RoPE block i is coded against the scalar quantizer's
// thresholds at its own width w_i, and the blocks' code pairs are packed widest first; values are
// coded at one width against the same quantizer.  The arithmetic is the one the tile quantizer
// k_quant spells out (fp32, one IEEE operation at a time, the per-token sum in element order), so
// codes and fp16 scales are the same bits.
//
// Two kernels, one wave per workgroup and one workgroup per tile of 64 positions of one
// (sequence, kv head), lane = token: k_quant_rows_keys codes the keys, then k_quant_rows_values
// the values (each is its own register allocation: one kernel holding both needs the registers of
// both).  A wave reads its 64 rows with 16-byte loads (four whole rows per instruction) and turns
// them through LDS in four rounds of 16 rows, so that lane t ends with token t's 128 elements in
// 64 registers (element pairs, as stored).  The per-token chains then read registers, not LDS,
// and a wave needs 4-10 KB of LDS instead of a staged tile of 16.6 KB.
//  * keys: the RMS chain over the 128 elements, then the blocks in index order, each block's two
//    binary searches over its scaled thresholds, the pair OR-ed into the token's record at the
//    bit position the width order gives it (positions from the widths of all blocks, computed
//    once per wave; the record is assembled in LDS, one row of dwords per lane);
//  * values: the RMS chain, the codes by counting the scaled thresholds each element reaches, 8
//    codes per dword in the order the lane streams read them, exchanged through LDS, then each
//    lane assembles its own stream of 64 fields with shifts known at compile time.
// Rows that are not 16-byte aligned, fp32 rows, affine formats and the rotations take k_quant.
#include "bgtq_internal.h"

#include <hip/hip_ext.h>

#include "../../include/bgtq.h"
#include "bgtq_device.h"
#include "generated/bgtq_codebook_data.h"

namespace bgtq {
namespace {

constexpr int QR_ROWS = 16;                    // rows per LDS round
constexpr int QR_STRIDE = 68;                  // dwords per staged row: 16-byte reads of 16 lanes hit distinct banks
constexpr int QR_STAGE = QR_ROWS * QR_STRIDE;  // dwords of one round's rows
constexpr int QR_VSTR = 20;                    // dwords per token in the value-code exchange (conflict-free both ways)
constexpr int QR_VAREA = cmax(QR_STAGE, TILE * QR_VSTR);
constexpr int QR_THR = (BGTQ_CB_THRESHOLDS + 3) & ~3;  // threshold words ahead of the key wave's area
constexpr int QR_RMAX = 32;                    // key record dwords at most (budget 512 units)

// LDS bytes of the key kernel for R-dword records: thresholds, then the larger of one round's
// rows and the records (an odd stride of R | 1 dwords per lane).
constexpr int qr_key_lds(int R) { return 4 * (QR_THR + cmax(QR_STAGE, TILE * (R | 1))); }

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

// Lane t receives token t's row: x[i] = elements 2i (low half) and 2i + 1 (high half).  Rows
// outside the append's range are zero.  area: QR_STAGE dwords of this wave's LDS.
template <int MODE>
__device__ __forceinline__ void qr_load_rows(const QuantArgs& a, const uint16_t* src, int64_t tile, int b, int h,
                                             int lane, uint32_t* area, uint32_t (&x)[64]) {
    // each lane finds its own token's row once; load instruction k reads rows 4k .. 4k + 3 (lane
    // 16 * (row - 4k) + 16-byte chunk) at the offsets their lanes found
    bool act_mine;
    const int64_t off_mine = qr_row(a, tile, b, h, lane, act_mine);
    const int32_t off_lo = (int32_t)(uint32_t)off_mine, off_hi = (int32_t)(off_mine >> 32);
    const int32_t act_i = act_mine ? 1 : 0;
    u32x4_t ld[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int u = 4 * k + (lane >> 4);
        const int64_t off =
            (int64_t)(((uint64_t)(uint32_t)__shfl(off_hi, u, 64) << 32) | (uint32_t)__shfl(off_lo, u, 64));
        ld[k] = u32x4_t{0u, 0u, 0u, 0u};
        if (__shfl(act_i, u, 64)) ld[k] = __builtin_nontemporal_load((const u32x4_t*)(src + off + 8 * (lane & 15)));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *(u32x4_t*)(area + (4 * k + (lane >> 4)) * QR_STRIDE + 4 * (lane & 15)) = ld[4 * r + k];
        wave_lds_fence();
        if ((lane >> 4) == r) {
            const uint32_t* row = area + (lane & 15) * QR_STRIDE;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
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
// element pairs it reads again instead of keeping all 128 fp32 elements live from the one before.
// `done`, the previous phase's result, passes first: that phase cannot sink below this point
// (which would keep the row twice).
__device__ __forceinline__ void qr_opaque(uint32_t (&x)[64], float& done) {
    asm volatile("" : "+v"(done));
#pragma unroll
    for (int i = 0; i < 64; ++i) asm volatile("" : "+v"(x[i]));
}

// fp16 RMS scale of the row: u = x_j * r_(j/2) (keys) or x_j (values), u*u summed in element
// order, mean over 128, square root, rounded to fp16.  rr: lane i holds block i's 1/sigma.
template <int MODE, bool KEYS>
__device__ __forceinline__ float qr_rms16(const uint32_t (&x)[64], float rr, uint16_t* s16) {
#pragma clang fp contract(off)
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        float u0 = qr_e0<MODE>(x[i]), u1 = qr_e1<MODE>(x[i]);
        if constexpr (KEYS) {
            const float r = lane_f(rr, i);
            u0 = u0 * r;
            u1 = u1 * r;
        }
        acc = acc + u0 * u0;
        acc = acc + u1 * u1;
    }
    const float ms = acc / 128.0f;
    const uint16_t h = f2h(sqrtf(ms));
    *s16 = h;
    return h2f(h);
}

// Codes of x0 and x1 among the 2^w - 1 thresholds t * thr[thr_base(w) + m]: the two binary
// searches side by side, each the number of thresholds its coordinate reaches.
__device__ __forceinline__ uint32_t qr_pair(float x0, float x1, float t, int w, const float* thr) {
#pragma clang fp contract(off)
    const float* tb = thr + thr_base(w);
    uint32_t c0 = 0, c1 = 0;
    for (int st = w - 1; st >= 0; --st) {
        const uint32_t n0 = c0 + (1u << st), n1 = c1 + (1u << st);
        const float th0 = t * tb[n0 - 1], th1 = t * tb[n1 - 1];
        if (x0 >= th0) c0 = n0;
        if (x1 >= th1) c1 = n1;
    }
    return c0 | (c1 << w);
}

// Keys: Block-GTQ records and fp16 scales of one tile.  Dynamic LDS: qr_key_lds(R) bytes.
template <int MODE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void k_quant_rows_keys(const QuantArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];
    const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int64_t tile = a.tile0[b] + blockIdx.x;
    if (tile * TILE >= a.pos_hi[b]) return;  // beyond this sequence's range
    float* s_thr = (float*)s_dyn;
    uint32_t* area = s_dyn + QR_THR;
    // block `lane`'s width (above 8 is invalid metadata: clamped), sigma and 1/sigma, requested
    // ahead of the rows
    int w = a.bits[h * 64 + lane];
    const float sg = a.sigma[h * 64 + lane], rr = a.inv_sigma[h * 64 + lane];
    for (int i = lane; i < BGTQ_CB_THRESHOLDS; i += 64) s_thr[i] = __builtin_bit_cast(float, c_thr32[i]);
    uint32_t x[64];
    qr_load_rows<MODE>(a, (const uint16_t*)a.src_k, tile, b, h, lane, area, x);
    w = w < 8 ? w : 8;
    // bit position of block lane's pair in the record: the pairs of wider blocks, and of equally
    // wide blocks of lower index, come first
    int bp = 0;
    for (int j = 0; j < 64; ++j) {
        const int wj = __builtin_amdgcn_readlane(w, j);
        bp += ((wj > w) | ((wj == w) & (j < lane))) ? 2 * wj : 0;
    }
    uint16_t s16;
    float S = qr_rms16<MODE, true>(x, rr, &s16);
    qr_opaque(x, S);
    const int R = a.R;
    uint32_t* rec = area + lane * (R | 1);  // odd stride: one bank per lane
    for (int k = 0; k < R; ++k) rec[k] = 0u;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        const int wi = __builtin_amdgcn_readlane(w, i);
        if (wi == 0) continue;
        float t;
        {
#pragma clang fp contract(off)
            t = S * lane_f(sg, i);
        }
        const uint32_t pr = qr_pair(qr_e0<MODE>(x[i]), qr_e1<MODE>(x[i]), t, wi, s_thr);
        const int bpi = __builtin_amdgcn_readlane(bp, i), d = bpi >> 5, sh = bpi & 31;
        // widths summing past the budget (invalid metadata) never write past the record
        if (d < R) __hip_atomic_fetch_or(rec + d, pr << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        if (sh + 2 * wi > 32 && d + 1 < R)
            __hip_atomic_fetch_or(rec + d + 1, pr >> (32 - sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
    wave_lds_fence();
    const int64_t pos = tile * TILE + lane;
    if (pos >= a.pos_lo[b] && pos < a.pos_hi[b]) {
        const size_t bh = (size_t)b * a.Hkv + h;
        uint32_t* kt = (uint32_t*)(a.k_codes + (bh * a.n_tiles + tile) * a.k_tile_bytes);
        for (int k = 0; k < R; ++k) __builtin_nontemporal_store(rec[k], kt + k * TILE + lane);
        a.k_scale[bh * a.n_cap + pos] = s16;
    }
}

// Values: codes at width VB, fp16 scales and the tile's lane streams (stream L = dd + 16 jj holds,
// at field phi = 32 sh + 4 db + m, the codes of dim 16 db + dd for tokens p = 16 sh + 4 jj + m and
// p + 32).
template <int MODE, int VB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void k_quant_rows_values(const QuantArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t area[QR_VAREA];
    const int h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int64_t tile = a.tile0[b] + blockIdx.x;
    if (tile * TILE >= a.pos_hi[b]) return;  // beyond this sequence's range
    const int64_t pos = tile * TILE + lane;
    const bool active = pos >= a.pos_lo[b] && pos < a.pos_hi[b];
    uint32_t x[64];
    qr_load_rows<MODE>(a, (const uint16_t*)a.src_v, tile, b, h, lane, area, x);
    uint16_t s16;
    float S = qr_rms16<MODE, false>(x, 0.f, &s16);
    qr_opaque(x, S);
    constexpr int NT = (1 << VB) - 1;
    float th[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma clang fp contract(off)
        th[m] = S * __builtin_bit_cast(float, c_thr32[thr_base_c(VB) + m]);
    }
    // dwords 2dp and 2dp + 1 of the token's exchange row: the codes of dims 16 db + 2dp and
    // 16 db + 2dp + 1 (the two halves of x[8 db + dp]) at bits 4 db, written as each pair is done
    uint32_t* mine = area + lane * QR_VSTR;
#pragma unroll
    for (int dp = 0; dp < 8; ++dp) {
        uint32_t n0 = 0u, n1 = 0u;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const float v0 = qr_e0<MODE>(x[8 * db + dp]), v1 = qr_e1<MODE>(x[8 * db + dp]);
            uint32_t c0 = 0, c1 = 0;
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                c0 += v0 >= th[m] ? 1u : 0u;
                c1 += v1 >= th[m] ? 1u : 0u;
            }
            n0 |= c0 << (4 * db);
            n1 |= c1 << (4 * db);
        }
        *(uint2*)(mine + 2 * dp) = active ? make_uint2(n0, n1) : make_uint2(0u, 0u);
    }
    wave_lds_fence();
    const int dd = lane & 15, jj = lane >> 4;
    uint32_t cw[2][4][2];  // [sh][m][+32]: the code dword of this lane's dim column for each token
#pragma unroll
    for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) cw[sh][m][t2] = area[(16 * sh + 4 * jj + m + 32 * t2) * QR_VSTR + dd];
    constexpr int NW = 4 * VB;  // dwords per stream
    constexpr uint32_t CM = (1u << VB) - 1u;
    uint32_t st[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) st[k] = 0u;
#pragma unroll
    for (int phi = 0; phi < 64; ++phi) {
        const int m = phi & 3, db = (phi >> 2) & 7, sh = phi >> 5;
        const uint32_t f = ((cw[sh][m][0] >> (4 * db)) & CM) | (((cw[sh][m][1] >> (4 * db)) & CM) << VB);
        const int bit = 2 * VB * phi;
        st[bit >> 5] |= f << (bit & 31);
        if ((bit & 31) + 2 * VB > 32) st[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
    }
    const size_t bh = (size_t)b * a.Hkv + h;
    uint32_t* vt = (uint32_t*)(a.v_codes + (bh * a.n_tiles + tile) * a.v_tile_bytes);
    const int64_t t0 = tile * TILE;
    const int lo = a.pos_lo[b] > t0 ? (int)(a.pos_lo[b] - t0) : 0;
    if (lo == 0) {
#pragma unroll
        for (int g = 0; g < VB; ++g)
            __builtin_nontemporal_store(u32x4_t{st[4 * g], st[4 * g + 1], st[4 * g + 2], st[4 * g + 3]},
                                        (u32x4_t*)(vt + (g * 64 + lane) * 4));
    } else {
        // the tile's first lo tokens were appended before: their fields keep their bits
        uint32_t mk[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) mk[k] = 0u;
#pragma unroll
        for (int phi = 0; phi < 64; ++phi) {
            const int m = phi & 3, sh = phi >> 5;
            const int p = 16 * sh + 4 * jj + m;
            const uint32_t f = (p >= lo ? CM : 0u) | (p + 32 >= lo ? CM << VB : 0u);
            const int bit = 2 * VB * phi;
            mk[bit >> 5] |= f << (bit & 31);
            if ((bit & 31) + 2 * VB > 32) mk[(bit >> 5) + 1] |= f >> (32 - (bit & 31));
        }
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            uint32_t* dst = vt + ((k >> 2) * 64 + lane) * 4 + (k & 3);
            if (mk[k] == 0xFFFFFFFFu) *dst = st[k];
            else if (mk[k]) *dst = (*dst & ~mk[k]) | (st[k] & mk[k]);
        }
    }
    if (active) a.v_scale[bh * a.n_cap + pos] = s16;
}

template <int MODE>
hipError_t launch_rows(const QuantArgs& a, dim3 grid, hipStream_t s) {
    // an armed event pair spans both launches: start with the keys, stop after the values
    hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    const bool keys = a.which & 1, values = (a.which >> 1) & 1;
    if (keys) {
        hipExtLaunchKernelGGL(k_quant_rows_keys<MODE>, grid, dim3(64), (size_t)qr_key_lds(a.R), s, e0,
                              values ? nullptr : e1, 0, a);
        if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (values) {
        auto kv = a.v_bits == 1 ? k_quant_rows_values<MODE, 1>
                : a.v_bits == 2 ? k_quant_rows_values<MODE, 2>
                : a.v_bits == 3 ? k_quant_rows_values<MODE, 3>
                                : k_quant_rows_values<MODE, 4>;
        hipExtLaunchKernelGGL(kv, grid, dim3(64), 0, s, keys ? nullptr : e0, e1, 0, a);
        if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

bool quant_rows_supported(const QuantArgs& a) {
    return a.dtype != BGTQ_F32 && a.vec16 && a.R >= 1 && a.R <= QR_RMAX && a.v_bits >= 1 && a.v_bits <= 4 &&
           (!(a.which & 1) || a.k_mode == BGTQ_K_BLOCKGTQ) && (!(a.which & 2) || a.v_mode == BGTQ_V_CODEBOOK);
}

hipError_t launch_quant_rows(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t s) {
    if (!quant_rows_supported(a)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)max_tiles, a.Hkv, B);
    if (a.dtype == BGTQ_F16) return launch_rows<QR_F16>(a, grid, s);
    if (a.round16) return launch_rows<QR_BF16_TO_F16>(a, grid, s);
    return launch_rows<QR_BF16>(a, grid, s);
}

}  // namespace bgtq
