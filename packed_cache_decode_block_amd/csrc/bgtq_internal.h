// Internal declarations shared by the host C-ABI (bgtq_host.cpp) and the HIP kernels
// (bgtq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define BGTQ_MAXB 64  // sequences per call carried in kernel arguments

namespace bgtq {

// Per-(batch, kv head) prep record written by k_prep and read by the decode kernels.
// Offsets in 32-bit words from the record start.
struct PrepLayout {
    int G;
    int qp_words;     // 64 slots x 2 x G q' (sorted Block-GTQ order, sigma folded)
    int qn_words;     // 64 blocks x 2 x G q'' (natural order, no sigma)
    int qs_words;     // affine: 16 groups x G per-group query sums
    int desc_words;   // 32 words: 64 x 16-bit slot descriptors; +1 word nnz_pad
    int stride;       // record size in words (multiple of 64)
    __host__ __device__ int qp() const { return 0; }
    __host__ __device__ int qn() const { return qp_words; }
    __host__ __device__ int qs() const { return qp_words + qn_words; }
    __host__ __device__ int desc() const { return qp_words + qn_words + qs_words; }
};

__host__ __device__ inline PrepLayout prep_layout(int G) {
    PrepLayout p;
    p.G = G;
    p.qp_words = 128 * G;
    p.qn_words = 128 * G;
    p.qs_words = 16 * G;
    p.desc_words = 64;
    int total = p.qp_words + p.qn_words + p.qs_words + p.desc_words;
    p.stride = (total + 63) / 64 * 64;
    return p;
}

// Byte geometry of one layer's buffers.
struct Geometry {
    int B, Hq, Hkv, G;
    int64_t n_cap, n_tiles;
    int k_mode, R;            // K record dwords
    int k_bits, k_group;      // affine keys
    int v_mode, v_bits;
    int n_recent;
    int64_t k_tile_bytes, v_tile_bytes;
    int64_t k_codes_layer, v_codes_layer;     // bytes per layer
    int64_t k_scale_layer, v_scale_layer;     // bytes per layer (fp16 arrays)
    int64_t recent_layer;                     // bytes per layer per ring (K or V)
};

struct PrepArgs {
    const void* q;              // [B][Hq][128] dtype
    int dtype;
    const uint8_t* bits;        // [Hkv][64] for this layer (BLOCKGTQ) or NULL
    const float* sigma;         // [Hkv][64] or NULL
    uint32_t* out;              // ws prep region [B][Hkv][stride]
    int Hkv, G, k_mode, k_group;
    int stride;
};

struct DecodeArgs {
    // layer buffers
    const uint8_t* k_codes;     // [B][Hkv][n_tiles][k_tile_bytes]
    const uint8_t* v_codes;
    const uint16_t* k_scale;    // fp16
    const uint16_t* k_zero;
    const uint16_t* v_scale;
    const uint16_t* v_zero;
    const uint16_t* recent_k;   // fp16 [B][Hkv][n_recent][128]
    const uint16_t* recent_v;
    const uint32_t* prep;       // [B][Hkv][prep stride]
    float* part;                // [B][Hq][n_parts][132]
    int Hkv, Hq, G;
    int64_t n_cap, n_tiles;
    int64_t k_tile_bytes, v_tile_bytes;
    int k_group;
    int n_recent;
    int n_splits;               // packed splits; split index n_splits = recent split
    int n_parts;                // n_splits + (recent ? 1 : 0)
    int tiles_per_split;
    int prep_stride;
    int v_affine;
    int64_t n_packed[BGTQ_MAXB];
    int32_t n_rec[BGTQ_MAXB];
};

struct CombineArgs {
    const float* part;          // [B*Hq][n_parts][132]
    float* out;                 // [B*Hq][128]
    int n_parts;
};

struct Fp16Args {
    const uint16_t* k16;        // [B][Hkv][N][128]
    const uint16_t* v16;
    const uint32_t* prep;
    float* part;
    int Hkv, Hq, G;
    int64_t N;
    int n_splits, tiles_per_split, prep_stride;
};

struct EnergyArgs {
    const void* k;              // [T][Hkv][128]
    const void* q;              // [T][Hq][128]
    int dtype;
    int64_t T;
    int Hkv, G;
    double* out;                // [Hkv][64][2]: sum_t |k_blk|^2, sum_{t,h} |q_blk|^2
};

// One quantize launch writes tokens [pos_lo[b], pos_hi[b]) of every sequence b; the row of
// position p is src + b*sB + ((p - off[b]) mod mod_n)*sT + h*sH (mod_n == 0: no modulo).
// tile0[b] = pos_lo[b] / 64; the grid's x extent covers the largest tile span.
struct QuantArgs {
    const void* src_k;          // key rows (same strides as src_v)
    const void* src_v;
    int dtype;
    int64_t sB, sT, sH;
    int64_t mod_n;
    // destination (one layer)
    uint8_t* k_codes;           // [B][Hkv][n_tiles][k_tile_bytes]
    uint8_t* v_codes;
    uint16_t* k_scale;
    uint16_t* k_zero;
    uint16_t* v_scale;
    uint16_t* v_zero;
    const uint8_t* bits;        // [Hkv][64]
    const float* sigma;
    const float* inv_sigma;
    int Hkv;
    int64_t n_cap, n_tiles, k_tile_bytes, v_tile_bytes;
    int k_mode, R, k_bits, k_group;
    int v_mode, v_bits;
    int which;                  // bit 0: keys, bit 1: values
    int64_t tile0[BGTQ_MAXB];   // first tile touched per sequence
    int64_t pos_lo[BGTQ_MAXB], pos_hi[BGTQ_MAXB], off[BGTQ_MAXB];
};

// Copy rows into the fp16 ring: position p -> slot p % n_recent, for p in [pos_lo[b], pos_hi[b]).
struct RingArgs {
    const void* k;
    const void* v;
    int dtype;
    int64_t sB, sT, sH;
    uint16_t* ring_k;           // [B][Hkv][n_recent][128] for this layer
    uint16_t* ring_v;
    int Hkv, n_recent;
    int64_t pos_lo[BGTQ_MAXB], pos_hi[BGTQ_MAXB], off[BGTQ_MAXB];
};

// Launchers (bgtq_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_prep(const PrepArgs& a, int B, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int B, int k_mode, int R, int v_bits, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int rows, hipStream_t s);
hipError_t launch_fp16(const Fp16Args& a, int B, hipStream_t s);
hipError_t launch_energy(const EnergyArgs& a, hipStream_t s);
hipError_t launch_quant(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t s);
hipError_t launch_ring(const RingArgs& a, int B, int64_t max_rows, hipStream_t s);
bool decode_supported(int k_mode, int R, int k_bits, int k_group, int v_bits, int G);

}  // namespace bgtq
