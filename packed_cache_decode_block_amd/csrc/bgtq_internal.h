// Internal declarations shared by the host C-ABI (bgtq_host.cpp) and the HIP kernels
// (bgtq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bgtq.h"

#define BGTQ_MAXB 64         // sequences per call carried in kernel arguments
#define BGTQ_MAX_PARTS 8192  // split partials per query head merged by the combine kernel
#define BGTQ_KST_ROW_BYTES 320  // stride of the K-record rows staged in LDS by the matrix-core decode

namespace bgtq {

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

struct DecodeArgs {
    // layer buffers
    const uint8_t* k_codes;     // [B][Hkv][n_tiles][k_tile_bytes]
    const uint8_t* v_codes;
    const uint16_t* k_scale;    // fp16
    const uint16_t* k_zero;
    const uint16_t* v_scale;
    const uint16_t* v_zero;
    const void* q;              // [B][Hq][128] in q_dtype
    const uint8_t* bits;        // [Hkv][64] this layer's widths (Block-GTQ)
    const float* sigma;         // [Hkv][64]
    const uint8_t* k_rot;       // [Hkv][16] sign bits of the key rotation (affine keys), or null
    const uint8_t* plan;        // [Hkv][BGTQ_PLAN_BYTES] this layer's decode plan (Block-GTQ keys)
    float* part;                // [B][Hq][n_parts][132]
    int q_dtype;
    int Hkv, Hq, G;
    int64_t n_cap, n_tiles;
    int64_t k_tile_bytes, v_tile_bytes;
    int k_group;
    int n_recent;
    int n_splits;               // packed splits (the fp16 ring, if any, is partial n_splits)
    int n_parts;                // n_splits + (recent ? 1 : 0)
    int tiles_per_split;
    int v_affine;
    int32_t n_packed[BGTQ_MAXB];
    // One-token append in the same launch (the plan-driven kernel, for bgtq_decode_step): with
    // app_k set, the last packed token of every sequence (position n_packed - 1) is quantized
    // from the rows app_k / app_v (element (b, h, j) at b * app_sB + h * app_sH + j, app_dtype)
    // and written to the cache through the app_* pointers (the same buffers as above) by the wave
    // whose tile holds it, which then attends to it with the rest of its tile.
    const void* app_k;
    const void* app_v;
    int app_dtype;
    int64_t app_sB, app_sH;
    const float* inv_sigma;     // [Hkv][64] this layer's 1/sigma
    uint8_t* app_k_codes;
    uint8_t* app_v_codes;
    uint16_t* app_k_scale;
    uint16_t* app_v_scale;
    uint16_t* app_v_zero;
};

struct CombineArgs {
    const float* part;          // [B*Hq][n_parts][132]
    float* out;                 // [B*Hq][128]
    int n_parts;
    const uint8_t* v_rot;       // [Hkv][16] sign bits of the value rotation of this layer, or null
    int Hq, G;                  // row r is query head r % Hq of sequence r / Hq, kv head (r % Hq) / G
    // The fp16 window of a packed cache, attended by the merge itself (k16 null: no window):
    // rows [B][Hkv][rows][128] fp16, the first n_valid[b] of sequence b valid, at most
    // kMergeWindowMax; q [B][Hq][128] in q_dtype.
    const uint16_t* k16;
    const uint16_t* v16;
    const void* q;
    int q_dtype;
    int Hkv;
    int64_t rows;
    int32_t n_valid[BGTQ_MAXB];
};

// Longest fp16 window the split merge attends to itself; a longer one is decoded by a split-K
// launch of its own that writes one more partial.
constexpr int kMergeWindowMax = 512;

// fp16 tiles: rows [B][Hkv][rows][128] fp16.  Used for the unquantized comparator (all splits)
// and for the fp16 recent ring of a packed cache (one extra split written at part index split0).
struct Fp16Args {
    const uint16_t* k16;
    const uint16_t* v16;
    const void* q;              // [B][Hq][128] in q_dtype
    float* part;
    int q_dtype;
    int Hkv, Hq, G;
    int64_t rows;               // rows per (b, h) in memory
    int n_splits, tiles_per_split;
    int split0, n_parts;        // partial index of split 0; partial records per query head
    int32_t n_valid[BGTQ_MAXB]; // valid rows per sequence
};

struct EnergyArgs {
    const void* k;              // [T][Hkv][128]
    const void* q;              // [T][Hq][128]
    int dtype;
    int64_t T;
    int Hkv, G;
    double* out;                // [n_chunks][Hkv][64][2]: sum_t |k_blk|^2, sum_{t,h} |q_blk|^2 per chunk
    int n_chunks;               // token chunks (grid y)
    int64_t tc;                 // tokens per chunk
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
    const uint8_t* k_rot;       // [Hkv][16] sign bits of the key rotation (affine keys), or null
    const uint8_t* v_rot;       // [Hkv][16] sign bits of the value rotation, or null
    int Hkv;
    int64_t n_cap, n_tiles, k_tile_bytes, v_tile_bytes;
    int k_mode, R, k_bits, k_group;
    int v_mode, v_bits;
    int which;                  // bit 0: keys, bit 1: values
    int vec16;                  // set by the launcher: rows and strides allow 16-byte row loads
    int64_t tile0[BGTQ_MAXB];   // first tile touched per sequence
    int64_t pos_lo[BGTQ_MAXB], pos_hi[BGTQ_MAXB], off[BGTQ_MAXB];
    // Gathered source rows (device int32, or null): position p of sequence b reads source row
    // gather[b * gather_stride + p - pos_lo[b]] instead of p - off[b].
    const int32_t* gather;
    int64_t gather_stride;
    int round16;                // rows are rounded to fp16 first (as if they had passed the fp16 store)
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
    const int32_t* gather;      // as QuantArgs::gather (null: row p - off[b])
    int64_t gather_stride;
};

// Reorder the rows of the high-precision store (log-based filter): for a sequence b with
// seq_first[b] >= 0, new row j of every kv head is old row perm[seq_first[b] + j], j < n_recent.
constexpr int BGTQ_PERM_MAX = 1536;   // permutation entries carried in the kernel arguments
constexpr int BGTQ_HP_ROWS_MAX = 512; // store rows a permutation workgroup stages in LDS
struct PermuteArgs {
    uint16_t* rows_k;           // [B][Hkv][n_recent][128] for this layer
    uint16_t* rows_v;
    int Hkv, n_recent;
    int32_t seq_first[BGTQ_MAXB];
    const int16_t* perm_dev;    // the permutation in device memory (caller workspace), or null: perm
    int16_t perm[BGTQ_PERM_MAX];
};

// Launchers (bgtq_kernels.hip; launch_permute in bgtq_logquant.hip).  Return hipSuccess or the
// launch error.
hipError_t launch_permute(const PermuteArgs& a, int B, hipStream_t s);
// Host memory to the device, enqueued on s (the log-based filter's permutations and gather indices).
hipError_t copy_to_device(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int B, int k_mode, int R, int v_bits, bool vector_only, hipStream_t s);
// Block-GTQ keys at g = 4 or 8 (bgtq_decode_gtq.hip): one workgroup of kGtqWaves waves per split.
hipError_t launch_decode_gtq(const DecodeArgs& a, int B, int R, int v_bits, hipStream_t s);
hipError_t launch_plan(const uint8_t* bits, uint8_t* plan, int Hkv, hipStream_t s);
// Waves per workgroup of the Block-GTQ matrix-core decode (one workgroup per compute unit): splits
// of at most kGtqWavesOneTile tiles run one tile per wave, longer ones loop on kGtqWavesLoop waves.
constexpr int kGtqWavesOneTile = 16;
constexpr int kGtqWavesLoop = 8;
// Event pair armed for the next main-kernel launch of this thread (see arm_launch_events).
extern thread_local hipEvent_t t_ev_start, t_ev_stop;
hipError_t launch_combine(const CombineArgs& a, int rows, hipStream_t s);
hipError_t launch_fp16(const Fp16Args& a, int B, hipStream_t s);
hipError_t launch_energy(const EnergyArgs& a, hipStream_t s);
hipError_t launch_quant(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t s);
// Bulk quantize with rows held in registers (bgtq_quant_rows.hip): 16-bit rows in 16-byte chunks,
// Block-GTQ keys and codebook values (either half may be absent).
bool quant_rows_supported(const QuantArgs& a);
hipError_t launch_quant_rows(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t s);
hipError_t launch_ring(const RingArgs& a, int B, int64_t max_rows, hipStream_t s);
bool decode_supported(int k_mode, int R, int k_bits, int k_group, int v_bits, int G);
// Tracing aid: the next decode, fp16-decode or quantize kernel launch on this thread records
// `start` and `stop` around the kernel itself (hipExtLaunchKernelGGL); disarm drops an unused pair.
void arm_launch_events(hipEvent_t start, hipEvent_t stop);
void disarm_launch_events();
int decode_wgs_per_cu(int k_mode, int G, int v_bits, int k_group, bool vector_only);  // resident decode workgroups per CU the split heuristic aims for
// Decode into a workspace the caller did not size (bgtq_decode_attention_noalloc): with
// n_splits == 0 the library's split choice is capped so that the partials fit ws_bytes; an explicit
// n_splits must fit.  Same validation, kernels and error reporting as bgtq_decode_attention.
int decode_capped(const bgtq_cache* c, int layer, const void* q, int dtype, float* out, void* ws, size_t ws_bytes,
                  int n_splits, void* stream);
// Sets the thread's error text (bgtq_last_error) and returns code.
int set_error(int code, const char* fmt, ...);

}  // namespace bgtq
