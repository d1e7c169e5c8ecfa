/*
 * bgtq.h — C ABI of the packed-cache decode library for MI355X (gfx950).
 *
 * Decode attention served directly from a low-bit packed KV cache.  Keys carry per-RoPE-block
 * integer bit widths chosen by Block-GTQ's greedy allocator; values carry one uniform width.
 * Sources: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (abstract; review §1 Key
 * Terms, §3 Method & Key Results, Figures 1-2), "Quantize What Counts" technical summary
 * (Results: group-size sensitivity, K4V2), "LogQuant" technical summary (Method 2 recent
 * window, Method 4 position-agnostic concatenation).
 *
 * Conventions shared by every call:
 *  - Every function returns an int status: BGTQ_OK (0) or a negative BGTQ_E_* code;
 *    bgtq_last_error() returns a thread-local message for the last failure.
 *  - Pointers named "device" are device memory the caller allocated (e.g. torch tensors) and
 *    still owns; "host" pointers are ordinary host memory.  The library never allocates,
 *    frees or synchronizes device memory, except where a call says it is synchronous.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Device work is
 *    enqueued on it and returns immediately.
 *  - Arguments are validated on the host before anything is enqueued; a failed check
 *    returns BGTQ_E_INVALID / BGTQ_E_UNSUPPORTED / BGTQ_E_BUDGET / BGTQ_E_CAPACITY and has no
 *    side effect.  A failed launch returns BGTQ_E_HIP.  No C++ exception crosses the ABI.
 *  - Head dimension d is 128 (64 RoPE blocks of 2 coordinates, interleaved pairs (2i, 2i+1)).
 *  - Cached values must be finite with |x| <= 65504 and give finite fp16 scales; other
 *    inputs give undefined codes (they cannot be checked without reading device memory).
 */
#ifndef BGTQ_H
#define BGTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    BGTQ_OK = 0,
    BGTQ_E_INVALID = -1,      /* bad pointer, shape, layer, size or workspace */
    BGTQ_E_UNSUPPORTED = -2,  /* valid request outside what the kernels implement */
    BGTQ_E_BUDGET = -3,       /* bit budget infeasible for the allocator */
    BGTQ_E_CAPACITY = -4,     /* append would exceed the cache capacity */
    BGTQ_E_HIP = -5           /* a HIP runtime call or kernel launch failed */
};

enum { BGTQ_F32 = 0, BGTQ_F16 = 1, BGTQ_BF16 = 2 };          /* activation dtypes */
enum { BGTQ_SCORE_QK = 0, BGTQ_SCORE_K = 1 };               /* energy score modes */
enum { BGTQ_K_BLOCKGTQ = 0, BGTQ_K_AFFINE = 1 };            /* key formats */
enum { BGTQ_V_CODEBOOK = 0, BGTQ_V_AFFINE = 1 };            /* value formats */

/* Buffer selectors for bgtq_cache_bytes. */
enum {
    BGTQ_BUF_K_CODES = 0, BGTQ_BUF_V_CODES = 1, BGTQ_BUF_K_SCALE = 2, BGTQ_BUF_K_ZERO = 3,
    BGTQ_BUF_V_SCALE = 4, BGTQ_BUF_V_ZERO = 5, BGTQ_BUF_RECENT_K = 6, BGTQ_BUF_RECENT_V = 7,
    BGTQ_BUF_META = 8,        /* bits + sigma + inv_sigma, for reference */
    BGTQ_BUF_PLAN = 9         /* decode plan: BGTQ_PLAN_BYTES per (layer, kv head), Block-GTQ keys */
};

#define BGTQ_HEAD_DIM 128
#define BGTQ_N_BLOCKS 64
#define BGTQ_TILE 64
#define BGTQ_MAX_BATCH 64
#define BGTQ_ENERGY_CHUNK 16   /* calibration tokens per workgroup of bgtq_block_energy */
#define BGTQ_PLAN_BYTES 512    /* decode plan bytes per (layer, kv head) */

/* Decode kernel family of a cache (bgtq_cache.decode_path). */
enum {
    BGTQ_DECODE_AUTO = 0,   /* the library's choice: matrix cores for g >= 4, vector ALUs below */
    BGTQ_DECODE_VECTOR = 1  /* q·k and P·V on the vector ALUs for every format and head ratio */
};

/*
 * Packed KV cache descriptor (plain data; the caller fills it and owns every buffer).
 *
 * Geometry: L layers, B sequences, Hq query heads, Hkv KV heads (Hq % Hkv == 0, g = Hq/Hkv in
 * {1, 2, 4, 8}), d = 128, n_cap = packed-token capacity per (layer, sequence), a multiple of 64.
 *
 * Key format (k_mode):
 *   BGTQ_K_BLOCKGTQ — per-block widths bits[l][h][i] in 0..8 with sum == budget_units (a
 *     multiple of 16); each token stores 2*budget_units bits plus one fp16 scale.
 *   BGTQ_K_AFFINE — every coordinate k_bits (2, 4 or 8) bits; fp16 scale and zero per group
 *     of k_group (8..128, divides 128) coordinates of one token.
 * Value format (v_mode): v_bits in 1..4 per coordinate;
 *   BGTQ_V_CODEBOOK — one fp16 scale per token (uniform TQ-MSE width);
 *   BGTQ_V_AFFINE — fp16 scale and zero per token (group = 128).
 * n_recent > 0 keeps the newest n_recent tokens of each (layer, sequence, kv head) in an fp16
 *   ring (slot = position % n_recent) outside the packed cache; 0 disables it.
 *
 * Device buffers (per layer blocks, layer-major; sizes from bgtq_cache_bytes):
 *   k_codes  uint8 [L][B][Hkv][n_cap/64][64 * K record bytes]   (tile layout, see below)
 *   v_codes  uint8 [L][B][Hkv][n_cap/64][1024 * v_bits]
 *   k_scale  fp16  [L][B][Hkv][n_cap]            (affine: [..][n_cap][128/k_group])
 *   k_zero   fp16  affine keys only, same shape as k_scale; else NULL
 *   v_scale  fp16  [L][B][Hkv][n_cap];  v_zero: affine values only, same shape; else NULL
 *   recent_k, recent_v  fp16 [L][B][Hkv][n_recent][128] when n_recent > 0; else NULL
 *   bits      uint8 [L][Hkv][64]   widths (BLOCKGTQ), from bgtq_allocate
 *   sigma     fp32  [L][Hkv][64]   per-block key scale sigma_i = sqrt(E_k[i]/2)
 *   inv_sigma fp32  [L][Hkv][64]   fp32(1/sigma_i), 0 for a dead block
 *   plan      uint8 [L][Hkv][BGTQ_PLAN_BYTES]: Block-GTQ keys only (else NULL).  What the decode needs
 *     that depends only on a layer's widths (block order, operand positions), written by
 *     bgtq_prepare_metadata after the layer's bits are set; its contents are the library's own.
 *   k_rot     uint8 [L][Hkv][16] or NULL: affine keys only.  Sign bits s_j (bit j % 8 of byte
 *     j / 8 set means s_j = -1) of a randomized Hadamard key rotation ("Quantize What Counts"
 *     summary, Results: rotating the keys alone recovers most of K4V4's accuracy at K4V2): each
 *     appended key row is stored as y = H (s * k) / 16 (H the 128x128 Sylvester Hadamard
 *     matrix, fast transform in stages 1, 2, ..., 64, fp32), and decode rotates the query to
 *     H (s * q) / 8 so that the logits are unchanged; the fp16 recent ring keeps rows unrotated.
 *     NULL disables it.  With Block-GTQ keys it is BGTQ_E_UNSUPPORTED.
 *   v_rot     uint8 [L][Hkv][16] or NULL: sign bits s_j (as k_rot) of a randomized Hadamard
 *     rotation of the values ("Quantize What Counts" summary, Results: the summary finds rotating
 *     the values alone marginal or harmful; offered for comparison).  Each appended value row is
 *     stored as y = H (s * v) / 16 (the transform of k_rot, fp32) and quantized; the split merge
 *     undoes the rotation once on the output, o = s * (H o') / 8.  Any key format; not with an fp16
 *     window (n_recent > 0 or a log-based filter): BGTQ_E_UNSUPPORTED.  NULL disables it.
 *   decode_path  BGTQ_DECODE_AUTO or BGTQ_DECODE_VECTOR (plain value, not a buffer): which decode
 *     kernels bgtq_decode_attention runs.  Both compute the same attention to the same tolerance;
 *     VECTOR keeps every product on the vector ALUs (no matrix-core instructions), for comparison
 *     and measurement.  Other values: BGTQ_E_INVALID from the decode calls.
 * Host state:
 *   n_tokens  int64 [L][B] host array: tokens appended so far per (layer, sequence) (packed +
 *     recent).  bgtq_quantize_append advances it on success only.
 *   n_hp      int32 [L][B] host array or NULL.  Non-NULL selects LogQuant's log-based filter
 *     for the recent buffers: they then hold n_hp[layer][b] high-precision rows in slots
 *     0..n_hp-1, in any order, and the other n_tokens - n_hp tokens are packed.  Appends go
 *     through bgtq_logquant_append; bgtq_quantize_append and bgtq_decode_step refuse such a cache.
 *     NULL keeps the positional ring: min(n_tokens, n_recent) recent rows, slot = position mod
 *     n_recent.
 *
 * Tile layout (64 consecutive tokens of one (batch, kv head)):
 *   K record = little-endian bit stream of R = 2U/32 dwords (affine: 4*k_bits dwords).  Block-GTQ
 *   record: blocks by width descending (ties: lower index first), width-0 blocks omitted; block i
 *   of width w holds code(2i) then code(2i+1), w bits each.  Affine: coordinate j at bits
 *   [k_bits*j, +k_bits).  Tile = dword-major, token-minor: dword k of token t at byte (k*64+t)*4.
 *   V tile ("lane streams"): 64 streams of 4*v_bits dwords, stream L = dd + 16j (dd 0..15,
 *   j 0..3) holding 64 fields of 2*v_bits bits, field phi = (s*8 + db)*4 + m (s 0..1, db 0..7,
 *   m 0..3) at bit 2*v_bits*phi: the codes of dim 16db + dd for tokens p and p + 32,
 *   p = 16s + 4j + m, token p in the low half.  Stream dword c is tile dword
 *   ((c/4)*64 + L)*4 + c%4.
 */
typedef struct bgtq_cache {
    int32_t L, B, Hq, Hkv, d;
    int64_t n_cap;
    int32_t k_mode, budget_units, k_bits, k_group;
    int32_t v_mode, v_bits;
    int32_t n_recent;
    void *k_codes, *v_codes, *k_scale, *k_zero, *v_scale, *v_zero, *recent_k, *recent_v;
    const uint8_t *bits;
    const float *sigma, *inv_sigma;
    int64_t *n_tokens;
    const uint8_t *k_rot;
    int32_t *n_hp;
    void *plan;
    int32_t decode_path;
    const uint8_t *v_rot;
} bgtq_cache;

/* Thread-local text describing the last non-OK status of this thread ("" if none). */
const char *bgtq_last_error(void);

/* Library version string. */
const char *bgtq_version(void);

/*
 * The library's frozen TQ-MSE scalar table for `bits` in 1..8 (host, synchronous).
 * TQ-MSE (review §1; abstract) quantizes coordinates with an MSE-optimal scalar quantizer
 * whose error falls as 4^-b.  Table: Lloyd-Max quantizer of N(0,1), centroids rounded to fp16,
 * thresholds = exact midpoints of adjacent centroids.  centroids_f16 (host, 2^bits uint16 fp16
 * bit patterns, ascending) and thresholds (host, 2^bits - 1 floats) may be NULL.
 */
int bgtq_codebook(int bits, uint16_t *centroids_f16, float *thresholds);

/*
 * Greedy integer bit allocation (host, synchronous).  Block-GTQ (abstract; review §3,
 * Figure 1): per layer and KV head, widths by marginal gain under the 4^-b rate.  Starting from
 * b_min on every block with a positive score (0 elsewhere), repeatedly add one bit to the block
 * maximizing s_i * 4^-b_i among blocks with b_i < b_max and s_i > 0; ties go to the lowest
 * index.  scores: host fp64 [n_heads][n_blk]; bits_out: host uint8 [n_heads][n_blk].
 * Errors: BGTQ_E_INVALID (NULL, n_blk not in 1..256, b_max not in 1..8, b_min > b_max,
 * negative or non-finite score), BGTQ_E_BUDGET (budget_units cannot be spent on any head).
 */
int bgtq_allocate(const double *scores, int n_heads, int n_blk, int budget_units,
                  int b_min, int b_max, uint8_t *bits_out);

/*
 * The same greedy ranked by a tabulated distortion-rate curve instead of the idealized 4^-b
 * (host, synchronous).  The review (§3) states the allocation with the TQ-MSE rate 4^-b; the
 * library's own scalar tables reach D(b) (their exact N(0,1) mean squared error: D(0) = 1,
 * D(1) = 1 - 2/pi, ...), whose ratios approach 4 only at wide codes.  With block distortion
 * s_i * D(b_i), each step adds one bit to the block maximizing s_i * (D(b_i) - D(b_i + 1)) among
 * blocks with b_i < b_max and s_i > 0 (ties: lowest index).  rate: host fp64 [b_max + 1], D(b)
 * for b = 0..b_max, strictly decreasing with non-increasing steps (a convex curve, for which this
 * greedy minimizes sum_i s_i D(b_i) exactly).  Other arguments and errors as bgtq_allocate, plus
 * BGTQ_E_INVALID for a NULL, non-finite, non-decreasing or non-convex rate.
 */
int bgtq_allocate_rate(const double *scores, int n_heads, int n_blk, int budget_units,
                       int b_min, int b_max, const double *rate, uint8_t *bits_out);

/*
 * Calibration energy (device reduction, then a synchronous copy to the host).  Block-GTQ
 * (abstract; review §3) scores each RoPE block from calibration data per layer and KV head:
 * E_k[i] = mean_t ||k_t,(2i,2i+1)||^2, E_q[i] = mean over t and the g query heads of the group of
 * ||q||^2, score = E_q*E_k (BGTQ_SCORE_QK) or E_k (BGTQ_SCORE_K); sigma_i = fp32(sqrt(E_k[i]/2)),
 * inv_sigma_i = fp32(1/sigma_i) (0 if sigma_i = 0).  Sums run in fp64 on the device.
 * k_cal: device [T_cal][Hkv][128], q_cal: device [T_cal][Hkv*g][128], contiguous, dtype.
 * Outputs (host, [Hkv][64]; any may be NULL): scores fp64, sigma fp32, inv_sigma fp32.
 * ws: device scratch of at least Hkv*64*16 bytes (caller-owned).  The tokens are reduced in
 * chunks of BGTQ_ENERGY_CHUNK, one workgroup each, as many as ws holds (Hkv*64*16 bytes per
 * chunk; ceil(T_cal / BGTQ_ENERGY_CHUNK) chunks use the whole GPU); the host adds the chunk sums
 * in order, so equal calls give equal results.  Synchronizes `stream`.
 * Errors: BGTQ_E_INVALID (NULL inputs, T_cal < 1, bad dtype, small ws), BGTQ_E_UNSUPPORTED (d).
 */
int bgtq_block_energy(const void *k_cal, const void *q_cal, int dtype, int64_t T_cal,
                      int Hkv, int g, int d, int score_mode, double *scores, float *sigma,
                      float *inv_sigma, void *ws, size_t ws_bytes, void *stream);

/*
 * LogQuant's log-based filter for one sequence (host, synchronous; LogQuant summary, Method 2):
 * at most 3W tokens stay at high precision, and when the set is full the density of its older
 * part is halved.  Reading: when a token arrives and the set holds 3W, the 2W oldest members
 * (by position) are halved, the 2nd, 4th, ... oldest leaving for the low-bit store; then the
 * new token joins.
 * State: a high-precision store of 3W row slots, of which slots 0..*n_hp-1 are filled;
 * hp_pos[slot] (capacity 3W) is the token position the row holds, in any slot order.
 * Planning the append of the token at position `pos` (above every held position):
 * - when *n_hp == 3W, the W leaving rows' slots are written to evict[0..W-1], oldest first.
 *   Their rows are to be quantized in that order.  The store is then compacted into slots
 *   0..2W-1 by copying row move_src[i] to slot move_dst[i], i < *n_moves, after the leaving
 *   rows were read.  No move reads a slot that another move writes.  evict, move_src and
 *   move_dst each hold W entries;
 * - the new token's row goes to slot *new_slot.
 * hp_pos and *n_hp are left as after the append.  Returns the number of leaving rows (0 or W),
 * or BGTQ_E_INVALID (W outside [1, 2^20], NULL pointers, *n_hp outside [0, 3W], pos not above a
 * held position, a repeated position) with nothing changed.
 */
int bgtq_logquant_plan(int W, int64_t *hp_pos, int *n_hp, int64_t pos, int32_t *evict,
                       int32_t *move_src, int32_t *move_dst, int *n_moves, int *new_slot);

/*
 * Device workspace of the log-based filter's calls (host, no side effects): the bytes that
 * bgtq_logquant_prefill needs for a prompt of n_prompt tokens (its gather indices), or, with
 * n_prompt = 0, that bgtq_logquant_append needs (the store permutation, once B * n_recent is above
 * 1536; 0 below, where the permutation travels in the kernel arguments).  <0 on error.
 */
int64_t bgtq_logquant_workspace_bytes(const bgtq_cache *c, int64_t n_prompt);

/*
 * Append one token per sequence under LogQuant's log-based filter (device, asynchronous; host
 * bookkeeping synchronous).  LogQuant summary, Method 2; the filter is bgtq_logquant_plan's,
 * with W = n_recent / 3.  Needs c->n_hp and n_recent a multiple of 3 in [3, 512].  For each
 * sequence the new token's row enters the high-precision store.  When the store already holds 3W
 * rows, the rows that leave are quantized first, oldest first, and appended to the packed cache.
 * The store is then compacted, as the plan describes.
 * k, v: device rows [B][1][Hkv][128] in `dtype` (strides as bgtq_quantize_append, n_new = 1).
 * hp_pos: host int64 [B][n_recent], the token position each store row holds; maintained here.
 * ws, ws_bytes: device workspace, 256-byte aligned, of bgtq_logquant_workspace_bytes(c, 0) bytes;
 * may be NULL when that is 0 (B * n_recent <= 1536).  The store permutation is then copied into
 * it from host memory on `stream`.
 * On success n_tokens, n_hp and hp_pos advance.  Errors found before any launch change nothing:
 * those of bgtq_quantize_append, BGTQ_E_INVALID (no n_hp, bad n_recent, inconsistent counts, a
 * missing or small workspace).  BGTQ_E_HIP (a launch failed after an earlier one of the same call
 * was enqueued) leaves the host bookkeeping unchanged and the layer's device store and packed tail
 * unspecified.
 */
int bgtq_logquant_append(bgtq_cache *c, int layer, const void *k, const void *v, int dtype,
                         const int64_t *strides, int64_t *hp_pos, void *ws, size_t ws_bytes,
                         void *stream);

/*
 * LogQuant's filter over a prompt, in one call (device, asynchronous; host planning synchronous;
 * LogQuant summary, Method 2).  Appends n_prompt tokens to every sequence of a layer whose
 * sequences are empty (n_tokens and n_hp 0), with the result of n_prompt calls of
 * bgtq_logquant_append up to the order of the store's slots: the filter's selection over
 * positions 0..n_prompt-1 decides which tokens stay at high precision (at most 3W = n_recent) and
 * in which order the others left; the leaving tokens are quantized into packed positions
 * 0, 1, ... in that order (one gathered quantize launch) and the kept tokens' fp16 rows go to
 * store slots 0..n_hp-1 in position order.  k, v: device rows [B][n_prompt][Hkv][128] in `dtype`
 * (strides as bgtq_quantize_append).  hp_pos: host int64 [B][n_recent], written (-1 past n_hp).
 * ws, ws_bytes: device workspace, 256-byte aligned, of bgtq_logquant_workspace_bytes(c, n_prompt)
 * bytes (the gather indices, copied from host memory on `stream`).  On success n_tokens = n_prompt
 * and n_hp = the kept count.  Errors before any launch change nothing: BGTQ_E_INVALID (no n_hp,
 * bad n_recent or n_prompt, a sequence not empty, NULL pointers, a missing or small workspace),
 * BGTQ_E_CAPACITY (the leaving tokens exceed n_cap), and the format errors of
 * bgtq_quantize_append.
 */
int bgtq_logquant_prefill(bgtq_cache *c, int layer, const void *k, const void *v, int dtype,
                          int64_t n_prompt, const int64_t *strides, int64_t *hp_pos, void *ws,
                          size_t ws_bytes, void *stream);

/*
 * Prepare a layer's decode plan (device, asynchronous) from its widths c->bits[layer]: the block
 * order of the Block-GTQ records (review §3: widths per RoPE block and KV head), where each block's
 * codes sit in the record and where its query coordinates go in the decode's operands.  Call it
 * after writing a layer's bits (and before decoding that layer); the decode of a Block-GTQ cache
 * reads the plan instead of deriving it in every workgroup.  Writes c->plan[layer] only.
 * Errors: BGTQ_E_INVALID (NULL descriptor, bits or plan, layer out of range, affine keys).
 */
int bgtq_prepare_metadata(const bgtq_cache *c, int layer, void *stream);

/* Bytes of one cache buffer (all L layers) for the descriptor's geometry; <0 on error. */
int64_t bgtq_cache_bytes(const bgtq_cache *c, int which);

/*
 * Quantize-append (device, asynchronous).  The packed-cache path (review §1 Packed-Cache;
 * abstract) writes each new K/V row as codes plus a per-token fp16 scale.  Per token:
 * S = fp16_rne(sqrt_f32(sum_j (x_j * inv_sigma_i)^2 / 128)) with the sum in fp32, sequential
 * over j, no FMA; code_j = number of thresholds tau_m with x_j >= fp32(fp32(S*sigma_i)*tau_m)
 * (values: sigma = 1).  Affine groups: scale = fp16(fp32(max-min)/(2^b-1)), zero = fp16(min),
 * code = clamp(rint((x-zero)/scale)).  With n_recent > 0, tokens that leave the fp16 window are
 * quantized and new tokens enter the ring.
 * k, v: device rows in `dtype`, element (b, t, h, j) at b*strides[0] + t*strides[1] +
 * h*strides[2] + j (strides in elements; NULL = contiguous [B][n_new][Hkv][128]).
 * Appends n_new tokens to every sequence of `layer`.  Errors: BGTQ_E_INVALID,
 * BGTQ_E_UNSUPPORTED (format outside the kernels), BGTQ_E_CAPACITY (packed tokens > n_cap).
 */
int bgtq_quantize_append(bgtq_cache *c, int layer, const void *k, const void *v, int dtype,
                         int64_t n_new, const int64_t *strides, void *stream);

/* Workspace bytes bgtq_decode_attention needs for n_splits (0 = the library's choice). */
int64_t bgtq_decode_workspace_bytes(const bgtq_cache *c, int n_splits);

/*
 * Decode attention from the packed cache (device, asynchronous).  Packed-cache serving
 * (review §1 Packed-Cache, Figure 2; abstract): in one pass over the codes, without an fp16
 * copy of K/V, compute z_t = q.k_hat_t/sqrt(128) with k_hat = S*sigma_i*c[code] (affine:
 * scale*code+zero), an online softmax, and o = sum_t p_t v_hat_t / sum_t p_t over the packed
 * tokens and the fp16 recent tokens (order-free concatenation, LogQuant summary Method 4).
 * Split-K over context; partials merged by log-sum-exp.  An fp16 window of at most 512 rows
 * (n_recent, or the log-based filter's store) is attended by the merge launch itself; a longer one
 * by a split-K launch of its own, which takes one more partial per query head of workspace.
 * q: device [B][Hq][128] in dtype; out: device fp32 [B][Hq][128]; ws: device scratch of at
 * least bgtq_decode_workspace_bytes(c, n_splits) bytes (256-byte aligned), contents undefined
 * after the call.  Errors: BGTQ_E_INVALID (NULL, layer, empty context, small workspace),
 * BGTQ_E_UNSUPPORTED.
 */
int bgtq_decode_attention(const bgtq_cache *c, int layer, const void *q, int dtype, float *out,
                          void *ws, size_t ws_bytes, int n_splits, void *stream);

/*
 * One decode step: quantize-append then attend, in one call (device, asynchronous).  Appends k, v
 * (as bgtq_quantize_append: n_new rows per sequence, same strides convention) and computes
 * bgtq_decode_attention for q over the grown context, all on `stream`; k, v and q share `dtype`.
 * The codes and scales written are those bgtq_quantize_append writes, and the output equals the
 * two calls made in turn (to the decode's rounding).
 * Launches: with one new token per sequence, Block-GTQ keys, g >= 4 on BGTQ_DECODE_AUTO and no
 * fp16 window (n_recent == 0, no log-based filter), the append is fused into the attention
 * launch — the operator fusion LogQuant names as future work (LogQuant summary, Conclusion): the
 * wave whose tile holds the new token quantizes it while its tile is in flight, writes it to the
 * cache and attends to it with the rest of the tile, so the step is the decode launch plus the
 * split merge.  Otherwise the append kernels run first, as dependent launches on `stream`.
 * Both halves are validated against the post-append lengths before anything is enqueued: an
 * error other than BGTQ_E_HIP leaves the cache and n_tokens untouched.  BGTQ_E_HIP from the
 * attention half is reported after the append was enqueued (n_tokens then includes the new rows).
 * ws, ws_bytes, n_splits and out as bgtq_decode_attention.  Errors: those of the two calls.
 */
int bgtq_decode_step(bgtq_cache *c, int layer, const void *k, const void *v, const void *q,
                     int dtype, int64_t n_new, const int64_t *strides, float *out, void *ws,
                     size_t ws_bytes, int n_splits, void *stream);

/*
 * bgtq_decode_attention without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The split-K partials go to a fixed array of BGTQ_NOALLOC_SCRATCH_BYTES bytes that the library
 * keeps on each GPU it runs on until the process ends (looked up on the first call on a device);
 * the call itself allocates nothing.  Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (other streams, other threads) race; calls in order on one stream do not.
 * n_splits = 0 takes the library's split count, reduced so that the partials
 * (B * Hq * (splits + 1 if n_recent > 512) * 528 bytes) fit the array; an explicit n_splits whose
 * partials do not fit is BGTQ_E_UNSUPPORTED, as is a geometry for which one split does not fit.
 * Other arguments, results and errors as bgtq_decode_attention.
 */
#define BGTQ_NOALLOC_SCRATCH_BYTES (4 << 20)
int bgtq_decode_attention_noalloc(const bgtq_cache *c, int layer, const void *q, int dtype, float *out,
                                  int n_splits, void *stream);

/* Workspace bytes for bgtq_fp16_decode_attention. */
int64_t bgtq_fp16_decode_workspace_bytes(int64_t N, int B, int Hq, int Hkv, int n_splits);

/*
 * Unquantized comparator (device, asynchronous): the same split-K decode attention over an fp16
 * cache, the role fp16 FlashAttention-2 plays in the abstract's serving comparison.
 * k16, v16: device fp16 [B][Hkv][N][128]; q: device [B][Hq][128] in dtype; out: fp32
 * [B][Hq][128]; ws as above.  Errors: BGTQ_E_INVALID, BGTQ_E_UNSUPPORTED.
 */
int bgtq_fp16_decode_attention(const void *k16, const void *v16, int64_t N, int B, int Hq,
                               int Hkv, int d, const void *q, int dtype, float *out, void *ws,
                               size_t ws_bytes, int n_splits, void *stream);

/*
 * Kernel tracing (host).  While enabled, every launch of a main kernel (packed decode, fp16
 * decode, quantize-append) records a pair of HIP events around the kernel's own execution
 * (hipExtLaunchKernelGGL; the dispatch gap before the kernel is not included), up to
 * `max_launches` launches; bgtq_profile_enable(0) disables and releases the events.
 * bgtq_profile_read waits for the recorded events of one kind (BGTQ_PROF_*), returns their
 * count and the total / min / max duration in milliseconds (any output may be NULL), and clears
 * that kind's records.  Not thread-safe against concurrent decode calls on other threads.
 */
enum { BGTQ_PROF_DECODE = 0, BGTQ_PROF_FP16_DECODE = 1, BGTQ_PROF_QUANTIZE = 2 };
int bgtq_profile_enable(int max_launches);
int bgtq_profile_read(int kind, int *n_launches, double *total_ms, double *min_ms, double *max_ms);

#ifdef __cplusplus
}
#endif

#endif /* BGTQ_H */
