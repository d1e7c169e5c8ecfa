// Host side of the C ABI declared in include/bgtq.h: argument validation, the greedy
// allocator, cache geometry, workspace carving and kernel launches.  No device allocation,
// no synchronization except in bgtq_block_energy (which returns host scores).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/bgtq.h"
#include "bgtq_internal.h"
#include "generated/bgtq_codebook_data.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return BGTQ_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(BGTQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int D = 128;
constexpr int TILE = 64;
constexpr int PART = 132;

bool dtype_ok(int dt) { return dt == BGTQ_F32 || dt == BGTQ_F16 || dt == BGTQ_BF16; }

// Validate the descriptor's geometry and format; fill g.  Pointers are checked by callers.
int geometry(const bgtq_cache* c, bgtq::Geometry& g) {
    if (!c) return fail(BGTQ_E_INVALID, "cache descriptor is NULL");
    if (c->d != D) return fail(BGTQ_E_UNSUPPORTED, "head dim %d unsupported (only 128)", c->d);
    if (c->L < 1 || c->B < 1 || c->Hq < 1 || c->Hkv < 1)
        return fail(BGTQ_E_INVALID, "L, B, Hq, Hkv must be positive");
    if (c->B > BGTQ_MAX_BATCH) return fail(BGTQ_E_UNSUPPORTED, "B=%d exceeds %d", c->B, BGTQ_MAX_BATCH);
    if (c->Hq % c->Hkv) return fail(BGTQ_E_INVALID, "Hq %% Hkv != 0");
    const int G = c->Hq / c->Hkv;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return fail(BGTQ_E_UNSUPPORTED, "group size %d unsupported", G);
    if (c->n_cap < TILE || c->n_cap % TILE) return fail(BGTQ_E_INVALID, "n_cap must be a positive multiple of 64");
    if (c->n_cap > INT32_MAX) return fail(BGTQ_E_UNSUPPORTED, "n_cap exceeds 2^31 - 1");
    if (c->n_recent < 0) return fail(BGTQ_E_INVALID, "n_recent < 0");
    g.B = c->B; g.Hq = c->Hq; g.Hkv = c->Hkv; g.G = G;
    g.n_cap = c->n_cap;
    g.n_tiles = c->n_cap / TILE;
    g.k_mode = c->k_mode;
    g.k_bits = c->k_bits;
    g.k_group = c->k_group;
    if (c->k_mode == BGTQ_K_BLOCKGTQ) {
        if (c->budget_units < 16 || c->budget_units > 8 * 64 || c->budget_units % 16)
            return fail(BGTQ_E_INVALID, "budget_units must be a multiple of 16 in [16, 512]");
        g.R = 2 * c->budget_units / 32;
    } else if (c->k_mode == BGTQ_K_AFFINE) {
        if (!(c->k_bits == 2 || c->k_bits == 4 || c->k_bits == 8))
            return fail(BGTQ_E_INVALID, "k_bits must be 2, 4 or 8");
        if (c->k_group < 8 || c->k_group > D || D % c->k_group)
            return fail(BGTQ_E_INVALID, "k_group must divide 128 and be >= 8");
        g.R = c->k_bits * D / 32;
    } else {
        return fail(BGTQ_E_INVALID, "unknown k_mode %d", c->k_mode);
    }
    if (c->k_rot && c->k_mode != BGTQ_K_AFFINE)
        return fail(BGTQ_E_UNSUPPORTED, "the key rotation applies to affine keys only");
    if (c->v_rot && (c->n_recent > 0 || c->n_hp))
        return fail(BGTQ_E_UNSUPPORTED, "the value rotation applies to caches without an fp16 window");
    if (c->v_mode != BGTQ_V_CODEBOOK && c->v_mode != BGTQ_V_AFFINE) return fail(BGTQ_E_INVALID, "unknown v_mode");
    if (c->v_bits < 1 || c->v_bits > 4) return fail(BGTQ_E_INVALID, "v_bits must be in 1..4");
    g.v_mode = c->v_mode;
    g.v_bits = c->v_bits;
    g.n_recent = c->n_recent;
    g.k_tile_bytes = (int64_t)TILE * g.R * 4;
    g.v_tile_bytes = (int64_t)1024 * g.v_bits;
    const int64_t bh = (int64_t)g.B * g.Hkv;
    g.k_codes_layer = bh * g.n_tiles * g.k_tile_bytes;
    g.v_codes_layer = bh * g.n_tiles * g.v_tile_bytes;
    g.k_scale_layer = bh * g.n_cap * 2 * (c->k_mode == BGTQ_K_AFFINE ? D / c->k_group : 1);
    g.v_scale_layer = bh * g.n_cap * 2;
    g.recent_layer = bh * (int64_t)g.n_recent * D * 2;
    return BGTQ_OK;
}

int default_splits(int64_t max_tiles, int bh, int n_cu, int per_cu, int waves = 4) {
    // One round of workgroups (per_cu resident per CU), each with a whole number of tiles per wave
    // (a multiple of the wave count; at least two tiles per wave with four waves, one with more) so
    // that the waves of a split finish together.
    const int64_t target = (int64_t)per_cu * n_cu;
    int64_t s = (target + bh - 1) / bh;
    if (s < 1) s = 1;
    int64_t tps = (max_tiles + s - 1) / s;
    tps = (tps + waves - 1) / waves * waves;
    if (tps < 8) tps = 8;
    s = (max_tiles + tps - 1) / tps;
    return (int)(s < 1 ? 1 : s);
}

int cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) n = p.multiProcessorCount;
        if (n <= 0) n = 256;
    }
    return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Block-GTQ keys with 4 or 8 query heads per kv head take the plan-driven matrix-core decode, one
// workgroup per compute unit.
bool vector_only(const bgtq_cache* c) { return c->decode_path == BGTQ_DECODE_VECTOR; }
bool uses_gtq_kernel(const bgtq_cache* c, int G) { return c->k_mode == BGTQ_K_BLOCKGTQ && G >= 4 && !vector_only(c); }

// The library's split count for a context of max_tiles tiles per (batch, kv head).  Block-GTQ at
// g >= 4: one tile per wave of a sixteen-wave workgroup when one round of workgroups covers the
// context, else one round of eight-wave workgroups that loop over their tiles.  Other formats: the
// per-CU heuristic of their kernel.
// A window longer than the merge attends to itself is decoded by a split-K launch of its own, which
// writes one more partial per query head.
bool ring_split(int64_t n_recent) { return n_recent > bgtq::kMergeWindowMax; }

int auto_splits(const bgtq_cache* c, int G, int64_t max_tiles, int bh) {
    const int n_cu = cu_count();
    if (uses_gtq_kernel(c, G)) {
        const int64_t one = (max_tiles + bgtq::kGtqWavesOneTile - 1) / bgtq::kGtqWavesOneTile;
        if (one * bh <= n_cu) return (int)std::max<int64_t>(one, 1);
        return default_splits(max_tiles, bh, n_cu, 1, bgtq::kGtqWavesLoop);
    }
    return default_splits(max_tiles, bh, n_cu, bgtq::decode_wgs_per_cu(c->k_mode, G, c->v_bits, c->k_group, vector_only(c)));
}

// Event pairs around main-kernel launches (tracing aid, see bgtq_profile_enable).
struct Profiler {
    int cap = 0;
    std::vector<hipEvent_t> ev;   // 2 per record
    std::vector<int> kind;
    int n = 0;
};
Profiler g_prof;

// Arms the slot's events for the next main-kernel launch, which records them around the kernel
// itself; an unused pair is disarmed when the scope ends.
struct ProfScope {
    ProfScope(int kind, hipStream_t) {
        if (g_prof.cap > 0 && g_prof.n < g_prof.cap) {
            const int slot = g_prof.n++;
            g_prof.kind[slot] = kind;
            bgtq::arm_launch_events(g_prof.ev[2 * slot], g_prof.ev[2 * slot + 1]);
        }
    }
    ~ProfScope() { bgtq::disarm_launch_events(); }
};

}  // namespace

extern "C" {

const char* bgtq_last_error(void) { return g_err.c_str(); }

int bgtq_profile_enable(int max_launches) {
    if (max_launches < 0) return fail(BGTQ_E_INVALID, "max_launches < 0");
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof = Profiler{};
    if (max_launches == 0) return ok();
    g_prof.ev.resize(2 * (size_t)max_launches);
    g_prof.kind.resize(max_launches);
    for (auto& e : g_prof.ev) {
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            g_prof.ev.clear();
            return hip_fail(r, "hipEventCreate");
        }
    }
    g_prof.cap = max_launches;
    return ok();
}

int bgtq_profile_read(int kind, int* n_launches, double* total_ms, double* min_ms, double* max_ms) {
    int cnt = 0;
    double tot = 0.0, mn = 0.0, mx = 0.0;
    std::vector<int> keep;
    for (int i = 0; i < g_prof.n; ++i) {
        if (g_prof.kind[i] != kind) {
            keep.push_back(i);
            continue;
        }
        hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        float ms = 0.f;
        if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r, "profile event");
        tot += ms;
        mn = cnt ? std::min(mn, (double)ms) : ms;
        mx = cnt ? std::max(mx, (double)ms) : ms;
        ++cnt;
    }
    // compact the records of other kinds to the front (swap their event pairs)
    for (size_t j = 0; j < keep.size(); ++j) {
        const int i = keep[j];
        if (i != (int)j) {
            std::swap(g_prof.ev[2 * j], g_prof.ev[2 * i]);
            std::swap(g_prof.ev[2 * j + 1], g_prof.ev[2 * i + 1]);
            g_prof.kind[j] = g_prof.kind[i];
        }
    }
    g_prof.n = (int)keep.size();
    if (n_launches) *n_launches = cnt;
    if (total_ms) *total_ms = tot;
    if (min_ms) *min_ms = mn;
    if (max_ms) *max_ms = mx;
    return ok();
}

const char* bgtq_version(void) { return "bgtq 0.1 (gfx950)"; }

int bgtq_codebook(int bits, uint16_t* centroids_f16, float* thresholds) {
    if (bits < 1 || bits > 8) return fail(BGTQ_E_INVALID, "bits must be in 1..8");
    const int n = 1 << bits;
    const int cb = n - 2, tb = n - bits - 1;
    if (centroids_f16)
        for (int m = 0; m < n; ++m) centroids_f16[m] = bgtq_cb_centroid_f16[cb + m];
    if (thresholds)
        for (int m = 0; m < n - 1; ++m) std::memcpy(&thresholds[m], &bgtq_cb_threshold_f32[tb + m], 4);
    return ok();
}

extern "C++" {
namespace {
// The greedy of both allocators: from b_min on every live block (positive score), repeatedly add
// one bit to the live block below b_max with the largest key(score, width); ties go to the
// lowest index.  Arguments are validated by the callers.
template <typename Key>
int greedy_widths(const double* scores, int n_heads, int n_blk, int budget_units, int b_min, int b_max,
                  uint8_t* bits_out, Key key_of) {
    std::vector<uint8_t> out((size_t)n_heads * n_blk);
    for (int hd = 0; hd < n_heads; ++hd) {
        const double* s = scores + (size_t)hd * n_blk;
        uint8_t* b = out.data() + (size_t)hd * n_blk;
        int spent = 0;
        for (int i = 0; i < n_blk; ++i) {
            b[i] = s[i] > 0.0 ? (uint8_t)b_min : 0;
            spent += b[i];
        }
        if (spent > budget_units) return fail(BGTQ_E_BUDGET, "b_min exceeds the budget (head %d)", hd);
        for (; spent < budget_units; ++spent) {
            int best = -1;
            double best_key = 0.0;
            for (int i = 0; i < n_blk; ++i) {
                if (b[i] >= b_max || !(s[i] > 0.0)) continue;
                const double key = key_of(s[i], (int)b[i]);
                if (best < 0 || key > best_key) {
                    best = i;
                    best_key = key;
                }
            }
            if (best < 0) return fail(BGTQ_E_BUDGET, "budget %d exceeds what head %d can hold", budget_units, hd);
            ++b[best];
        }
    }
    std::memcpy(bits_out, out.data(), out.size());
    return ok();
}

int check_allocate_args(const double* scores, int n_heads, int n_blk, int budget_units, int b_min, int b_max,
                        const uint8_t* bits_out) {
    if (!scores || !bits_out) return fail(BGTQ_E_INVALID, "NULL pointer");
    if (n_heads < 1 || n_blk < 1 || n_blk > 256) return fail(BGTQ_E_INVALID, "bad n_heads/n_blk");
    if (b_max < 1 || b_max > 8 || b_min < 0 || b_min > b_max) return fail(BGTQ_E_INVALID, "bad b_min/b_max");
    if (budget_units < 0) return fail(BGTQ_E_INVALID, "negative budget");
    for (int64_t i = 0; i < (int64_t)n_heads * n_blk; ++i)
        if (!(scores[i] >= 0.0) || !std::isfinite(scores[i]))
            return fail(BGTQ_E_INVALID, "score %lld is negative or not finite", (long long)i);
    return 0;
}
}  // namespace
}  // extern "C++"

int bgtq_allocate(const double* scores, int n_heads, int n_blk, int budget_units, int b_min, int b_max,
                  uint8_t* bits_out) {
    if (int rc = check_allocate_args(scores, n_heads, n_blk, budget_units, b_min, b_max, bits_out)) return rc;
    // s * 4^-b exactly
    return greedy_widths(scores, n_heads, n_blk, budget_units, b_min, b_max, bits_out,
                         [](double s, int b) { return std::ldexp(s, -2 * b); });
}

int bgtq_allocate_rate(const double* scores, int n_heads, int n_blk, int budget_units, int b_min, int b_max,
                       const double* rate, uint8_t* bits_out) {
    if (int rc = check_allocate_args(scores, n_heads, n_blk, budget_units, b_min, b_max, bits_out)) return rc;
    if (!rate) return fail(BGTQ_E_INVALID, "NULL rate");
    double gain[8];
    for (int b = 0; b < b_max; ++b) {
        if (!std::isfinite(rate[b]) || !std::isfinite(rate[b + 1])) return fail(BGTQ_E_INVALID, "rate not finite");
        gain[b] = rate[b] - rate[b + 1];
        if (!(gain[b] > 0.0)) return fail(BGTQ_E_INVALID, "rate does not decrease at width %d", b);
        if (b > 0 && gain[b] > gain[b - 1])
            return fail(BGTQ_E_INVALID, "rate steps grow at width %d (the curve must be convex)", b);
    }
    // marginal gain of one more bit: s * (D(b) - D(b + 1))
    return greedy_widths(scores, n_heads, n_blk, budget_units, b_min, b_max, bits_out,
                         [&gain](double s, int b) { return s * gain[b]; });
}

int bgtq_logquant_plan(int W, int64_t* hp_pos, int* n_hp, int64_t pos, int32_t* evict, int32_t* move_src,
                       int32_t* move_dst, int* n_moves, int* new_slot) {
    if (W < 1 || W > (1 << 20)) return fail(BGTQ_E_INVALID, "W=%d out of range", W);
    if (!hp_pos || !n_hp || !n_moves || !new_slot) return fail(BGTQ_E_INVALID, "NULL argument");
    const int n = *n_hp;
    if (n < 0 || n > 3 * W) return fail(BGTQ_E_INVALID, "n_hp=%d outside [0, 3W]", n);
    for (int i = 0; i < n; ++i)
        if (hp_pos[i] >= pos) return fail(BGTQ_E_INVALID, "position %lld not above held position %lld", (long long)pos,
                                          (long long)hp_pos[i]);
    int kept = n, n_ev = 0;
    *n_moves = 0;
    if (n == 3 * W) {
        if (!evict || !move_src || !move_dst) return fail(BGTQ_E_INVALID, "NULL evict or move arrays");
        std::vector<int> order(n);
        for (int i = 0; i < n; ++i) order[i] = i;
        std::sort(order.begin(), order.end(), [&](int a, int b) { return hp_pos[a] < hp_pos[b]; });
        for (int i = 1; i < n; ++i)
            if (hp_pos[order[i]] == hp_pos[order[i - 1]]) return fail(BGTQ_E_INVALID, "repeated position");
        // the 2W oldest rows are halved: the 2nd, 4th, ... oldest leave, oldest first
        std::vector<char> gone(n, 0);
        for (int i = 1; i < 2 * W; i += 2) {
            evict[n_ev++] = order[i];
            gone[order[i]] = 1;
        }
        // compaction into slots [0, 2W): kept rows above 2W fill the vacated slots below it, in
        // ascending slot order on both sides (a vacated slot is never a source)
        int h = 0, m = 0;
        for (int src = 2 * W; src < n; ++src) {
            if (gone[src]) continue;
            while (!gone[h]) ++h;
            move_src[m] = src;
            move_dst[m] = h;
            hp_pos[h] = hp_pos[src];
            ++m;
            ++h;
        }
        *n_moves = m;
        kept = 2 * W;
    }
    hp_pos[kept] = pos;
    *new_slot = kept;
    *n_hp = kept + 1;
    return n_ev;
}

int bgtq_block_energy(const void* k_cal, const void* q_cal, int dtype, int64_t T_cal, int Hkv, int g, int d,
                      int score_mode, double* scores, float* sigma, float* inv_sigma, void* ws, size_t ws_bytes,
                      void* stream) {
    if (!k_cal || !q_cal || !ws) return fail(BGTQ_E_INVALID, "NULL pointer");
    if (!dtype_ok(dtype)) return fail(BGTQ_E_INVALID, "bad dtype");
    if (d != D) return fail(BGTQ_E_UNSUPPORTED, "head dim must be 128");
    if (T_cal < 1 || Hkv < 1 || g < 1) return fail(BGTQ_E_INVALID, "bad sizes");
    if (score_mode != BGTQ_SCORE_QK && score_mode != BGTQ_SCORE_K) return fail(BGTQ_E_INVALID, "bad score mode");
    const size_t per_chunk = (size_t)Hkv * 64 * 2 * sizeof(double);
    if (ws_bytes < per_chunk) return fail(BGTQ_E_INVALID, "workspace too small (%zu < %zu)", ws_bytes, per_chunk);
    // tokens in chunks of BGTQ_ENERGY_CHUNK, one workgroup each, as far as the workspace holds them
    const int64_t want = (T_cal + BGTQ_ENERGY_CHUNK - 1) / BGTQ_ENERGY_CHUNK;
    const int64_t n_chunks = std::max<int64_t>(1, std::min<int64_t>({want, (int64_t)(ws_bytes / per_chunk), 65535}));
    const int64_t tc = (T_cal + n_chunks - 1) / n_chunks;
    hipStream_t s = (hipStream_t)stream;
    bgtq::EnergyArgs a{k_cal, q_cal, dtype, T_cal, Hkv, g, (double*)ws, (int)n_chunks, tc};
    hipError_t e = bgtq::launch_energy(a, s);
    if (e != hipSuccess) return hip_fail(e, "energy launch");
    std::vector<double> host((size_t)n_chunks * Hkv * 128);
    e = hipMemcpyAsync(host.data(), ws, (size_t)n_chunks * per_chunk, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "energy copy");
    for (int h = 0; h < Hkv; ++h)
        for (int i = 0; i < 64; ++i) {
            double sk = 0.0, sq = 0.0;  // chunks in order: the same sums for the same chunk count
            for (int64_t c = 0; c < n_chunks; ++c) {
                sk += host[((c * Hkv + h) * 64 + i) * 2];
                sq += host[((c * Hkv + h) * 64 + i) * 2 + 1];
            }
            const double ek = sk / (double)T_cal;
            const double eq = sq / ((double)T_cal * g);
            const float sg = (float)std::sqrt(ek / 2.0);
            if (scores) scores[h * 64 + i] = score_mode == BGTQ_SCORE_QK ? eq * ek : ek;
            if (sigma) sigma[h * 64 + i] = sg;
            if (inv_sigma) inv_sigma[h * 64 + i] = sg > 0.f ? 1.0f / sg : 0.f;
        }
    return ok();
}

int bgtq_prepare_metadata(const bgtq_cache* c, int layer, void* stream) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (layer < 0 || layer >= c->L) return fail(BGTQ_E_INVALID, "layer %d out of range", layer);
    if (c->k_mode != BGTQ_K_BLOCKGTQ) return fail(BGTQ_E_INVALID, "the decode plan is for Block-GTQ keys");
    if (!c->bits || !c->plan) return fail(BGTQ_E_INVALID, "NULL bits or plan");
    hipError_t e = bgtq::launch_plan(c->bits + (size_t)layer * g.Hkv * 64,
                                     (uint8_t*)c->plan + (size_t)layer * g.Hkv * BGTQ_PLAN_BYTES, g.Hkv,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    return ok();
}

int64_t bgtq_cache_bytes(const bgtq_cache* c, int which) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    const int64_t L = c->L;
    switch (which) {
        case BGTQ_BUF_K_CODES: return L * g.k_codes_layer;
        case BGTQ_BUF_V_CODES: return L * g.v_codes_layer;
        case BGTQ_BUF_K_SCALE: return L * g.k_scale_layer;
        case BGTQ_BUF_K_ZERO: return c->k_mode == BGTQ_K_AFFINE ? L * g.k_scale_layer : 0;
        case BGTQ_BUF_V_SCALE: return L * g.v_scale_layer;
        case BGTQ_BUF_V_ZERO: return c->v_mode == BGTQ_V_AFFINE ? L * g.v_scale_layer : 0;
        case BGTQ_BUF_RECENT_K:
        case BGTQ_BUF_RECENT_V: return L * g.recent_layer;
        case BGTQ_BUF_META: return L * g.Hkv * 64 * (1 + 4 + 4);
        case BGTQ_BUF_PLAN: return c->k_mode == BGTQ_K_BLOCKGTQ ? L * g.Hkv * BGTQ_PLAN_BYTES : 0;
    }
    return fail(BGTQ_E_INVALID, "unknown buffer selector %d", which);
}

}  // extern "C"

namespace {

// Per-layer destination and format fields of the quantize-append arguments.
void fill_quant_layer(const bgtq_cache* c, const bgtq::Geometry& g, int layer, bgtq::QuantArgs& q) {
    q.k_codes = (uint8_t*)c->k_codes + (size_t)layer * g.k_codes_layer;
    q.v_codes = (uint8_t*)c->v_codes + (size_t)layer * g.v_codes_layer;
    q.k_scale = (uint16_t*)((uint8_t*)c->k_scale + (size_t)layer * g.k_scale_layer);
    q.k_zero = c->k_zero ? (uint16_t*)((uint8_t*)c->k_zero + (size_t)layer * g.k_scale_layer) : nullptr;
    q.v_scale = (uint16_t*)((uint8_t*)c->v_scale + (size_t)layer * g.v_scale_layer);
    q.v_zero = c->v_zero ? (uint16_t*)((uint8_t*)c->v_zero + (size_t)layer * g.v_scale_layer) : nullptr;
    if (c->k_mode == BGTQ_K_BLOCKGTQ) {
        q.bits = c->bits + (size_t)layer * g.Hkv * 64;
        q.sigma = c->sigma + (size_t)layer * g.Hkv * 64;
        q.inv_sigma = c->inv_sigma + (size_t)layer * g.Hkv * 64;
    }
    q.k_rot = c->k_rot ? c->k_rot + (size_t)layer * g.Hkv * 16 : nullptr;
    q.v_rot = c->v_rot ? c->v_rot + (size_t)layer * g.Hkv * 16 : nullptr;
    q.Hkv = g.Hkv;
    q.n_cap = g.n_cap;
    q.n_tiles = g.n_tiles;
    q.k_tile_bytes = g.k_tile_bytes;
    q.v_tile_bytes = g.v_tile_bytes;
    q.k_mode = c->k_mode;
    q.R = g.R;
    q.k_bits = c->k_bits;
    q.k_group = c->k_group;
    q.v_mode = c->v_mode;
    q.v_bits = c->v_bits;
    q.which = 3;
}

// Quantize-append body.  With dry_run the call validates and plans only: nothing is launched and
// n_tokens is untouched, so a caller can check both halves of a combined step before either runs.
int quantize_append_impl(bgtq_cache* c, int layer, const void* k, const void* v, int dtype, int64_t n_new,
                         const int64_t* strides, void* stream, bool dry_run) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (layer < 0 || layer >= c->L) return fail(BGTQ_E_INVALID, "layer %d out of range", layer);
    if (c->n_hp) return fail(BGTQ_E_INVALID, "the cache uses the log-based filter: append with bgtq_logquant_append");
    if (!k || !v) return fail(BGTQ_E_INVALID, "NULL k/v");
    if (!dtype_ok(dtype)) return fail(BGTQ_E_INVALID, "bad dtype");
    if (n_new < 0) return fail(BGTQ_E_INVALID, "n_new < 0");
    if (!c->n_tokens) return fail(BGTQ_E_INVALID, "n_tokens is NULL");
    if (!c->k_codes || !c->v_codes || !c->k_scale || !c->v_scale) return fail(BGTQ_E_INVALID, "NULL cache buffer");
    if (c->k_mode == BGTQ_K_BLOCKGTQ && (!c->bits || !c->sigma || !c->inv_sigma))
        return fail(BGTQ_E_INVALID, "Block-GTQ keys need bits, sigma and inv_sigma");
    if (c->k_mode == BGTQ_K_AFFINE && !c->k_zero) return fail(BGTQ_E_INVALID, "affine keys need k_zero");
    if (c->v_mode == BGTQ_V_AFFINE && !c->v_zero) return fail(BGTQ_E_INVALID, "affine values need v_zero");
    if (c->n_recent > 0 && (!c->recent_k || !c->recent_v)) return fail(BGTQ_E_INVALID, "recent ring buffers are NULL");
    int64_t sB, sT, sH;
    if (strides) {
        sB = strides[0]; sT = strides[1]; sH = strides[2];
    } else {
        sH = D; sT = (int64_t)g.Hkv * D; sB = n_new * sT;
    }
    int64_t* nt = c->n_tokens + (size_t)layer * c->B;
    const int R = c->n_recent;
    // Plan: positions [packed_old, packed_new) get quantized; the new fp16 window is written last.
    std::vector<int64_t> packed_old(c->B), packed_new(c->B), total_old(c->B), total_new(c->B);
    for (int b = 0; b < c->B; ++b) {
        if (nt[b] < 0) return fail(BGTQ_E_INVALID, "n_tokens[%d] < 0", b);
        total_old[b] = nt[b];
        total_new[b] = nt[b] + n_new;
        packed_old[b] = total_old[b] - (R > 0 ? std::min<int64_t>(total_old[b], R) : 0);
        packed_new[b] = total_new[b] - (R > 0 ? std::min<int64_t>(total_new[b], R) : 0);
        if (packed_new[b] > c->n_cap)
            return fail(BGTQ_E_CAPACITY, "sequence %d: %lld packed tokens exceed n_cap %lld", b,
                        (long long)packed_new[b], (long long)c->n_cap);
    }
    if (n_new == 0 || dry_run) return ok();
    hipStream_t s = (hipStream_t)stream;
    const size_t bh = (size_t)g.B * g.Hkv;
    bgtq::QuantArgs q{};
    fill_quant_layer(c, g, layer, q);
    q.dtype = dtype;
    hipError_t e;
    auto run = [&](const void* sk, const void* sv, int dt, int64_t b_, int64_t t_, int64_t h_, int64_t mod_n,
                   const std::vector<int64_t>& lo, const std::vector<int64_t>& hi,
                   const std::vector<int64_t>& off) -> hipError_t {
        q.src_k = sk;
        q.src_v = sv;
        q.dtype = dt;
        q.sB = b_; q.sT = t_; q.sH = h_;
        q.mod_n = mod_n;
        int64_t max_tiles = 0;
        for (int b = 0; b < c->B; ++b) {
            q.pos_lo[b] = lo[b];
            q.pos_hi[b] = hi[b];
            q.off[b] = off[b];
            q.tile0[b] = lo[b] / TILE;
            if (hi[b] > lo[b]) max_tiles = std::max(max_tiles, (hi[b] - 1) / TILE - lo[b] / TILE + 1);
        }
        if (max_tiles == 0) return hipSuccess;  // nothing in range: no launch, and no profiler slot
        ProfScope ps(BGTQ_PROF_QUANTIZE, s);
        return bgtq::launch_quant(q, c->B, max_tiles, s);
    };
    std::vector<int64_t> lo(c->B), hi(c->B), off(c->B);
    if (R > 0) {
        // 1) tokens leaving the fp16 ring: positions [packed_old, min(packed_new, total_old)), from ring slots
        const uint16_t* rk = (const uint16_t*)c->recent_k + (size_t)layer * bh * R * D;
        const uint16_t* rv = (const uint16_t*)c->recent_v + (size_t)layer * bh * R * D;
        for (int b = 0; b < c->B; ++b) {
            lo[b] = packed_old[b];
            hi[b] = std::min(packed_new[b], total_old[b]);
            if (hi[b] < lo[b]) hi[b] = lo[b];
            off[b] = 0;
        }
        e = run(rk, rv, BGTQ_F16, (int64_t)g.Hkv * R * D, D, (int64_t)R * D, R, lo, hi, off);
        if (e != hipSuccess) return hip_fail(e, "quantize (ring eviction)");
    }
    // 2) new rows that go straight to the packed cache: positions [max(total_old, packed_old), packed_new)
    for (int b = 0; b < c->B; ++b) {
        lo[b] = std::max(total_old[b], packed_old[b]);
        hi[b] = std::max(packed_new[b], lo[b]);
        off[b] = total_old[b];
    }
    e = run(k, v, dtype, sB, sT, sH, 0, lo, hi, off);
    if (e != hipSuccess) return hip_fail(e, "quantize (new rows)");
    if (R > 0) {
        // 3) new rows that stay in the fp16 window: positions [max(packed_new, total_old), total_new)
        bgtq::RingArgs ra{};
        ra.k = k;
        ra.v = v;
        ra.dtype = dtype;
        ra.sB = sB; ra.sT = sT; ra.sH = sH;
        ra.ring_k = (uint16_t*)c->recent_k + (size_t)layer * bh * R * D;
        ra.ring_v = (uint16_t*)c->recent_v + (size_t)layer * bh * R * D;
        ra.Hkv = g.Hkv;
        ra.n_recent = R;
        int64_t max_rows = 0;
        for (int b = 0; b < c->B; ++b) {
            ra.pos_lo[b] = std::max(packed_new[b], total_old[b]);
            ra.pos_hi[b] = total_new[b];
            ra.off[b] = total_old[b];
            max_rows = std::max(max_rows, ra.pos_hi[b] - ra.pos_lo[b]);
        }
        e = bgtq::launch_ring(ra, c->B, max_rows, s);
        if (e != hipSuccess) return hip_fail(e, "ring write");
    }
    for (int b = 0; b < c->B; ++b) nt[b] = total_new[b];
    return ok();
}

}  // namespace

extern "C" {

int bgtq_quantize_append(bgtq_cache* c, int layer, const void* k, const void* v, int dtype, int64_t n_new,
                         const int64_t* strides, void* stream) {
    return quantize_append_impl(c, layer, k, v, dtype, n_new, strides, stream, false);
}

int64_t bgtq_logquant_workspace_bytes(const bgtq_cache* c, int64_t n_prompt) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (n_prompt < 0) return fail(BGTQ_E_INVALID, "n_prompt < 0");
    const int64_t R = c->n_recent;
    // the store permutation of every sequence (int16), when it does not fit the kernel arguments
    const int64_t perm = (int64_t)c->B * R > bgtq::BGTQ_PERM_MAX ? (int64_t)c->B * R * 2 : 0;
    // a prefill's gather indices (int32): the leaving tokens in leaving order, then the kept ones
    const int64_t gather = n_prompt > 0 ? (n_prompt + R) * 4 : 0;
    const int64_t need = std::max(perm, gather);
    return need ? (need + 255) / 256 * 256 : 0;
}

int bgtq_logquant_append(bgtq_cache* c, int layer, const void* k, const void* v, int dtype, const int64_t* strides,
                         int64_t* hp_pos, void* ws, size_t ws_bytes, void* stream) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (layer < 0 || layer >= c->L) return fail(BGTQ_E_INVALID, "layer %d out of range", layer);
    if (!c->n_hp) return fail(BGTQ_E_INVALID, "the log-based filter needs n_hp");
    const int R = c->n_recent;
    if (R < 3 || R % 3 || R > bgtq::BGTQ_HP_ROWS_MAX)
        return fail(BGTQ_E_INVALID, "n_recent=%d must be a multiple of 3 in [3, %d]", R, bgtq::BGTQ_HP_ROWS_MAX);
    const bool perm_in_ws = (int64_t)c->B * R > bgtq::BGTQ_PERM_MAX;
    if (perm_in_ws && (!ws || ws_bytes < (size_t)c->B * R * 2 || ((uintptr_t)ws & 255)))
        return fail(BGTQ_E_INVALID, "B * n_recent above %d: the store permutation needs a 256-byte aligned workspace "
                    "of bgtq_logquant_workspace_bytes(c, 0) bytes", bgtq::BGTQ_PERM_MAX);
    if (!k || !v || !hp_pos) return fail(BGTQ_E_INVALID, "NULL k/v/hp_pos");
    if (!dtype_ok(dtype)) return fail(BGTQ_E_INVALID, "bad dtype");
    if (!c->n_tokens) return fail(BGTQ_E_INVALID, "n_tokens is NULL");
    if (!c->k_codes || !c->v_codes || !c->k_scale || !c->v_scale || !c->recent_k || !c->recent_v)
        return fail(BGTQ_E_INVALID, "NULL cache buffer");
    if (c->k_mode == BGTQ_K_BLOCKGTQ && (!c->bits || !c->sigma || !c->inv_sigma))
        return fail(BGTQ_E_INVALID, "Block-GTQ keys need bits, sigma and inv_sigma");
    if (c->k_mode == BGTQ_K_AFFINE && !c->k_zero) return fail(BGTQ_E_INVALID, "affine keys need k_zero");
    if (c->v_mode == BGTQ_V_AFFINE && !c->v_zero) return fail(BGTQ_E_INVALID, "affine values need v_zero");
    const int W = R / 3;
    int64_t sB, sT, sH;
    if (strides) {
        sB = strides[0]; sT = strides[1]; sH = strides[2];
    } else {
        sH = D; sT = (int64_t)g.Hkv * D; sB = sT;
    }
    int64_t* nt = c->n_tokens + (size_t)layer * c->B;
    int32_t* nhp = c->n_hp + (size_t)layer * c->B;
    // Plan every sequence on copies of the bookkeeping: nothing changes unless all plans succeed.
    std::vector<int64_t> pos(hp_pos, hp_pos + (size_t)c->B * R);
    std::vector<int> nh(c->B), slot(c->B), leaving(c->B);
    std::vector<int32_t> ev(W), ms(W), md(W);
    std::vector<int16_t> perm_host(perm_in_ws ? (size_t)c->B * R : 0);
    bgtq::PermuteArgs pa{};
    pa.Hkv = g.Hkv;
    pa.n_recent = R;
    int n_perm = 0, n_thin = 0;
    for (int b = 0; b < c->B; ++b) {
        pa.seq_first[b] = -1;
        if (nhp[b] < 0 || nhp[b] > R || nhp[b] > nt[b])
            return fail(BGTQ_E_INVALID, "sequence %d: n_hp %d inconsistent with n_tokens", b, nhp[b]);
        const int64_t packed = nt[b] - nhp[b];
        nh[b] = nhp[b];
        int n_moves = 0;
        rc = bgtq_logquant_plan(W, pos.data() + (size_t)b * R, &nh[b], nt[b], ev.data(), ms.data(), md.data(), &n_moves,
                                &slot[b]);
        if (rc < 0) return rc;
        leaving[b] = rc;
        if (rc == 0) continue;
        if (packed + W > c->n_cap)
            return fail(BGTQ_E_CAPACITY, "sequence %d: %lld packed tokens exceed n_cap %lld", b,
                        (long long)(packed + W), (long long)c->n_cap);
        // kept rows stay or fill the vacated slots below 2W; the leaving rows go to [2W, 3W) in order
        int16_t* perm = (perm_in_ws ? perm_host.data() : pa.perm) + n_perm;
        for (int j = 0; j < R; ++j) perm[j] = (int16_t)j;
        for (int m = 0; m < n_moves; ++m) perm[md[m]] = (int16_t)ms[m];
        for (int i = 0; i < W; ++i) perm[2 * W + i] = (int16_t)ev[i];
        pa.seq_first[b] = n_perm;
        n_perm += R;
        ++n_thin;
    }
    hipStream_t s = (hipStream_t)stream;
    const size_t bh = (size_t)g.B * g.Hkv;
    uint16_t* rk = (uint16_t*)c->recent_k + (size_t)layer * bh * R * D;
    uint16_t* rv = (uint16_t*)c->recent_v + (size_t)layer * bh * R * D;
    hipError_t e;
    if (n_thin) {
        pa.rows_k = rk;
        pa.rows_v = rv;
        if (perm_in_ws) {
            e = bgtq::copy_to_device(ws, perm_host.data(), (size_t)n_perm * 2, s);
            if (e != hipSuccess) return hip_fail(e, "store permutation copy");
            pa.perm_dev = (const int16_t*)ws;
        }
        e = bgtq::launch_permute(pa, c->B, s);
        if (e != hipSuccess) return hip_fail(e, "store reorder");
        // the leaving rows, now in store slots [2W, 3W), become packed positions [packed, packed + W)
        bgtq::QuantArgs q{};
        fill_quant_layer(c, g, layer, q);
        q.src_k = rk;
        q.src_v = rv;
        q.dtype = BGTQ_F16;
        q.sB = (int64_t)g.Hkv * R * D;
        q.sT = D;
        q.sH = (int64_t)R * D;
        q.mod_n = 0;
        int64_t max_tiles = 0;
        for (int b = 0; b < c->B; ++b) {
            const int64_t packed = nt[b] - nhp[b];
            q.pos_lo[b] = packed;
            q.pos_hi[b] = packed + leaving[b];
            q.off[b] = packed - 2 * W;
            q.tile0[b] = packed / TILE;
            if (leaving[b]) max_tiles = std::max(max_tiles, (packed + leaving[b] - 1) / TILE - packed / TILE + 1);
        }
        {
            ProfScope ps(BGTQ_PROF_QUANTIZE, s);
            e = bgtq::launch_quant(q, c->B, max_tiles, s);
        }
        if (e != hipSuccess) return hip_fail(e, "quantize (leaving rows)");
    }
    // the new token's row enters its store slot (slot = position mod n_recent with position = slot)
    bgtq::RingArgs ra{};
    ra.k = k;
    ra.v = v;
    ra.dtype = dtype;
    ra.sB = sB; ra.sT = sT; ra.sH = sH;
    ra.ring_k = rk;
    ra.ring_v = rv;
    ra.Hkv = g.Hkv;
    ra.n_recent = R;
    for (int b = 0; b < c->B; ++b) {
        ra.pos_lo[b] = slot[b];
        ra.pos_hi[b] = slot[b] + 1;
        ra.off[b] = slot[b];
    }
    e = bgtq::launch_ring(ra, c->B, 1, s);
    if (e != hipSuccess) return hip_fail(e, "store write");
    std::copy(pos.begin(), pos.end(), hp_pos);
    for (int b = 0; b < c->B; ++b) {
        nhp[b] = nh[b];
        nt[b] += 1;
    }
    return ok();
}

int bgtq_logquant_prefill(bgtq_cache* c, int layer, const void* k, const void* v, int dtype, int64_t n_prompt,
                          const int64_t* strides, int64_t* hp_pos, void* ws, size_t ws_bytes, void* stream) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (layer < 0 || layer >= c->L) return fail(BGTQ_E_INVALID, "layer %d out of range", layer);
    if (!c->n_hp) return fail(BGTQ_E_INVALID, "the log-based filter needs n_hp");
    const int R = c->n_recent;
    if (R < 3 || R % 3 || R > bgtq::BGTQ_HP_ROWS_MAX)
        return fail(BGTQ_E_INVALID, "n_recent=%d must be a multiple of 3 in [3, %d]", R, bgtq::BGTQ_HP_ROWS_MAX);
    if (!k || !v || !hp_pos) return fail(BGTQ_E_INVALID, "NULL k/v/hp_pos");
    if (!dtype_ok(dtype)) return fail(BGTQ_E_INVALID, "bad dtype");
    if (n_prompt < 1 || n_prompt > INT32_MAX) return fail(BGTQ_E_INVALID, "n_prompt must be in [1, 2^31)");
    if (!c->n_tokens) return fail(BGTQ_E_INVALID, "n_tokens is NULL");
    if (!c->k_codes || !c->v_codes || !c->k_scale || !c->v_scale || !c->recent_k || !c->recent_v)
        return fail(BGTQ_E_INVALID, "NULL cache buffer");
    if (c->k_mode == BGTQ_K_BLOCKGTQ && (!c->bits || !c->sigma || !c->inv_sigma))
        return fail(BGTQ_E_INVALID, "Block-GTQ keys need bits, sigma and inv_sigma");
    if (c->k_mode == BGTQ_K_AFFINE && !c->k_zero) return fail(BGTQ_E_INVALID, "affine keys need k_zero");
    if (c->v_mode == BGTQ_V_AFFINE && !c->v_zero) return fail(BGTQ_E_INVALID, "affine values need v_zero");
    int64_t* nt = c->n_tokens + (size_t)layer * c->B;
    int32_t* nhp = c->n_hp + (size_t)layer * c->B;
    for (int b = 0; b < c->B; ++b)
        if (nt[b] != 0 || nhp[b] != 0) return fail(BGTQ_E_INVALID, "sequence %d is not empty: prefill starts a layer", b);
    const int64_t need = bgtq_logquant_workspace_bytes(c, n_prompt);
    if (!ws || ws_bytes < (size_t)need || ((uintptr_t)ws & 255))
        return fail(BGTQ_E_INVALID, "workspace must be 256-byte aligned and hold %lld bytes", (long long)need);
    // The filter's selection over positions 0..n_prompt-1 (the same for every sequence): a store of
    // at most 3W positions; at 3W, of its 2W oldest the 2nd, 4th, ... leave, oldest first.
    const int W = R / 3;
    std::vector<int32_t> hp, leave;
    hp.reserve(R + 1);
    leave.reserve((size_t)n_prompt);
    std::vector<int32_t> keep;
    keep.reserve(R);
    for (int64_t p = 0; p < n_prompt; ++p) {
        if ((int)hp.size() == R) {
            keep.clear();
            for (int i = 0; i < 2 * W; ++i) (i % 2 ? leave : keep).push_back(hp[i]);
            for (int i = 2 * W; i < R; ++i) keep.push_back(hp[i]);
            hp.swap(keep);
        }
        hp.push_back((int32_t)p);
    }
    const int64_t n_leave = (int64_t)leave.size(), n_keep = (int64_t)hp.size();
    if (n_leave > c->n_cap)
        return fail(BGTQ_E_CAPACITY, "%lld packed tokens exceed n_cap %lld", (long long)n_leave, (long long)c->n_cap);
    int64_t sB, sT, sH;
    if (strides) {
        sB = strides[0]; sT = strides[1]; sH = strides[2];
    } else {
        sH = D; sT = (int64_t)g.Hkv * D; sB = n_prompt * sT;
    }
    hipStream_t s = (hipStream_t)stream;
    // gather indices in the workspace: the leaving tokens (packed positions 0..n_leave-1), then the kept
    std::vector<int32_t> idx(leave);
    idx.insert(idx.end(), hp.begin(), hp.end());
    hipError_t e = bgtq::copy_to_device(ws, idx.data(), idx.size() * 4, s);
    if (e != hipSuccess) return hip_fail(e, "prefill index copy");
    const int32_t* g_leave = (const int32_t*)ws;
    const int32_t* g_keep = g_leave + n_leave;
    if (n_leave > 0) {
        bgtq::QuantArgs q{};
        fill_quant_layer(c, g, layer, q);
        q.src_k = k;
        q.src_v = v;
        q.dtype = dtype;
        q.sB = sB; q.sT = sT; q.sH = sH;
        q.gather = g_leave;
        q.gather_stride = 0;
        q.round16 = 1;  // every leaving token was an fp16 store row first
        for (int b = 0; b < c->B; ++b) {
            q.pos_lo[b] = 0;
            q.pos_hi[b] = n_leave;
            q.off[b] = 0;
            q.tile0[b] = 0;
        }
        ProfScope ps(BGTQ_PROF_QUANTIZE, s);
        e = bgtq::launch_quant(q, c->B, (n_leave + TILE - 1) / TILE, s);
        if (e != hipSuccess) return hip_fail(e, "prefill quantize");
    }
    const size_t bh = (size_t)g.B * g.Hkv;
    bgtq::RingArgs ra{};
    ra.k = k;
    ra.v = v;
    ra.dtype = dtype;
    ra.sB = sB; ra.sT = sT; ra.sH = sH;
    ra.ring_k = (uint16_t*)c->recent_k + (size_t)layer * bh * R * D;
    ra.ring_v = (uint16_t*)c->recent_v + (size_t)layer * bh * R * D;
    ra.Hkv = g.Hkv;
    ra.n_recent = R;
    ra.gather = g_keep;
    ra.gather_stride = 0;
    for (int b = 0; b < c->B; ++b) {
        ra.pos_lo[b] = 0;
        ra.pos_hi[b] = n_keep;
        ra.off[b] = 0;
    }
    e = bgtq::launch_ring(ra, c->B, n_keep, s);
    if (e != hipSuccess) return hip_fail(e, "prefill store write");
    for (int b = 0; b < c->B; ++b) {
        int64_t* hb = hp_pos + (size_t)b * R;
        for (int64_t j = 0; j < n_keep; ++j) hb[j] = hp[j];
        for (int64_t j = n_keep; j < R; ++j) hb[j] = -1;
        nhp[b] = (int32_t)n_keep;
        nt[b] = n_prompt;
    }
    return ok();
}

int64_t bgtq_decode_workspace_bytes(const bgtq_cache* c, int n_splits) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (n_splits < 0) return fail(BGTQ_E_INVALID, "n_splits < 0");
    const int64_t max_tiles = g.n_tiles;
    // the largest count the library picks for any length up to the capacity
    int ns = n_splits;
    if (!ns) {
        const int bh = g.B * g.Hkv;
        ns = auto_splits(c, g.G, max_tiles, bh);
        if (uses_gtq_kernel(c, g.G)) ns = std::max(ns, std::max(1, cu_count() / bh));
    }
    const int parts = ns + (ring_split(g.n_recent) ? 1 : 0);
    if (parts > BGTQ_MAX_PARTS) return fail(BGTQ_E_UNSUPPORTED, "n_splits above %d", BGTQ_MAX_PARTS - 1);
    return (int64_t)g.B * g.Hq * parts * PART * 4;
}

}  // extern "C"

namespace {

// Decode body over the context lengths `lens` ([B]; the descriptor's n_tokens row, or the lengths a
// pending append will leave).  With dry_run the call validates only and launches nothing.
// Rows of a one-token append that the decode launch quantizes and writes itself (element (b, h, j)
// at b * sB + h * sH + j).
struct AppendRows {
    const void* k;
    const void* v;
    int dtype;
    int64_t sB, sH;
};

int decode_attention_impl(const bgtq_cache* c, int layer, const void* q, int dtype, float* out, void* ws,
                          size_t ws_bytes, int n_splits, void* stream, const int64_t* lens, bool dry_run,
                          bool cap_to_ws = false, const AppendRows* app = nullptr) {
    bgtq::Geometry g;
    int rc = geometry(c, g);
    if (rc) return rc;
    if (layer < 0 || layer >= c->L) return fail(BGTQ_E_INVALID, "layer %d out of range", layer);
    if (!q || !out || !ws) return fail(BGTQ_E_INVALID, "NULL q/out/ws");
    if (((uintptr_t)ws) & 255) return fail(BGTQ_E_INVALID, "workspace must be 256-byte aligned");
    if (!dtype_ok(dtype)) return fail(BGTQ_E_INVALID, "bad dtype");
    if (!c->n_tokens || !lens) return fail(BGTQ_E_INVALID, "n_tokens is NULL");
    if (n_splits < 0) return fail(BGTQ_E_INVALID, "n_splits < 0");
    if (!c->k_codes || !c->v_codes || !c->k_scale || !c->v_scale) return fail(BGTQ_E_INVALID, "NULL cache buffer");
    if (c->k_mode == BGTQ_K_BLOCKGTQ && (!c->bits || !c->sigma))
        return fail(BGTQ_E_INVALID, "NULL key metadata");
    if (c->decode_path != BGTQ_DECODE_AUTO && c->decode_path != BGTQ_DECODE_VECTOR)
        return fail(BGTQ_E_INVALID, "decode_path %d is neither BGTQ_DECODE_AUTO nor BGTQ_DECODE_VECTOR", c->decode_path);
    if (uses_gtq_kernel(c, g.G) && !c->plan)
        return fail(BGTQ_E_INVALID, "NULL decode plan (Block-GTQ keys need bgtq_prepare_metadata)");
    if (c->k_mode == BGTQ_K_AFFINE && !c->k_zero) return fail(BGTQ_E_INVALID, "affine keys need k_zero");
    if (c->v_mode == BGTQ_V_AFFINE && !c->v_zero) return fail(BGTQ_E_INVALID, "affine values need v_zero");
    if (c->n_recent > 0 && (!c->recent_k || !c->recent_v)) return fail(BGTQ_E_INVALID, "recent ring buffers are NULL");
    if (!bgtq::decode_supported(c->k_mode, g.R, c->k_bits, c->k_group, c->v_bits, g.G))
        return fail(BGTQ_E_UNSUPPORTED, "no decode kernel for this format (k_mode %d, R %d, k_bits %d, k_group %d, "
                    "v_bits %d, g %d)", c->k_mode, g.R, c->k_bits, c->k_group, c->v_bits, g.G);
    const int64_t* nt = lens;
    bgtq::DecodeArgs a{};
    int32_t n_rec[BGTQ_MAX_BATCH] = {};
    int64_t max_tiles = 0;
    bool any_recent = false;
    for (int b = 0; b < c->B; ++b) {
        if (nt[b] <= 0) return fail(BGTQ_E_INVALID, "sequence %d has an empty context", b);
        const int64_t rec = c->n_hp ? (int64_t)c->n_hp[(size_t)layer * c->B + b]
                                    : (c->n_recent > 0 ? std::min<int64_t>(nt[b], c->n_recent) : 0);
        if (rec < 0 || rec > c->n_recent || rec > nt[b])
            return fail(BGTQ_E_INVALID, "sequence %d: %lld high-precision rows do not fit", b, (long long)rec);
        a.n_packed[b] = (int32_t)(nt[b] - rec);
        n_rec[b] = (int32_t)rec;
        if (a.n_packed[b] > c->n_cap) return fail(BGTQ_E_INVALID, "sequence %d exceeds n_cap", b);
        max_tiles = std::max<int64_t>(max_tiles, ((int64_t)a.n_packed[b] + TILE - 1) / TILE);
        any_recent |= rec > 0;
    }
    // Default splits follow the current length; never more than the capacity-sized workspace holds.
    int ns = n_splits ? n_splits : auto_splits(c, g.G, std::max<int64_t>(max_tiles, 1), g.B * g.Hkv);
    const int ring = ring_split(c->n_recent) ? 1 : 0;  // the window's own partial, when it has a launch
    int parts = ns + ring;
    const size_t per_part = (size_t)g.B * g.Hq * PART * 4;
    if (cap_to_ws && n_splits == 0 && ws_bytes < parts * per_part) {
        // the library's choice, reduced to what the fixed workspace holds
        const int64_t fit = (int64_t)(ws_bytes / per_part) - ring;
        if (fit < 1)
            return fail(BGTQ_E_UNSUPPORTED, "B*Hq = %d needs %zu bytes of partials per split, above the %zu-byte "
                        "scratch", g.B * g.Hq, per_part * (1 + ring), ws_bytes);
        ns = (int)fit;
        parts = ns + ring;
    }
    if (parts > BGTQ_MAX_PARTS) return fail(BGTQ_E_UNSUPPORTED, "n_splits above %d", BGTQ_MAX_PARTS - 1);
    const size_t need = parts * per_part;
    if (ws_bytes < need)
        return fail(cap_to_ws ? BGTQ_E_UNSUPPORTED : BGTQ_E_INVALID, "%s too small (%zu < %zu bytes for %d splits)",
                    cap_to_ws ? "scratch" : "workspace", ws_bytes, need, ns);
    (void)any_recent;
    if (dry_run) return ok();
    hipStream_t s = (hipStream_t)stream;
    float* part = (float*)ws;
    hipError_t e;
    const size_t bh = (size_t)g.B * g.Hkv;
    a.k_codes = (const uint8_t*)c->k_codes + (size_t)layer * g.k_codes_layer;
    a.v_codes = (const uint8_t*)c->v_codes + (size_t)layer * g.v_codes_layer;
    a.k_scale = (const uint16_t*)((const uint8_t*)c->k_scale + (size_t)layer * g.k_scale_layer);
    a.k_zero = c->k_zero ? (const uint16_t*)((const uint8_t*)c->k_zero + (size_t)layer * g.k_scale_layer) : nullptr;
    a.v_scale = (const uint16_t*)((const uint8_t*)c->v_scale + (size_t)layer * g.v_scale_layer);
    a.v_zero = c->v_zero ? (const uint16_t*)((const uint8_t*)c->v_zero + (size_t)layer * g.v_scale_layer) : nullptr;
    a.q = q;
    a.q_dtype = dtype;
    a.bits = c->k_mode == BGTQ_K_BLOCKGTQ ? c->bits + (size_t)layer * g.Hkv * 64 : nullptr;
    a.sigma = c->k_mode == BGTQ_K_BLOCKGTQ ? c->sigma + (size_t)layer * g.Hkv * 64 : nullptr;
    a.k_rot = c->k_rot ? c->k_rot + (size_t)layer * g.Hkv * 16 : nullptr;
    a.plan = uses_gtq_kernel(c, g.G) ? (const uint8_t*)c->plan + (size_t)layer * g.Hkv * BGTQ_PLAN_BYTES : nullptr;
    bgtq::Fp16Args ra{};
    if (ring) {
        ra.k16 = (const uint16_t*)c->recent_k + (size_t)layer * bh * c->n_recent * D;
        ra.v16 = (const uint16_t*)c->recent_v + (size_t)layer * bh * c->n_recent * D;
        ra.q = q;
        ra.q_dtype = dtype;
        ra.part = part;
        ra.Hkv = g.Hkv;
        ra.Hq = g.Hq;
        ra.G = g.G;
        ra.rows = c->n_recent;
        ra.n_splits = 1;
        ra.tiles_per_split = (c->n_recent + TILE - 1) / TILE;
        ra.split0 = ns;
        ra.n_parts = parts;
        for (int b = 0; b < c->B; ++b) ra.n_valid[b] = n_rec[b];
    }
    a.part = part;
    a.Hkv = g.Hkv;
    a.Hq = g.Hq;
    a.G = g.G;
    a.n_cap = g.n_cap;
    a.n_tiles = g.n_tiles;
    a.k_tile_bytes = g.k_tile_bytes;
    a.v_tile_bytes = g.v_tile_bytes;
    a.k_group = c->k_group;
    a.n_recent = c->n_recent;
    a.n_splits = ns;
    a.n_parts = parts;
    a.tiles_per_split = (int)((max_tiles + ns - 1) / ns);
    if (a.tiles_per_split < 1) a.tiles_per_split = 1;
    a.v_affine = c->v_mode == BGTQ_V_AFFINE;
    if (app) {  // the last packed token of every sequence is written by this launch
        a.app_k = app->k;
        a.app_v = app->v;
        a.app_dtype = app->dtype;
        a.app_sB = app->sB;
        a.app_sH = app->sH;
        a.inv_sigma = c->inv_sigma + (size_t)layer * g.Hkv * 64;
        a.app_k_codes = (uint8_t*)c->k_codes + (size_t)layer * g.k_codes_layer;
        a.app_v_codes = (uint8_t*)c->v_codes + (size_t)layer * g.v_codes_layer;
        a.app_k_scale = (uint16_t*)((uint8_t*)c->k_scale + (size_t)layer * g.k_scale_layer);
        a.app_v_scale = (uint16_t*)((uint8_t*)c->v_scale + (size_t)layer * g.v_scale_layer);
        a.app_v_zero = c->v_zero ? (uint16_t*)((uint8_t*)c->v_zero + (size_t)layer * g.v_scale_layer) : nullptr;
    }
    {
        ProfScope ps(BGTQ_PROF_DECODE, s);
        e = uses_gtq_kernel(c, g.G) ? bgtq::launch_decode_gtq(a, g.B, g.R, c->v_bits, s)
                                    : bgtq::launch_decode(a, g.B, c->k_mode, g.R, c->v_bits, vector_only(c), s);
    }
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    bgtq::CombineArgs ca{part, out, parts, c->v_rot ? c->v_rot + (size_t)layer * g.Hkv * 16 : nullptr, g.Hq, g.G};
    if (ring) {
        e = bgtq::launch_fp16(ra, g.B, s);
        if (e != hipSuccess) return hip_fail(e, "recent-ring decode launch");
    } else if (c->n_recent > 0) {  // the merge attends to the window itself
        ca.k16 = (const uint16_t*)c->recent_k + (size_t)layer * bh * c->n_recent * D;
        ca.v16 = (const uint16_t*)c->recent_v + (size_t)layer * bh * c->n_recent * D;
        ca.q = q;
        ca.q_dtype = dtype;
        ca.Hkv = g.Hkv;
        ca.rows = c->n_recent;
        for (int b = 0; b < c->B; ++b) ca.n_valid[b] = n_rec[b];
    }
    e = bgtq::launch_combine(ca, g.B * g.Hq, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

}  // namespace

namespace bgtq {

int decode_capped(const bgtq_cache* c, int layer, const void* q, int dtype, float* out, void* ws, size_t ws_bytes,
                  int n_splits, void* stream) {
    const int64_t* lens = (c && c->n_tokens && layer >= 0 && layer < c->L && c->B >= 1)
                              ? c->n_tokens + (size_t)layer * c->B
                              : nullptr;
    return decode_attention_impl(c, layer, q, dtype, out, ws, ws_bytes, n_splits, stream, lens, false, true);
}

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

}  // namespace bgtq

extern "C" {

int bgtq_decode_attention(const bgtq_cache* c, int layer, const void* q, int dtype, float* out, void* ws,
                          size_t ws_bytes, int n_splits, void* stream) {
    if (c && c->n_tokens && layer >= 0 && layer < c->L && c->B >= 1)
        return decode_attention_impl(c, layer, q, dtype, out, ws, ws_bytes, n_splits, stream,
                                     c->n_tokens + (size_t)layer * c->B, false);
    return decode_attention_impl(c, layer, q, dtype, out, ws, ws_bytes, n_splits, stream, nullptr, false);
}

int bgtq_decode_step(bgtq_cache* c, int layer, const void* k, const void* v, const void* q, int dtype,
                     int64_t n_new, const int64_t* strides, float* out, void* ws, size_t ws_bytes, int n_splits,
                     void* stream) {
    // Both halves are validated against the post-append lengths before anything is enqueued.
    int rc = quantize_append_impl(c, layer, k, v, dtype, n_new, strides, stream, true);
    if (rc) return rc;
    int64_t lens[BGTQ_MAX_BATCH];
    int64_t* nt = c->n_tokens + (size_t)layer * c->B;
    for (int b = 0; b < c->B; ++b) lens[b] = nt[b] + n_new;
    rc = decode_attention_impl(c, layer, q, dtype, out, ws, ws_bytes, n_splits, stream, lens, true);
    if (rc) return rc;
    // One token per sequence into a cache without an fp16 window, on the plan-driven kernel: the
    // decode launch quantizes and writes the token itself (the wave whose tile holds it, while the
    // tile is in flight) and attends to it; otherwise the append kernels run first.
    if (n_new == 1 && !c->n_hp && c->n_recent == 0 && !c->v_rot && uses_gtq_kernel(c, c->Hq / c->Hkv)) {
        const AppendRows rows{k, v, dtype, strides ? strides[0] : (int64_t)c->Hkv * D, strides ? strides[2] : D};
        rc = decode_attention_impl(c, layer, q, dtype, out, ws, ws_bytes, n_splits, stream, lens, false, false,
                                   &rows);
        if (rc) return rc;
        for (int b = 0; b < c->B; ++b) nt[b] = lens[b];
        return ok();
    }
    rc = quantize_append_impl(c, layer, k, v, dtype, n_new, strides, stream, false);
    if (rc) return rc;
    return decode_attention_impl(c, layer, q, dtype, out, ws, ws_bytes, n_splits, stream, nt, false);
}

int64_t bgtq_fp16_decode_workspace_bytes(int64_t N, int B, int Hq, int Hkv, int n_splits) {
    if (N < 1 || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || n_splits < 0) return fail(BGTQ_E_INVALID, "bad sizes");
    const int G = Hq / Hkv;
    const int ns = n_splits ? n_splits : default_splits((N + TILE - 1) / TILE, B * Hkv, cu_count(), 2);
    if (ns > BGTQ_MAX_PARTS) return fail(BGTQ_E_UNSUPPORTED, "n_splits above %d", BGTQ_MAX_PARTS);
    (void)G;
    return (int64_t)B * Hq * ns * PART * 4;
}

int bgtq_fp16_decode_attention(const void* k16, const void* v16, int64_t N, int B, int Hq, int Hkv, int d,
                               const void* q, int dtype, float* out, void* ws, size_t ws_bytes, int n_splits,
                               void* stream) {
    if (!k16 || !v16 || !q || !out || !ws) return fail(BGTQ_E_INVALID, "NULL pointer");
    if (d != D) return fail(BGTQ_E_UNSUPPORTED, "head dim must be 128");
    if (N < 1 || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(BGTQ_E_INVALID, "bad sizes");
    if (B > BGTQ_MAX_BATCH) return fail(BGTQ_E_UNSUPPORTED, "B=%d exceeds %d", B, BGTQ_MAX_BATCH);
    if (N > INT32_MAX) return fail(BGTQ_E_UNSUPPORTED, "N too large");
    if (!dtype_ok(dtype)) return fail(BGTQ_E_INVALID, "bad dtype");
    if (n_splits < 0) return fail(BGTQ_E_INVALID, "n_splits < 0");
    if (((uintptr_t)ws) & 255) return fail(BGTQ_E_INVALID, "workspace must be 256-byte aligned");
    if (((uintptr_t)k16) & 15 || ((uintptr_t)v16) & 15) return fail(BGTQ_E_INVALID, "fp16 cache must be 16-byte aligned");
    const int G = Hq / Hkv;
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return fail(BGTQ_E_UNSUPPORTED, "group size %d unsupported", G);
    const int64_t n_tiles = (N + TILE - 1) / TILE;
    const int ns = n_splits ? n_splits : default_splits(n_tiles, B * Hkv, cu_count(), 2);
    if (ns > BGTQ_MAX_PARTS) return fail(BGTQ_E_UNSUPPORTED, "n_splits above %d", BGTQ_MAX_PARTS);
    const size_t need = (size_t)B * Hq * ns * PART * 4;
    if (ws_bytes < need) return fail(BGTQ_E_INVALID, "workspace too small (%zu < %zu)", ws_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    float* part = (float*)ws;
    hipError_t e;
    bgtq::Fp16Args a{};
    a.k16 = (const uint16_t*)k16;
    a.v16 = (const uint16_t*)v16;
    a.q = q;
    a.q_dtype = dtype;
    a.part = part;
    a.Hkv = Hkv;
    a.Hq = Hq;
    a.G = G;
    a.rows = N;
    a.n_splits = ns;
    a.tiles_per_split = (int)((n_tiles + ns - 1) / ns);
    a.split0 = 0;
    a.n_parts = ns;
    for (int b = 0; b < B; ++b) a.n_valid[b] = (int32_t)N;
    {
        ProfScope ps(BGTQ_PROF_FP16_DECODE, s);
        e = bgtq::launch_fp16(a, B, s);
    }
    if (e != hipSuccess) return hip_fail(e, "fp16 decode launch");
    bgtq::CombineArgs ca{part, out, ns, nullptr, Hq, Hq / Hkv};
    e = bgtq::launch_combine(ca, B * Hq, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

}  // extern "C"
