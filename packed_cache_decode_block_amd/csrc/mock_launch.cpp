// Test-only stand-ins for the kernel launchers (linked with bgtq_host.cpp instead of the HIP kernels).
// Each mock checks the argument block the real kernel would read — every pointer it dereferences is
// set, sizes and index ranges are consistent — and records the launch, so host logic can be tested
// without a GPU.  Not part of libbgtq.so.
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/bgtq.h"
#include "bgtq_internal.h"

namespace {
std::string g_log;
int g_launches = 0;
// the last host-to-device copy: destination and bytes (stands in for the device memory it filled)
const void* g_copy_dst = nullptr;
std::string g_copy;
// partial records per query head of the last decode launch (0: none since the reset); the merge
// after it must read exactly these
int g_decode_parts = 0;
hipError_t bad(const char* what) {
    g_log += std::string("BAD ") + what + "\n";
    return hipErrorInvalidValue;
}
void note(const char* what) {
    g_log += std::string(what) + "\n";
    ++g_launches;
}
}  // namespace

extern "C" const char* bgtq_mock_log(void) { return g_log.c_str(); }
extern "C" int bgtq_mock_launches(void) { return g_launches; }
extern "C" void bgtq_mock_reset(void) {
    g_log.clear();
    g_launches = 0;
    g_copy_dst = nullptr;
    g_copy.clear();
    g_decode_parts = 0;
}
// Bytes of the last host-to-device copy (up to max), for tests; returns how many there were.
extern "C" int64_t bgtq_mock_last_copy(void* out, int64_t max) {
    const int64_t n = (int64_t)g_copy.size();
    if (out) std::memcpy(out, g_copy.data(), (size_t)(n < max ? n : max));
    return n;
}

namespace bgtq {

thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

static hipError_t check_decode(const DecodeArgs& a, int B, int k_mode, int R, int v_bits) {
    if (!a.k_codes || !a.v_codes || !a.k_scale || !a.v_scale || !a.q || !a.part) return bad("decode: null pointer");
    if (k_mode == BGTQ_K_BLOCKGTQ && (!a.bits || !a.sigma)) return bad("decode: null key metadata");
    if (k_mode == BGTQ_K_AFFINE && !a.k_zero) return bad("decode: null k_zero");
    if (a.v_affine && !a.v_zero) return bad("decode: null v_zero");
    if (B < 1 || B > BGTQ_MAXB || a.Hkv < 1 || a.Hq != a.Hkv * a.G) return bad("decode: geometry");
    if (a.q_dtype < 0 || a.q_dtype > 2) return bad("decode: q dtype");
    if (a.k_tile_bytes != 64 * 4 * R || a.v_tile_bytes != 1024 * v_bits) return bad("decode: tile bytes");
    if (a.n_splits < 1 || a.n_parts < a.n_splits || a.n_parts > BGTQ_MAX_PARTS || a.tiles_per_split < 1)
        return bad("decode: splits");
    for (int b = 0; b < B; ++b) {
        if (a.n_packed[b] < 0 || a.n_packed[b] > a.n_cap) return bad("decode: n_packed");
        const int64_t tiles = (a.n_packed[b] + 63) / 64;
        if (tiles > (int64_t)a.n_splits * a.tiles_per_split) return bad("decode: splits do not cover the context");
    }
    if (a.n_tiles * 64 != a.n_cap) return bad("decode: n_tiles");
    g_decode_parts = a.n_parts;
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int B, int k_mode, int R, int v_bits, bool vector_only, hipStream_t) {
    if (hipError_t e = check_decode(a, B, k_mode, R, v_bits)) return e;
    note(vector_only ? "decode_vector" : "decode");
    return hipSuccess;
}

hipError_t launch_decode_gtq(const DecodeArgs& a, int B, int R, int v_bits, hipStream_t) {
    if (!a.plan) return bad("decode: null plan");
    if (a.G != 4 && a.G != 8) return bad("decode: group size of the plan-driven decode");
    if (hipError_t e = check_decode(a, B, BGTQ_K_BLOCKGTQ, R, v_bits)) return e;
    if (a.app_k) {
        if (!a.app_v || !a.inv_sigma || !a.app_k_codes || !a.app_v_codes || !a.app_k_scale || !a.app_v_scale ||
            (a.v_affine && !a.app_v_zero))
            return bad("decode: append pointers");
        if (a.app_dtype < 0 || a.app_dtype > 2) return bad("decode: append dtype");
        for (int b = 0; b < B; ++b)
            if (a.n_packed[b] < 1) return bad("decode: append into an empty sequence");
        note("decode_gtq_append");
        return hipSuccess;
    }
    note("decode_gtq");
    return hipSuccess;
}

hipError_t launch_plan(const uint8_t* bits, uint8_t* plan, int Hkv, hipStream_t) {
    if (!bits || !plan || Hkv < 1) return bad("plan");
    note("plan");
    return hipSuccess;
}

hipError_t launch_fp16(const Fp16Args& a, int B, hipStream_t) {
    if (!a.k16 || !a.v16 || !a.q || !a.part) return bad("fp16: null pointer");
    if (B < 1 || B > BGTQ_MAXB || a.Hq != a.Hkv * a.G) return bad("fp16: geometry");
    if (a.q_dtype < 0 || a.q_dtype > 2) return bad("fp16: q dtype");
    if (a.n_splits < 1 || a.split0 + a.n_splits > a.n_parts || a.n_parts > BGTQ_MAX_PARTS) return bad("fp16: splits");
    for (int b = 0; b < B; ++b) {
        if (a.n_valid[b] < 0 || a.n_valid[b] > a.rows) return bad("fp16: n_valid");
        if ((a.n_valid[b] + 63) / 64 > (int64_t)a.n_splits * a.tiles_per_split) return bad("fp16: coverage");
    }
    note("fp16");
    return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, int rows, hipStream_t) {
    if (!a.part || !a.out || a.n_parts < 1 || a.n_parts > BGTQ_MAX_PARTS || rows < 1) return bad("combine");
    if (a.v_rot && (a.Hq < 1 || a.G < 1 || a.Hq % a.G || rows % a.Hq)) return bad("combine: rotation geometry");
    if (g_decode_parts && a.n_parts != g_decode_parts) return bad("combine: partial count differs from the decode's");
    g_decode_parts = 0;
    if (a.k16) {
        if (!a.v16 || !a.q || a.rows < 1 || a.Hkv < 1 || a.G < 1 || a.Hq != a.Hkv * a.G || rows % a.Hq)
            return bad("combine: window geometry");
        if (a.q_dtype < 0 || a.q_dtype > 2) return bad("combine: q dtype");
        for (int b = 0; b < rows / a.Hq; ++b)
            if (a.n_valid[b] < 0 || a.n_valid[b] > a.rows || a.n_valid[b] > kMergeWindowMax)
                return bad("combine: window rows");
        note("combine_window");
        return hipSuccess;
    }
    note("combine");
    return hipSuccess;
}

hipError_t launch_energy(const EnergyArgs& a, hipStream_t) {
    if (!a.k || !a.q || !a.out || a.T < 1 || a.Hkv < 1 || a.G < 1) return bad("energy");
    note("energy");
    return hipSuccess;
}

hipError_t copy_to_device(void* dst, const void* src, size_t bytes, hipStream_t) {
    if (!dst || !src || bytes == 0) return bad("copy: args");
    g_copy_dst = dst;
    g_copy.assign((const char*)src, bytes);
    note("copy");
    return hipSuccess;
}

// Device int32 indices the host copied just before (the mock's only device memory).
static bool copied_range(const void* p, int64_t n) {
    const char* c = (const char*)p;
    const char* d = (const char*)g_copy_dst;
    return d && c >= d && c + n * 4 <= d + g_copy.size();
}

hipError_t launch_quant(const QuantArgs& a, int B, int64_t max_tiles, hipStream_t) {
    if (max_tiles <= 0) return hipSuccess;
    if (a.gather) {
        for (int b = 0; b < B; ++b)
            if (!copied_range(a.gather + b * a.gather_stride, a.pos_hi[b] - a.pos_lo[b])) return bad("quant: gather");
    }
    if (!a.src_k || !a.src_v || !a.k_codes || !a.v_codes || !a.k_scale || !a.v_scale) return bad("quant: null");
    if (a.k_mode == BGTQ_K_BLOCKGTQ && (!a.bits || !a.sigma || !a.inv_sigma)) return bad("quant: null metadata");
    if (a.k_mode == BGTQ_K_AFFINE && !a.k_zero) return bad("quant: null k_zero");
    if (a.v_mode == BGTQ_V_AFFINE && !a.v_zero) return bad("quant: null v_zero");
    for (int b = 0; b < B; ++b) {
        if (a.pos_lo[b] < 0 || a.pos_hi[b] < a.pos_lo[b] || a.pos_hi[b] > a.n_cap) return bad("quant: range");
        if (a.tile0[b] != a.pos_lo[b] / 64) return bad("quant: tile0");
        if (a.pos_hi[b] > a.pos_lo[b] && (a.pos_hi[b] - 1) / 64 - a.tile0[b] + 1 > max_tiles) return bad("quant: grid");
        if (!a.gather && a.mod_n == 0 && a.pos_hi[b] > a.pos_lo[b] && a.pos_lo[b] - a.off[b] < 0)
            return bad("quant: source row");
    }
    note("quant");
    return hipSuccess;
}

hipError_t launch_ring(const RingArgs& a, int B, int64_t max_rows, hipStream_t) {
    if (max_rows <= 0) return hipSuccess;
    if (!a.k || !a.v || !a.ring_k || !a.ring_v || a.n_recent < 1) return bad("ring: null");
    for (int b = 0; b < B; ++b) {
        if (a.pos_hi[b] - a.pos_lo[b] > max_rows || a.pos_hi[b] > a.n_recent + a.pos_lo[b]) return bad("ring: range");
        if (a.gather ? !copied_range(a.gather + b * a.gather_stride, a.pos_hi[b] - a.pos_lo[b]) : a.pos_lo[b] < a.off[b])
            return bad("ring: source rows");
    }
    note("ring");
    return hipSuccess;
}

hipError_t launch_permute(const PermuteArgs& a, int B, hipStream_t) {
    if (!a.rows_k || !a.rows_v || a.n_recent < 1 || a.n_recent > BGTQ_HP_ROWS_MAX) return bad("permute: args");
    for (int b = 0; b < B; ++b) {
        const int f = a.seq_first[b];
        if (f < 0) continue;
        const int16_t* perm = a.perm;
        if (a.perm_dev) {
            if (!copied_range(a.perm_dev, 0) || (int64_t)(f + a.n_recent) * 2 > (int64_t)g_copy.size())
                return bad("permute: device permutation");
            perm = (const int16_t*)g_copy.data();
        } else if (f + a.n_recent > BGTQ_PERM_MAX) {
            return bad("permute: range");
        }
        std::string seen(a.n_recent, 0);
        for (int j = 0; j < a.n_recent; ++j) {
            const int r = perm[f + j];
            if (r < 0 || r >= a.n_recent || seen[r]) return bad("permute: not a permutation");
            seen[r] = 1;
        }
    }
    note("permute");
    return hipSuccess;
}

void arm_launch_events(hipEvent_t, hipEvent_t) {}
void disarm_launch_events() {}

int decode_wgs_per_cu(int k_mode, int G, int v_bits, int k_group, bool) {
    if (G >= 4 && k_mode == BGTQ_K_BLOCKGTQ) return v_bits == 3 ? 2 : 3;
    (void)k_group;
    return 2;
}

bool decode_supported(int k_mode, int R, int k_bits, int k_group, int v_bits, int G) {
    if (!(G == 1 || G == 2 || G == 4 || G == 8)) return false;
    if (v_bits < 2 || v_bits > 4) return false;
    if (k_mode == BGTQ_K_AFFINE) return k_bits == 4 && (k_group == 32 || k_group == 64 || k_group == 128);
    return R == 8 || R == 12 || R == 16;
}

}  // namespace bgtq
