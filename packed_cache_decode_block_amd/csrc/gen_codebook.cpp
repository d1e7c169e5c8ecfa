// Build-time generator of the library's frozen TQ-MSE scalar tables.
//
// TQ-MSE (review page §1 Key Terms; abstract of "RoPE-Aware Bit Allocation for KV-Cache
// Quantization") quantizes each coordinate with a distortion-optimal scalar quantizer whose
// error falls as 4^-b.  The table used by this library for b = 1..8: the minimum-MSE scalar
// quantizer of N(0,1) with 2^b levels (every centroid the mean of its cell, every threshold the
// midpoint of its two centroids), centroids rounded to the nearest fp16, thresholds = exact
// midpoints of the rounded centroids (exact in fp32).
//
// Method: Max's shooting procedure (J. Max, "Quantizing for minimum distortion", 1960, §III).
// The quantizer is symmetric, so with an even level count the positive half starts at the
// threshold 0.  A trial first centroid c_0 fixes the whole positive half by marching outward:
// the next threshold t_{k+1} is the point where the mean of the cell [t_k, t_{k+1}] equals c_k
// (found by bisection; the cell mean grows with its right end), and the next centroid is the
// mirror c_{k+1} = 2 t_{k+1} - c_k.  The last cell [t_{h-1}, inf) must then have mean c_{h-1};
// c_0 is bisected on the sign of that mismatch (a march that cannot place a threshold means c_0
// was too large).  Cell means of finite cells are ratios of two 32-point Gauss-Legendre sums of
// x phi(x) and phi(x) over the cell; the tail cell's mean is phi(a) / Q(a).  Long double
// throughout; bisections run until the interval stops shrinking.
//
// Usage: gen_codebook <out.h>   writes constant tables consumed by host and device code.
#include <cinttypes>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

typedef long double ld;

const ld kPi = 3.14159265358979323846264338327950288L;

ld pdf(ld x) { return std::exp(-0.5L * x * x) / std::sqrt(2.0L * kPi); }

// Nodes and weights of n-point Gauss-Legendre quadrature on [-1, 1]: roots of P_n by Newton's
// method from the Chebyshev-like first guesses, weights 2 / ((1 - x^2) P_n'(x)^2).
struct GaussLegendre {
    std::vector<ld> x, w;
    explicit GaussLegendre(int n) : x(n), w(n) {
        for (int i = 0; i < n; ++i) {
            ld z = std::cos(kPi * (i + 0.75L) / (n + 0.5L)), dp = 0;
            for (int it = 0; it < 100; ++it) {
                ld p0 = 1, p1 = z;
                for (int k = 2; k <= n; ++k) {
                    const ld p2 = ((2 * k - 1) * z * p1 - (k - 1) * p0) / k;
                    p0 = p1;
                    p1 = p2;
                }
                dp = n * (z * p1 - p0) / (z * z - 1);
                const ld dz = p1 / dp;
                z -= dz;
                if (std::fabs(dz) < 1e-19L) break;
            }
            x[i] = z;
            w[i] = 2 / ((1 - z * z) * dp * dp);
        }
    }
};

const GaussLegendre& gl() {
    static const GaussLegendre q(32);
    return q;
}

// Mean of N(0,1) restricted to [a, b] (b may be +inf).
ld cell_mean(ld a, ld b) {
    if (std::isinf(b)) return pdf(a) / (0.5L * std::erfc(a / std::sqrt(2.0L)));
    const ld mid = 0.5L * (a + b), half = 0.5L * (b - a);
    ld m0 = 0, m1 = 0;
    for (size_t i = 0; i < gl().x.size(); ++i) {
        const ld x = mid + half * gl().x[i], f = gl().w[i] * pdf(x);
        m0 += f;
        m1 += f * x;
    }
    return m1 / m0;
}

// March the positive half from first centroid c0 (h centroids).  Returns false when some
// threshold cannot be placed (c0 too large); else fills c and the tail mismatch
// mean(last cell) - c[h-1].
bool march(ld c0, int h, std::vector<ld>& c, ld& mismatch) {
    c.assign(1, c0);
    ld t = 0;
    for (int k = 0; k + 1 < h; ++k) {
        const ld ck = c.back();
        if (!(ck < cell_mean(t, INFINITY))) return false;
        ld lo = t, hi = t + 1;
        while (cell_mean(t, hi) < ck) hi = t + 2 * (hi - t);
        for (;;) {
            const ld mid = 0.5L * (lo + hi);
            if (mid <= lo || mid >= hi) break;
            (cell_mean(t, mid) < ck ? lo : hi) = mid;
        }
        t = 0.5L * (lo + hi);
        c.push_back(2 * t - ck);
    }
    mismatch = cell_mean(t, INFINITY) - c.back();
    return true;
}

// Positive-half centroids c[0..h-1] of the 2^b-level quantizer.
std::vector<double> solve(int b) {
    const int h = (1 << b) / 2;
    ld lo = 0, hi = std::sqrt(2.0L / kPi);  // c0 lies below the mean of the whole half line
    std::vector<ld> c;
    ld mis = 0;
    for (;;) {
        const ld mid = 0.5L * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        const bool ok = march(mid, h, c, mis);
        (ok && mis >= 0 ? lo : hi) = mid;
    }
    if (!march(lo, h, c, mis)) {
        std::fprintf(stderr, "march failed at the converged first centroid (b=%d)\n", b);
        std::exit(1);
    }
    return std::vector<double>(c.begin(), c.end());
}

// Round a double to the nearest fp16 (ties to even) directly, without passing through float.
uint16_t to_half(double v) {
    uint16_t sign = 0;
    if (std::signbit(v)) { sign = 0x8000; v = -v; }
    if (v == 0.0) return sign;
    int e;
    std::frexp(v, &e);                       // v = m * 2^e, m in [0.5, 1)
    int exp_h = e - 1;                       // v = 1.f * 2^exp_h
    if (exp_h < -14) exp_h = -14;            // subnormal range shares the minimum exponent
    const double ulp = std::ldexp(1.0, exp_h - 10);
    double q = v / ulp;                      // exact (power-of-two scaling)
    double fl = std::floor(q);
    double rem = q - fl;
    uint64_t mant = (uint64_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (mant & 1))) ++mant;
    // mant counts ulps at exponent exp_h: normal values have mant in [1024, 2048)
    if (mant >= 2048) { mant >>= 1; ++exp_h; }
    if (exp_h > 15) return sign | 0x7C00;
    uint16_t bits;
    if (mant < 1024) bits = (uint16_t)mant;  // subnormal
    else bits = (uint16_t)(((exp_h + 15) << 10) | (mant - 1024));
    return sign | bits;
}

double half_to_double(uint16_t h) {
    const int e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v = e == 0 ? std::ldexp((double)m, -24) : std::ldexp((double)(m | 1024), e - 25);
    return (h & 0x8000) ? -v : v;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 2) { std::fprintf(stderr, "usage: %s out.h\n", argv[0]); return 2; }
    FILE* f = std::fopen(argv[1], "w");
    if (!f) { std::perror("fopen"); return 1; }
    std::fprintf(f, "// Generated by gen_codebook.cpp — frozen Lloyd-Max N(0,1) tables, b = 1..8.\n");
    std::fprintf(f, "// Entry for width b starts at index (1<<b) - 2 (centroids) / (1<<b) - b - 1 (thresholds).\n");
    std::fprintf(f, "#pragma once\n#include <stdint.h>\n");
    std::vector<uint16_t> cent;
    std::vector<uint32_t> thr;
    for (int b = 1; b <= 8; ++b) {
        std::vector<double> pos = solve(b);
        const int h = (int)pos.size();
        std::vector<uint16_t> ch(2 * h);
        for (int k = 0; k < h; ++k) {
            // the fp16 rounding must not depend on the solver's last digits
            if (to_half(pos[k] * (1 + 1e-10)) != to_half(pos[k]) || to_half(pos[k] * (1 - 1e-10)) != to_half(pos[k])) {
                std::fprintf(stderr, "centroid %d of width %d lies within 1e-10 of an fp16 rounding tie\n", k, b);
                return 1;
            }
            ch[h + k] = to_half(pos[k]);
            ch[h - 1 - k] = to_half(-pos[k]);
        }
        for (int m = 0; m < 2 * h; ++m) cent.push_back(ch[m]);
        for (int m = 1; m < 2 * h; ++m) {
            const double mid = 0.5 * (half_to_double(ch[m - 1]) + half_to_double(ch[m]));
            const float mf = (float)mid;
            if ((double)mf != mid) { std::fprintf(stderr, "midpoint not exact b=%d m=%d\n", b, m); return 1; }
            uint32_t u;
            std::memcpy(&u, &mf, 4);
            thr.push_back(u);
        }
    }
    std::fprintf(f, "#define BGTQ_CB_CENTROIDS %zu\n#define BGTQ_CB_THRESHOLDS %zu\n", cent.size(), thr.size());
    auto sep = [](size_t i, size_t per) { return i == 0 ? "\n  " : (i % per ? "," : ",\n  "); };
    std::fprintf(f, "static const uint16_t bgtq_cb_centroid_f16[%zu] = {", cent.size());
    for (size_t i = 0; i < cent.size(); ++i) std::fprintf(f, "%s0x%04x", sep(i, 12), cent[i]);
    std::fprintf(f, "};\n// the same centroids widened exactly to fp32 (bit patterns)\n");
    std::fprintf(f, "static const uint32_t bgtq_cb_centroid_f32[%zu] = {", cent.size());
    for (size_t i = 0; i < cent.size(); ++i) {
        const float v = (float)half_to_double(cent[i]);
        uint32_t u;
        std::memcpy(&u, &v, 4);
        std::fprintf(f, "%s0x%08" PRIx32, sep(i, 8), u);
    }
    std::fprintf(f, "};\nstatic const uint32_t bgtq_cb_threshold_f32[%zu] = {", thr.size());
    for (size_t i = 0; i < thr.size(); ++i) std::fprintf(f, "%s0x%08" PRIx32, sep(i, 8), thr[i]);
    std::fprintf(f, "};\n");
    // initializer lists for device-side __constant__ copies
    std::fprintf(f, "#define BGTQ_CB_CENTROID_F16_INIT {");
    for (size_t i = 0; i < cent.size(); ++i) std::fprintf(f, "%s0x%04x", i ? "," : "", cent[i]);
    std::fprintf(f, "}\n#define BGTQ_CB_CENTROID_F32_INIT {");
    for (size_t i = 0; i < cent.size(); ++i) {
        const float v = (float)half_to_double(cent[i]);
        uint32_t u;
        std::memcpy(&u, &v, 4);
        std::fprintf(f, "%s0x%08" PRIx32 "u", i ? "," : "", u);
    }
    std::fprintf(f, "}\n#define BGTQ_CB_THRESHOLD_F32_INIT {");
    for (size_t i = 0; i < thr.size(); ++i) std::fprintf(f, "%s0x%08" PRIx32 "u", i ? "," : "", thr[i]);
    std::fprintf(f, "}\n");
    // Decode-side LDS image (8 KiB).  Pair table of width w (entry a | b << w = fp16 c[a] | fp16 c[b] << 16,
    // 4 bytes) at byte 4 * 4^w; fp16 coordinate table of width w (entry a = c[a], 2 bytes) at byte
    // 2048 + 2^(w+1).  Each table starts at a multiple of its size and its offset is the index mask
    // plus a constant (4 for pairs, 2050 for coordinates), so an entry address is (bits & mask) | base
    // with base = mask + constant; a zero entry sits at 4 and at 2050 for empty slots (mask 0).
    const size_t img_bytes = 8192;
    std::vector<uint8_t> img(img_bytes, 0);
    auto put16 = [&](size_t at, uint16_t v) { img[at] = (uint8_t)(v & 0xFF); img[at + 1] = (uint8_t)(v >> 8); };
    std::vector<int> owner(img_bytes, 0);
    auto claim = [&](size_t at, size_t n, int id) {
        for (size_t i = at; i < at + n; ++i) {
            if (i >= img_bytes || owner[i]) return false;
            owner[i] = id;
        }
        return true;
    };
    if (!claim(4, 4, 1) || !claim(2050, 2, 2)) { std::fprintf(stderr, "zero entries collide\n"); return 1; }
    for (int w = 1; w <= 5; ++w) {
        const int cb = (1 << w) - 2;
        const size_t n = (size_t)1 << (2 * w), at = 4 * n;
        if (!claim(at, 4 * n, 10 + w)) { std::fprintf(stderr, "pair table %d collides\n", w); return 1; }
        for (size_t idx = 0; idx < n; ++idx) {
            put16(at + 4 * idx, cent[cb + (idx & ((1u << w) - 1))]);
            put16(at + 4 * idx + 2, cent[cb + (idx >> w)]);
        }
    }
    for (int w = 1; w <= 8; ++w) {
        const int cb = (1 << w) - 2;
        const size_t n = (size_t)1 << w, at = 2048 + 2 * n;
        if (!claim(at, 2 * n, 20 + w)) { std::fprintf(stderr, "coordinate table %d collides\n", w); return 1; }
        for (size_t idx = 0; idx < n; ++idx) put16(at + 2 * idx, cent[cb + idx]);
    }
    std::fprintf(f, "#define BGTQ_CB_MX_BYTES %zu\n#define BGTQ_CB_MX_WORDS %zu\n", img.size(), img.size() / 4);
    std::fprintf(f, "#define BGTQ_CB_MX_PAIR_BIAS 4u\n#define BGTQ_CB_MX_COORD_BIAS 2050u\n");
    std::fprintf(f, "#define BGTQ_CB_MX_INIT {");
    for (size_t i = 0; i < img.size(); i += 4) {
        const uint32_t v = (uint32_t)img[i] | ((uint32_t)img[i + 1] << 8) | ((uint32_t)img[i + 2] << 16) |
                           ((uint32_t)img[i + 3] << 24);
        std::fprintf(f, "%s0x%08" PRIx32 "u", i ? "," : "", v);
    }
    std::fprintf(f, "}\n");
    std::fclose(f);
    return 0;
}
