// Build-time generator of the library's frozen TQ-MSE scalar tables.
//
// TQ-MSE (review page §1 Key Terms; abstract of "RoPE-Aware Bit Allocation for KV-Cache
// Quantization") quantizes each coordinate with a distortion-optimal scalar quantizer whose
// error falls as 4^-b.  The table used by this library for b = 1..8: the Lloyd-Max quantizer
// of N(0,1) (every centroid the mean of its cell, every threshold the midpoint of its two
// centroids), centroids rounded to the nearest fp16, thresholds = exact midpoints of the
// rounded centroids (exact in fp32).  The fixed point is solved with Newton's method on the
// symmetric positive half (tridiagonal Jacobian).
//
// Usage: gen_codebook <out.h>   writes constant tables consumed by host and device code.
#include <cinttypes>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

namespace {

const double kInvSqrt2Pi = 0.3989422804014327;  // 1/sqrt(2*pi)

double pdf(double x) { return std::exp(-0.5 * x * x) * kInvSqrt2Pi; }
double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }

// Inverse normal CDF by bisection on the upper tail (only used for the starting point).
double probit(double p) {
    double lo = -40, hi = 40;
    for (int i = 0; i < 200; ++i) {
        double mid = 0.5 * (lo + hi);
        if (1.0 - upper_tail(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

// Positive-half centroids c[0..h-1] of the 2^b-level Lloyd-Max quantizer.
std::vector<double> solve(int b) {
    const int n = 1 << b, h = n / 2;
    std::vector<double> c(h), t(h + 1), mu(h), da(h), db(h);
    for (int k = 0; k < h; ++k) c[k] = probit((k + 0.5) / n + 0.5);
    for (int it = 0; it < 100; ++it) {
        t[0] = 0.0;
        for (int k = 1; k < h; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        for (int k = 0; k < h; ++k) {
            const double a = t[k];
            const bool last = (k == h - 1);
            const double fa = pdf(a);
            double num, mass, fb = 0.0, bb = 0.0;
            if (last) {
                num = fa;
                mass = upper_tail(a);
            } else {
                bb = t[k + 1];
                fb = pdf(bb);
                num = -fa * std::expm1(-0.5 * (bb - a) * (bb + a));
                mass = upper_tail(a) - upper_tail(bb);
            }
            mu[k] = num / mass;
            da[k] = fa / mass * (mu[k] - a);
            db[k] = last ? 0.0 : fb / mass * (bb - mu[k]);
        }
        // (I - J) x = mu - c with J tridiagonal: J[k][k-1] = da/2, J[k][k] = (da+db)/2, J[k][k+1] = db/2
        std::vector<double> sub(h, 0.0), dia(h, 1.0), sup(h, 0.0), rhs(h), cp(h), dp(h), x(h);
        for (int k = 0; k < h; ++k) {
            if (k >= 1) { sub[k] = -0.5 * da[k]; dia[k] -= 0.5 * da[k]; }
            if (k + 1 < h) { sup[k] = -0.5 * db[k]; dia[k] -= 0.5 * db[k]; }
            rhs[k] = mu[k] - c[k];
        }
        cp[0] = sup[0] / dia[0];
        dp[0] = rhs[0] / dia[0];
        for (int k = 1; k < h; ++k) {
            const double m = dia[k] - sub[k] * cp[k - 1];
            cp[k] = sup[k] / m;
            dp[k] = (rhs[k] - sub[k] * dp[k - 1]) / m;
        }
        x[h - 1] = dp[h - 1];
        for (int k = h - 2; k >= 0; --k) x[k] = dp[k] - cp[k] * x[k + 1];
        double step = 0.0;
        for (int k = 0; k < h; ++k) {
            c[k] += x[k];
            step = std::fmax(step, std::fabs(x[k]));
        }
        if (step < 1e-13) break;
    }
    return c;
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
