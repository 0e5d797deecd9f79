// fc_oracle.cpp -- plain, slow, single-threaded CPU oracle for the flash all-reduce data path.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file: only the
// tests, the package's smoke check and the benchmark's CPU-baseline leg use it.  It shares no code,
// header, table or constant with the HIP kernels.
//
// Build: g++ -O2 -ffp-contract=off -fPIC -shared (no -ffast-math).  Every float operation below is one
// IEEE binary32 operation with round-to-nearest-even; contraction is off, so a*b+c is two roundings.
//
// What it computes, and the passages it follows:
//  * group quantization of activations to low bit widths -- Flash Communication (abstract; summary,
//    "Core ideas of the solution": low-bit fine-grained quantization of activation values);
//  * the two-step all-reduce, reduce-scatter then all-gather -- Flash Communication (summary, "Core
//    ideas of the solution": two-step All-Reduce), with a fixed reduction order -- flash-comm (abstract:
//    transport order decoupled from reduction order);
//  * the fused residual-add + RMSNorm after the all-reduce -- TokenWeave (abstract: fused
//    AllReduce-RMSNorm);
//  * self-synchronizing blocks whose readiness is validated by the receiver -- flash-comm (abstract:
//    each data block carries evidence of its readiness).
// The pages give no formula, bit width or layout.  Where they are silent this file takes the plainest
// reading; each such reading is marked "reading:" at the point where it is used.
//
// Parity status: every function here is pinned by CPU tests against mathematics (closed forms,
// brute force, invariants, exact double arithmetic); no function is "parity unpinned".

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------------------------------------------
// Number formats.  A binary format with P significand bits (hidden bit included), minimum normal
// exponent EMIN and largest finite value MAXF.  Rounding is done on the exact double value, by
// definition: scale by the quantum of the binade, round to an integer with ties to even, scale back.
// Every value handled here (fp32 inputs) is exact in double, so this is a single correct rounding.
// ---------------------------------------------------------------------------------------------------

struct Fmt {
    int p;        // significand bits incl. hidden bit: fp16 11, bf16 8
    int emin;     // exponent of the smallest normal: fp16 -14, bf16 -126
    int ebits;    // exponent field width: fp16 5, bf16 8
};
const Fmt kF16 = {11, -14, 5};
const Fmt kBF16 = {8, -126, 8};

// Round |v| (finite, >= 0) to the format with ties-to-even; returns the rounded magnitude as double
// (may be the overflow threshold 2^(emax+1), which the caller encodes as infinity).
double round_mag_rne(double mag, const Fmt& f) {
    if (mag == 0.0) return 0.0;
    int e;
    std::frexp(mag, &e);          // mag = m * 2^e, m in [0.5, 1): binade exponent is e-1
    int binade = e - 1;
    if (binade < f.emin) binade = f.emin;  // subnormal range has the quantum of the smallest binade
    double quantum = std::ldexp(1.0, binade - (f.p - 1));
    double q = mag / quantum;     // exact: division by a power of two
    double r = std::nearbyint(q); // default rounding mode: to nearest, ties to even
    return r * quantum;           // exact
}

// Encode a magnitude that is exactly representable (or the overflow threshold) into format bits
// (without sign).
uint32_t encode_mag(double mag, const Fmt& f) {
    const int emax = (1 << (f.ebits - 1)) - 1;
    const uint32_t inf_bits = ((1u << f.ebits) - 1u) << (f.p - 1);
    if (mag == 0.0) return 0;
    int e;
    std::frexp(mag, &e);
    int binade = e - 1;
    if (binade > emax) return inf_bits;                       // rounded past the largest finite value
    if (binade < f.emin) {                                    // subnormal: integer multiple of quantum
        double quantum = std::ldexp(1.0, f.emin - (f.p - 1));
        return (uint32_t)(mag / quantum);
    }
    uint32_t biased = (uint32_t)(binade + emax);
    double frac = mag / std::ldexp(1.0, binade) - 1.0;        // in [0,1), exact
    uint32_t m = (uint32_t)(frac * std::ldexp(1.0, f.p - 1)); // exact integer
    return (biased << (f.p - 1)) | m;
}

uint32_t to_fmt_rne(float x, const Fmt& f) {
    const int total = 1 + f.ebits + (f.p - 1);
    const uint32_t sign = std::signbit(x) ? (1u << (total - 1)) : 0u;
    const uint32_t inf_bits = ((1u << f.ebits) - 1u) << (f.p - 1);
    if (std::isnan(x)) return sign | inf_bits | (1u << (f.p - 2));  // a quiet NaN
    if (std::isinf(x)) return sign | inf_bits;
    double mag = std::fabs((double)x);
    return sign | encode_mag(round_mag_rne(mag, f), f);
}

double from_fmt(uint32_t bits, const Fmt& f) {
    const int total = 1 + f.ebits + (f.p - 1);
    const int emax = (1 << (f.ebits - 1)) - 1;
    const bool neg = (bits >> (total - 1)) & 1u;
    const uint32_t ef = (bits >> (f.p - 1)) & ((1u << f.ebits) - 1u);
    const uint32_t mf = bits & ((1u << (f.p - 1)) - 1u);
    double v;
    if (ef == ((1u << f.ebits) - 1u)) {
        v = mf ? NAN : INFINITY;
    } else if (ef == 0) {
        v = std::ldexp((double)mf, f.emin - (f.p - 1));
    } else {
        v = std::ldexp(1.0 + std::ldexp((double)mf, -(f.p - 1)), (int)ef - emax);
    }
    return neg ? -v : v;
}

inline float bits_to_f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
inline uint32_t f32_to_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

// fp16 helpers
inline uint16_t f16_rne(float x) { return (uint16_t)to_fmt_rne(x, kF16); }
inline float f16_val(uint16_t h) { return (float)from_fmt(h, kF16); }  // exact widening

// Largest fp16 that is <= v ("round down").  Start from the nearest value and, when it lies above v,
// step one fp16 value toward -infinity.  From +-0 the step goes to the smallest negative subnormal.
uint16_t f16_rd(float v) {
    uint16_t h = f16_rne(v);
    if (std::isnan(v)) return h;
    if ((double)f16_val(h) > (double)v) {
        if ((h & 0x7fffu) == 0) h = 0x8001u;            // +-0 -> -2^-24
        else if (h & 0x8000u) h = (uint16_t)(h + 1u);   // negative: grow the magnitude
        else h = (uint16_t)(h - 1u);                    // positive: shrink the magnitude
    }
    return h;
}

// Smallest fp16 that is >= v ("round up").
uint16_t f16_ru(float v) {
    uint16_t h = f16_rne(v);
    if (std::isnan(v)) return h;
    if ((double)f16_val(h) < (double)v) {
        if ((h & 0x7fffu) == 0) h = 0x0001u;            // +-0 -> +2^-24
        else if (h & 0x8000u) h = (uint16_t)(h - 1u);   // negative: shrink the magnitude
        else h = (uint16_t)(h + 1u);                    // positive: grow the magnitude
    }
    return h;
}

// bf16 helpers
inline uint16_t bf16_rne(float x) { return (uint16_t)to_fmt_rne(x, kBF16); }
inline float bf16_val(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }  // exact widening

// ---------------------------------------------------------------------------------------------------
// Group quantization.  reading: asymmetric min/max quantization with a real-valued zero-point (the
// group minimum) and scale = range / (2^b - 1), both stored as fp16; codes are unsigned in [0, 2^b-1].
// The zero-point is rounded down and the scale up so that every element stays in range; a code is
// round((x - zero) / scale) with ties to even, computed as (x - zero) * (1/scale).
// ---------------------------------------------------------------------------------------------------

struct GroupMeta { uint16_t scale; uint16_t zero; };

inline uint32_t pack_meta(GroupMeta m) { return (uint32_t)m.scale | ((uint32_t)m.zero << 16); }
inline GroupMeta unpack_meta(uint32_t w) { return GroupMeta{(uint16_t)(w & 0xffffu), (uint16_t)(w >> 16)}; }

// Quantize one group of g fp32 values to unsigned codes of `bits` bits.
GroupMeta quantize_group(const float* x, int g, int bits, uint32_t* codes) {
    const int qmax = (1 << bits) - 1;
    float lo = x[0], hi = x[0];
    for (int i = 1; i < g; ++i) {
        if (x[i] < lo) lo = x[i];
        if (x[i] > hi) hi = x[i];
    }
    lo = lo + 0.0f;  // -0 becomes +0, so the zero-point never depends on which zero was the minimum
    GroupMeta m;
    m.zero = f16_rd(lo);
    const float z = f16_val(m.zero);
    const float diff = hi - z;
    float inv;
    if (diff == 0.0f) {          // constant group whose value is an fp16: scale 0, all codes 0
        m.scale = 0;
        inv = 0.0f;
    } else {
        const float t = diff / (float)qmax;
        m.scale = f16_ru(t);
        const float s = f16_val(m.scale);
        inv = 1.0f / s;
    }
    for (int i = 0; i < g; ++i) {
        const float d = x[i] - z;
        const float v = d * inv;
        float r = std::nearbyint(v);  // ties to even
        if (r < 0.0f) r = 0.0f;
        if (r > (float)qmax) r = (float)qmax;
        codes[i] = (uint32_t)r;
    }
    return m;
}

// Dequantize one code: fl(fl(q * scale) + zero).
inline float dequant_one(uint32_t q, GroupMeta m) {
    const float s = f16_val(m.scale);
    const float z = f16_val(m.zero);
    const float p = (float)q * s;
    return p + z;
}

// Code storage: bits = 8, byte i holds code i; bits = 4, byte i holds code 2i in its low nibble and
// code 2i+1 in its high nibble.
inline void put_code(uint8_t* codes, int64_t i, int bits, uint32_t q) {
    if (bits == 8) {
        codes[i] = (uint8_t)q;
    } else {
        uint8_t& b = codes[i >> 1];
        if ((i & 1) == 0) b = (uint8_t)((b & 0xf0u) | (q & 0x0fu));
        else b = (uint8_t)((b & 0x0fu) | ((q & 0x0fu) << 4));
    }
}
inline uint32_t get_code(const uint8_t* codes, int64_t i, int bits) {
    if (bits == 8) return codes[i];
    const uint8_t b = codes[i >> 1];
    return (i & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 0x0fu);
}

void quantize_f32(const float* x, int64_t n, int bits, int group, uint8_t* codes, uint32_t* meta) {
    std::vector<uint32_t> q(group);
    for (int64_t g0 = 0, k = 0; g0 < n; g0 += group, ++k) {
        GroupMeta m = quantize_group(x + g0, group, bits, q.data());
        meta[k] = pack_meta(m);
        for (int i = 0; i < group; ++i) put_code(codes, g0 + i, bits, q[i]);
    }
}

void dequant_f32(const uint8_t* codes, const uint32_t* meta, int64_t n, int bits, int group, float* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = dequant_one(get_code(codes, i, bits), unpack_meta(meta[i / group]));
}

// ---------------------------------------------------------------------------------------------------
// RMSNorm epilogue on one row: h = y + residual (fp32), residual_out = bf16(h),
// r = 1/sqrt(mean(h^2) + eps), out = bf16((h * r) * gamma).  reading: eps inside the square root,
// the product taken in fp32 before the single rounding to bf16, gamma applied last.
// ---------------------------------------------------------------------------------------------------

// Sum of squares of a row as the plain reading of the epilogue has it: the left fold of fl(h_j * h_j) over
// j = 0 .. H-1 (each square rounded, then added; no fused multiply-add).
float sumsq_seq(const float* h, int64_t hidden) {
    float ss = 0.0f;
    for (int64_t j = 0; j < hidden; ++j) {
        const float sq = h[j] * h[j];
        ss = ss + sq;
    }
    return ss;
}

void rmsnorm_row(const float* y, const uint16_t* residual, const uint16_t* gamma, float eps, int64_t hidden,
                 uint16_t* out, uint16_t* residual_out, float* hbuf) {
    for (int64_t j = 0; j < hidden; ++j) {
        float h = y[j];
        if (residual) h = h + bf16_val(residual[j]);
        hbuf[j] = h;
    }
    if (residual_out)
        for (int64_t j = 0; j < hidden; ++j) residual_out[j] = bf16_rne(hbuf[j]);
    const float ss = sumsq_seq(hbuf, hidden);
    const float ms = ss / (float)hidden;
    const float rinv = 1.0f / std::sqrt(ms + eps);
    for (int64_t j = 0; j < hidden; ++j) {
        const float a = hbuf[j] * rinv;
        const float b = a * bf16_val(gamma[j]);
        out[j] = bf16_rne(b);
    }
}

// ---------------------------------------------------------------------------------------------------
// Sum of squares of a row in the tree order of the kernels' reproducibility contract, for the variant
// that normalizes the reduce-scattered shard before the all-gather (TokenWeave, abstract: RMSNorm fused
// with, and moved relative to, the communication).  The plain reading of that variant sums the squares
// as the epilogue does (sumsq_seq above); the pages fix no order, and the normalized values decide
// integer codes, so the GPU commits to one fixed order of its own, independent of its launch shape, and
// this function restates that order so that the kernels' other steps can be checked bit for bit: chunk
// c is elements [8c, 8c+8) of the row; its partial p_c is the left fold of fl(h*h) over its 8 elements;
// the row sum is the pairwise tree over p_0 .. p_{m-1}, m = the chunk count rounded up to a power of
// two, absent chunks 0: level 0 = p, level k+1 [i] = level k [2i] + level k [2i+1].
// ---------------------------------------------------------------------------------------------------
float sumsq_tree(const float* h, int64_t hidden) {
    const int64_t nch = hidden / 8;
    int64_t m = 1;
    while (m < nch) m *= 2;
    std::vector<float> lvl(m, 0.0f);
    for (int64_t c = 0; c < nch; ++c) {
        float p = h[8 * c] * h[8 * c];
        for (int e = 1; e < 8; ++e) {
            const float sq = h[8 * c + e] * h[8 * c + e];
            p = p + sq;
        }
        lvl[c] = p;
    }
    for (int64_t w = m; w > 1; w /= 2)
        for (int64_t i = 0; i < w / 2; ++i) lvl[i] = lvl[2 * i] + lvl[2 * i + 1];
    return lvl[0];
}

// Normalized rows in fp32, for quantization: h = y + residual, residual_out = bf16(h),
// r = 1/sqrt(ss/H + eps) with ss = sumsq_seq(h) (order 0, the plain reading) or sumsq_tree(h) (order 1),
// o = fl(fl(h * r) * gamma) (not rounded to bf16: the next step quantizes it, as the all-gather payload
// is quantized from fp32 sums in the other variant).
void norm_row_f32(const float* y, const uint16_t* residual, const uint16_t* gamma, float eps, int64_t hidden,
                  int order, float* o, uint16_t* residual_out, float* hbuf) {
    for (int64_t j = 0; j < hidden; ++j) {
        float h = y[j];
        if (residual) h = h + bf16_val(residual[j]);
        hbuf[j] = h;
    }
    if (residual_out)
        for (int64_t j = 0; j < hidden; ++j) residual_out[j] = bf16_rne(hbuf[j]);
    const float ss = order == 1 ? sumsq_tree(hbuf, hidden) : sumsq_seq(hbuf, hidden);
    const float ms = ss / (float)hidden;
    const float rinv = 1.0f / std::sqrt(ms + eps);
    for (int64_t j = 0; j < hidden; ++j) {
        const float a = hbuf[j] * rinv;
        o[j] = a * bf16_val(gamma[j]);
    }
}

}  // namespace

extern "C" {

int or_version(void) { return 1; }

// ---- conversions (exposed so the tests can pin them) ------------------------------------------------
// mode 0 = nearest-even, 1 = down, 2 = up
void or_f32_to_f16(const float* x, int64_t n, int mode, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = mode == 0 ? f16_rne(x[i]) : mode == 1 ? f16_rd(x[i]) : f16_ru(x[i]);
}
void or_f16_to_f32(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = f16_val(h[i]);
}
void or_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(x[i]);
}

// ---- group quantization -----------------------------------------------------------------------------
// x: n fp32 (or bf16) values; n % group == 0.  codes: n*bits/8 bytes; meta: n/group words,
// bits 0..15 = fp16 scale, bits 16..31 = fp16 zero-point.
void or_quantize_f32(const float* x, int64_t n, int bits, int group, uint8_t* codes, uint32_t* meta) {
    quantize_f32(x, n, bits, group, codes, meta);
}
void or_quantize_bf16(const uint16_t* x, int64_t n, int bits, int group, uint8_t* codes, uint32_t* meta) {
    std::vector<float> f(n);
    for (int64_t i = 0; i < n; ++i) f[i] = bf16_val(x[i]);
    quantize_f32(f.data(), n, bits, group, codes, meta);
}
void or_dequant(const uint8_t* codes, const uint32_t* meta, int64_t n, int bits, int group, float* y) {
    dequant_f32(codes, meta, n, bits, group, y);
}

// ---- reduce-scatter receive side: one shard ----------------------------------------------------------
// codes[r], meta[r]: rank r's quantized chunk of this shard (L elements).  The R chunks are
// dequantized and summed in fp32 as a left fold in ascending rank order, starting from rank 0's value
// (flash-comm, abstract: reduction order fixed, independent of arrival order).  The fp32 sum S (if
// requested) is then requantized at bits_out for the all-gather hop.
void or_reduce_shard(const uint8_t* const* codes, const uint32_t* const* meta, int R, int64_t L,
                     int bits_in, int bits_out, int group, float* S_out, uint8_t* out_codes,
                     uint32_t* out_meta) {
    std::vector<float> S(L);
    for (int64_t i = 0; i < L; ++i) {
        float acc = dequant_one(get_code(codes[0], i, bits_in), unpack_meta(meta[0][i / group]));
        for (int r = 1; r < R; ++r) {
            const float d = dequant_one(get_code(codes[r], i, bits_in), unpack_meta(meta[r][i / group]));
            acc = acc + d;
        }
        S[i] = acc;
    }
    if (S_out) std::memcpy(S_out, S.data(), sizeof(float) * L);
    if (out_codes && out_meta) quantize_f32(S.data(), L, bits_out, group, out_codes, out_meta);
}

// ---- RMSNorm of fp32 rows ------------------------------------------------------------------------------
void or_rmsnorm(const float* y, const uint16_t* residual, const uint16_t* gamma, float eps, int64_t rows,
                int64_t hidden, uint16_t* out, uint16_t* residual_out) {
    std::vector<float> h(hidden);
    for (int64_t t = 0; t < rows; ++t)
        rmsnorm_row(y + t * hidden, residual ? residual + t * hidden : nullptr, gamma, eps, hidden,
                    out + t * hidden, residual_out ? residual_out + t * hidden : nullptr, h.data());
}

// ---- all-gather receive side ------------------------------------------------------------------------------
// shards[s] (codes, meta): the requantized shard s, elements [s*L, (s+1)*L) of the [rows, hidden]
// output.  Plain mode (y != NULL): y = bf16(dequant).  Norm mode (gamma != NULL): residual-add +
// RMSNorm epilogue on the fp32 dequantized values.
void or_gather(const uint8_t* const* codes, const uint32_t* const* meta, int R, int64_t L, int bits, int group,
               uint16_t* y, const uint16_t* residual, const uint16_t* gamma, float eps, int64_t hidden,
               uint16_t* out, uint16_t* residual_out) {
    const int64_t n = (int64_t)R * L;
    std::vector<float> f(n);
    for (int s = 0; s < R; ++s) dequant_f32(codes[s], meta[s], L, bits, group, f.data() + (int64_t)s * L);
    if (y)
        for (int64_t i = 0; i < n; ++i) y[i] = bf16_rne(f[i]);
    if (gamma) or_rmsnorm(f.data(), residual, gamma, eps, n / hidden, hidden, out, residual_out);
}

// ---- the whole quantized two-step all-reduce, as seen by every rank ---------------------------------
// parts: R pointers to bf16 [n] partial sums.  Writes the per-rank messages (codes1 [R][n*b1/8],
// meta1 [R][n/group]), the requantized shards (codes2 [n*b2/8], meta2 [n/group], shard s at offset
// s*L), and the gathered output (plain y and/or norm out + residual_out).
void or_two_step(const uint16_t* const* parts, int R, int64_t n, int bits1, int bits2, int group,
                 uint8_t* codes1, uint32_t* meta1, uint8_t* codes2, uint32_t* meta2, uint16_t* y,
                 const uint16_t* residual, const uint16_t* gamma, float eps, int64_t hidden, uint16_t* out,
                 uint16_t* residual_out) {
    const int64_t L = n / R;
    const int64_t c1 = n * bits1 / 8, c2 = L * bits2 / 8, g1 = n / group, g2 = L / group;
    for (int r = 0; r < R; ++r) or_quantize_bf16(parts[r], n, bits1, group, codes1 + r * c1, meta1 + r * g1);
    std::vector<const uint8_t*> cin(R);
    std::vector<const uint32_t*> min_(R);
    for (int s = 0; s < R; ++s) {
        for (int r = 0; r < R; ++r) {
            cin[r] = codes1 + r * c1 + s * (L * bits1 / 8);
            min_[r] = meta1 + r * g1 + s * (L / group);
        }
        or_reduce_shard(cin.data(), min_.data(), R, L, bits1, bits2, group, nullptr, codes2 + s * c2,
                        meta2 + s * g2);
    }
    std::vector<const uint8_t*> gc(R);
    std::vector<const uint32_t*> gm(R);
    for (int s = 0; s < R; ++s) { gc[s] = codes2 + s * c2; gm[s] = meta2 + s * g2; }
    or_gather(gc.data(), gm.data(), R, L, bits2, group, y, residual, gamma, eps, hidden, out, residual_out);
}

// ---- norm before the all-gather (TokenWeave, abstract) ---------------------------------------------------
// The fixed-order sum of squares of one row (exposed for the tests).
float or_sumsq_tree(const float* h, int64_t hidden) { return sumsq_tree(h, hidden); }
float or_sumsq_seq(const float* h, int64_t hidden) { return sumsq_seq(h, hidden); }

// fp32 normalized rows (norm_row_f32, order 0 plain or 1 tree) of y [rows*hidden].
void or_norm_rows_f32(const float* y, const uint16_t* residual, const uint16_t* gamma, float eps, int64_t rows,
                      int64_t hidden, int order, float* o, uint16_t* residual_out) {
    std::vector<float> h(hidden);
    for (int64_t t = 0; t < rows; ++t)
        norm_row_f32(y + t * hidden, residual ? residual + t * hidden : nullptr, gamma, eps, hidden, order,
                     o + t * hidden, residual_out ? residual_out + t * hidden : nullptr, h.data());
}

// One shard, norm first: S = the fixed-order fold of the R dequantized chunks (as or_reduce_shard); the
// shard holds whole rows (L % hidden == 0); h = S + residual (the shard's rows), residual_out = bf16(h),
// o = the normalized rows (norm_row_f32), quantized at bits_out for the all-gather.  o_out (may be NULL)
// receives o.  order: the sum of squares' order (0 plain, 1 tree; norm_row_f32).
void or_reduce_norm_quant(const uint8_t* const* codes, const uint32_t* const* meta, int R, int64_t L, int bits_in,
                          int bits_out, int group, const uint16_t* residual, const uint16_t* gamma, float eps,
                          int64_t hidden, int order, uint16_t* residual_out, uint8_t* out_codes, uint32_t* out_meta,
                          float* o_out) {
    std::vector<float> S(L), o(L);
    or_reduce_shard(codes, meta, R, L, bits_in, bits_out, group, S.data(), nullptr, nullptr);
    or_norm_rows_f32(S.data(), residual, gamma, eps, L / hidden, hidden, order, o.data(), residual_out);
    if (o_out) std::memcpy(o_out, o.data(), sizeof(float) * L);
    quantize_f32(o.data(), L, bits_out, group, out_codes, out_meta);
}

// The whole two-step all-reduce with the norm before the all-gather: every rank's message (as
// or_two_step), every shard's reduce + residual-add + norm + quantization (residual_out of every row,
// codes2/meta2 as in or_two_step), then the gather: y = bf16(dequant) of the normalized rows.
void or_two_step_normfirst(const uint16_t* const* parts, int R, int64_t n, int bits1, int bits2, int group,
                           uint8_t* codes1, uint32_t* meta1, uint8_t* codes2, uint32_t* meta2,
                           const uint16_t* residual, const uint16_t* gamma, float eps, int64_t hidden, int order,
                           uint16_t* residual_out, uint16_t* y) {
    const int64_t L = n / R;
    const int64_t c1 = n * bits1 / 8, c2 = L * bits2 / 8, g1 = n / group, g2 = L / group;
    for (int r = 0; r < R; ++r) or_quantize_bf16(parts[r], n, bits1, group, codes1 + r * c1, meta1 + r * g1);
    std::vector<const uint8_t*> cin(R);
    std::vector<const uint32_t*> min_(R);
    for (int s = 0; s < R; ++s) {
        for (int r = 0; r < R; ++r) {
            cin[r] = codes1 + r * c1 + s * (L * bits1 / 8);
            min_[r] = meta1 + r * g1 + s * (L / group);
        }
        or_reduce_norm_quant(cin.data(), min_.data(), R, L, bits1, bits2, group, residual ? residual + s * L : nullptr,
                             gamma, eps, hidden, order, residual_out ? residual_out + s * L : nullptr,
                             codes2 + s * c2, meta2 + s * g2, nullptr);
    }
    std::vector<const uint8_t*> gc(R);
    std::vector<const uint32_t*> gm(R);
    for (int s = 0; s < R; ++s) { gc[s] = codes2 + s * c2; gm[s] = meta2 + s * g2; }
    or_gather(gc.data(), gm.data(), R, L, bits2, group, y, nullptr, nullptr, 0.0f, hidden, nullptr, nullptr);
}

// ---- unquantized fused reduce + residual-add + RMSNorm (TokenWeave, abstract) -------------------------
void or_reduce_rmsnorm(const uint16_t* const* parts, int R, int64_t rows, int64_t hidden, const uint16_t* residual,
                       const uint16_t* gamma, float eps, uint16_t* out, uint16_t* residual_out, uint16_t* y_out) {
    const int64_t n = rows * hidden;
    std::vector<float> y(n);
    for (int64_t i = 0; i < n; ++i) {
        float acc = bf16_val(parts[0][i]);
        for (int r = 1; r < R; ++r) acc = acc + bf16_val(parts[r][i]);
        y[i] = acc;
    }
    if (y_out)
        for (int64_t i = 0; i < n; ++i) y_out[i] = bf16_rne(y[i]);
    if (gamma) or_rmsnorm(y.data(), residual, gamma, eps, rows, hidden, out, residual_out);
}

// ---- self-synchronizing slots (flash-comm, abstract) ----------------------------------------------------
// A slot is a little-endian 64-bit word: bits 0..15 = bf16 element 2k, bits 16..31 = element 2k+1,
// bits 32..63 = the epoch of the round that wrote it.  A block is `block_slots` consecutive slots.
// order (may be NULL) is the order in which the sender writes its blocks; the result does not depend on it.
void or_ll_pack(const uint16_t* x, int64_t n, int block_slots, uint32_t epoch, const int32_t* order,
                uint64_t* slots) {
    const int64_t nslots = n / 2, nblk = nslots / block_slots;
    for (int64_t j = 0; j < nblk; ++j) {
        const int64_t b = order ? order[j] : j;
        for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k)
            slots[k] = (uint64_t)x[2 * k] | ((uint64_t)x[2 * k + 1] << 16) | ((uint64_t)epoch << 32);
    }
}

// Receiver: for every block not yet done, rank r's copy is stale if any of its slots carries an epoch
// other than the expected one.  A block whose R copies are all valid is reduced (fp32 left fold in
// ascending rank order, one rounding to bf16) and marked done; otherwise its output is left untouched
// and it counts as pending.  reading: only complete blocks are reduced (a sum over a subset of ranks
// would not be an all-reduce, and would depend on arrival timing).
// counters[0] += number of stale (rank, block) pairs examined; counters[1] += pending blocks.
void or_ll_unpack_reduce(const uint64_t* const* slots, int R, int64_t n, int block_slots, uint32_t epoch,
                         uint16_t* out, uint8_t* stale, uint8_t* done, uint32_t* counters) {
    const int64_t nslots = n / 2, nblk = nslots / block_slots;
    for (int64_t b = 0; b < nblk; ++b) {
        if (done[b]) continue;
        bool all_valid = true;
        for (int r = 0; r < R; ++r) {
            bool st = false;
            for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k)
                if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;
            stale[(int64_t)r * nblk + b] = st ? 1 : 0;
            if (st) { all_valid = false; counters[0] += 1; }
        }
        if (!all_valid) { counters[1] += 1; continue; }
        for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k) {
            for (int e = 0; e < 2; ++e) {
                float acc = bf16_val((uint16_t)(slots[0][k] >> (16 * e)));
                for (int r = 1; r < R; ++r) acc = acc + bf16_val((uint16_t)(slots[r][k] >> (16 * e)));
                out[2 * k + e] = bf16_rne(acc);
            }
        }
        done[b] = 1;
    }
}

// ---- readiness by one flag word per block (flash-comm, abstract: the readiness evidence may also be a
// per-block word published after the block's data; the cost-guided choice among encodings trades its
// fence against the 8-byte slots' doubled bytes).  Rank r's payload is a dense bf16 [n] buffer; block b is
// elements [b*E, (b+1)*E); flags[r][b] is written after the block (release) and read before it (acquire).
// For every block not done: rank r's copy is stale iff flags[r][b] != epoch (its payload is then not read);
// a block whose R copies are all valid is reduced (fp32 left fold in ascending rank order, one rounding to
// bf16) and marked done, otherwise it is left untouched and pending.  counters as for the slots.
void or_flag_unpack_reduce(const uint16_t* const* payload, const uint32_t* const* flags, int R, int64_t n,
                           int block_elems, uint32_t epoch, uint16_t* out, uint8_t* stale, uint8_t* done,
                           uint32_t* counters) {
    const int64_t nblk = n / block_elems;
    for (int64_t b = 0; b < nblk; ++b) {
        if (done[b]) continue;
        bool all_valid = true;
        for (int r = 0; r < R; ++r) {
            const bool st = flags[r][b] != epoch;
            stale[(int64_t)r * nblk + b] = st ? 1 : 0;
            if (st) { all_valid = false; counters[0] += 1; }
        }
        if (!all_valid) { counters[1] += 1; continue; }
        for (int64_t i = b * block_elems; i < (b + 1) * block_elems; ++i) {
            float acc = bf16_val(payload[0][i]);
            for (int r = 1; r < R; ++r) acc = acc + bf16_val(payload[r][i]);
            out[i] = bf16_rne(acc);
        }
        done[b] = 1;
    }
}

// ---- standalone all-gather on self-synchronizing blocks (flash-comm, abstract: readiness evidence per
// block; the all-gather is the second workload of the mechanism).  Rank r's payload is nwords 32-bit words
// (bf16 pairs, or the words of a quantized message: codes then meta) carried in the low halves of its
// slots, epoch words in the high halves; a block is `block_slots` consecutive slots.  For every
// (rank, block) not yet done: the copy is stale if any slot carries an epoch other than the expected one;
// a valid block's words are copied to out[r] and it is marked done; a stale one is left untouched and
// pending.  counters[0] += stale (rank, block) pairs, counters[1] += pending (rank, block) pairs (here the
// same pairs: nothing is reduced across ranks, so every pair stands alone).
void or_ll_gather(const uint64_t* const* slots, int R, int64_t nwords, int block_slots, uint32_t epoch,
                  uint32_t* const* out, uint8_t* stale, uint8_t* done, uint32_t* counters) {
    const int64_t nblk = nwords / block_slots;
    for (int r = 0; r < R; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            const int64_t f = (int64_t)r * nblk + b;
            if (done[f]) continue;
            bool st = false;
            for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k)
                if ((uint32_t)(slots[r][k] >> 32) != epoch) st = true;
            stale[f] = st ? 1 : 0;
            if (st) {
                counters[0] += 1;
                counters[1] += 1;
                continue;
            }
            for (int64_t k = b * block_slots; k < (b + 1) * block_slots; ++k) out[r][k] = (uint32_t)slots[r][k];
            done[f] = 1;
        }
    }
}

}  // extern "C"
