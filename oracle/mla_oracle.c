/*
 * CPU oracle for the fused MLA decode epilogue.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke entry point and the benchmark's CPU-baseline
 * leg may load or call this code.  The product path never does; it shares no
 * code, header, table or constant with the GPU library.
 *
 * What is computed (prhub summary of vLLM PR #54896, "Kimi-K3 MLA decode
 * kernel", sections "implementation breakdown" items 1-4 and "key source
 * snippets"): for every token t and every head h the 576-wide latent query
 * row is the 512-wide no-position part followed by the (optionally rotated)
 * 64-wide positional part; in the same call the token's latent cache row,
 * kv_c followed by the (optionally rotated) k_pe, is written into a paged cache
 * at the token's slot.  Either output may be stored as OCP FP8 E4M3 under a
 * per-tensor scale.  The page's own test fixes the plain case: with rotation
 * and FP8 off, q equals cat(ql_nope, q_pe) and the cache rows at the slots
 * equal cat(kv_c, k_pe); the cache starts as zeros and every other byte stays.
 *
 * Readings where the page is silent:
 *  - rotation is the NeoX half-split form (element i pairs with element
 *    i+32) unless the interleaved GPT-J pairing (2i with 2i+1) is asked for;
 *    the rope table row for position p holds cos[0:32] then sin[0:32]
 *    (fp32, or bf16 when asked for);
 *  - activations are bf16 (the page's configuration) or fp16 (the page's
 *    kernel is templated on the element type); unquantised outputs keep the
 *    activation type;
 *  - the rotation is evaluated in fp32 as two rounded products and one rounded
 *    add/sub (no fused multiply-add), because its result decides bf16 and E4M3
 *    codes and both sides must take that decision in the same precision;
 *  - FP8 storage is x * (1/scale): inv = fl32(1/scale), v = fl32(x * inv),
 *    clamped to [-448, 448], then rounded to nearest-even E4M3 (OCP OFP8
 *    definition: bias 7, subnormal step 2^-9, max 448, NaN = S.1111.111);
 *  - positions outside [0, max_position) are clamped into the table;
 *  - slots outside [0, num_slots) leave the cache untouched (padding tokens);
 *  - with duplicate slots the later token's row is the one left in the cache;
 *  - for the epilogue fused into the absorbed key projection ahead of it,
 *    ql_nope is that product's exact value (a double sum of exact products,
 *    W_UK handed over transposed as [H, 512, 128]), encoded once: the fused
 *    path never rounds ql_nope to the activation type before encoding.
 *
 * Every function here is pinned by tests against format definitions, closed
 * forms, library routines and brute force (see tests/test_oracle_pins.py).
 */
/* Every fp32 operation below must round on its own: the library is built
 * with -ffp-contract=off and without fast-math. */
#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif

#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ROW 576
#define NOPE 512
#define PE 64
#define HALF 32

/* Round-half-even of a non-negative value that is exact in double. */
static double round_half_even(double q) {
    double f = floor(q);
    double r = q - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* ---- bf16 <-> fp32 (bf16 is the top half of an IEEE binary32) ---------- */

float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round an fp32 value to bf16, nearest with ties to even.  The 16 dropped
 * bits are compared with one half of the last kept bit; a carry out of the
 * mantissa correctly moves into the exponent (and to infinity past the top).
 * A NaN stays a NaN: the quiet bit is set so truncation cannot make it Inf. */
uint16_t oracle_f32_to_bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16, lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

/* ---- IEEE 754 binary16 (fp16): 1 sign, 5 exponent (bias 15), 10 mantissa */

/* Exact value of an fp16 bit pattern, from the format definition. */
float oracle_fp16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);                  /* subnormal: m * 2^-24 */
    else
        v = ldexp(1.0 + m / 1024.0, e - 15);
    return (float)(sign ? -v : v);
}

/* Round an fp32 value to fp16, nearest with ties to even.  Magnitudes from
 * 65520 (halfway between 65504 and 2^16) upward become infinity; the
 * subnormal step is 2^-24; NaN stays a (quiet) NaN. */
uint16_t oracle_f32_to_fp16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)x);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: m * 2^-24, m in 0..1024 (1024 is the smallest
         * normal 2^-14, whose code 0x0400 is exponent 1 mantissa 0) */
        double m = round_half_even(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e2;
    double f = frexp(a, &e2);
    int ue = e2 - 1;
    double m = round_half_even((2.0 * f - 1.0) * 1024.0);
    if (m == 1024.0) { m = 0.0; ue += 1; }
    return (uint16_t)(sign | (uint16_t)((ue + 15) << 10) | (uint16_t)m);
}

/* ---- OCP FP8 E4M3 (OFP8 "E4M3FN": no infinities, one NaN per sign) ----- */

/* Encode an fp32 value as E4M3: NaN -> S.1111.111, |v| >= 448 (incl. Inf)
 * saturates to S.1111.110 = 448, otherwise the nearest representable value,
 * ties to the even code.  Subnormals (exponent field 0) step by 2^-9. */
uint8_t oracle_f32_to_e4m3(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9, m in 0..8 (m = 8 is 2^-6, the
         * smallest normal, whose code 0x08 is also exponent 1 mantissa 0) */
        double m = round_half_even(a * 512.0);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e2;
    double f = frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1) */
    int ue = e2 - 1;               /* a = (2f) * 2^ue, 2f in [1, 2) */
    double mant = 2.0 * f;
    double m = round_half_even((mant - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; ue += 1; }
    int be = ue + 7;               /* biased exponent, 1..15 */
    int code = (be << 3) | (int)m;
    if (code > 0x7E) code = 0x7E;  /* cannot happen below 448; kept defensive */
    return (uint8_t)(sign | code);
}

/* Quantise under a per-tensor scale: x * fl32(1/scale), clamped to +-448
 * with NaN kept, then E4M3.  inv is passed in already rounded to fp32. */
uint8_t oracle_quant_e4m3(float x, float inv) {
    float c = x * inv;             /* one fp32 rounding */
    if (!isnan(c)) {
        if (c > 448.0f) c = 448.0f;
        if (c < -448.0f) c = -448.0f;
    }
    return oracle_f32_to_e4m3(c);
}

/* ---- rotation of one 64-wide positional tail ----------------------------- */

/* Pair p (p = 0..31) of the tail rotates by the angle of table column p:
 * NeoX pairs element p with element p+32, GPT-J ("interleaved") pairs element
 * 2p with element 2p+1.  With a the first and b the second element of the
 * pair, c = cos and s = sin of the angle:
 *     first  = a*c - b*s,    second = b*c + a*s,
 * each product and the sum rounded to fp32 separately. */
static void pair_index(int p, int gptj, int* i0, int* i1) {
    if (gptj) { *i0 = 2 * p; *i1 = 2 * p + 1; }
    else      { *i0 = p;     *i1 = p + HALF; }
}

void oracle_rope_f32(const float* x, const float* cos_row, const float* sin_row, int gptj,
                     float* y) {
    for (int p = 0; p < HALF; ++p) {
        int i0, i1;
        pair_index(p, gptj, &i0, &i1);
        float a = x[i0], b = x[i1], c = cos_row[p], s = sin_row[p];
        float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        y[i0] = ac - bs;
        y[i1] = bc + as;
    }
}

/* Same rotation in float64, used only to bound the fp32 one in tests. */
void oracle_rope_f64(const float* x, const float* cos_row, const float* sin_row, int gptj,
                     double* y) {
    for (int p = 0; p < HALF; ++p) {
        int i0, i1;
        pair_index(p, gptj, &i0, &i1);
        double a = x[i0], b = x[i1], c = cos_row[p], s = sin_row[p];
        y[i0] = a * c - b * s;
        y[i1] = b * c + a * s;
    }
}

/* NeoX rotation of a bf16 tail by an fp32 table row (cos[0:32] | sin[0:32]). */
void oracle_rope_neox_f32(const uint16_t* x, const float* cs, float* y) {
    float xf[PE];
    for (int i = 0; i < PE; ++i) xf[i] = oracle_bf16_to_f32(x[i]);
    oracle_rope_f32(xf, cs, cs + HALF, 0, y);
}

void oracle_rope_neox_f64(const uint16_t* x, const float* cs, double* y) {
    float xf[PE];
    for (int i = 0; i < PE; ++i) xf[i] = oracle_bf16_to_f32(x[i]);
    oracle_rope_f64(xf, cs, cs + HALF, 0, y);
}

/* ---- one 576-wide output row -------------------------------------------- */

/* Element type of the activations and of unquantised outputs. */
static float elem_to_f32(uint16_t v, int fp16) {
    return fp16 ? oracle_fp16_to_f32(v) : oracle_bf16_to_f32(v);
}

/* The absorbed key projection whose output the epilogue reads (the page's
 * kernel waits for that product before it touches ql_nope, "implementation
 * breakdown" item 2).  With W_UK given transposed, w_uk_t[h, n, k] =
 * W_UK[h, k, n]:
 *   ql[t, h, n] = sum over k < 128 of q_nope[t, h, k] * w_uk_t[h, n, k],  n < 512
 *   mag[t, h, n] = sum over k < 128 of |q_nope[t, h, k] * w_uk_t[h, n, k]|
 * Inputs are activation bit patterns (bf16, or fp16 when asked for),
 * contiguous: [T, H, 128] and [H, 512, 128].  Each product of two such values
 * is exact in double and the sums are formed in double in increasing k, so
 * ql is the exact value up to double rounding; mag (may be NULL) bounds how
 * far any fp32 evaluation of the sum can stray from it. */
void oracle_uk_product(double* ql, double* mag, const uint16_t* q_nope, const uint16_t* w_uk_t,
                       int64_t T, int64_t H, int fp16) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            const uint16_t* q = q_nope + ((size_t)t * H + h) * 128;
            for (int64_t n = 0; n < NOPE; ++n) {
                const uint16_t* w = w_uk_t + ((size_t)h * NOPE + n) * 128;
                double acc = 0.0, acc_abs = 0.0;
                for (int k = 0; k < 128; ++k) {
                    const double prod = (double)elem_to_f32(q[k], fp16) * (double)elem_to_f32(w[k], fp16);
                    acc += prod;
                    acc_abs += fabs(prod);
                }
                const size_t o = ((size_t)t * H + h) * NOPE + n;
                ql[o] = acc;
                if (mag) mag[o] = acc_abs;
            }
        }
}


static uint16_t f32_to_elem(float x, int fp16) {
    return fp16 ? oracle_f32_to_fp16_rne(x) : oracle_f32_to_bf16_rne(x);
}

/* Writes one latent row from its 512-wide and 64-wide parts (bit patterns of
 * bf16 or fp16) into dst, either in the activation type (2 bytes per
 * element) or as E4M3 (1 byte per element).  table_row points at the
 * token's rope table row (fp32, or bf16 bit patterns). */
static void write_row(uint8_t* dst, const uint16_t* nope, const uint16_t* pe, int rope, int gptj,
                      const void* table_row, int table_bf16, int fp16, int fp8, float inv) {
    float y[PE];
    if (rope) {
        float x[PE], c[HALF], s[HALF];
        for (int i = 0; i < PE; ++i) x[i] = elem_to_f32(pe[i], fp16);
        for (int p = 0; p < HALF; ++p) {
            if (table_bf16) {
                const uint16_t* t = (const uint16_t*)table_row;
                c[p] = oracle_bf16_to_f32(t[p]);
                s[p] = oracle_bf16_to_f32(t[HALF + p]);
            } else {
                const float* t = (const float*)table_row;
                c[p] = t[p];
                s[p] = t[HALF + p];
            }
        }
        oracle_rope_f32(x, c, s, gptj, y);
    }
    if (fp8) {
        for (int i = 0; i < NOPE; ++i)
            dst[i] = oracle_quant_e4m3(elem_to_f32(nope[i], fp16), inv);
        for (int i = 0; i < PE; ++i) {
            float v = rope ? y[i] : elem_to_f32(pe[i], fp16);
            dst[NOPE + i] = oracle_quant_e4m3(v, inv);
        }
    } else {
        uint16_t* d16 = (uint16_t*)dst;
        for (int i = 0; i < NOPE; ++i) d16[i] = nope[i];  /* bit copy */
        for (int i = 0; i < PE; ++i)
            d16[NOPE + i] = rope ? f32_to_elem(y[i], fp16) : pe[i];
    }
}

static int64_t clamp_pos(int64_t p, int64_t max_position) {
    if (p < 0) return 0;
    if (p >= max_position) return max_position - 1;
    return p;
}

/* The whole epilogue on host arrays, all contiguous:
 *   q_out   [T, H, 576]  activation type (q_fp8 = 0) or E4M3 bytes (q_fp8 = 1)
 *   ql_nope [T, H, 512], q_pe [T, H, 64], kv_c [T, 512], k_pe [T, 64]:
 *           bf16, or fp16 when fp16 = 1 (bit patterns)
 *   cache   [num_slots, 576]  activation type or E4M3 bytes (kv_fp8), in place
 *   slots   [T] int64, positions [T] int64 (read only when rope)
 *   table   [max_position, 64] rope table, fp32 or bf16 (table_bf16), read
 *           only when rope; gptj selects the interleaved pairing
 *   q_scale, kv_scale: per-tensor scales (read only for an FP8 output)
 * Returns 0, or -1 on a shape that cannot be evaluated. */
int oracle_mla_decode_ex(uint8_t* q_out, const uint16_t* ql_nope, const uint16_t* q_pe,
                         const uint16_t* kv_c, const uint16_t* k_pe, uint8_t* cache,
                         const int64_t* slots, const int64_t* positions, const void* table,
                         float q_scale, float kv_scale, int64_t T, int64_t H, int64_t num_slots,
                         int64_t max_position, int rope, int q_fp8, int kv_fp8, int fp16, int gptj,
                         int table_bf16) {
    if (T < 0 || H < 1 || num_slots < 0) return -1;
    if (rope && max_position < 1) return -1;
    float qi = q_fp8 ? 1.0f / q_scale : 1.0f;   /* correctly rounded fp32 */
    float ki = kv_fp8 ? 1.0f / kv_scale : 1.0f;
    size_t q_row_bytes = (size_t)ROW * (q_fp8 ? 1 : 2);
    size_t kv_row_bytes = (size_t)ROW * (kv_fp8 ? 1 : 2);
    size_t table_row_bytes = (size_t)PE * (table_bf16 ? 2 : 4);

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const void* trow = rope ? (const uint8_t*)table +
                                      (size_t)clamp_pos(positions[t], max_position) * table_row_bytes
                                : 0;
        for (int64_t h = 0; h < H; ++h) {
            int64_t r = t * H + h;
            write_row(q_out + (size_t)r * q_row_bytes, ql_nope + (size_t)r * NOPE,
                      q_pe + (size_t)r * PE, rope, gptj, trow, table_bf16, fp16, q_fp8, qi);
        }
    }
    /* The scatter runs in token order so that a repeated slot keeps the
     * later token's row. */
    for (int64_t t = 0; t < T; ++t) {
        int64_t s = slots[t];
        if (s < 0 || s >= num_slots) continue;
        const void* trow = rope ? (const uint8_t*)table +
                                      (size_t)clamp_pos(positions[t], max_position) * table_row_bytes
                                : 0;
        write_row(cache + (size_t)s * kv_row_bytes, kv_c + (size_t)t * NOPE,
                  k_pe + (size_t)t * PE, rope, gptj, trow, table_bf16, fp16, kv_fp8, ki);
    }
    return 0;
}

/* The page's configuration: bf16 activations, NeoX rotation, fp32 table. */
int oracle_mla_decode_q_concat_kv_insert(
    uint8_t* q_out, const uint16_t* ql_nope, const uint16_t* q_pe,
    const uint16_t* kv_c, const uint16_t* k_pe, uint8_t* cache,
    const int64_t* slots, const int64_t* positions, const float* cs,
    float q_scale, float kv_scale, int64_t T, int64_t H, int64_t num_slots,
    int64_t max_position, int rope, int q_fp8, int kv_fp8) {
    return oracle_mla_decode_ex(q_out, ql_nope, q_pe, kv_c, k_pe, cache, slots, positions, cs,
                                q_scale, kv_scale, T, H, num_slots, max_position, rope, q_fp8,
                                kv_fp8, 0, 0, 0);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- array forms of the encoders (for exhaustive pins) ------------------ */

void oracle_f32_to_e4m3_n(const float* x, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(x[i]);
}

void oracle_quant_e4m3_n(const float* x, float inv, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_quant_e4m3(x[i], inv);
}

void oracle_f32_to_bf16_n(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16_rne(x[i]);
}

void oracle_f32_to_fp16_n(const float* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_fp16_rne(x[i]);
}

void oracle_fp16_to_f32_n(const uint16_t* x, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp16_to_f32(x[i]);
}

/* Thread count of the OpenMP loop (timing only; results do not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
