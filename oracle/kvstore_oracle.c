/*
 * CPU oracle for the KV-cache store.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path loads this file or
 * the library built from it: only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or helper
 * with the HIP library; the two meet only in the seeded inputs they are fed.
 *
 * Plain, slow, single-threaded C.  Build: gcc -O2 -ffp-contract=off -shared
 * -fPIC kvstore_oracle.c -lm.  No vectorisation tricks, no blocking, no
 * fusion: one token at a time, one element at a time, in the order the pages
 * describe.
 *
 * What it follows:
 *   - Scatter copy: sglang "kvcache.cuh", section store_kvcache / copy_kv_warp:
 *     token t's K and V rows are copied byte for byte to cache row indices[t];
 *     the index must satisfy 0 <= index < size_limit (the page asserts it on
 *     the device).  Here a bad index is counted and its row skipped.
 *   - Fused FP8 paged store: sglang "trtllm_fp8_kv_kernel.py", kernel
 *     _fused_fp8_set_kv_buffer_kernel and helper _process_kv_tensor:
 *     page = loc / page_size, offset = loc % page_size; each element is
 *     loaded, multiplied in fp32 by the tensor's inverse scale (1.0 when no
 *     scale is given) and cast to float8 e4m3; the byte lands at
 *     page*s_page + offset*s_offset + head*s_head + dim.
 *   - The e4m3fn encoding is written from the format definition named on that
 *     page (torch.float8_e4m3fn): 1 sign bit, 4 exponent bits with bias 7,
 *     3 mantissa bits, no infinities, NaN = S.1111.111, largest finite 448.
 *     The cast's rounding and overflow are not stated on the pages; the reading
 *     taken is round-to-nearest-even with saturation to +-448 (a NaN stays a
 *     NaN and keeps its sign).
 *
 *   - e5m2 caches: the page's unfused path stores into float8_e5m2 as well as
 *     float8_e4m3fn caches (its uint8-view condition names both).  The e5m2
 *     encoding is written from its definition: 1 sign bit, 5 exponent bits
 *     with bias 15, 2 mantissa bits, exponent 31 = infinity (mantissa 0) or
 *     NaN, largest finite 57344.  Same reading as for e4m3fn: round to nearest
 *     even, saturate to +-57344 (infinities too), NaN -> 0x7F | sign.
 *   - Dynamic scales (the docstring of "trtllm_fp8_kv_kernel.py" lists
 *     per-token scale computation among the fused kernel's steps; its code
 *     only takes a given per-tensor scale).  Reading taken: per group (a
 *     token's whole K or V row, or one head of it), amax = max |x| with NaN
 *     ignored, scale = max(amax / 448, 2^-126) in fp32 (the floor, the
 *     smallest normal float, keeps 1 / scale finite for all-zero and tiny
 *     groups), and inv = 1 / scale in fp32 as the page's wrapper inverts a
 *     scale; each element becomes e4m3fn(x * inv) and the fp32 scale is
 *     stored beside the slot.
 *
 * Parity pins (all in tests/, CPU only): exhaustive nearest-value search over
 * the decoded e4m3fn table for every bf16 and fp16 pattern, torch's own
 * float8_e4m3fn cast where it does not overflow, hand-derived closed-form
 * values, and store invariants (sentinel, round trip, paged == flat, OOB
 * skip, permutation invariance, brute force on tiny inputs).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Input element decoding.                                                  */
/* ---------------------------------------------------------------------- */

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
static float bf16_to_float(uint16_t b) {
    uint32_t w = (uint32_t)b << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}

/* IEEE binary16: 1 sign, 5 exponent bits (bias 15), 10 fraction bits. */
static float fp16_to_float(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double mag;
    if (e == 0) {
        mag = ldexp((double)m, -24);             /* subnormal: m * 2^-24 */
    } else if (e == 31) {
        if (m != 0) {
            /* NaN: keep the sign, keep it quiet */
            uint32_t w = ((uint32_t)sign << 31) | 0x7FC00000u | ((uint32_t)m << 13);
            float f;
            memcpy(&f, &w, sizeof f);
            return f;
        }
        mag = INFINITY;
    } else {
        mag = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return (float)(sign ? -mag : mag);           /* exact: fits in binary32 */
}

static float src_to_float(uint16_t bits, int src_is_fp16) {
    return src_is_fp16 ? fp16_to_float(bits) : bf16_to_float(bits);
}

/* ---------------------------------------------------------------------- */
/* fp32 multiply by the inverse scale.                                      */
/* ---------------------------------------------------------------------- */

/*
 * y = x * inv rounded once to binary32.  Both operands are binary32, so their
 * exact product has at most 48 significant bits and is exact in binary64;
 * converting it to float is then the single round-to-nearest of an fp32
 * multiply, independent of FMA contraction or x87 excess precision.
 * A NaN operand propagates itself (keeping its sign; the input before the
 * scale).  A NaN made from two non-NaN operands (inf * 0) is the negative
 * default NaN 0xFFC00000: IEEE 754 leaves its sign open, and an fp32 multiply
 * in torch on the CPU (the arithmetic of the page's unfused path) returns
 * that pattern.
 */
static float mul_f32(float x, float inv) {
    if (isnan(x)) return x;
    if (isnan(inv)) return inv;
    double p = (double)x * (double)inv;
    if (isnan(p)) return -NAN;
    return (float)p;
}

/* ---------------------------------------------------------------------- */
/* float -> e4m3fn, round to nearest even, saturate to +-448.               */
/* ---------------------------------------------------------------------- */

/* Round-half-to-even of a non-negative double whose fractional part is exact. */
static double round_half_even(double q) {
    double fl = floor(q);
    double frac = q - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint8_t oracle_e4m3fn_from_float(float y) {
    uint8_t s = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(0x7F | s);
    double a = fabs((double)y);
    if (a > 448.0) return (uint8_t)(0x7E | s);   /* includes +-inf */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9, m in 0..7; m == 8 is the
           smallest normal 2^-6, whose code 0x08 continues the sequence. */
        double m = round_half_even(a * 512.0);   /* exact scaling by 2^9 */
        return (uint8_t)((uint8_t)m | s);
    }
    int ex;
    frexp(a, &ex);                               /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                              /* floor(log2 a), >= -6 */
    double m = round_half_even(ldexp(a, 3 - e)); /* a / 2^(e-3), in [8, 16] */
    if (m == 16.0) {                             /* rounding carried into the exponent */
        e += 1;
        m = 8.0;
    }
    return (uint8_t)((((e + 7) << 3) | ((int)m - 8)) | s);
}

uint8_t oracle_e5m2_from_float(float y) {
    uint8_t s = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(0x7F | s);
    double a = fabs((double)y);
    if (a > 57344.0) return (uint8_t)(0x7B | s); /* includes +-inf */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-16, m in 0..3; m == 4 is the
           smallest normal 2^-14, whose code 0x04 continues the sequence. */
        double m = round_half_even(a * 65536.0); /* exact scaling by 2^16 */
        return (uint8_t)((uint8_t)m | s);
    }
    int ex;
    frexp(a, &ex);                               /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                              /* floor(log2 a), >= -14 */
    double m = round_half_even(ldexp(a, 2 - e)); /* a / 2^(e-2), in [4, 8] */
    if (m == 8.0) {                              /* rounding carried into the exponent */
        e += 1;
        m = 4.0;
    }
    return (uint8_t)((((e + 15) << 2) | ((int)m - 4)) | s);
}

/* FP8 storage formats of the fused stores. */
enum { FMT_E4M3FN = 0, FMT_E5M2 = 1 };

/* One element of the fused store: decode, scale, encode. */
static uint8_t quantize_fmt(uint16_t bits, int src_is_fp16, float inv, int fmt) {
    float x = src_to_float(bits, src_is_fp16);
    float y = mul_f32(x, inv);
    return fmt == FMT_E5M2 ? oracle_e5m2_from_float(y) : oracle_e4m3fn_from_float(y);
}

static uint8_t quantize_one(uint16_t bits, int src_is_fp16, float inv) {
    return quantize_fmt(bits, src_is_fp16, inv, FMT_E4M3FN);
}

/* ---------------------------------------------------------------------- */
/* Exported element helpers (for pins).                                    */
/* ---------------------------------------------------------------------- */

float oracle_src_to_float(uint16_t bits, int src_is_fp16) {
    return src_to_float(bits, src_is_fp16);
}

float oracle_mul_f32(float x, float inv) { return mul_f32(x, inv); }

/* out[i] = e4m3fn(src[i] * inv); inv == NULL means 1.0. */
void oracle_quantize(const uint16_t* src, int64_t n, int src_is_fp16, const float* inv,
                     uint8_t* out) {
    float s = inv ? *inv : 1.0f;
    for (int64_t i = 0; i < n; ++i) out[i] = quantize_one(src[i], src_is_fp16, s);
}

void oracle_e4m3fn_array(const float* y, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3fn_from_float(y[i]);
}

void oracle_e5m2_array(const float* y, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e5m2_from_float(y[i]);
}

/* out[i] = e5m2(src[i] * inv); inv == NULL means 1.0. */
void oracle_quantize_e5m2(const uint16_t* src, int64_t n, int src_is_fp16, const float* inv,
                          uint8_t* out) {
    float s = inv ? *inv : 1.0f;
    for (int64_t i = 0; i < n; ++i) out[i] = quantize_fmt(src[i], src_is_fp16, s, FMT_E5M2);
}

/* ---------------------------------------------------------------------- */
/* Stores.                                                                  */
/* ---------------------------------------------------------------------- */

static int64_t read_index(const void* indices, int idx_is_i64, int64_t pos) {
    if (idx_is_i64) return ((const int64_t*)indices)[pos];
    return (int64_t)((const int32_t*)indices)[pos];
}

/* Records a rejected token: count it, keep the smallest token id. */
static void note_bad(int64_t t, int64_t* first_bad, uint64_t* bad_count) {
    *bad_count += 1;
    if (*first_bad < 0 || t < *first_bad) *first_bad = t;
}

/*
 * Scatter copy.  All strides are in bytes except idx_stride (elements).
 * first_bad is set to -1 and bad_count to 0 on entry.  Returns the number of
 * rows written.
 */
int64_t oracle_copy(const uint8_t* k, const uint8_t* v, uint8_t* k_cache, uint8_t* v_cache,
                    const void* indices, int idx_is_i64, int64_t idx_stride,
                    int64_t row_bytes, int64_t k_stride, int64_t v_stride,
                    int64_t cache_stride, int64_t batch, int64_t size_limit,
                    int64_t* first_bad, uint64_t* bad_count) {
    int64_t written = 0;
    *first_bad = -1;
    *bad_count = 0;
    for (int64_t t = 0; t < batch; ++t) {
        int64_t loc = read_index(indices, idx_is_i64, t * idx_stride);
        if (loc < 0 || loc >= size_limit) {
            note_bad(t, first_bad, bad_count);
            continue;
        }
        memcpy(k_cache + loc * cache_stride, k + t * k_stride, (size_t)row_bytes);
        memcpy(v_cache + loc * cache_stride, v + t * v_stride, (size_t)row_bytes);
        ++written;
    }
    return written;
}

/* One tensor (K or V) of one token into its paged cache slot. */
static void store_fp8_row(const uint8_t* src, int64_t s_tok, int64_t s_head, int64_t t,
                          uint8_t* cache, int64_t s_page, int64_t s_off, int64_t s_chead,
                          int64_t page, int64_t off, int64_t num_heads, int64_t head_dim,
                          int src_is_fp16, float inv, int fmt) {
    for (int64_t h = 0; h < num_heads; ++h) {
        for (int64_t d = 0; d < head_dim; ++d) {
            uint16_t bits;
            memcpy(&bits, src + t * s_tok + h * s_head + 2 * d, sizeof bits);
            cache[page * s_page + off * s_off + h * s_chead + d] =
                quantize_fmt(bits, src_is_fp16, inv, fmt);
        }
    }
}

/*
 * Fused FP8 paged store.  Input strides in bytes (dim stride is one element),
 * cache strides in bytes (dim stride is one byte).  inv_k / inv_v are host
 * pointers to fp32 inverse scales, NULL meaning 1.0.  Returns rows written.
 */
static int64_t fp8_paged_fmt(const uint8_t* k, const uint8_t* v, uint8_t* k_cache,
                             uint8_t* v_cache, const void* indices, int idx_is_i64,
                             int64_t idx_stride, int src_is_fp16, int64_t num_heads,
                             int64_t head_dim, int64_t k_stride_token, int64_t k_stride_head,
                             int64_t v_stride_token, int64_t v_stride_head,
                             int64_t kc_stride_page, int64_t kc_stride_offset,
                             int64_t kc_stride_head, int64_t vc_stride_page,
                             int64_t vc_stride_offset, int64_t vc_stride_head, int64_t batch,
                             int64_t size_limit, int64_t page_size, const float* inv_k,
                             const float* inv_v, int fmt, int64_t* first_bad,
                             uint64_t* bad_count) {
    int64_t written = 0;
    float ik = inv_k ? *inv_k : 1.0f;
    float iv = inv_v ? *inv_v : 1.0f;
    *first_bad = -1;
    *bad_count = 0;
    for (int64_t t = 0; t < batch; ++t) {
        int64_t loc = read_index(indices, idx_is_i64, t * idx_stride);
        if (loc < 0 || loc >= size_limit) {
            note_bad(t, first_bad, bad_count);
            continue;
        }
        int64_t page = loc / page_size;
        int64_t off = loc % page_size;
        store_fp8_row(k, k_stride_token, k_stride_head, t, k_cache, kc_stride_page,
                      kc_stride_offset, kc_stride_head, page, off, num_heads, head_dim,
                      src_is_fp16, ik, fmt);
        store_fp8_row(v, v_stride_token, v_stride_head, t, v_cache, vc_stride_page,
                      vc_stride_offset, vc_stride_head, page, off, num_heads, head_dim,
                      src_is_fp16, iv, fmt);
        ++written;
    }
    return written;
}

/* e4m3fn caches (the fused kernel's format). */
int64_t oracle_fp8_paged(const uint8_t* k, const uint8_t* v, uint8_t* k_cache,
                         uint8_t* v_cache, const void* indices, int idx_is_i64,
                         int64_t idx_stride, int src_is_fp16, int64_t num_heads,
                         int64_t head_dim, int64_t k_stride_token, int64_t k_stride_head,
                         int64_t v_stride_token, int64_t v_stride_head,
                         int64_t kc_stride_page, int64_t kc_stride_offset,
                         int64_t kc_stride_head, int64_t vc_stride_page,
                         int64_t vc_stride_offset, int64_t vc_stride_head, int64_t batch,
                         int64_t size_limit, int64_t page_size, const float* inv_k,
                         const float* inv_v, int64_t* first_bad, uint64_t* bad_count) {
    return fp8_paged_fmt(k, v, k_cache, v_cache, indices, idx_is_i64, idx_stride, src_is_fp16,
                         num_heads, head_dim, k_stride_token, k_stride_head, v_stride_token,
                         v_stride_head, kc_stride_page, kc_stride_offset, kc_stride_head,
                         vc_stride_page, vc_stride_offset, vc_stride_head, batch, size_limit,
                         page_size, inv_k, inv_v, FMT_E4M3FN, first_bad, bad_count);
}

/* e5m2 caches, same arguments. */
int64_t oracle_fp8_paged_e5m2(const uint8_t* k, const uint8_t* v, uint8_t* k_cache,
                              uint8_t* v_cache, const void* indices, int idx_is_i64,
                              int64_t idx_stride, int src_is_fp16, int64_t num_heads,
                              int64_t head_dim, int64_t k_stride_token, int64_t k_stride_head,
                              int64_t v_stride_token, int64_t v_stride_head,
                              int64_t kc_stride_page, int64_t kc_stride_offset,
                              int64_t kc_stride_head, int64_t vc_stride_page,
                              int64_t vc_stride_offset, int64_t vc_stride_head, int64_t batch,
                              int64_t size_limit, int64_t page_size, const float* inv_k,
                              const float* inv_v, int64_t* first_bad, uint64_t* bad_count) {
    return fp8_paged_fmt(k, v, k_cache, v_cache, indices, idx_is_i64, idx_stride, src_is_fp16,
                         num_heads, head_dim, k_stride_token, k_stride_head, v_stride_token,
                         v_stride_head, kc_stride_page, kc_stride_offset, kc_stride_head,
                         vc_stride_page, vc_stride_offset, vc_stride_head, batch, size_limit,
                         page_size, inv_k, inv_v, FMT_E5M2, first_bad, bad_count);
}

/* ---------------------------------------------------------------------- */
/* Fused FP8 paged store with dynamic per-token / per-token-head scales.    */
/* ---------------------------------------------------------------------- */

/* Scale of one group: amax / 448 in fp32, at least the smallest normal float. */
static float group_scale(float amax) {
    float scale = amax / 448.0f;
    if (scale < FLT_MIN) scale = FLT_MIN;
    return scale;
}

/* max |x| over heads [h0, h1) of one token row, NaN ignored. */
static float group_amax(const uint8_t* src, int64_t s_tok, int64_t s_head, int64_t t, int64_t h0,
                        int64_t h1, int64_t head_dim, int src_is_fp16) {
    float amax = 0.0f;
    for (int64_t h = h0; h < h1; ++h) {
        for (int64_t d = 0; d < head_dim; ++d) {
            uint16_t bits;
            memcpy(&bits, src + t * s_tok + h * s_head + 2 * d, sizeof bits);
            float a = fabsf(src_to_float(bits, src_is_fp16));
            if (a > amax) amax = a;                 /* false for NaN: ignored */
        }
    }
    return amax;
}

/*
 * As oracle_fp8_paged, without given scales: for each valid token and each of
 * K and V, the groups are the whole row (per_head = 0) or each head
 * (per_head = 1).  The fp32 scale of group g lands at byte offset
 * page * s_page + offset * s_offset + g * s_head of k_scales / v_scales.
 */
int64_t oracle_fp8_paged_dynamic(const uint8_t* k, const uint8_t* v, uint8_t* k_cache,
                                 uint8_t* v_cache, const void* indices, int idx_is_i64,
                                 int64_t idx_stride, int src_is_fp16, int64_t num_heads,
                                 int64_t head_dim, int64_t k_stride_token, int64_t k_stride_head,
                                 int64_t v_stride_token, int64_t v_stride_head,
                                 int64_t kc_stride_page, int64_t kc_stride_offset,
                                 int64_t kc_stride_head, int64_t vc_stride_page,
                                 int64_t vc_stride_offset, int64_t vc_stride_head,
                                 uint8_t* k_scales, uint8_t* v_scales, int64_t ks_stride_page,
                                 int64_t ks_stride_offset, int64_t ks_stride_head,
                                 int64_t vs_stride_page, int64_t vs_stride_offset,
                                 int64_t vs_stride_head, int per_head, int64_t batch,
                                 int64_t size_limit, int64_t page_size, int64_t* first_bad,
                                 uint64_t* bad_count) {
    int64_t written = 0;
    int64_t groups = per_head ? num_heads : 1;
    int64_t heads_per_group = per_head ? 1 : num_heads;
    *first_bad = -1;
    *bad_count = 0;
    for (int64_t t = 0; t < batch; ++t) {
        int64_t loc = read_index(indices, idx_is_i64, t * idx_stride);
        if (loc < 0 || loc >= size_limit) {
            note_bad(t, first_bad, bad_count);
            continue;
        }
        int64_t page = loc / page_size;
        int64_t off = loc % page_size;
        for (int x = 0; x < 2; ++x) {
            const uint8_t* src = x ? v : k;
            int64_t s_tok = x ? v_stride_token : k_stride_token;
            int64_t s_head = x ? v_stride_head : k_stride_head;
            uint8_t* cache = x ? v_cache : k_cache;
            int64_t c_page = x ? vc_stride_page : kc_stride_page;
            int64_t c_off = x ? vc_stride_offset : kc_stride_offset;
            int64_t c_head = x ? vc_stride_head : kc_stride_head;
            uint8_t* scales = x ? v_scales : k_scales;
            int64_t sc_page = x ? vs_stride_page : ks_stride_page;
            int64_t sc_off = x ? vs_stride_offset : ks_stride_offset;
            int64_t sc_head = x ? vs_stride_head : ks_stride_head;
            for (int64_t g = 0; g < groups; ++g) {
                int64_t h0 = g * heads_per_group, h1 = h0 + heads_per_group;
                float amax = group_amax(src, s_tok, s_head, t, h0, h1, head_dim, src_is_fp16);
                float scale = group_scale(amax);
                float inv = 1.0f / scale;
                memcpy(scales + page * sc_page + off * sc_off + g * sc_head, &scale, sizeof scale);
                for (int64_t h = h0; h < h1; ++h) {
                    for (int64_t d = 0; d < head_dim; ++d) {
                        uint16_t bits;
                        memcpy(&bits, src + t * s_tok + h * s_head + 2 * d, sizeof bits);
                        cache[page * c_page + off * c_off + h * c_head + d] =
                            quantize_one(bits, src_is_fp16, inv);
                    }
                }
            }
        }
        ++written;
    }
    return written;
}

