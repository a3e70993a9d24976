/*
 * CPU oracle for the quantized routed-expert MoE feed-forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the package smoke check
 * and the CPU-baseline leg of the benchmark may load it; the GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What it computes (sources are the minnow README, sections "Quantization" and
 * "Build and run", and the LLaDA2.2-flash-minnow model card, section
 * "Checkpoints and precision" and its precision table):
 *
 *  - routed-expert weights are signed INT4 or INT8 with one FP16 scale per 128
 *    weights; the 128 weights of a group are contiguous along the input
 *    (reduction) dimension of each projection (model card precision table,
 *    INT8 and INT4 rows);
 *  - default mode (W4A16 / W8A16): the expert matmuls take BF16 inputs and
 *    dequantized weights, accumulating in floating point (README
 *    "Quantization"; model card, paragraph after the table);
 *  - INT8-activation mode (W4A8 / W8A8): expert inputs are quantized per 128
 *    values to signed INT8 with an FP32 scale, group dot products are exact
 *    INT32 sums, and scaled groups are combined in FP32; expert outputs return
 *    to BF16 (model card, paragraph on --int8-expert-activations);
 *  - each expert is a gate/up/down feed-forward with SiLU on the gate (README
 *    "Quantization": fused gate/up/SiLU kernels; model card: gate, up and down
 *    projection weights);
 *  - the CPU path keeps experts compressed and expands one selected expert at a
 *    time (README "Build and run"); this oracle does the same;
 *  - NVFP4 (W4A4): E2M1 weights and inputs, an E4M3 scale per 16 values, an
 *    FP32 outer scale per expert matrix (weights) or per input row (inputs),
 *    FP32 accumulation (model card precision table, NVFP4 row; README
 *    "Quantization").  Its readings are listed in the NVFP4 section below.
 *
 * Readings where the pages are silent (each one is a choice, listed with the
 * design notes):
 *  - weight scale s = fp16(max|w| / qmax) with qmax 7 (INT4) or 127 (INT8);
 *    codes q = clamp(rint(w / s), -8..7 | -127..127), computed with the stored
 *    FP16 scale, ties to even; an all-zero group (or a scale that underflows
 *    FP16) stores s = 0 and q = 0;
 *  - INT4 packing: element 2j in the low nibble of byte j, element 2j+1 in the
 *    high nibble, two's complement; rows are [out][in];
 *  - activation scale s = max|v| / 127 in FP32, q = clamp(rint(v / s), -127, 127);
 *    s = 0 gives q = 0;
 *  - INT8 activations feed all three projections: x into gate/up, the BF16
 *    intermediate h into down;
 *  - h = bf16(silu(g) * u) and y = bf16(W_down h) are materialized in BF16;
 *  - the per-token combine is out = sum_k w_k * y_k in FP32, k ascending, with
 *    one fused multiply-add per term, then a single rounding to BF16;
 *  - a routed id outside [0, E) drops that slot (it contributes zero).
 *
 * Precision: where the pages do not fix it, sums are taken in double (the
 * dequantized FP32 weights and BF16 inputs multiply exactly in double), so the
 * oracle gives the exactly rounded value of each materialized BF16 quantity.
 * The INT8-activation mode combines its scaled groups in FP32 because the model
 * card says so.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fopenmp
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GROUP 128

/* ------------------------------------------------------------------------ */
/* Number formats, from their IEEE-style definitions.                        */
/* ------------------------------------------------------------------------ */

/* Round v to a binary format with `sig` significant bits, smallest normal
 * 2^emin and largest finite value `maxf`: nearest, ties to even, gradual
 * underflow, overflow to infinity. */
static double orc_round_format(double v, int sig, int emin, double maxf)
{
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    int ex;
    frexp(v, &ex);                 /* |v| = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                /* |v| in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;        /* subnormal range: fixed quantum */
    int qexp = e - (sig - 1);      /* weight of the last kept bit */
    double r = nearbyint(ldexp(v, -qexp)); /* default rounding mode: ties to even */
    double res = ldexp(r, qexp);
    if (fabs(res) > maxf) return v > 0 ? INFINITY : -INFINITY;
    return res;
}

static const double ORC_BF16_MAX = 3.38953138925153547590e+38; /* (2-2^-7)*2^127 */
static const double ORC_FP16_MAX = 65504.0;

double orc_round_bf16(double v) { return orc_round_format(v, 8, -126, ORC_BF16_MAX); }
double orc_round_fp16(double v) { return orc_round_format(v, 11, -14, ORC_FP16_MAX); }

/* Encode a value to bf16 bits by rounding it first. */
uint16_t orc_bf16_from_double(double v)
{
    if (isnan(v)) return 0x7FC0;
    float f = (float)orc_round_bf16(v); /* exactly representable: conversion is exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

float orc_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t orc_fp16_from_double(double v)
{
    if (isnan(v)) return 0x7E00;
    double r = orc_round_fp16(v);
    uint16_t sign = (signbit(r) ? 0x8000 : 0);
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7C00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {           /* subnormal: a = mant * 2^-24 */
        return sign | (uint16_t)ldexp(a, 24);
    }
    int ex;
    double m = frexp(a, &ex);            /* a = m * 2^ex, m in [0.5,1) */
    int e = ex - 1;                      /* a = (2m) * 2^e, 2m in [1,2) */
    uint16_t mant = (uint16_t)((2.0 * m - 1.0) * 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | mant;
}

double orc_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)mant, -24);
    else if (e == 31) v = mant ? NAN : INFINITY;
    else v = ldexp(1.0 + mant / 1024.0, e - 15);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Weight format: symmetric signed INT4 / INT8, one FP16 scale per 128 inputs. */
/* ------------------------------------------------------------------------ */

static int orc_qmax(int bits) { return bits == 4 ? 7 : 127; }
static int orc_qmin(int bits) { return bits == 4 ? -8 : -127; }

/* Bytes of one packed row of `cols` codes. */
int64_t orc_packed_row_bytes(int64_t cols, int bits) { return bits == 4 ? cols / 2 : cols; }

static void orc_put_code(uint8_t* row, int64_t j, int bits, int q)
{
    if (bits == 8) {
        row[j] = (uint8_t)(int8_t)q;
    } else {
        uint8_t nib = (uint8_t)(q & 0xF);
        if (j % 2 == 0) row[j / 2] = (uint8_t)((row[j / 2] & 0xF0) | nib);
        else            row[j / 2] = (uint8_t)((row[j / 2] & 0x0F) | (nib << 4));
    }
}

static int orc_get_code(const uint8_t* row, int64_t j, int bits)
{
    if (bits == 8) return (int)(int8_t)row[j];
    int nib = (j % 2 == 0) ? (row[j / 2] & 0xF) : (row[j / 2] >> 4);
    return nib >= 8 ? nib - 16 : nib;    /* two's complement nibble */
}

/* Quantize w[rows][cols] (float32) into packed codes q[rows][row_bytes] and
 * FP16 scales s[rows][cols/128].  Returns 0, or -1 on bad arguments. */
int orc_quantize_weights(const float* w, int64_t rows, int64_t cols, int bits,
                         uint8_t* q, uint16_t* s)
{
    if ((bits != 4 && bits != 8) || cols % ORC_GROUP != 0 || rows < 0) return -1;
    const int64_t G = cols / ORC_GROUP, rb = orc_packed_row_bytes(cols, bits);
    const int qmax = orc_qmax(bits), qmin = orc_qmin(bits);
    for (int64_t r = 0; r < rows; ++r) {
        const float* wr = w + r * cols;
        uint8_t* qr = q + r * rb;
        for (int64_t g = 0; g < G; ++g) {
            float m = 0.0f;
            for (int64_t j = g * ORC_GROUP; j < (g + 1) * ORC_GROUP; ++j) {
                float a = fabsf(wr[j]);
                if (a > m) m = a;
            }
            float ratio = m / (float)qmax;                   /* FP32 division */
            uint16_t s16 = orc_fp16_from_double((double)ratio);
            s[r * G + g] = s16;
            float sf = (float)orc_fp16_to_double(s16);
            for (int64_t j = g * ORC_GROUP; j < (g + 1) * ORC_GROUP; ++j) {
                int qv = 0;
                if (sf != 0.0f) {
                    float t = rintf(wr[j] / sf);
                    if (t > (float)qmax) t = (float)qmax;
                    if (t < (float)qmin) t = (float)qmin;
                    qv = (int)t;
                }
                orc_put_code(qr, j, bits, qv);
            }
        }
    }
    return 0;
}

/* Unpack codes to int8 [rows][cols]. */
void orc_unpack_codes(const uint8_t* q, int64_t rows, int64_t cols, int bits, int8_t* codes)
{
    const int64_t rb = orc_packed_row_bytes(cols, bits);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j)
            codes[r * cols + j] = (int8_t)orc_get_code(q + r * rb, j, bits);
}

/* Dequantize to float32: w = s * q.  The product of an 11-bit FP16 significand
 * and a code of at most 8 bits is exact in FP32. */
void orc_dequantize(const uint8_t* q, const uint16_t* s, int64_t rows, int64_t cols, int bits, float* w)
{
    const int64_t G = cols / ORC_GROUP, rb = orc_packed_row_bytes(cols, bits);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            double sc = orc_fp16_to_double(s[r * G + j / ORC_GROUP]);
            w[r * cols + j] = (float)(sc * (double)orc_get_code(q + r * rb, j, bits));
        }
}

/* ------------------------------------------------------------------------ */
/* Activation quantizer: per row and 128-group, FP32 scale max|v|/127.        */
/* ------------------------------------------------------------------------ */

static void orc_quantize_act_row(const float* v, int64_t cols, int8_t* q, float* s)
{
    for (int64_t g = 0; g < cols / ORC_GROUP; ++g) {
        float m = 0.0f;
        for (int64_t j = g * ORC_GROUP; j < (g + 1) * ORC_GROUP; ++j) {
            float a = fabsf(v[j]);
            if (a > m) m = a;
        }
        float sc = m / 127.0f;                               /* FP32 division */
        s[g] = sc;
        for (int64_t j = g * ORC_GROUP; j < (g + 1) * ORC_GROUP; ++j) {
            int qv = 0;
            if (sc != 0.0f) {
                float t = rintf(v[j] / sc);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                qv = (int)t;
            }
            q[j] = (int8_t)qv;
        }
    }
}

/* v: bf16 bits [rows][cols] -> q int8 [rows][cols], s float [rows][cols/128]. */
int orc_quantize_act(const uint16_t* v, int64_t rows, int64_t cols, int8_t* q, float* s)
{
    if (cols % ORC_GROUP != 0 || rows < 0) return -1;
    float* row = (float*)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
    if (!row) return -2;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < cols; ++j) row[j] = orc_bf16_to_float(v[r * cols + j]);
        orc_quantize_act_row(row, cols, q + r * cols, s + r * (cols / ORC_GROUP));
    }
    free(row);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Routing permutation: stable counting sort of slots s = t*K + k by expert.  */
/* ------------------------------------------------------------------------ */

/* counts[E], offsets[E+1], sorted_slot[S] (first offsets[E] entries valid),
 * slot_row[S] (-1 for a dropped slot).  Returns the number of dropped slots. */
int orc_route(const int32_t* ids, int32_t T, int32_t K, int32_t E,
              int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row)
{
    const int64_t S = (int64_t)T * K;
    int bad = 0;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < S; ++s) {
        int32_t id = ids[s];
        if (id < 0 || id >= E) ++bad;
        else ++counts[id];
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t s = 0; s < S; ++s) {
        int32_t id = ids[s];
        if (id < 0 || id >= E) { slot_row[s] = -1; continue; }
        int32_t pos = cursor[id]++;
        sorted_slot[pos] = (int32_t)s;
        slot_row[s] = pos;
    }
    for (int64_t p = offsets[E]; p < S; ++p) sorted_slot[p] = -1;
    free(cursor);
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Expert feed-forward.                                                       */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t T, H, I, E, K;
    int32_t bits;      /* 4 or 8 */
    int32_t act_int8;  /* 0: BF16 activations; 1: INT8 activations */
} orc_shape;

typedef struct {
    const uint8_t* gate_q; const uint16_t* gate_s;   /* [E][I][H*bits/8], [E][I][H/128] */
    const uint8_t* up_q;   const uint16_t* up_s;
    const uint8_t* down_q; const uint16_t* down_s;   /* [E][H][I*bits/8], [E][H][I/128] */
} orc_weights;

static double orc_silu(double g) { return g / (1.0 + exp(-g)); }

static int64_t orc_mat_bytes(int64_t rows, int64_t cols, int bits) { return rows * orc_packed_row_bytes(cols, bits); }

/* FP32 combination of scaled INT32 group dot products:
 * acc = sum over groups (ascending) of float(isum_g) * (xs_g * ws_g). */
static float orc_int8_dot(const int8_t* xq, const float* xs, const int8_t* wq, const uint16_t* ws,
                          int64_t n, int* overflow)
{
    float acc = 0.0f;
    for (int64_t g = 0; g < n / ORC_GROUP; ++g) {
        int64_t isum = 0;
        for (int64_t j = g * ORC_GROUP; j < (g + 1) * ORC_GROUP; ++j) isum += (int64_t)xq[j] * wq[j];
        if (isum > INT32_MAX || isum < INT32_MIN) *overflow = 1;
        float wsf = (float)orc_fp16_to_double(ws[g]);
        float sc = xs[g] * wsf;
        acc = acc + (float)isum * sc;
    }
    return acc;
}

/* Work items of the expert loops: runs of at most ORC_CHUNK sorted rows of
 * one expert, so that one expert with many rows is spread over threads (each
 * item expands its expert's weights itself).  Returns a malloc'ed array
 * {n, e0, r0_0, r1_0, e1, ...}. */
#define ORC_CHUNK 64
static int32_t* orc_row_chunks(const int32_t* offsets, int32_t E)
{
    int64_t n = 0;
    for (int32_t e = 0; e < E; ++e) n += (offsets[e + 1] - offsets[e] + ORC_CHUNK - 1) / ORC_CHUNK;
    int32_t* c = (int32_t*)malloc(sizeof(int32_t) * (size_t)(1 + 3 * n));
    c[0] = (int32_t)n;
    int64_t k = 0;
    for (int32_t e = 0; e < E; ++e)
        for (int32_t r = offsets[e]; r < offsets[e + 1]; r += ORC_CHUNK, ++k) {
            c[1 + 3 * k] = e;
            c[2 + 3 * k] = r;
            c[3 + 3 * k] = r + ORC_CHUNK < offsets[e + 1] ? r + ORC_CHUNK : offsets[e + 1];
        }
    return c;
}

/* Gate/up for every sorted row of every expert, or only for rows whose flag is
 * set in row_mask (may be NULL).  A16: x bf16 [T][H].  A8: xq [T][H], xs [T][H/128].
 * h: bf16 bits [S][I] indexed by sorted row. */
int orc_gate_up(const orc_shape* d, const uint16_t* x, const int8_t* xq, const float* xs,
                const int32_t* sorted_slot, const int32_t* offsets, const orc_weights* W,
                const uint8_t* row_mask, uint16_t* h)
{
    const int64_t H = d->H, I = d->I, G_H = H / ORC_GROUP;
    const int bits = d->bits;
    int overflow = 0;
    int32_t* chunks = orc_row_chunks(offsets, d->E);
    const int64_t nchunks = chunks[0];
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:overflow)
    for (int64_t c = 0; c < nchunks; ++c) {
        const int32_t e = chunks[1 + 3 * c], r0 = chunks[2 + 3 * c], r1 = chunks[3 + 3 * c];
        int any = 0;
        for (int32_t r = r0; r < r1; ++r) if (!row_mask || row_mask[r]) { any = 1; break; }
        if (!any) continue;
        const uint8_t* gq = W->gate_q + e * orc_mat_bytes(I, H, bits);
        const uint8_t* uq = W->up_q + e * orc_mat_bytes(I, H, bits);
        const uint16_t* gs = W->gate_s + e * I * G_H;
        const uint16_t* us = W->up_s + e * I * G_H;
        float* wg = NULL; float* wu = NULL; int8_t* cg = NULL; int8_t* cu = NULL;
        float* xr = (float*)malloc(sizeof(float) * (size_t)H);
        if (!d->act_int8) {    /* expand this expert: exact FP32 dequantized weights */
            wg = (float*)malloc(sizeof(float) * (size_t)(I * H));
            wu = (float*)malloc(sizeof(float) * (size_t)(I * H));
            orc_dequantize(gq, gs, I, H, bits, wg);
            orc_dequantize(uq, us, I, H, bits, wu);
        } else {               /* expand codes only: the group dot products are integer */
            cg = (int8_t*)malloc((size_t)(I * H));
            cu = (int8_t*)malloc((size_t)(I * H));
            orc_unpack_codes(gq, I, H, bits, cg);
            orc_unpack_codes(uq, I, H, bits, cu);
        }
        for (int32_t r = r0; r < r1; ++r) {
            if (row_mask && !row_mask[r]) continue;
            const int64_t t = sorted_slot[r] / d->K;
            if (!d->act_int8)
                for (int64_t k = 0; k < H; ++k) xr[k] = orc_bf16_to_float(x[t * H + k]);
            for (int64_t i = 0; i < I; ++i) {
                double g, u;
                if (!d->act_int8) {
                    double sg = 0.0, su = 0.0;
                    for (int64_t k = 0; k < H; ++k) {
                        sg += (double)xr[k] * (double)wg[i * H + k];
                        su += (double)xr[k] * (double)wu[i * H + k];
                    }
                    g = sg; u = su;
                } else {
                    g = orc_int8_dot(xq + t * H, xs + t * G_H, cg + i * H, gs + i * G_H, H, &overflow);
                    u = orc_int8_dot(xq + t * H, xs + t * G_H, cu + i * H, us + i * G_H, H, &overflow);
                }
                h[(int64_t)r * I + i] = orc_bf16_from_double(orc_silu(g) * u);
            }
        }
        free(xr); free(wg); free(wu); free(cg); free(cu);
    }
    free(chunks);
    return overflow ? -3 : 0;
}

/* Down projection for sorted rows.  A16: h bf16 [S][I].  A8: hq [S][I], hs [S][I/128].
 * y: bf16 bits [S][H] indexed by sorted row. */
int orc_down(const orc_shape* d, const uint16_t* h, const int8_t* hq, const float* hs,
             const int32_t* offsets, const orc_weights* W, const uint8_t* row_mask, uint16_t* y)
{
    const int64_t H = d->H, I = d->I, G_I = I / ORC_GROUP;
    const int bits = d->bits;
    int overflow = 0;
    int32_t* chunks = orc_row_chunks(offsets, d->E);
    const int64_t nchunks = chunks[0];
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:overflow)
    for (int64_t c = 0; c < nchunks; ++c) {
        const int32_t e = chunks[1 + 3 * c], r0 = chunks[2 + 3 * c], r1 = chunks[3 + 3 * c];
        int any = 0;
        for (int32_t r = r0; r < r1; ++r) if (!row_mask || row_mask[r]) { any = 1; break; }
        if (!any) continue;
        const uint8_t* dq = W->down_q + e * orc_mat_bytes(H, I, bits);
        const uint16_t* ds = W->down_s + e * H * G_I;
        float* wd = NULL; int8_t* cd = NULL;
        float* hr = (float*)malloc(sizeof(float) * (size_t)I);
        if (!d->act_int8) {
            wd = (float*)malloc(sizeof(float) * (size_t)(H * I));
            orc_dequantize(dq, ds, H, I, bits, wd);
        } else {
            cd = (int8_t*)malloc((size_t)(H * I));
            orc_unpack_codes(dq, H, I, bits, cd);
        }
        for (int32_t r = r0; r < r1; ++r) {
            if (row_mask && !row_mask[r]) continue;
            if (!d->act_int8)
                for (int64_t i = 0; i < I; ++i) hr[i] = orc_bf16_to_float(h[(int64_t)r * I + i]);
            for (int64_t j = 0; j < H; ++j) {
                double acc;
                if (!d->act_int8) {
                    double s = 0.0;
                    for (int64_t i = 0; i < I; ++i) s += (double)hr[i] * (double)wd[j * I + i];
                    acc = s;
                } else {
                    acc = orc_int8_dot(hq + (int64_t)r * I, hs + (int64_t)r * G_I, cd + j * I,
                                       ds + j * G_I, I, &overflow);
                }
                y[(int64_t)r * H + j] = orc_bf16_from_double(acc);
            }
        }
        free(hr); free(wd); free(cd);
    }
    free(chunks);
    return overflow ? -3 : 0;
}

/* Per-token weighted combine, k ascending, one FP32 fused multiply-add per
 * term.  out_f32 (may be NULL) receives the FP32 sum before rounding; out_bf16
 * (may be NULL) the BF16 result.  tokens (may be NULL = all T) lists the rows
 * to produce; output row n belongs to tokens[n]. */
void orc_combine(const uint16_t* y, const int32_t* slot_row, const float* topk_w,
                 int32_t T, int32_t K, int32_t H, const int64_t* tokens, int64_t ntok,
                 float* out_f32, uint16_t* out_bf16)
{
    const int64_t n_out = tokens ? ntok : T;
    for (int64_t n = 0; n < n_out; ++n) {
        const int64_t t = tokens ? tokens[n] : n;
        for (int64_t j = 0; j < H; ++j) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int32_t r = slot_row[t * K + k];
                if (r < 0) continue;
                acc = fmaf(topk_w[t * K + k], orc_bf16_to_float(y[(int64_t)r * H + j]), acc);
            }
            if (out_f32) out_f32[n * H + j] = acc;
            if (out_bf16) out_bf16[n * H + j] = orc_bf16_from_double((double)acc);
        }
    }
}

/* The whole feed-forward.  tokens (may be NULL = all tokens) restricts the
 * work to the listed tokens; out rows follow the list.  Scratch h/y are
 * allocated here at [S][I] and [S][H] (only the needed rows are written).
 * y_tok (may be NULL) receives the BF16 expert outputs that each listed token
 * combines, [n][K][H] in slot order (zeros for a dropped slot).
 * Returns the number of dropped slots (>= 0), or a negative error. */
int orc_moe_forward(const orc_shape* d, const uint16_t* x, const int32_t* ids, const float* topk_w,
                    const orc_weights* W, const int64_t* tokens, int64_t ntok,
                    float* out_f32, uint16_t* out_bf16, uint16_t* y_tok)
{
    const int64_t T = d->T, H = d->H, I = d->I, K = d->K, S = T * K;
    if (H % ORC_GROUP || I % ORC_GROUP || (d->bits != 4 && d->bits != 8)) return -1;
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)(d->E > 0 ? d->E : 1));
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(d->E + 1));
    int32_t* sorted_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    int32_t* slot_row = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    uint8_t* mask = (uint8_t*)calloc((size_t)(S > 0 ? S : 1), 1);
    uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(S * I > 0 ? S * I : 1));
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(S * H > 0 ? S * H : 1));
    int8_t* xq = NULL; float* xs = NULL; int8_t* hq = NULL; float* hs = NULL;
    int rc = orc_route(ids, d->T, d->K, d->E, counts, offsets, sorted_slot, slot_row);
    const int nbad = rc;
    const int64_t n_out = tokens ? ntok : T;
    for (int64_t n = 0; n < n_out; ++n) {
        const int64_t t = tokens ? tokens[n] : n;
        for (int64_t k = 0; k < K; ++k) if (slot_row[t * K + k] >= 0) mask[slot_row[t * K + k]] = 1;
    }
    if (d->act_int8) {
        xq = (int8_t*)calloc((size_t)(T * H > 0 ? T * H : 1), 1);
        xs = (float*)calloc((size_t)(T * (H / ORC_GROUP) > 0 ? T * (H / ORC_GROUP) : 1), sizeof(float));
        hq = (int8_t*)calloc((size_t)(S * I > 0 ? S * I : 1), 1);
        hs = (float*)calloc((size_t)(S * (I / ORC_GROUP) > 0 ? S * (I / ORC_GROUP) : 1), sizeof(float));
        for (int64_t n = 0; n < n_out; ++n) {
            const int64_t t = tokens ? tokens[n] : n;
            orc_quantize_act(x + t * H, 1, H, xq + t * H, xs + t * (H / ORC_GROUP));
        }
    }
    rc = orc_gate_up(d, x, xq, xs, sorted_slot, offsets, W, mask, h);
    if (rc == 0 && d->act_int8) {
        for (int64_t r = 0; r < S; ++r)
            if (mask[r]) orc_quantize_act(h + r * I, 1, I, hq + r * I, hs + r * (I / ORC_GROUP));
    }
    if (rc == 0) rc = orc_down(d, h, hq, hs, offsets, W, mask, y);
    if (rc == 0) orc_combine(y, slot_row, topk_w, d->T, d->K, d->H, tokens, ntok, out_f32, out_bf16);
    if (rc == 0 && y_tok) {
        for (int64_t n = 0; n < n_out; ++n) {
            const int64_t t = tokens ? tokens[n] : n;
            for (int64_t k = 0; k < K; ++k) {
                const int32_t r = slot_row[t * K + k];
                uint16_t* dst = y_tok + (n * K + k) * H;
                if (r < 0) memset(dst, 0, sizeof(uint16_t) * (size_t)H);
                else memcpy(dst, y + (int64_t)r * H, sizeof(uint16_t) * (size_t)H);
            }
        }
    }
    free(counts); free(offsets); free(sorted_slot); free(slot_row); free(mask);
    free(h); free(y); free(xq); free(xs); free(hq); free(hs);
    return rc == 0 ? nbad : rc;
}

/* Router ahead of the permutation: per token, the K experts with the largest
 * logits, in descending order of logit, ties going to the lower expert id,
 * and their combine weights, a softmax over the K selected logits with the
 * largest one subtracted.  The README's "Quantization" section puts the
 * routing of decode blocks on the GPU and the model card ("Checkpoints and
 * precision", paragraph under the heading about routed experts) keeps the
 * router in floating point; the selection and weighting rule itself is not
 * on the pages: this is the plain top-K softmax reading.  Selection is K
 * passes of a linear scan (strict comparison, so the first, lowest, id wins a
 * tie); exponentials and the normalising sum are taken in double and each
 * weight is rounded once to FP32.  Requires 1 <= K <= E; returns -1 otherwise.
 * Non-finite logits give unspecified results. */
int orc_topk_softmax(const float* logits, int32_t T, int32_t E, int32_t K, int32_t* ids, float* w)
{
    if (K < 1 || K > E) return -1;
    uint8_t* taken = (uint8_t*)malloc((size_t)E);
    double* z = (double*)malloc(sizeof(double) * (size_t)K);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int32_t k = 0; k < K; ++k) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            ids[t * K + k] = best;
        }
        const double m = (double)l[ids[t * K]];
        double sum = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            z[k] = exp((double)l[ids[t * K + k]] - m);
            sum += z[k];
        }
        for (int32_t k = 0; k < K; ++k) w[t * K + k] = (float)(z[k] / sum);
    }
    free(taken);
    free(z);
    return 0;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the expert loops use from now on (benchmark baselines). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* NVFP4 (W4A4).  Model card "LLaDA2.2-flash for minnow", precision table,    */
/* NVFP4 row: E2M1 FP4 weights with an E4M3 scale per 16 weights and an FP32  */
/* outer scale per expert matrix; expert inputs dynamically quantized to E2M1 */
/* with an E4M3 scale per 16 values and an FP32 outer scale per input row.    */
/* README "Quantization": FP32 accumulation.  Model card, paragraph after the */
/* table: the non-native path rebuilds the already quantized FP4 operands and */
/* keeps the activation quantization.                                        */
/*                                                                            */
/* Readings where the pages are silent (listed with the design notes):        */
/*  - outer scale S = max|v| / (6 * 448) in FP32 over the expert matrix        */
/*    (weights) or the row (activations), so the largest block scale is the   */
/*    E4M3 maximum 448 and the largest code the E2M1 maximum 6;              */
/*  - block scale b = E4M3(max|block| / (S * 6)): the FP32 product S * 6, the */
/*    FP32 quotient, rounded to E4M3 to nearest, ties to even, saturating at  */
/*    448; S = 0 gives b = 0;                                                 */
/*  - code c = E2M1(v / (b * S)): the FP32 product b * S, the FP32 quotient,  */
/*    rounded to E2M1 to nearest, ties to even, saturating at 6; a zero      */
/*    divisor, or a magnitude that rounds to zero, gives code 0 (+0);         */
/*  - packing: element 2j in the low nibble of byte j, element 2j + 1 in the  */
/*    high nibble (as INT4); blocks are 16 consecutive values along the       */
/*    reduction dimension; scales are stored [rows][cols / 16], one byte each; */
/*  - the product v = E2M1(c) * E4M3(b) * S is the dequantized value; the     */
/*    expert matmuls sum exact products of such values (here in double) and   */
/*    h, y are materialized in BF16 as in the other formats; h is quantized   */
/*    again (per sorted row) before the down projection.                      */
/* ------------------------------------------------------------------------ */

#define ORC_FP4_BLOCK 16

/* E2M1: sign, two exponent bits (bias 1), one mantissa bit; exponent field 0
 * is subnormal (0 or 0.5).  Code bit 3 is the sign. */
double orc_e2m1_value(int code)
{
    const int e = (code >> 1) & 3, m = code & 1;
    const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (code & 8) ? -mag : mag;
}

/* E4M3 (the FN variant of the OCP 8-bit formats): sign, four exponent bits
 * (bias 7), three mantissa bits; exponent field 0 is subnormal; all-ones
 * exponent and mantissa is NaN; no infinities; largest finite 448. */
double orc_e4m3_value(uint8_t b)
{
    const int e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7) mag = NAN;
    else if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return (b & 0x80) ? -mag : mag;
}

/* Nearest E4M3 (ties to even), saturating to +-448; NaN stays NaN. */
uint8_t orc_e4m3_encode(double v)
{
    if (isnan(v)) return 0x7F;
    double r = orc_round_format(v, 4, -6, 448.0);
    if (isinf(r)) r = r > 0 ? 448.0 : -448.0;
    const uint8_t sign = signbit(r) ? 0x80 : 0;
    const double a = fabs(r);
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -6)) return sign | (uint8_t)ldexp(a, 9);       /* subnormal: a = m * 2^-9 */
    int ex;
    const double fr = frexp(a, &ex);                                  /* a = fr * 2^ex, fr in [0.5, 1) */
    const int e = ex - 1;
    return sign | (uint8_t)((e + 7) << 3) | (uint8_t)((2.0 * fr - 1.0) * 8.0);
}

/* Nearest E2M1 code (ties to even), saturating to +-6; a magnitude that
 * rounds to zero gives code 0. */
int orc_e2m1_encode(double v)
{
    double r = orc_round_format(v, 2, 0, 6.0);
    if (isinf(r)) r = r > 0 ? 6.0 : -6.0;
    if (r == 0.0) return 0;
    const double a = fabs(r);
    int code = 0;
    for (int c = 1; c < 8; ++c)
        if (orc_e2m1_value(c) == a) code = c;
    return (r < 0 ? 8 : 0) | code;
}

/* The FP32 outer scale of a set of values with largest magnitude amax. */
static float orc_fp4_outer(float amax) { return amax / (6.0f * 448.0f); }

/* Quantize one row of `cols` values (float32) with outer scale S into packed
 * codes (cols / 2 bytes) and E4M3 block scales (cols / 16 bytes). */
static void orc_fp4_row(const float* v, int64_t cols, float S, uint8_t* q, uint8_t* b)
{
    memset(q, 0, (size_t)(cols / 2));
    const float den = S * 6.0f;
    for (int64_t blk = 0; blk < cols / ORC_FP4_BLOCK; ++blk) {
        const float* vb = v + blk * ORC_FP4_BLOCK;
        float m = 0.0f;
        for (int j = 0; j < ORC_FP4_BLOCK; ++j) {
            float a = fabsf(vb[j]);
            if (a > m) m = a;
        }
        const float d = den > 0.0f ? m / den : 0.0f;
        const uint8_t bs = orc_e4m3_encode((double)d);
        b[blk] = bs;
        const float den2 = (float)orc_e4m3_value(bs) * S;
        for (int j = 0; j < ORC_FP4_BLOCK; ++j) {
            const int c = den2 > 0.0f ? orc_e2m1_encode((double)(vb[j] / den2)) : 0;
            const int64_t k = blk * ORC_FP4_BLOCK + j;
            q[k / 2] |= (uint8_t)(k % 2 == 0 ? c : c << 4);
        }
    }
}

/* Weights: `mats` matrices of [rows][cols] float32, each with its own outer
 * scale.  q [mats][rows][cols/2], b [mats][rows][cols/16], outer [mats].
 * Returns 0, or -1 on bad arguments. */
int orc_fp4_quantize_weights(const float* w, int64_t mats, int64_t rows, int64_t cols,
                             uint8_t* q, uint8_t* b, float* outer)
{
    if (mats < 0 || rows < 0 || cols % ORC_FP4_BLOCK != 0) return -1;
    for (int64_t mt = 0; mt < mats; ++mt) {
        const float* wm = w + mt * rows * cols;
        float amax = 0.0f;
        for (int64_t i = 0; i < rows * cols; ++i) {
            float a = fabsf(wm[i]);
            if (a > amax) amax = a;
        }
        const float S = orc_fp4_outer(amax);
        outer[mt] = S;
        for (int64_t r = 0; r < rows; ++r)
            orc_fp4_row(wm + r * cols, cols, S, q + (mt * rows + r) * (cols / 2),
                        b + (mt * rows + r) * (cols / ORC_FP4_BLOCK));
    }
    return 0;
}

/* Activations: bf16 rows [rows][cols], an outer scale per row. */
int orc_fp4_quantize_act(const uint16_t* v, int64_t rows, int64_t cols, uint8_t* q, uint8_t* b, float* row_scale)
{
    if (rows < 0 || cols % ORC_FP4_BLOCK != 0) return -1;
    float* f = (float*)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
    if (!f) return -2;
    for (int64_t r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int64_t j = 0; j < cols; ++j) {
            f[j] = orc_bf16_to_float(v[r * cols + j]);
            float a = fabsf(f[j]);
            if (a > amax) amax = a;
        }
        row_scale[r] = orc_fp4_outer(amax);
        orc_fp4_row(f, cols, row_scale[r], q + r * (cols / 2), b + r * (cols / ORC_FP4_BLOCK));
    }
    free(f);
    return 0;
}

/* E2M1(c) * E4M3(b) of element k of a packed row, without the outer scale
 * (a product of at most 6 significant bits, exact in double). */
static double orc_fp4_elem(const uint8_t* q, const uint8_t* b, int64_t k)
{
    const int c = (k % 2 == 0) ? (q[k / 2] & 0xF) : (q[k / 2] >> 4);
    return orc_e2m1_value(c) * orc_e4m3_value(b[k / ORC_FP4_BLOCK]);
}

/* Dequantize rows: out[r][k] = E2M1 * E4M3 * scale[r / rows_per_scale]
 * (float64; one outer scale per `rows_per_scale` rows). */
void orc_fp4_dequantize(const uint8_t* q, const uint8_t* b, const float* scale, int64_t rows, int64_t cols,
                        int64_t rows_per_scale, double* out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k)
            out[r * cols + k] = orc_fp4_elem(q + r * (cols / 2), b + r * (cols / ORC_FP4_BLOCK), k) *
                                (double)scale[r / rows_per_scale];
}

typedef struct {
    const uint8_t* q;   /* [E][rows][cols/2] */
    const uint8_t* b;   /* [E][rows][cols/16] */
    const float* o;     /* [E] */
} orc_fp4_mat;

typedef struct {
    orc_fp4_mat gate, up, down;   /* gate/up [E][I][H], down [E][H][I] */
} orc_fp4_weights;

/* One expert matrix (rows x cols) as unscaled doubles E2M1 * E4M3 (the outer
 * scale is applied to the dot product). */
static double* orc_fp4_expand(const orc_fp4_mat* m, int32_t e, int64_t rows, int64_t cols)
{
    double* w = (double*)malloc(sizeof(double) * (size_t)(rows * cols));
    const uint8_t* q = m->q + (int64_t)e * rows * (cols / 2);
    const uint8_t* b = m->b + (int64_t)e * rows * (cols / ORC_FP4_BLOCK);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k)
            w[r * cols + k] = orc_fp4_elem(q + r * (cols / 2), b + r * (cols / ORC_FP4_BLOCK), k);
    return w;
}

/* Gate/up from quantized x: xq [T][H/2], xb [T][H/16], xr [T].  h bf16 [S][I]
 * by sorted row; only rows whose row_mask flag is set (NULL = all). */
int orc_fp4_gate_up(const orc_shape* d, const uint8_t* xq, const uint8_t* xb, const float* xr,
                    const int32_t* sorted_slot, const int32_t* offsets, const orc_fp4_weights* W,
                    const uint8_t* row_mask, uint16_t* h)
{
    const int64_t H = d->H, I = d->I;
    int32_t* chunks = orc_row_chunks(offsets, d->E);
    const int64_t nchunks = chunks[0];
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nchunks; ++c) {
        const int32_t e = chunks[1 + 3 * c], r0 = chunks[2 + 3 * c], r1 = chunks[3 + 3 * c];
        int any = 0;
        for (int32_t r = r0; r < r1; ++r) if (!row_mask || row_mask[r]) { any = 1; break; }
        if (!any) continue;
        double* wg = orc_fp4_expand(&W->gate, e, I, H);
        double* wu = orc_fp4_expand(&W->up, e, I, H);
        double* xv = (double*)malloc(sizeof(double) * (size_t)H);
        for (int32_t r = r0; r < r1; ++r) {
            if (row_mask && !row_mask[r]) continue;
            const int64_t t = sorted_slot[r] / d->K;
            for (int64_t k = 0; k < H; ++k) xv[k] = orc_fp4_elem(xq + t * (H / 2), xb + t * (H / ORC_FP4_BLOCK), k);
            for (int64_t i = 0; i < I; ++i) {
                double sg = 0.0, su = 0.0;
                for (int64_t k = 0; k < H; ++k) {
                    sg += xv[k] * wg[i * H + k];
                    su += xv[k] * wu[i * H + k];
                }
                const double g = sg * (double)xr[t] * (double)W->gate.o[e];
                const double u = su * (double)xr[t] * (double)W->up.o[e];
                h[(int64_t)r * I + i] = orc_bf16_from_double(orc_silu(g) * u);
            }
        }
        free(wg); free(wu); free(xv);
    }
    free(chunks);
    return 0;
}

/* Down from quantized h: hq [S][I/2], hb [S][I/16], hr [S] by sorted row.
 * y bf16 [S][H] by sorted row. */
int orc_fp4_down(const orc_shape* d, const uint8_t* hq, const uint8_t* hb, const float* hr,
                 const int32_t* offsets, const orc_fp4_weights* W, const uint8_t* row_mask, uint16_t* y)
{
    const int64_t H = d->H, I = d->I;
    int32_t* chunks = orc_row_chunks(offsets, d->E);
    const int64_t nchunks = chunks[0];
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < nchunks; ++c) {
        const int32_t e = chunks[1 + 3 * c], r0 = chunks[2 + 3 * c], r1 = chunks[3 + 3 * c];
        int any = 0;
        for (int32_t r = r0; r < r1; ++r) if (!row_mask || row_mask[r]) { any = 1; break; }
        if (!any) continue;
        double* wd = orc_fp4_expand(&W->down, e, H, I);
        double* hv = (double*)malloc(sizeof(double) * (size_t)I);
        for (int32_t r = r0; r < r1; ++r) {
            if (row_mask && !row_mask[r]) continue;
            for (int64_t i = 0; i < I; ++i) hv[i] = orc_fp4_elem(hq + (int64_t)r * (I / 2), hb + (int64_t)r * (I / ORC_FP4_BLOCK), i);
            for (int64_t j = 0; j < H; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < I; ++i) s += hv[i] * wd[j * I + i];
                y[(int64_t)r * H + j] = orc_bf16_from_double(s * (double)hr[r] * (double)W->down.o[e]);
            }
        }
        free(wd); free(hv);
    }
    free(chunks);
    return 0;
}

/* The whole NVFP4 feed-forward (same contract as orc_moe_forward; d->bits and
 * d->act_int8 are ignored).  Returns the number of dropped slots, or < 0. */
int orc_fp4_moe_forward(const orc_shape* d, const uint16_t* x, const int32_t* ids, const float* topk_w,
                        const orc_fp4_weights* W, const int64_t* tokens, int64_t ntok,
                        float* out_f32, uint16_t* out_bf16, uint16_t* y_tok)
{
    const int64_t T = d->T, H = d->H, I = d->I, K = d->K, S = T * K;
    if (H % ORC_FP4_BLOCK || I % ORC_FP4_BLOCK) return -1;
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)(d->E > 0 ? d->E : 1));
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(d->E + 1));
    int32_t* sorted_slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    int32_t* slot_row = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
    uint8_t* mask = (uint8_t*)calloc((size_t)(S > 0 ? S : 1), 1);
    uint16_t* h = (uint16_t*)calloc((size_t)(S * I > 0 ? S * I : 1), sizeof(uint16_t));
    uint16_t* y = (uint16_t*)calloc((size_t)(S * H > 0 ? S * H : 1), sizeof(uint16_t));
    uint8_t* xq = (uint8_t*)calloc((size_t)(T * H / 2 > 0 ? T * H / 2 : 1), 1);
    uint8_t* xb = (uint8_t*)calloc((size_t)(T * H / ORC_FP4_BLOCK > 0 ? T * H / ORC_FP4_BLOCK : 1), 1);
    float* xr = (float*)calloc((size_t)(T > 0 ? T : 1), sizeof(float));
    uint8_t* hq = (uint8_t*)calloc((size_t)(S * I / 2 > 0 ? S * I / 2 : 1), 1);
    uint8_t* hb = (uint8_t*)calloc((size_t)(S * I / ORC_FP4_BLOCK > 0 ? S * I / ORC_FP4_BLOCK : 1), 1);
    float* hr = (float*)calloc((size_t)(S > 0 ? S : 1), sizeof(float));
    const int nbad = orc_route(ids, d->T, d->K, d->E, counts, offsets, sorted_slot, slot_row);
    const int64_t n_out = tokens ? ntok : T;
    for (int64_t n = 0; n < n_out; ++n) {
        const int64_t t = tokens ? tokens[n] : n;
        for (int64_t k = 0; k < K; ++k) if (slot_row[t * K + k] >= 0) mask[slot_row[t * K + k]] = 1;
        orc_fp4_quantize_act(x + t * H, 1, H, xq + t * (H / 2), xb + t * (H / ORC_FP4_BLOCK), xr + t);
    }
    int rc = orc_fp4_gate_up(d, xq, xb, xr, sorted_slot, offsets, W, mask, h);
    for (int64_t r = 0; rc == 0 && r < S; ++r)
        if (mask[r]) orc_fp4_quantize_act(h + r * I, 1, I, hq + r * (I / 2), hb + r * (I / ORC_FP4_BLOCK), hr + r);
    if (rc == 0) rc = orc_fp4_down(d, hq, hb, hr, offsets, W, mask, y);
    if (rc == 0) orc_combine(y, slot_row, topk_w, d->T, d->K, d->H, tokens, ntok, out_f32, out_bf16);
    if (rc == 0 && y_tok) {
        for (int64_t n = 0; n < n_out; ++n) {
            const int64_t t = tokens ? tokens[n] : n;
            for (int64_t k = 0; k < K; ++k) {
                const int32_t r = slot_row[t * K + k];
                uint16_t* dst = y_tok + (n * K + k) * H;
                if (r < 0) memset(dst, 0, sizeof(uint16_t) * (size_t)H);
                else memcpy(dst, y + (int64_t)r * H, sizeof(uint16_t) * (size_t)H);
            }
        }
    }
    free(counts); free(offsets); free(sorted_slot); free(slot_row); free(mask); free(h); free(y);
    free(xq); free(xb); free(xr); free(hq); free(hb); free(hr);
    return rc == 0 ? nbad : rc;
}
