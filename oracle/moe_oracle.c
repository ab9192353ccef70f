/*
 * moe_oracle.c -- plain CPU reference of the routed-MoE layer.
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): single-threaded, binary64,
 * no blocking, no fusion, no library beyond libm.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Subnormals: fraction * 2^-24.  Inf/NaN scales are an input error: NaN. */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int fr = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + fr), ex - 25);
    return sign ? -v : v;
}

/* bf16 is the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a binary64 value to bf16 (8 significant bits, binary32 exponent
 * range), round-to-nearest-even, overflow to infinity, NaN stays NaN. */
uint16_t orc_f64_to_bf16(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0 : 0x7FC0);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    uint32_t bits;
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: quantum 2^-133 */
        double q = rint(a / ldexp(1.0, -133));        /* rint: ties to even */
        bits = (uint32_t)q;                            /* 128 becomes the min normal */
    } else {
        int e;
        frexp(a, &e);                                  /* a = m 2^e, 0.5 <= m < 1 */
        int E = e - 1;                                 /* a in [2^E, 2^(E+1)) */
        double q = rint(a / ldexp(1.0, E - 7));        /* 128..256 */
        bits = ((uint32_t)(E + 127) << 7) + ((uint32_t)q - 128u);
        if (bits >= 0x7F80u) return sign | 0x7F80;    /* overflow */
    }
    return (uint16_t)(sign | bits);
}

double orc_round_act(double v, int act) {
    if (act == ORC_F32) return (double)(float)v;
    return orc_bf16_to_f64(orc_f64_to_bf16(v));
}

double orc_load_act(const void* base, int act, int64_t idx) {
    if (act == ORC_F32) return (double)((const float*)base)[idx];
    return orc_bf16_to_f64(((const uint16_t*)base)[idx]);
}

/* ------------------------------------------------------------------------ */
/* ggml Q4_0 block (byte-for-byte ggml blocks, multiplied in place)          */

void orc_q4_0_decode(const uint8_t* blk, double out[32]) {
    uint16_t dbits = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));   /* little-endian */
    double d = orc_f16_to_f64(dbits);
    const uint8_t* qs = blk + 2;
    for (int j = 0; j < 16; ++j) {
        int lo = qs[j] & 0x0F;
        int hi = qs[j] >> 4;
        out[j] = (double)(lo - 8) * d;
        out[j + 16] = (double)(hi - 8) * d;
    }
}

double orc_gelu_tanh(double z) {
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* dot of one Q4_0 row (nb blocks) with a binary64 vector */
static double q4_0_row_dot(const uint8_t* row, int nb, const double* v) {
    double acc = 0.0, wv[32];
    for (int b = 0; b < nb; ++b) {
        orc_q4_0_decode(row + (size_t)b * 18, wv);
        for (int j = 0; j < 32; ++j) acc += wv[j] * v[b * 32 + j];
    }
    return acc;
}

/* ------------------------------------------------------------------------ */
/* Router                                                                    */

int orc_router_logits(const void* x, int x_dt, int64_t T, int H, const float* w_r,
                      const float* r_scale, const float* bias, int E, double* logits) {
    if (T < 0 || H <= 0 || E <= 0 || !w_r || !logits || (T > 0 && !x)) return 1;
    for (int64_t t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int j = 0; j < H; ++j) {
                double xv = orc_load_act(x, x_dt, t * (int64_t)H + j);
                if (r_scale) xv *= (double)r_scale[j];
                acc += xv * (double)w_r[(size_t)e * H + j];
            }
            if (bias) acc += (double)bias[e];
            logits[t * E + e] = acc;
        }
    return 0;
}

/* Renormalised softmax weights of given experts: p = softmax over all E
 * logits, w[t,k] = p[ids[t,k]] / sum_k p[ids[t,k]]. */
int orc_topk_weights(const double* logits, int64_t T, int E, int K, const int32_t* ids, double* w) {
    if (T < 0 || E <= 0 || K <= 0 || K > E || !logits || !ids || !w) return 1;
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    if (!p) return 2;
    for (int64_t t = 0; t < T; ++t) {
        const double* l = logits + t * E;
        double mx = l[0];
        for (int e = 1; e < E; ++e) if (l[e] > mx) mx = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) { p[e] = exp(l[e] - mx); z += p[e]; }
        for (int e = 0; e < E; ++e) p[e] /= z;
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += p[ids[t * K + k]];
        for (int k = 0; k < K; ++k) w[t * K + k] = p[ids[t * K + k]] / s;
    }
    free(p);
    return 0;
}

/* Stable insertion sort of expert indices by descending logit: equal logits
 * keep ascending expert order; the first K are the chosen experts. */
int orc_topk_softmax(const double* logits, int64_t T, int E, int K, int32_t* ids, double* w) {
    if (T < 0 || E <= 0 || K <= 0 || K > E || !logits || !ids || !w) return 1;
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    if (!order) return 2;
    for (int64_t t = 0; t < T; ++t) {
        const double* l = logits + t * E;
        for (int e = 0; e < E; ++e) {
            int i = e;
            while (i > 0 && l[order[i - 1]] < l[e]) { order[i] = order[i - 1]; --i; }
            order[i] = e;
        }
        for (int k = 0; k < K; ++k) ids[t * K + k] = order[k];
    }
    free(order);
    return orc_topk_weights(logits, T, E, K, ids, w);
}

/* ------------------------------------------------------------------------ */
/* Permutation: stable counting sort                                         */

int orc_permute(const int32_t* ids, int64_t T, int K, int E, int32_t* offsets,
                int32_t* sorted_slots, int32_t* slot_pos) {
    if (T < 0 || K <= 0 || E <= 0 || !offsets) return 1;
    int64_t n = T * K;
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t s = 0; s < n; ++s) {
        if (ids[s] < 0 || ids[s] >= E) return 3;
        offsets[ids[s] + 1] += 1;
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!fill) return 2;
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t s = 0; s < n; ++s) {
        int32_t pos = fill[ids[s]]++;
        sorted_slots[pos] = (int32_t)s;
        slot_pos[s] = pos;
    }
    free(fill);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN                                                                */

int orc_expert_ffn_token(const void* x_row, int x_dt, int H, const uint8_t* w_gate_up,
                         const uint8_t* w_down, int I, int e, double* h_out, double* y_out) {
    if (H <= 0 || I <= 0 || H % 32 || I % 32 || !x_row || !w_gate_up || !w_down) return 1;
    int nbh = H / 32, nbi = I / 32;
    size_t gu_row = (size_t)nbh * 18, dn_row = (size_t)nbi * 18;
    const uint8_t* gu = w_gate_up + (size_t)e * (size_t)(2 * I) * gu_row;
    const uint8_t* dn = w_down + (size_t)e * (size_t)H * dn_row;
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    if (!xv || !h) { free(xv); free(h); return 2; }
    for (int j = 0; j < H; ++j) xv[j] = orc_load_act(x_row, x_dt, j);
    for (int i = 0; i < I; ++i) {
        double g = q4_0_row_dot(gu + (size_t)i * gu_row, nbh, xv);          /* gate row i */
        double u = q4_0_row_dot(gu + (size_t)(I + i) * gu_row, nbh, xv);    /* up row i */
        h[i] = orc_round_act(orc_gelu_tanh(g) * u, x_dt);
        if (h_out) h_out[i] = h[i];
    }
    if (y_out)
        for (int o = 0; o < H; ++o) y_out[o] = q4_0_row_dot(dn + (size_t)o * dn_row, nbi, h);
    free(xv);
    free(h);
    return 0;
}

int orc_linear_q4_0(const void* x, int x_dt, int64_t T, int H, const uint8_t* w, int R, double* y) {
    if (T < 0 || H <= 0 || H % 32 || R <= 0 || !x || !w || !y) return 1;
    int nb = H / 32;
    size_t row = (size_t)nb * 18, esz = (x_dt == ORC_F32) ? 4 : 2;
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    if (!xv) return 2;
    for (int64_t t = 0; t < T; ++t) {
        const uint8_t* xr = (const uint8_t*)x + (size_t)t * (size_t)H * esz;
        for (int j = 0; j < H; ++j) xv[j] = orc_load_act(xr, x_dt, j);
        for (int r = 0; r < R; ++r) y[(size_t)t * R + r] = q4_0_row_dot(w + (size_t)r * row, nb, xv);
    }
    free(xv);
    return 0;
}

int orc_expert_ffn(const void* x, int x_dt, int64_t T, int H, const uint8_t* w_gate_up,
                   const uint8_t* w_down, int I, int E, int K, const int32_t* offsets,
                   const int32_t* sorted_slots, const uint8_t* slot_mask, double* y_sorted) {
    if (T < 0 || K <= 0 || E <= 0 || !offsets || !sorted_slots || !y_sorted) return 1;
    size_t esz = (x_dt == ORC_F32) ? 4 : 2;
    for (int e = 0; e < E; ++e)
        for (int32_t p = offsets[e]; p < offsets[e + 1]; ++p) {
            int32_t s = sorted_slots[p];
            if (slot_mask && !slot_mask[s]) continue;
            int64_t t = s / K;
            const uint8_t* xr = (const uint8_t*)x + (size_t)t * (size_t)H * esz;
            int rc = orc_expert_ffn_token(xr, x_dt, H, w_gate_up, w_down, I, e, NULL,
                                          y_sorted + (size_t)p * H);
            if (rc) return rc;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */

int orc_combine(const double* y_sorted, const int32_t* slot_pos, const int32_t* ids,
                const double* w, const float* scale, int64_t T, int K, int H,
                const uint8_t* token_mask, double* out) {
    if (T < 0 || K <= 0 || H <= 0 || !out) return 1;
    for (int64_t t = 0; t < T; ++t) {
        if (token_mask && !token_mask[t]) continue;
        for (int o = 0; o < H; ++o) out[t * H + o] = 0.0;
        for (int k = 0; k < K; ++k) {
            int64_t s = t * K + k;
            double c = w[s] * (scale ? (double)scale[ids[s]] : 1.0);
            const double* y = y_sorted + (size_t)slot_pos[s] * H;
            for (int o = 0; o < H; ++o) out[t * H + o] += c * y[o];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm (pre-norm of the stack)                                           */

int orc_rmsnorm(const void* x, int x_dt, const float* w, double eps, int64_t T, int H,
                uint16_t* out_bf16) {
    if (T < 0 || H <= 0 || !w || !out_bf16) return 1;
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int j = 0; j < H; ++j) {
            double v = orc_load_act(x, x_dt, t * (int64_t)H + j);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / H + eps);
        for (int j = 0; j < H; ++j) {
            double v = orc_load_act(x, x_dt, t * (int64_t)H + j);
            out_bf16[t * H + j] = orc_f64_to_bf16(v * r * (double)w[j]);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Whole layer, step by step                                                 */

int orc_moe_layer(const void* x, int x_dt, int64_t T, int H, const float* w_r,
                  const float* logits_in, const float* r_scale, const float* bias, int E, int K,
                  const uint8_t* w_gate_up, const uint8_t* w_down, int I, const float* scale,
                  const uint8_t* token_mask, double* logits, int32_t* ids, double* w,
                  int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, double* out) {
    if (T < 0 || K <= 0 || K > E) return 1;
    double* l = logits ? logits : (double*)malloc(sizeof(double) * (size_t)(T * E + 1));
    if (!l) return 2;
    int rc = 0;
    if (w_r) {
        rc = orc_router_logits(x, x_dt, T, H, w_r, r_scale, bias, E, l);
    } else {
        if (!logits_in) rc = 1;
        else for (int64_t i = 0; i < T * E; ++i) l[i] = (double)logits_in[i];
    }
    if (!rc) rc = orc_topk_softmax(l, T, E, K, ids, w);
    if (!rc) rc = orc_permute(ids, T, K, E, offsets, sorted_slots, slot_pos);
    /* expert FFN and combine, token by token (tokens are independent): the
     * expert output of slot s is produced exactly as in orc_expert_ffn and
     * weighted exactly as in orc_combine. */
    double* y = (double*)malloc(sizeof(double) * (size_t)H * (size_t)K);
    if (!y) rc = 2;
    size_t esz = (x_dt == ORC_F32) ? 4 : 2;
    for (int64_t t = 0; !rc && t < T; ++t) {
        if (token_mask && !token_mask[t]) continue;
        const uint8_t* xr = (const uint8_t*)x + (size_t)t * (size_t)H * esz;
        for (int k = 0; k < K && !rc; ++k)
            rc = orc_expert_ffn_token(xr, x_dt, H, w_gate_up, w_down, I, ids[t * K + k], NULL,
                                      y + (size_t)k * H);
        for (int o = 0; !rc && o < H; ++o) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                int32_t e = ids[t * K + k];
                acc += (w[t * K + k] * (scale ? (double)scale[e] : 1.0)) * y[(size_t)k * H + o];
            }
            out[t * H + o] = acc;
        }
    }
    free(y);
    if (!logits) free(l);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Stack: residual add and one pre-norm block                                */

/* The stack's residual stream is bf16 (the stack workload's activations);
 * the layer output is added to it and the sum rounded once to bf16. */
int orc_residual(const uint16_t* x_bf16, const double* out, int64_t T, int H,
                 const uint8_t* token_mask, uint16_t* x_next) {
    if (T < 0 || H <= 0 || !x_bf16 || !out || !x_next) return 1;
    for (int64_t t = 0; t < T; ++t) {
        if (token_mask && !token_mask[t]) continue;
        for (int j = 0; j < H; ++j) {
            size_t i = (size_t)t * (size_t)H + (size_t)j;
            x_next[i] = orc_f64_to_bf16(orc_bf16_to_f64(x_bf16[i]) + out[i]);
        }
    }
    return 0;
}

/* Model card, table "What is inside": the norms are FP32 (here binary64 in the
 * oracle); the norm precedes the routed layer and the residual follows it. */
int orc_stack_layer(const uint16_t* x_bf16, int64_t T, int H, const float* rms_w, double eps,
                    const float* w_r, const float* bias, int E, int K, const uint8_t* w_gate_up,
                    const uint8_t* w_down, int I, const float* scale, const uint8_t* token_mask,
                    uint16_t* xhat_out, int32_t* ids_out, double* out_out, uint16_t* x_next) {
    if (T < 0 || H <= 0 || K <= 0 || K > E || !x_bf16 || !rms_w || !w_r || !x_next) return 1;
    size_t n = (size_t)T * (size_t)H;
    uint16_t* xhat = (uint16_t*)malloc(sizeof(uint16_t) * (n + 1));
    double* out = (double*)malloc(sizeof(double) * (n + 1));
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
    double* w = (double*)malloc(sizeof(double) * ((size_t)T * K + 1));
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t* ss = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
    int32_t* sp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
    int rc = (!xhat || !out || !ids || !w || !off || !ss || !sp) ? 2 : 0;
    for (size_t i = 0; !rc && i < n; ++i) out[i] = NAN;  /* rows of unselected tokens */
    if (!rc) rc = orc_rmsnorm(x_bf16, ORC_BF16, rms_w, eps, T, H, xhat);
    if (!rc)
        rc = orc_moe_layer(xhat, ORC_BF16, T, H, w_r, NULL, NULL, bias, E, K, w_gate_up, w_down, I,
                           scale, token_mask, NULL, ids, w, off, ss, sp, out);
    if (!rc) rc = orc_residual(x_bf16, out, T, H, token_mask, x_next);
    if (!rc && xhat_out) memcpy(xhat_out, xhat, sizeof(uint16_t) * n);
    if (!rc && ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * K);
    if (!rc && out_out) memcpy(out_out, out, sizeof(double) * n);
    free(xhat); free(out); free(ids); free(w); free(off); free(ss); free(sp);
    return rc;
}
