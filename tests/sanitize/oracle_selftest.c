/*
 * Runs every function of the CPU oracle (oracle/moe_oracle.c) on small inputs,
 * including the edge cases its callers reach (T = 0, K = E, exact ties, masks,
 * injected logits, subnormal / NaN / overflowing values), and checks a few
 * invariants.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py: any out-of-bounds access, use after free, leak or
 * undefined operation aborts the run.  Exit status 0 = every check passed.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {  /* splitmix64 */
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }
static float normalf(void) { return (float)((uniform() + uniform() + uniform() - 1.5) * 2.0); }

/* random Q4_0 rows: fp16 scale of a small magnitude (either sign), random nibbles */
static void q4_0_fill(uint8_t* q, size_t nblocks) {
    for (size_t b = 0; b < nblocks; ++b) {
        uint16_t d = (uint16_t)(0x2000 + (next_u64() & 0x0FFF));  /* ~1e-3 .. 1e-2 */
        if (next_u64() & 1) d |= 0x8000;
        q[b * 18] = (uint8_t)(d & 0xFF);
        q[b * 18 + 1] = (uint8_t)(d >> 8);
        for (int j = 0; j < 16; ++j) q[b * 18 + 2 + j] = (uint8_t)next_u64();
    }
}

static void codecs(void) {
    for (uint32_t h = 0; h < 65536; ++h) {
        double a = orc_f16_to_f64((uint16_t)h), b = orc_bf16_to_f64((uint16_t)h);
        if (!isnan(b)) CHECK(orc_f64_to_bf16(b) == (uint16_t)h || b == 0.0);
        (void)a;
    }
    const double cases[] = {0.0, -0.0, 1.0, -1.0, 1e-45, 1e-40, 3e38, 4e38, -4e38, INFINITY,
                            -INFINITY, NAN, 1.0 + 0x1p-8, 1.0 + 0x1p-9, 1.0 + 3 * 0x1p-9};
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
        uint16_t e = orc_f64_to_bf16(cases[i]);
        double r = orc_round_act(cases[i], ORC_BF16), f = orc_round_act(cases[i], ORC_F32);
        CHECK(isnan(cases[i]) ? isnan(r) : (r == orc_bf16_to_f64(e)));
        (void)f;
    }
    uint8_t blk[18];
    double out[32];
    q4_0_fill(blk, 1);
    orc_q4_0_decode(blk, out);
    blk[0] = 0; blk[1] = 0;
    orc_q4_0_decode(blk, out);
    for (int j = 0; j < 32; ++j) CHECK(out[j] == 0.0);
    CHECK(orc_gelu_tanh(0.0) == 0.0);
    CHECK(isfinite(orc_gelu_tanh(50.0)) && isfinite(orc_gelu_tanh(-50.0)));
}

static void routing(void) {
    enum { T = 5, H = 64, E = 8, K = 3 };
    float x[T * H], w[E * H], rs[H], bias[E];
    for (int i = 0; i < T * H; ++i) x[i] = normalf();
    for (int i = 0; i < E * H; ++i) w[i] = normalf() / 8;
    for (int i = 0; i < H; ++i) rs[i] = 1.0f + normalf() / 10;
    for (int i = 0; i < E; ++i) bias[i] = normalf();
    double logits[T * E], wts[T * K];
    int32_t ids[T * K];
    CHECK(orc_router_logits(x, ORC_F32, T, H, w, rs, bias, E, logits) == 0);
    CHECK(orc_router_logits(x, ORC_F32, 0, H, w, NULL, NULL, E, logits) == 0);
    CHECK(orc_router_logits(NULL, ORC_F32, T, H, w, NULL, NULL, E, logits) != 0);
    CHECK(orc_topk_softmax(logits, T, E, K, ids, wts) == 0);
    for (int t = 0; t < T; ++t) {
        double s = 0;
        for (int k = 0; k < K; ++k) s += wts[t * K + k];
        CHECK(fabs(s - 1.0) < 1e-12);
        for (int k = 1; k < K; ++k) CHECK(logits[t * E + ids[t * K + k - 1]] >= logits[t * E + ids[t * K + k]]);
    }
    /* exact ties and K = E */
    double flat[2 * E];
    int32_t all[2 * E];
    double wall[2 * E];
    for (int i = 0; i < 2 * E; ++i) flat[i] = (i % 3) ? 0.5 : -0.0;
    CHECK(orc_topk_softmax(flat, 2, E, E, all, wall) == 0);
    for (int t = 0; t < 2; ++t)
        for (int k = 1; k < E; ++k)
            CHECK(flat[t * E + all[t * E + k - 1]] > flat[t * E + all[t * E + k]] ||
                  (flat[t * E + all[t * E + k - 1]] == flat[t * E + all[t * E + k]] &&
                   all[t * E + k - 1] < all[t * E + k]));
    CHECK(orc_topk_softmax(logits, T, E, E + 1, ids, wts) != 0);
    CHECK(orc_topk_weights(logits, T, E, K, ids, wts) == 0);
    int32_t off[E + 1], ss[T * K], sp[T * K];
    CHECK(orc_permute(ids, T, K, E, off, ss, sp) == 0);
    CHECK(off[E] == T * K);
    for (int s = 0; s < T * K; ++s) CHECK(ss[sp[s]] == s);
    int32_t bad[2] = {0, E};
    CHECK(orc_permute(bad, 1, 2, E, off, ss, sp) == 3);
    CHECK(orc_permute(ids, 0, K, E, off, ss, sp) == 0 && off[E] == 0);
}

static void experts_and_layer(void) {
    enum { T = 4, H = 64, E = 4, K = 2, I = 32 };
    uint16_t x[T * H];
    float xf[T * H], wr[E * H], sc[E], rmsw[H], bias[E];
    uint8_t* gu = malloc((size_t)E * 2 * I * (H / 32) * 18);
    uint8_t* dn = malloc((size_t)E * H * (I / 32) * 18);
    q4_0_fill(gu, (size_t)E * 2 * I * (H / 32));
    q4_0_fill(dn, (size_t)E * H * (I / 32));
    for (int i = 0; i < T * H; ++i) {
        xf[i] = normalf();
        x[i] = orc_f64_to_bf16(xf[i]);
    }
    for (int i = 0; i < E * H; ++i) wr[i] = normalf() / 8;
    for (int i = 0; i < E; ++i) {
        sc[i] = 1.0f + normalf() / 10;
        bias[i] = -(float)i / 3;
    }
    for (int i = 0; i < H; ++i) rmsw[i] = 1.0f + normalf() / 20;
    double h[I], y[H];
    CHECK(orc_expert_ffn_token(x, ORC_BF16, H, gu, dn, I, E - 1, h, y) == 0);
    CHECK(orc_expert_ffn_token(xf, ORC_F32, H, gu, dn, I, 0, NULL, y) == 0);
    CHECK(orc_expert_ffn_token(x, ORC_BF16, 48, gu, dn, I, 0, h, y) != 0);  /* H % 32 */
    double lin[T * 2 * I];
    CHECK(orc_linear_q4_0(x, ORC_BF16, T, H, gu, 2 * I, lin) == 0);
    double logits[T * E], w[T * K], out[T * H], ys[T * K * H];
    int32_t ids[T * K], off[E + 1], ss[T * K], sp[T * K];
    uint8_t tmask[T] = {1, 0, 1, 1}, smask[T * K];
    for (int s = 0; s < T * K; ++s) smask[s] = tmask[s / K];
    CHECK(orc_moe_layer(x, ORC_BF16, T, H, wr, NULL, NULL, bias, E, K, gu, dn, I, sc, NULL, logits,
                        ids, w, off, ss, sp, out) == 0);
    CHECK(orc_expert_ffn(x, ORC_BF16, T, H, gu, dn, I, E, K, off, ss, smask, ys) == 0);
    CHECK(orc_combine(ys, sp, ids, w, sc, T, K, H, tmask, out) == 0);
    float li[T * E];
    for (int i = 0; i < T * E; ++i) li[i] = (float)uniform();
    CHECK(orc_moe_layer(xf, ORC_F32, T, H, NULL, li, NULL, NULL, E, K, gu, dn, I, NULL, tmask, NULL,
                        ids, w, off, ss, sp, out) == 0);
    CHECK(orc_moe_layer(xf, ORC_F32, T, H, NULL, NULL, NULL, NULL, E, K, gu, dn, I, NULL, NULL, NULL,
                        ids, w, off, ss, sp, out) != 0);  /* neither router nor logits */
    uint16_t xh[T * H], xn[T * H];
    int32_t sids[T * K];
    CHECK(orc_rmsnorm(x, ORC_BF16, rmsw, 1e-6, T, H, xh) == 0);
    CHECK(orc_residual(x, out, T, H, tmask, xn) == 0);
    CHECK(orc_stack_layer(x, T, H, rmsw, 1e-6, wr, bias, E, K, gu, dn, I, sc, NULL, xh, sids, out,
                          xn) == 0);
    CHECK(orc_stack_layer(x, T, H, rmsw, 1e-6, wr, bias, E, K, gu, dn, I, sc, tmask, NULL, NULL,
                          NULL, xn) == 0);
    memset(x, 0, sizeof x);
    CHECK(orc_stack_layer(x, T, H, rmsw, 1e-6, wr, bias, E, K, gu, dn, I, sc, NULL, xh, sids, out,
                          xn) == 0);
    for (int i = 0; i < T * H; ++i) CHECK(xn[i] == 0 && xh[i] == 0);
    free(gu);
    free(dn);
}

int main(void) {
    codecs();
    routing();
    experts_and_layer();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle self-test passed\n");
    return 0;
}
