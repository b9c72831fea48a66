/* Driver for a sanitizer build of the CPU oracle (AddressSanitizer + UndefinedBehaviorSanitizer):
 * calls every oracle entry on a small shard with edge routing (duplicates, dropped ids, a
 * non-local pair, an empty expert) and on the sizes' boundaries, so an out-of-bounds index or
 * undefined arithmetic in the oracle aborts the run.  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_rows_capacity(int T, int k, int EL, int BM);
int oracle_route(int T, int k, int E, int e_lo, int EL, int BM, const int32_t* topk_idx, int32_t* counts,
                 int32_t* padded_offsets, int32_t* row_pair, int32_t* pair_row, int32_t* tile_expert,
                 int32_t* tok_nloc, int32_t* meta);
int oracle_forward(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x, const int32_t* topk_idx,
                   const float* topk_w, const uint16_t* W1, const uint16_t* W2, const int32_t* tokens, int ntok,
                   double* y);
int oracle_l1_rows(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x, const int32_t* topk_idx,
                   const uint16_t* W1, const int32_t* pairs, int np, double* h_out, double* a_out);
int oracle_swiglu(int64_t nrows, int I, const double* hgu, double* a);
int oracle_swiglu_bwd(int64_t nrows, int I, const double* hgu, const double* da, double* dhgu);
int oracle_backward_rows(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x,
                         const int32_t* topk_idx, const float* topk_w, const uint16_t* W1, const uint16_t* W2,
                         const uint16_t* dy, const int32_t* pairs, int np, double* dA_out, double* dhgu_out);
int oracle_backward(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x, const int32_t* topk_idx,
                    const float* topk_w, const uint16_t* W1, const uint16_t* W2, const uint16_t* dy,
                    const int32_t* experts, int nexp, double* dW1, double* dW2);
int oracle_backward_tokens(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x,
                           const int32_t* topk_idx, const float* topk_w, const uint16_t* W1, const uint16_t* W2,
                           const uint16_t* dy, const int32_t* tokens, int ntok, double* dx, double* dtopk_w);
int oracle_mx_quantize(int fmt, int64_t n, const double* v, uint8_t* codes, uint8_t* scales);
int oracle_mx_dequantize(int fmt, int64_t n, const uint8_t* codes, const uint8_t* scales, double* v);
int oracle_forward_mx(int T, int H, int I, int E, int e_lo, int EL, int k, const uint8_t* x_codes,
                      const uint8_t* x_scales, const int32_t* topk_idx, const float* topk_w, const uint8_t* w1_codes,
                      const uint8_t* w1_scales, const uint8_t* w2_codes, const uint8_t* w2_scales, double clamp,
                      int quant_act, const int32_t* tokens, int ntok, double* y);
int oracle_mx_l1_rows(int T, int H, int I, int E, int e_lo, int EL, int k, const uint8_t* x_codes,
                      const uint8_t* x_scales, const int32_t* topk_idx, const uint8_t* w1_codes,
                      const uint8_t* w1_scales, double clamp, const int32_t* pairs, int np, double* a_out);
int oracle_mx_l2_rows(int H, int I, int EL, const uint8_t* w2_codes, const uint8_t* w2_scales, const int32_t* experts,
                      int np, const uint8_t* act_codes, const uint8_t* act_scales, double* o_out);

static uint32_t rng = 12345u;
static uint32_t next_u32(void) { rng ^= rng << 13; rng ^= rng >> 17; rng ^= rng << 5; return rng; }
static double next_unit(void) { return (next_u32() & 0xffffff) / 16777216.0 * 2.0 - 1.0; }
static uint16_t bf16_of(double v) {   /* truncation suffices for test data */
    float f = (float)v;
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}
#define CHECK(x) do { if ((x) != 0) { fprintf(stderr, "call failed: %s\n", #x); return 1; } } while (0)

int main(void) {
    enum { T = 9, H = 64, I = 32, E = 7, EL = 3, e_lo = 2, k = 3, BM = 4 };
    int32_t idx[T * k];
    for (int i = 0; i < T * k; ++i) idx[i] = (int32_t)(next_u32() % (E + 2)) - 1;   /* includes -1 and E */
    idx[0] = idx[1] = e_lo;           /* a duplicate */
    idx[3] = e_lo + EL;               /* non-local */
    for (int i = 0; i < T * k; ++i)
        if (idx[i] == e_lo + 1) idx[i] = e_lo + 2;   /* local expert 1 stays empty */
    float w[T * k];
    uint16_t x[T * H], W1[EL * H * 2 * I], W2[EL * I * H], dy[T * H];
    for (int i = 0; i < T * k; ++i) w[i] = (float)next_unit();
    for (int i = 0; i < T * H; ++i) { x[i] = bf16_of(next_unit()); dy[i] = bf16_of(next_unit()); }
    for (int i = 0; i < EL * H * 2 * I; ++i) W1[i] = bf16_of(0.2 * next_unit());
    for (int i = 0; i < EL * I * H; ++i) W2[i] = bf16_of(0.2 * next_unit());

    const int64_t R = oracle_rows_capacity(T, k, EL, BM);
    int32_t *row_pair = malloc(sizeof(int32_t) * R), *tile_expert = malloc(sizeof(int32_t) * (R / BM));
    int32_t counts[EL], offs[EL + 1], pair_row[T * k], tok_nloc[T], meta[2];
    CHECK(oracle_route(T, k, E, e_lo, EL, BM, idx, counts, offs, row_pair, pair_row, tile_expert, tok_nloc, meta));
    int32_t tokens[T], pairs[T * k], experts[EL];
    for (int t = 0; t < T; ++t) tokens[t] = t;
    for (int p = 0; p < T * k; ++p) pairs[p] = p;
    for (int e = 0; e < EL; ++e) experts[e] = e;
    double *y = malloc(sizeof(double) * T * H), *h = malloc(sizeof(double) * T * k * 2 * I);
    double *a = malloc(sizeof(double) * T * k * I), *dA = malloc(sizeof(double) * T * k * I);
    double *dh = malloc(sizeof(double) * T * k * 2 * I), *dW1 = malloc(sizeof(double) * EL * H * 2 * I);
    double *dW2 = malloc(sizeof(double) * EL * I * H), *dx = malloc(sizeof(double) * T * H);
    double *dtw = malloc(sizeof(double) * T * k), *a2 = malloc(sizeof(double) * T * k * I);
    CHECK(oracle_forward(T, H, I, E, e_lo, EL, k, x, idx, w, W1, W2, tokens, T, y));
    CHECK(oracle_l1_rows(T, H, I, E, e_lo, EL, k, x, idx, W1, pairs, T * k, h, a));
    CHECK(oracle_swiglu(T * k, I, h, a2));
    CHECK(oracle_backward_rows(T, H, I, E, e_lo, EL, k, x, idx, w, W1, W2, dy, pairs, T * k, dA, dh));
    CHECK(oracle_swiglu_bwd(T * k, I, h, dA, dh));
    CHECK(oracle_backward(T, H, I, E, e_lo, EL, k, x, idx, w, W1, W2, dy, experts, EL, dW1, dW2));
    CHECK(oracle_backward_tokens(T, H, I, E, e_lo, EL, k, x, idx, w, W1, W2, dy, tokens, T, dx, dtw));

    /* MX: FP8 x and activations, FP4 weights in [EL, N, K] order */
    double *xv = malloc(sizeof(double) * T * H), *w1t = malloc(sizeof(double) * EL * 2 * I * H);
    double *w2t = malloc(sizeof(double) * EL * H * I), *back = malloc(sizeof(double) * EL * 2 * I * H);
    uint8_t *xc = malloc(T * H), *xs = malloc(T * H / 32), *w1c = malloc(EL * 2 * I * H), *w1s = malloc(EL * 2 * I * H / 32);
    uint8_t *w2c = malloc(EL * H * I), *w2s = malloc(EL * H * I / 32), *ac = malloc(T * k * I), *as = malloc(T * k * I / 32);
    for (int i = 0; i < T * H; ++i) xv[i] = 3.0 * next_unit();
    xv[0] = 0.0; xv[1] = -0.0; xv[2] = 1e300; xv[3] = -1e-300;   /* saturating and tiny blocks */
    for (int i = 0; i < EL * 2 * I * H; ++i) w1t[i] = next_unit();
    for (int i = 0; i < EL * H * I; ++i) w2t[i] = next_unit();
    CHECK(oracle_mx_quantize(0, T * H, xv, xc, xs));
    CHECK(oracle_mx_quantize(1, EL * 2 * I * H, w1t, w1c, w1s));
    CHECK(oracle_mx_quantize(1, EL * H * I, w2t, w2c, w2s));
    CHECK(oracle_mx_dequantize(1, EL * 2 * I * H, w1c, w1s, back));
    CHECK(oracle_forward_mx(T, H, I, E, e_lo, EL, k, xc, xs, idx, w, w1c, w1s, w2c, w2s, 10.0, 1, tokens, T, y));
    CHECK(oracle_mx_l1_rows(T, H, I, E, e_lo, EL, k, xc, xs, idx, w1c, w1s, 10.0, pairs, T * k, a));
    CHECK(oracle_mx_quantize(0, T * k * I, a, ac, as));
    int32_t ex_of[T * k];
    for (int p = 0; p < T * k; ++p) ex_of[p] = (idx[p] >= e_lo && idx[p] < e_lo + EL) ? idx[p] - e_lo : -1;
    double* o = malloc(sizeof(double) * T * k * H);
    CHECK(oracle_mx_l2_rows(H, I, EL, w2c, w2s, ex_of, T * k, ac, as, o));
    printf("oracle sanitizer run: ok (R = %lld, dropped %d)\n", (long long)R, meta[1]);
    return 0;
}
