/*
 * CPU oracle for the MoE expert layer on one GPU's share of the experts.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls this file:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * It is the plain definition of what the layer computes, written as slow per-token and
 * per-expert loops in fp64 on the bf16 input values, so that a reader can check it against
 * the pages by eye:
 *   - "Mega MoE" page, Pipeline: x -> dispatch + L1 grouped GEMM (NT) -> SwiGLU ->
 *     L2 grouped GEMM (NT) + combine -> y, where the combine is a top-k weighted
 *     scatter-add that sums the num_topk contributions of each token.
 *   - "Mega MoE" page, Implementation Map: a dispatch prologue builds the routing tables.
 *   - "How Mega MoE Overlaps ..." page, Block-M alignment: each expert's token count is padded
 *     up to the GEMM block size.
 *   - "Mega MoE" page, Pipeline (backward): L2 dgrad, SwiGLU transpose, dW2 with a variable K,
 *     and dW1 (TN) on the recomputed dispatched x.
 *
 * Readings where the pages are silent or leave a step open:
 *   - weights are taken in the logical x @ W layouts W1 [EL, H, 2I] and W2 [EL, I, H];
 *   - columns [0, I) of the L1 output are the gate, [I, 2I) the up projection,
 *     a = silu(gate) * up with silu(g) = g / (1 + exp(-g));
 *   - a pair (t, j) is local when 0 <= id < E and e_lo <= id < e_lo + EL; ids outside
 *     [0, E) are dropped and counted; a duplicated id gives two independent pairs;
 *   - rows inside an expert's segment are in ascending pair order p = t * k + j;
 *   - topk_weights are used as given and applied in the combine;
 *   - y of a token with no local pair is zero;
 *   - the backward gradient of the L2 output row of pair p is w_p * dy[t].
 *
 * All int32 tables use -1 for "no entry".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* Expert slot of a pair, or -1 when the pair is not handled by this GPU. */
static int local_expert(int32_t id, int E, int e_lo, int EL) {
    if (id < 0 || id >= E) return -1;
    int e = id - e_lo;
    return (e >= 0 && e < EL) ? e : -1;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Row capacity of the tables: all T*k pairs local, plus up to BM-1 padding rows per expert,
 * rounded up to a whole block. */
int64_t oracle_rows_capacity(int T, int k, int EL, int BM) {
    int64_t r = (int64_t)T * k + (int64_t)EL * (BM - 1);
    return (r + BM - 1) / BM * BM;
}

/*
 * Routing tables (dispatch prologue; Block-M alignment).
 *   counts[EL]            rows of each local expert
 *   padded_offsets[EL+1]  start row of each expert's segment; segments are padded to BM
 *   row_pair[R_max]       pair id held by each row, -1 for padding and unused rows
 *   pair_row[T*k]         row of each pair, -1 for pairs that are not local
 *   tile_expert[R_max/BM] expert owning each block of BM rows, -1 past the last segment
 *   tok_nloc[T]           number of local pairs of each token
 *   meta[0] = padded row total R, meta[1] = number of ids outside [0, E)
 */
int oracle_route(int T, int k, int E, int e_lo, int EL, int BM, const int32_t* topk_idx,
                 int32_t* counts, int32_t* padded_offsets, int32_t* row_pair, int32_t* pair_row,
                 int32_t* tile_expert, int32_t* tok_nloc, int32_t* meta) {
    if (T < 0 || k <= 0 || E <= 0 || EL <= 0 || e_lo < 0 || BM <= 0) return -1;
    const int64_t npairs = (int64_t)T * k;
    const int64_t R_max = oracle_rows_capacity(T, k, EL, BM);

    int32_t dropped = 0;
    for (int e = 0; e < EL; ++e) counts[e] = 0;
    for (int64_t p = 0; p < npairs; ++p) {
        int32_t id = topk_idx[p];
        if (id < 0 || id >= E) ++dropped;
        int e = local_expert(id, E, e_lo, EL);
        if (e >= 0) ++counts[e];
    }

    padded_offsets[0] = 0;
    for (int e = 0; e < EL; ++e) {
        int32_t padded = (counts[e] + BM - 1) / BM * BM;
        padded_offsets[e + 1] = padded_offsets[e] + padded;
    }

    for (int64_t r = 0; r < R_max; ++r) row_pair[r] = -1;
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)EL);
    if (!next) return -2;
    for (int e = 0; e < EL; ++e) next[e] = padded_offsets[e];
    for (int64_t p = 0; p < npairs; ++p) {
        int e = local_expert(topk_idx[p], E, e_lo, EL);
        if (e < 0) {
            pair_row[p] = -1;
            continue;
        }
        int32_t row = next[e]++;
        row_pair[row] = (int32_t)p;
        pair_row[p] = row;
    }
    free(next);

    for (int64_t m = 0; m < R_max / BM; ++m) {
        int64_t r0 = m * BM;
        tile_expert[m] = -1;
        for (int e = 0; e < EL; ++e)
            if (padded_offsets[e] <= r0 && r0 < padded_offsets[e + 1]) tile_expert[m] = e;
    }

    for (int t = 0; t < T; ++t) {
        int32_t n = 0;
        for (int j = 0; j < k; ++j) n += local_expert(topk_idx[(int64_t)t * k + j], E, e_lo, EL) >= 0;
        tok_nloc[t] = n;
    }
    meta[0] = padded_offsets[EL];
    meta[1] = dropped;
    return 0;
}

/* L1 row of one pair: h[n] = sum_q x[t,q] * W1[e,q,n] for n < 2I (the dispatched token row
 * times the expert's [gate | up] weight). */
static void l1_row(const uint16_t* xrow, const uint16_t* W1e, int H, int I, double* h) {
    const int N = 2 * I;
    for (int n = 0; n < N; ++n) h[n] = 0.0;
    for (int q = 0; q < H; ++q) {
        const double xq = bf16_value(xrow[q]);
        const uint16_t* wrow = W1e + (size_t)q * N;
        for (int n = 0; n < N; ++n) h[n] += xq * bf16_value(wrow[n]);
    }
}

/*
 * Forward for a list of tokens: y[i, :] = sum over local pairs (t_i, j) of
 *   topk_weights[t_i, j] * ( SwiGLU(x[t_i] @ W1[e]) @ W2[e] ).
 * y is [ntok, H] fp64.
 */
int oracle_forward(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x,
                   const int32_t* topk_idx, const float* topk_w, const uint16_t* W1,
                   const uint16_t* W2, const int32_t* tokens, int ntok, double* y) {
    if (H <= 0 || I <= 0 || k <= 0) return -1;
    int err = 0;
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        double* o = (double*)malloc(sizeof(double) * (size_t)H);
        const int ok = h && a && o;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < ntok; ++i) {
            if (!ok) continue;
            {
                const int t = tokens[i];
                double* acc = y + (size_t)i * H;
                for (int m = 0; m < H; ++m) acc[m] = 0.0;
                if (t < 0 || t >= T) continue;
                for (int j = 0; j < k; ++j) {
                    const int e = local_expert(topk_idx[(int64_t)t * k + j], E, e_lo, EL);
                    if (e < 0) continue;
                    l1_row(x + (size_t)t * H, W1 + (size_t)e * H * 2 * I, H, I, h);
                    for (int c = 0; c < I; ++c) a[c] = silu(h[c]) * h[I + c];
                    for (int m = 0; m < H; ++m) o[m] = 0.0;
                    const uint16_t* W2e = W2 + (size_t)e * I * H;
                    for (int c = 0; c < I; ++c) {
                        const uint16_t* wrow = W2e + (size_t)c * H;
                        for (int m = 0; m < H; ++m) o[m] += a[c] * bf16_value(wrow[m]);
                    }
                    const double w = (double)topk_w[(int64_t)t * k + j];
                    for (int m = 0; m < H; ++m) acc[m] += w * o[m];
                }
            }
        }
        free(h);
        free(a);
        free(o);
    }
    return err;
}

/* L1 output (pre-activation [gate | up], [npairs_list, 2I]) and its SwiGLU ([.., I]) for a
 * list of pair ids; rows of non-local pairs are zero. */
int oracle_l1_rows(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x,
                   const int32_t* topk_idx, const uint16_t* W1, const int32_t* pairs, int np,
                   double* h_out, double* a_out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < np; ++i) {
        double* h = h_out + (size_t)i * 2 * I;
        double* a = a_out + (size_t)i * I;
        const int64_t p = pairs[i];
        const int e = (p >= 0 && p < (int64_t)T * k) ? local_expert(topk_idx[p], E, e_lo, EL) : -1;
        if (e < 0) {
            for (int n = 0; n < 2 * I; ++n) h[n] = 0.0;
            for (int c = 0; c < I; ++c) a[c] = 0.0;
            continue;
        }
        l1_row(x + (size_t)(p / k) * H, W1 + (size_t)e * H * 2 * I, H, I, h);
        for (int c = 0; c < I; ++c) a[c] = silu(h[c]) * h[I + c];
    }
    return 0;
}

/* SwiGLU on given [gate | up] rows (real values, fp64): a[r, c] = silu(hgu[r, c]) * hgu[r, I + c]. */
int oracle_swiglu(int64_t nrows, int I, const double* hgu, double* a) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r)
        for (int c = 0; c < I; ++c)
            a[r * I + c] = silu(hgu[r * 2 * I + c]) * hgu[r * 2 * I + I + c];
    return 0;
}

/* SwiGLU backward on given [gate | up] rows (real values, fp64) and an upstream gradient
 * da [nrows, I] (fp64): with s = sigmoid(g): dgate = da * up * s * (1 + g * (1 - s)),
 * dup = da * g * s. */
int oracle_swiglu_bwd(int64_t nrows, int I, const double* hgu, const double* da,
                      double* dhgu) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r)
        for (int c = 0; c < I; ++c) {
            const double g = hgu[r * 2 * I + c];
            const double u = hgu[r * 2 * I + I + c];
            const double d = da[r * I + c];
            const double s = 1.0 / (1.0 + exp(-g));
            dhgu[r * 2 * I + c] = d * u * s * (1.0 + g * (1.0 - s));
            dhgu[r * 2 * I + I + c] = d * g * s;
        }
    return 0;
}

/* Backward of one pair: from the upstream gradient dy[t], the L2 dgrad
 * dA[c] = sum_m (w_p * dy[t, m]) * W2[e, c, m], then the SwiGLU transpose into dHgu [2I]. */
static void pair_backward(const uint16_t* dyrow, double w, const uint16_t* W2e, int H, int I,
                          const double* h, double* dO, double* dA, double* dhgu) {
    for (int m = 0; m < H; ++m) dO[m] = w * bf16_value(dyrow[m]);
    for (int c = 0; c < I; ++c) {
        const uint16_t* wrow = W2e + (size_t)c * H;
        double s = 0.0;
        for (int m = 0; m < H; ++m) s += dO[m] * bf16_value(wrow[m]);
        dA[c] = s;
    }
    for (int c = 0; c < I; ++c) {
        const double g = h[c], u = h[I + c];
        const double sg = 1.0 / (1.0 + exp(-g));
        dhgu[c] = dA[c] * u * sg * (1.0 + g * (1.0 - sg));
        dhgu[I + c] = dA[c] * g * sg;
    }
}

/* Per-pair backward intermediates for a list of pair ids: dA [np, I], dHgu [np, 2I]. */
int oracle_backward_rows(int T, int H, int I, int E, int e_lo, int EL, int k,
                         const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                         const uint16_t* W1, const uint16_t* W2, const uint16_t* dy,
                         const int32_t* pairs, int np, double* dA_out, double* dhgu_out) {
    int err = 0;
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        double* dO = (double*)malloc(sizeof(double) * (size_t)H);
        const int ok = h && dO;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < np; ++i) {
            if (!ok) continue;
            {
                double* dA = dA_out + (size_t)i * I;
                double* dhgu = dhgu_out + (size_t)i * 2 * I;
                const int64_t p = pairs[i];
                const int e = (p >= 0 && p < (int64_t)T * k) ? local_expert(topk_idx[p], E, e_lo, EL) : -1;
                if (e < 0) {
                    for (int c = 0; c < I; ++c) dA[c] = 0.0;
                    for (int n = 0; n < 2 * I; ++n) dhgu[n] = 0.0;
                    continue;
                }
                const int64_t t = p / k;
                l1_row(x + (size_t)t * H, W1 + (size_t)e * H * 2 * I, H, I, h);
                pair_backward(dy + (size_t)t * H, (double)topk_w[p], W2 + (size_t)e * I * H, H, I,
                              h, dO, dA, dhgu);
            }
        }
        free(h);
        free(dO);
    }
    return err;
}

/*
 * Weight gradients of a list of local experts (variable K: an expert's K is its row count).
 *   dW2[e, c, m] = sum over pairs p of e of a_p[c] * (w_p * dy[t_p, m])      [I, H]
 *   dW1[e, q, n] = sum over pairs p of e of x[t_p, q] * dHgu_p[n]           [H, 2I]
 * Pairs are accumulated in ascending pair order; an expert with no pair gets exact zeros.
 * Outputs are [nexp, H, 2I] and [nexp, I, H] fp64, in the logical weight layouts.
 */
int oracle_backward(int T, int H, int I, int E, int e_lo, int EL, int k, const uint16_t* x,
                    const int32_t* topk_idx, const float* topk_w, const uint16_t* W1,
                    const uint16_t* W2, const uint16_t* dy, const int32_t* experts, int nexp,
                    double* dW1, double* dW2) {
    int err = 0;
    const int64_t npairs = (int64_t)T * k;
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        double* dO = (double*)malloc(sizeof(double) * (size_t)H);
        double* dA = (double*)malloc(sizeof(double) * (size_t)I);
        double* dhgu = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        const int ok = h && a && dO && dA && dhgu;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int s = 0; s < nexp; ++s) {
            if (!ok) continue;
            {
                const int e = experts[s];
                double* g1 = dW1 + (size_t)s * H * 2 * I;
                double* g2 = dW2 + (size_t)s * I * H;
                memset(g1, 0, sizeof(double) * (size_t)H * 2 * I);
                memset(g2, 0, sizeof(double) * (size_t)I * H);
                if (e < 0 || e >= EL) continue;
                for (int64_t p = 0; p < npairs; ++p) {
                    if (local_expert(topk_idx[p], E, e_lo, EL) != e) continue;
                    const int64_t t = p / k;
                    const uint16_t* xrow = x + (size_t)t * H;
                    l1_row(xrow, W1 + (size_t)e * H * 2 * I, H, I, h);
                    for (int c = 0; c < I; ++c) a[c] = silu(h[c]) * h[I + c];
                    pair_backward(dy + (size_t)t * H, (double)topk_w[p], W2 + (size_t)e * I * H,
                                  H, I, h, dO, dA, dhgu);
                    for (int c = 0; c < I; ++c) {
                        double* row = g2 + (size_t)c * H;
                        for (int m = 0; m < H; ++m) row[m] += a[c] * dO[m];
                    }
                    for (int q = 0; q < H; ++q) {
                        const double xq = bf16_value(xrow[q]);
                        double* row = g1 + (size_t)q * 2 * I;
                        for (int n = 0; n < 2 * I; ++n) row[n] += xq * dhgu[n];
                    }
                }
            }
        }
        free(h);
        free(a);
        free(dO);
        free(dA);
        free(dhgu);
    }
    return err;
}

/*
 * Token-side gradients of a list of tokens ("Mega MoE" page, Pipeline, backward: the
 * conjugate of dispatch + L1 is an L1 dgrad whose rows are summed back to token order; the
 * routing weights get the gradient of the weighted scatter-add).  For token t:
 *   dx[t, q]      = sum over local pairs p = (t, j) of sum_n W1[e, q, n] * dHgu_p[n]
 *   dtopk_w[t, j] = sum_m dy[t, m] * o_p[m]      for a local pair, where o_p is the L2 output
 *                   row SwiGLU(x[t] @ W1[e]) @ W2[e] before weighting; 0 for a pair that is not
 *                   local (this GPU's partial of the gradient, like y).
 * dHgu_p is the per-pair gradient of pair_backward (w_p * dy[t] through L2 and SwiGLU).
 * dx is [ntok, H] and dtopk_w [ntok, k], fp64.
 */
int oracle_backward_tokens(int T, int H, int I, int E, int e_lo, int EL, int k,
                           const uint16_t* x, const int32_t* topk_idx, const float* topk_w,
                           const uint16_t* W1, const uint16_t* W2, const uint16_t* dy,
                           const int32_t* tokens, int ntok, double* dx, double* dtopk_w) {
    if (H <= 0 || I <= 0 || k <= 0) return -1;
    int err = 0;
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        double* o = (double*)malloc(sizeof(double) * (size_t)H);
        double* dO = (double*)malloc(sizeof(double) * (size_t)H);
        double* dA = (double*)malloc(sizeof(double) * (size_t)I);
        double* dhgu = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        const int ok = h && a && o && dO && dA && dhgu;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < ntok; ++i) {
            if (!ok) continue;
            {
                const int t = tokens[i];
                double* gx = dx + (size_t)i * H;
                double* gw = dtopk_w + (size_t)i * k;
                for (int q = 0; q < H; ++q) gx[q] = 0.0;
                for (int j = 0; j < k; ++j) gw[j] = 0.0;
                if (t < 0 || t >= T) continue;
                const uint16_t* xrow = x + (size_t)t * H;
                const uint16_t* dyrow = dy + (size_t)t * H;
                for (int j = 0; j < k; ++j) {
                    const int e = local_expert(topk_idx[(int64_t)t * k + j], E, e_lo, EL);
                    if (e < 0) continue;
                    const uint16_t* W1e = W1 + (size_t)e * H * 2 * I;
                    const uint16_t* W2e = W2 + (size_t)e * I * H;
                    l1_row(xrow, W1e, H, I, h);
                    for (int c = 0; c < I; ++c) a[c] = silu(h[c]) * h[I + c];
                    for (int m = 0; m < H; ++m) o[m] = 0.0;
                    for (int c = 0; c < I; ++c) {
                        const uint16_t* wrow = W2e + (size_t)c * H;
                        for (int m = 0; m < H; ++m) o[m] += a[c] * bf16_value(wrow[m]);
                    }
                    double s = 0.0;
                    for (int m = 0; m < H; ++m) s += bf16_value(dyrow[m]) * o[m];
                    gw[j] = s;
                    pair_backward(dyrow, (double)topk_w[(int64_t)t * k + j], W2e, H, I, h, dO,
                                  dA, dhgu);
                    for (int q = 0; q < H; ++q) {
                        const uint16_t* wrow = W1e + (size_t)q * 2 * I;
                        double d = 0.0;
                        for (int n = 0; n < 2 * I; ++n) d += bf16_value(wrow[n]) * dhgu[n];
                        gx[q] += d;
                    }
                }
            }
        }
        free(h);
        free(a);
        free(o);
        free(dO);
        free(dA);
        free(dhgu);
    }
    return err;
}

/*
 * ---------------------------------------------------------------------------------------------
 * MX variant: FP8 activations and FP4 weights with power-of-two block scales ("How Mega MoE
 * Overlaps ..." page, Code Example: activations cast per token to FP8 with UE8M0 scale factors
 * over groups of 32 along K; weights transformed to FP4; the fused call takes an activation clamp
 * of 10).  Readings where the page only names the calls:
 *   - A block of 32 consecutive values along K shares one scale 2^E, E an integer in [-127, 127]
 *     (the UE8M0 byte is E + 127).  E is the smallest integer with amax <= fmax * 2^E, where amax is
 *     the block's largest magnitude and fmax the element format's largest value (448 for FP8 E4M3,
 *     6 for FP4 E2M1), so no element saturates; a block of zeros takes E = 0.
 *   - Elements are v / 2^E rounded to the nearest value of the format, ties to the even mantissa
 *     (OCP FP8 E4M3: 1 sign, 4 exponent bits of bias 7, 3 mantissa bits, subnormals, largest 448;
 *     OCP FP4 E2M1: 1 sign, 2 exponent bits of bias 1, 1 mantissa bit, values 0, 0.5, 1, 1.5, 2,
 *     3, 4, 6).  A value that rounds to zero keeps its sign.
 *   - The SwiGLU inputs are clamped: gate to at most `clamp`, up to [-clamp, clamp].
 *   - The SwiGLU output is cast again, per row and group of 32 along I, to FP8 for L2.
 * ---------------------------------------------------------------------------------------------
 */
static double pow2i(int e) { return ldexp(1.0, e); }

/* Value of exponent field e_field and mantissa field m of a format with `mbits` mantissa bits and
 * exponent bias `bias` (e_field 0: subnormal). */
static double fmt_value(int e_field, int m, int mbits, int bias) {
    const double frac = (double)m / (double)(1 << mbits);
    return e_field == 0 ? frac * pow2i(1 - bias) : (1.0 + frac) * pow2i(e_field - bias);
}

/* Nearest code (sign-magnitude: sign << (ebits + mbits) | e << mbits | m) of a finite value v whose
 * magnitude does not exceed the format's largest value; ties to the even mantissa. */
static int fmt_encode(double v, int ebits, int mbits, int bias, double vmax) {
    const int sign = v < 0 || (v == 0 && signbit(v));
    const double a = fabs(v) > vmax ? vmax : fabs(v);
    int best = 0;
    double best_err = INFINITY;
    const int ncode = 1 << (ebits + mbits);
    for (int c = 0; c < ncode; ++c) {
        const int e = c >> mbits, m = c & ((1 << mbits) - 1);
        const double x = fmt_value(e, m, mbits, bias);
        if (x > vmax) continue;
        const double err = fabs(x - a);
        /* codes are scanned in increasing value, so an equal error is the upper neighbour: it wins
         * the tie only when its mantissa is even */
        if (err < best_err || (err == best_err && (m & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (sign << (ebits + mbits)) | best;
}

static double fmt_decode(int code, int ebits, int mbits, int bias) {
    const int mag = code & ((1 << (ebits + mbits)) - 1);
    const double x = fmt_value(mag >> mbits, mag & ((1 << mbits) - 1), mbits, bias);
    return (code >> (ebits + mbits)) & 1 ? -x : x;
}

/* Block exponent: the smallest E with amax <= vmax * 2^E, in [-127, 127]; 0 for amax == 0. */
static int block_exponent(double amax, double vmax) {
    if (!(amax > 0)) return 0;
    int E = (int)ceil(log2(amax / vmax));
    while (E > -127 && amax <= vmax * pow2i(E - 1)) --E;   /* exact correction of log2 rounding */
    while (E < 127 && amax > vmax * pow2i(E)) ++E;
    return E < -127 ? -127 : (E > 127 ? 127 : E);
}

/* fmt: 0 = FP8 E4M3, 1 = FP4 E2M1.  Quantizes n values (n a multiple of 32) in blocks of 32:
 * codes[n] (one code per byte), scales[n / 32] (UE8M0 bytes, E + 127). */
int oracle_mx_quantize(int fmt, int64_t n, const double* v, uint8_t* codes, uint8_t* scales) {
    const int ebits = fmt == 0 ? 4 : 2, mbits = fmt == 0 ? 3 : 1, bias = fmt == 0 ? 7 : 1;
    const double vmax = fmt == 0 ? 448.0 : 6.0;
    if (n % 32) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < n / 32; ++b) {
        double amax = 0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[b * 32 + i]));
        const int E = block_exponent(amax, vmax);
        scales[b] = (uint8_t)(E + 127);
        for (int i = 0; i < 32; ++i)
            codes[b * 32 + i] = (uint8_t)fmt_encode(v[b * 32 + i] / pow2i(E), ebits, mbits, bias, vmax);
    }
    return 0;
}

/* Value of a code times its block scale. */
int oracle_mx_dequantize(int fmt, int64_t n, const uint8_t* codes, const uint8_t* scales, double* v) {
    const int ebits = fmt == 0 ? 4 : 2, mbits = fmt == 0 ? 3 : 1, bias = fmt == 0 ? 7 : 1;
    if (n % 32) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        v[i] = fmt_decode(codes[i], ebits, mbits, bias) * pow2i((int)scales[i / 32] - 127);
    return 0;
}

/*
 * MX forward for a list of tokens, on already quantized inputs:
 *   x_codes [T, H] FP8 codes with x_scales [T, H/32] (blocks along H);
 *   w1_codes [EL, 2I, H] FP4 codes (one per byte) with w1_scales [EL, 2I, H/32]: column n of the
 *     [gate | up] output, blocks along the reduction index H;
 *   w2_codes [EL, H, I] with w2_scales [EL, H, I/32]: output column m, blocks along I.
 *   h = x . W1 on the dequantized values; a = silu(min(g, clamp)) * clamp(u, -clamp, clamp);
 *   a cast to FP8 per group of 32 along I when quant_act is nonzero; o = a . W2;
 *   y[t] = sum over local pairs of w * o.  clamp <= 0 disables the clamp.  y is [ntok, H] fp64.
 */
int oracle_forward_mx(int T, int H, int I, int E, int e_lo, int EL, int k, const uint8_t* x_codes,
                      const uint8_t* x_scales, const int32_t* topk_idx, const float* topk_w,
                      const uint8_t* w1_codes, const uint8_t* w1_scales, const uint8_t* w2_codes,
                      const uint8_t* w2_scales, double clamp, int quant_act, const int32_t* tokens,
                      int ntok, double* y) {
    if (H % 32 || I % 32 || k <= 0) return -1;
    int err = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* wr = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
        double* h = (double*)malloc(sizeof(double) * 2 * (size_t)I);
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        uint8_t* ac = (uint8_t*)malloc((size_t)I);
        uint8_t* as = (uint8_t*)malloc((size_t)I / 32);
        double* o = (double*)malloc(sizeof(double) * (size_t)H);
        const int ok = xr && wr && h && a && ac && as && o;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < ntok; ++i) {
            if (!ok) continue;
            {
                const int t = tokens[i];
                double* acc = y + (size_t)i * H;
                for (int m = 0; m < H; ++m) acc[m] = 0.0;
                if (t < 0 || t >= T) continue;
                oracle_mx_dequantize(0, H, x_codes + (size_t)t * H, x_scales + (size_t)t * (H / 32), xr);
                for (int j = 0; j < k; ++j) {
                    const int e = local_expert(topk_idx[(int64_t)t * k + j], E, e_lo, EL);
                    if (e < 0) continue;
                    for (int n = 0; n < 2 * I; ++n) {
                        const size_t row = ((size_t)e * 2 * I + n);
                        oracle_mx_dequantize(1, H, w1_codes + row * H, w1_scales + row * (H / 32), wr);
                        double s = 0.0;
                        for (int q = 0; q < H; ++q) s += xr[q] * wr[q];
                        h[n] = s;
                    }
                    for (int c = 0; c < I; ++c) {
                        double g = h[c], u = h[I + c];
                        if (clamp > 0) {
                            if (g > clamp) g = clamp;
                            if (u > clamp) u = clamp;
                            if (u < -clamp) u = -clamp;
                        }
                        a[c] = silu(g) * u;
                    }
                    if (quant_act) {
                        oracle_mx_quantize(0, I, a, ac, as);
                        oracle_mx_dequantize(0, I, ac, as, a);
                    }
                    for (int m = 0; m < H; ++m) {
                        const size_t row = ((size_t)e * H + m);
                        oracle_mx_dequantize(1, I, w2_codes + row * I, w2_scales + row * (I / 32), wr);
                        double s = 0.0;
                        for (int c = 0; c < I; ++c) s += a[c] * wr[c];
                        o[m] = s;
                    }
                    const double w = (double)topk_w[(int64_t)t * k + j];
                    for (int m = 0; m < H; ++m) acc[m] += w * o[m];
                }
            }
        }
        free(xr);
        free(wr);
        free(h);
        free(a);
        free(ac);
        free(as);
        free(o);
    }
    return err;
}

/* MX L1 rows for a list of pair ids: a = silu(min(g, clamp)) * clamp(u, -clamp, clamp) of the
 * dequantized x row times the dequantized W1 (before the FP8 cast of the activation); [np, I] fp64,
 * zero for a pair that is not local.  Layouts as in oracle_forward_mx. */
int oracle_mx_l1_rows(int T, int H, int I, int E, int e_lo, int EL, int k, const uint8_t* x_codes,
                      const uint8_t* x_scales, const int32_t* topk_idx, const uint8_t* w1_codes,
                      const uint8_t* w1_scales, double clamp, const int32_t* pairs, int np, double* a_out) {
    if (H % 32 || I % 32 || k <= 0) return -1;
    int err = 0;
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* wr = (double*)malloc(sizeof(double) * (size_t)H);
        const int ok = xr && wr;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < np; ++i) {
            if (!ok) continue;
            {
                double* a = a_out + (size_t)i * I;
                for (int c = 0; c < I; ++c) a[c] = 0.0;
                const int64_t p = pairs[i];
                const int e = (p >= 0 && p < (int64_t)T * k) ? local_expert(topk_idx[p], E, e_lo, EL) : -1;
                if (e < 0) continue;
                const int64_t t = p / k;
                oracle_mx_dequantize(0, H, x_codes + (size_t)t * H, x_scales + (size_t)t * (H / 32), xr);
                for (int c = 0; c < I; ++c) {
                    double h2[2];
                    for (int half = 0; half < 2; ++half) {
                        const size_t row = (size_t)e * 2 * I + (size_t)half * I + c;
                        oracle_mx_dequantize(1, H, w1_codes + row * H, w1_scales + row * (H / 32), wr);
                        double s = 0.0;
                        for (int q = 0; q < H; ++q) s += xr[q] * wr[q];
                        h2[half] = s;
                    }
                    double g = h2[0], u = h2[1];
                    if (clamp > 0) {
                        if (g > clamp) g = clamp;
                        if (u > clamp) u = clamp;
                        if (u < -clamp) u = -clamp;
                    }
                    a[c] = silu(g) * u;
                }
            }
        }
        free(xr);
        free(wr);
    }
    return err;
}

/* MX L2 rows: o = (dequantized FP8 activation row) . (dequantized W2 of expert experts[i]) for np
 * given activation rows (codes [np, I], scales [np, I/32]); [np, H] fp64, unweighted; a row whose
 * expert is outside [0, EL) is zero. */
int oracle_mx_l2_rows(int H, int I, int EL, const uint8_t* w2_codes, const uint8_t* w2_scales,
                      const int32_t* experts, int np, const uint8_t* act_codes, const uint8_t* act_scales,
                      double* o_out) {
    if (H % 32 || I % 32) return -1;
    int err = 0;
#pragma omp parallel
    {
        double* ar = (double*)malloc(sizeof(double) * (size_t)I);
        double* wr = (double*)malloc(sizeof(double) * (size_t)I);
        const int ok = ar && wr;
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < np; ++i) {
            if (!ok) continue;
            {
                double* o = o_out + (size_t)i * H;
                for (int m = 0; m < H; ++m) o[m] = 0.0;
                const int e = experts[i];
                if (e < 0 || e >= EL) continue;
                oracle_mx_dequantize(0, I, act_codes + (size_t)i * I, act_scales + (size_t)i * (I / 32), ar);
                for (int m = 0; m < H; ++m) {
                    const size_t row = (size_t)e * H + m;
                    oracle_mx_dequantize(1, I, w2_codes + row * I, w2_scales + row * (I / 32), wr);
                    double s = 0.0;
                    for (int c = 0; c < I; ++c) s += ar[c] * wr[c];
                    o[m] = s;
                }
            }
        }
        free(ar);
        free(wr);
    }
    return err;
}
