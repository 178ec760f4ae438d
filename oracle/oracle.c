/*
 * oracle.c - plain, slow, obviously correct CPU reference for the MoE expert-layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library.  The HIP library never links, includes or calls it, and the two share
 * no code: this file has its own storage decoders, routing, FFN and MX quantiser.
 *
 * What it computes is the expert part of the EP-MC2 forward described on the page
 * "NPU Training Operators - MC2", section 执行路径 (execution path), on one device and without the
 * All-to-All exchange:
 *   step 1   flatten the tokens to [T, H];
 *   step 2   count the slots routed to each expert (histc with E bins over [0, E));
 *   step 6   permute token rows into expert-contiguous order;
 *   step 7   grouped matmul with the fc1 weights (gate and up projections);
 *   step 8   SwiGLU;
 *   step 9   grouped matmul with the fc2 (down) weights;
 *   step 10  unpermute: each token sums its k expert outputs weighted by the routing probabilities.
 * The operand set follows mc2_fused_expert on the page "MC2 通算融合" (hwcomputing.csdn.net),
 * section 用法: x [tokens, hidden], up/gate weights [E, hidden, ff], down weights [E, ff, hidden],
 * expert_ids [tokens, topk]; the probabilities come from step 10 above.
 *
 * Arithmetic: every stored input value (fp32, bf16, or OCP-MX E4M3 element times its E8M0 block
 * scale) is widened exactly to double; every sum is a double sum in ascending index order.
 * The one non-exact step is the MX variant's encoding of the SwiGLU output h before fc2, which
 * follows OCP Microscaling Formats v1.0 step by step (see oracle_mx_quantize).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_MXFP8 = 2 };

/* ------------------------------------------------------------------------------------------------
 * Storage decoders (exact).
 * ---------------------------------------------------------------------------------------------- */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3 (the "FN" variant used by OCP-MX): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals at exponent field 0, no infinities, S.1111.111 is NaN, max normal 448. */
double oracle_e4m3_value(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int ef = (c >> 3) & 0xF;
    int mf = c & 7;
    double mag;
    if (ef == 0xF && mf == 7)
        return NAN;
    if (ef == 0)
        mag = ldexp((double)mf, -9);              /* (m / 8) * 2^(1 - 7) */
    else
        mag = ldexp(8.0 + mf, ef - 7 - 3);        /* (1 + m / 8) * 2^(e - 7) */
    return sign ? -mag : mag;
}

/* E8M0 shared scale: 2^(code - 127); code 255 is NaN. */
double oracle_e8m0_value(uint8_t s)
{
    if (s == 0xFF)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

/* Decode a row-major [rows, cols] matrix.  MX blocks run along the contraction axis:
 *   blocks_along_rows = 1 : scale is [rows/32, cols]   (weights [K, N], blocks along K)
 *   blocks_along_rows = 0 : scale is [rows, cols/32]   (activations [M, K], blocks along K)
 * MX values are the E4M3 element value times the E8M0 block scale (both exact in double). */
static void decode_matrix(int dtype, const void* data, const uint8_t* scale, int64_t rows,
                          int64_t cols, int blocks_along_rows, double* out)
{
    double e4m3[256], e8m0[256];
    int64_t r;
    for (int i = 0; i < 256; ++i) {
        e4m3[i] = oracle_e4m3_value((uint8_t)i);
        e8m0[i] = oracle_e8m0_value((uint8_t)i);
    }
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const int64_t i = r * cols + c;
            switch (dtype) {
            case O_F32:
                out[i] = (double)((const float*)data)[i];
                break;
            case O_BF16:
                out[i] = oracle_bf16_value(((const uint16_t*)data)[i]);
                break;
            default: {
                const uint8_t s = blocks_along_rows ? scale[(r / 32) * cols + c]
                                                    : scale[r * (cols / 32) + c / 32];
                out[i] = e4m3[((const uint8_t*)data)[i]] * e8m0[s];
            }
            }
        }
}

/* ------------------------------------------------------------------------------------------------
 * OCP-MX encoding (MX variant of the h operand; Microscaling Formats v1.0, E4M3 elements).
 * ---------------------------------------------------------------------------------------------- */

/* Nearest E4M3 code to v: scan the 127 finite non-negative codes (values increase with the code),
 * keep the closest, and on an exact tie keep the even code (even mantissa).  Magnitudes above the
 * largest finite value 448 saturate to 448.  The sign bit is copied from v. */
uint8_t oracle_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    int best = 0;
    double best_d = a;                             /* distance to code 0 (value 0) */
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(oracle_e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* Encode `nblocks` consecutive blocks of 32 values.  Shared scale X = 2^(floor(log2(amax)) - 8),
 * 8 being the exponent of E4M3's largest normal (448 = 1.75 * 2^8); the exponent is clamped to the
 * E8M0 range [-127, 127] and an all-zero block takes -127.  Elements are v / X encoded as above. */
void oracle_mx_quantize(const double* v, int64_t nblocks, uint8_t* codes, uint8_t* scales)
{
    for (int64_t b = 0; b < nblocks; ++b) {
        const double* blk = v + b * 32;
        double amax = 0.0;
        int e, ex;
        for (int i = 0; i < 32; ++i)
            if (fabs(blk[i]) > amax)
                amax = fabs(blk[i]);
        if (amax > 0.0) {
            frexp(amax, &ex);                      /* amax = m * 2^ex, 0.5 <= m < 1 */
            e = (ex - 1) - 8;
        } else {
            e = -127;
        }
        if (e < -127) e = -127;
        if (e > 127) e = 127;
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i)
            codes[b * 32 + i] = oracle_e4m3_encode(ldexp(blk[i], -e));
    }
}

/* ------------------------------------------------------------------------------------------------
 * Routing: histc counts, offsets, stable per-expert slot list.
 * NPU Training Operators - MC2, 执行路径 step 2 (counts), step 6 (permute), step 10 (the inverse
 * map used by unpermute); 迁移检查 requires every id to lie in [0, E).
 * ---------------------------------------------------------------------------------------------- */

/* Returns 0, or -1 if an id is out of range (nothing written then). */
int oracle_route(const int32_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* pos)
{
    const int64_t M = T * k;                       /* slots, flattened token-major: s = t*k + j */
    int32_t* cursor;
    for (int64_t s = 0; s < M; ++s)
        if (ids[s] < 0 || ids[s] >= E)
            return -1;
    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t s = 0; s < M; ++s)
        counts[ids[s]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t s = 0; s < M; ++s) {             /* ascending s: stable within each expert */
        int32_t p = cursor[ids[s]]++;
        perm[p] = (int32_t)s;
        pos[s] = p;
    }
    free(cursor);
    return 0;
}

/* Permute, step 6: row p of the output is token perm[p] / k's row (a byte copy). */
void oracle_permute(const void* x, int64_t row_bytes, const int32_t* perm, int64_t M, int64_t k,
                    void* x_perm)
{
    for (int64_t p = 0; p < M; ++p)
        memcpy((char*)x_perm + p * row_bytes, (const char*)x + (int64_t)(perm[p] / k) * row_bytes,
               (size_t)row_bytes);
}

/* ------------------------------------------------------------------------------------------------
 * Expert FFN on a set of rows that all use one expert (steps 7-9).
 *   g = x Wg,  u = x Wu  (sums over h ascending),  a = silu(g) * u with silu(z) = z / (1 + e^-z),
 *   [MX variant: a is OCP-MX encoded in blocks of 32 along F and decoded again],
 *   y = a Wd (sum over f ascending).
 * ---------------------------------------------------------------------------------------------- */
static void expert_ffn(int64_t R, int64_t H, int64_t F, const double* x, const double* wg,
                       const double* wu, const double* wd, int h_mx, double* a, double* y)
{
    enum { CB = 64 };                              /* output columns per parallel task */
    int64_t c0;
    /* Each accumulator g[r][f] (u, y likewise) is a sum over the contraction index in ascending
     * order starting from 0; the loops below only choose which accumulators advance together. */
#pragma omp parallel for schedule(dynamic)
    for (c0 = 0; c0 < F; c0 += CB) {
        const int64_t nc = F - c0 < CB ? F - c0 : CB;
        double* g = (double*)calloc((size_t)(R * CB), sizeof(double));
        double* u = (double*)calloc((size_t)(R * CB), sizeof(double));
        for (int64_t h = 0; h < H; ++h) {
            const double* wgr = wg + h * F + c0;
            const double* wur = wu + h * F + c0;
            for (int64_t r = 0; r < R; ++r) {
                const double xv = x[r * H + h];
                for (int64_t f = 0; f < nc; ++f) {
                    g[r * CB + f] += xv * wgr[f];
                    u[r * CB + f] += xv * wur[f];
                }
            }
        }
        for (int64_t r = 0; r < R; ++r)
            for (int64_t f = 0; f < nc; ++f) {
                const double gv = g[r * CB + f];
                a[r * F + c0 + f] = gv / (1.0 + exp(-gv)) * u[r * CB + f];
            }
        free(g);
        free(u);
    }
    if (h_mx) {
        int64_t nb = R * F / 32;
        uint8_t* q = (uint8_t*)malloc((size_t)(R * F));
        uint8_t* s = (uint8_t*)malloc((size_t)nb);
        oracle_mx_quantize(a, nb, q, s);
        for (int64_t i = 0; i < R * F; ++i)
            a[i] = oracle_e4m3_value(q[i]) * oracle_e8m0_value(s[i / 32]);
        free(q);
        free(s);
    }
#pragma omp parallel for schedule(dynamic)
    for (c0 = 0; c0 < H; c0 += CB) {
        const int64_t nc = H - c0 < CB ? H - c0 : CB;
        double* acc = (double*)calloc((size_t)(R * CB), sizeof(double));
        for (int64_t f = 0; f < F; ++f) {
            const double* wdr = wd + f * H + c0;
            for (int64_t r = 0; r < R; ++r) {
                const double av = a[r * F + f];
                for (int64_t c = 0; c < nc; ++c)
                    acc[r * CB + c] += av * wdr[c];
            }
        }
        for (int64_t r = 0; r < R; ++r)
            for (int64_t c = 0; c < nc; ++c)
                y[r * H + c0 + c] = acc[r * CB + c];
        free(acc);
    }
}

/* FFN of n rows, row i through expert row_expert[i].  `x` holds n stored rows [n, H] (+ MX scales
 * [n, H/32]).  Weights are all E experts in storage format: w_gate/w_up [E, H, F] (MX scales
 * [E, H/32, F]), w_down [E, F, H] (MX scales [E, F/32, H]).  Output y is double [n, H].
 * Each expert's weights are decoded once.  Returns 0, or -1 on a bad expert index. */
int oracle_ffn_rows(int dtype, int64_t n, int64_t H, int64_t F, int64_t E, const void* x,
                    const uint8_t* x_scale, const int32_t* row_expert, const void* w_gate,
                    const uint8_t* wg_scale, const void* w_up, const uint8_t* wu_scale,
                    const void* w_down, const uint8_t* wd_scale, double* y)
{
    const int64_t esz = dtype == O_F32 ? 4 : dtype == O_BF16 ? 2 : 1;
    double *wg, *wu, *wd, *xr, *a, *yr;
    int64_t* rows;
    for (int64_t i = 0; i < n; ++i)
        if (row_expert[i] < 0 || row_expert[i] >= E)
            return -1;
    wg = (double*)malloc(sizeof(double) * (size_t)(H * F));
    wu = (double*)malloc(sizeof(double) * (size_t)(H * F));
    wd = (double*)malloc(sizeof(double) * (size_t)(F * H));
    xr = (double*)malloc(sizeof(double) * (size_t)(n * H + 1));
    a = (double*)malloc(sizeof(double) * (size_t)(n * F + 1));
    yr = (double*)malloc(sizeof(double) * (size_t)(n * H + 1));
    rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
    for (int64_t e = 0; e < E; ++e) {
        int64_t R = 0;
        for (int64_t i = 0; i < n; ++i)
            if (row_expert[i] == e)
                rows[R++] = i;
        if (R == 0)
            continue;
        decode_matrix(dtype, (const char*)w_gate + e * H * F * esz,
                      wg_scale ? wg_scale + e * (H / 32) * F : NULL, H, F, 1, wg);
        decode_matrix(dtype, (const char*)w_up + e * H * F * esz,
                      wu_scale ? wu_scale + e * (H / 32) * F : NULL, H, F, 1, wu);
        decode_matrix(dtype, (const char*)w_down + e * F * H * esz,
                      wd_scale ? wd_scale + e * (F / 32) * H : NULL, F, H, 1, wd);
        for (int64_t r = 0; r < R; ++r)
            decode_matrix(dtype, (const char*)x + rows[r] * H * esz,
                          x_scale ? x_scale + rows[r] * (H / 32) : NULL, 1, H, 0, xr + r * H);
        expert_ffn(R, H, F, xr, wg, wu, wd, dtype == O_MXFP8, a, yr);
        for (int64_t r = 0; r < R; ++r)
            memcpy(y + rows[r] * H, yr + r * H, sizeof(double) * (size_t)H);
    }
    free(wg); free(wu); free(wd); free(xr); free(a); free(yr); free(rows);
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Whole layer, in the pages' order: route -> permute -> FFN over the permuted rows (optionally in
 * chunks of `chunk` rows, processed in chunk order) -> weighted unpermute.
 * `chunk` = 0 means one chunk.  The M-axis split into fixed-size row chunks is the one on the page
 * "MC2 通算融合架构总览", §6 切分策略; the claim that splitting leaves the result unchanged is on the
 * page "MC2 通算融合", section 流水线设计 (third stage).
 * Outputs: out double [T, H] plus the route results.  Returns 0 or -1 (bad ids / arguments).
 * ---------------------------------------------------------------------------------------------- */
int oracle_forward(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                   const void* x, const uint8_t* x_scale, const void* w_gate, const uint8_t* wg_scale,
                   const void* w_up, const uint8_t* wu_scale, const void* w_down,
                   const uint8_t* wd_scale, const int32_t* ids, const float* probs, int64_t chunk,
                   double* out, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos)
{
    const int64_t M = T * k;
    const int64_t esz = dtype == O_F32 ? 4 : dtype == O_BF16 ? 2 : 1;
    const int64_t ssz = dtype == O_MXFP8 ? H / 32 : 0;
    char* x_perm;
    uint8_t* xs_perm = NULL;
    int32_t* row_expert;
    double* y_perm;
    int rc = 0;
    if (chunk < 0 || (dtype == O_MXFP8 && (H % 32 || F % 32)))
        return -1;
    if (oracle_route(ids, T, k, E, counts, offsets, perm, pos) != 0)
        return -1;
    x_perm = (char*)malloc((size_t)(M * H * esz + 1));
    oracle_permute(x, H * esz, perm, M, k, x_perm);
    if (dtype == O_MXFP8) {
        xs_perm = (uint8_t*)malloc((size_t)(M * ssz + 1));
        oracle_permute(x_scale, ssz, perm, M, k, xs_perm);
    }
    row_expert = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M + 1));
    for (int64_t e = 0; e < E; ++e)
        for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p)
            row_expert[p] = (int32_t)e;
    y_perm = (double*)malloc(sizeof(double) * (size_t)(M * H + 1));
    if (chunk == 0 || chunk > M)
        chunk = M > 0 ? M : 1;
    for (int64_t c0 = 0; c0 < M && rc == 0; c0 += chunk) {
        int64_t n = M - c0 < chunk ? M - c0 : chunk;
        rc = oracle_ffn_rows(dtype, n, H, F, E, x_perm + c0 * H * esz,
                             xs_perm ? xs_perm + c0 * ssz : NULL, row_expert + c0, w_gate, wg_scale,
                             w_up, wu_scale, w_down, wd_scale, y_perm + c0 * H);
    }
    /* unpermute, step 10: out[t] = sum over j = 0..k-1 (ascending) of probs[t, j] * y_perm[pos[t*k+j]] */
    for (int64_t t = 0; t < T && rc == 0; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)probs[t * k + j] * y_perm[(int64_t)pos[t * k + j] * H + h];
            out[t * H + h] = acc;
        }
    free(x_perm); free(xs_perm); free(row_expert); free(y_perm);
    return rc;
}

/* Per-token form of the same layer for a list of tokens: out[i] = sum_j probs[t, j] * FFN_{ids[t, j]}(x[t])
 * with t = tokens[i] (the definition itself, with no routing or permutation).  Used where the grouped
 * forward over every row would take too long on a CPU.  Output: double [ntok, H]. */
int oracle_forward_tokens(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                          const void* x, const uint8_t* x_scale, const void* w_gate,
                          const uint8_t* wg_scale, const void* w_up, const uint8_t* wu_scale,
                          const void* w_down, const uint8_t* wd_scale, const int32_t* ids,
                          const float* probs, const int32_t* tokens, int64_t ntok, double* out)
{
    const int64_t esz = dtype == O_F32 ? 4 : dtype == O_BF16 ? 2 : 1;
    const int64_t ssz = dtype == O_MXFP8 ? H / 32 : 0;
    const int64_t n = ntok * k;
    char* xr = (char*)malloc((size_t)(n * H * esz + 1));
    uint8_t* xs = ssz ? (uint8_t*)malloc((size_t)(n * ssz)) : NULL;
    int32_t* re = (int32_t*)calloc((size_t)(n + 1), sizeof(int32_t));
    double* y = (double*)malloc(sizeof(double) * (size_t)(n * H + 1));
    int rc = 0;
    for (int64_t i = 0; i < ntok && rc == 0; ++i) {
        int64_t t = tokens[i];
        if (t < 0 || t >= T) { rc = -1; break; }
        for (int64_t j = 0; j < k; ++j) {
            memcpy(xr + (i * k + j) * H * esz, (const char*)x + t * H * esz, (size_t)(H * esz));
            if (ssz)
                memcpy(xs + (i * k + j) * ssz, x_scale + t * ssz, (size_t)ssz);
            re[i * k + j] = ids[t * k + j];
        }
    }
    if (rc == 0)
        rc = oracle_ffn_rows(dtype, n, H, F, E, xr, xs, re, w_gate, wg_scale, w_up, wu_scale,
                             w_down, wd_scale, y);
    for (int64_t i = 0; i < ntok && rc == 0; ++i)
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)probs[tokens[i] * k + j] * y[(i * k + j) * H + h];
            out[i * H + h] = acc;
        }
    free(xr); free(xs); free(re); free(y);
    return rc;
}

/* ------------------------------------------------------------------------------------------------
 * Router in front of the path: the gate's top-k (the "Gate 计算" step of the step breakdown on the
 * page "MC2 通算融合"; the router top-k distribution is one of the checks listed on the page "NPU
 * Training Operators - MC2").  Reading taken: the k experts with the largest logits, in descending
 * logit order, ties broken towards the lower expert id; the probability of each is the softmax over
 * the k selected logits, which equals the softmax over all E experts renormalised over the k.
 * Per token: k passes of a plain scan for the largest not yet taken logit (strictly greater wins,
 * so the first of equal logits is kept), then exp(l_j - l_max) / sum_i exp(l_i - l_max) in double.
 * Logits must not be NaN, and the largest logit of a token must be finite.
 * ---------------------------------------------------------------------------------------------- */
void oracle_router(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids, double* probs)
{
    char* taken = (char*)malloc(E > 0 ? (size_t)E : 1);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        const double m = (double)l[ids[t * k]];
        double sum = 0.0;
        for (int64_t j = 0; j < k; ++j)
            sum += exp((double)l[ids[t * k + j]] - m);
        for (int64_t j = 0; j < k; ++j)
            probs[t * k + j] = exp((double)l[ids[t * k + j]] - m) / sum;
    }
    free(taken);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------------------------------
 * Backward of the layer: the gradients of the scalar L = sum_{t,h} dout[t,h] * out[t,h] with
 * respect to x, the three weight stacks and the routing probabilities, for given routing.  The
 * page "NPU Training Operators - MC2" wraps the forward and the backward of each step in its fused
 * ops, and its 验证项 list the fc1 / fc2 gradients among the checks.  Written from the chain rule
 * on the forward's definition (steps 6-10), per slot s = t*k + j with expert e = ids[s]:
 *   g = x_t Wg[e], u = x_t Wu[e], sg = sigmoid(g), a = g sg u, y = a Wd[e]
 *   dprobs[s]  = <dout_t, y>
 *   dy         = probs[s] dout_t
 *   da         = dy Wd[e]^T                      (sum over h)
 *   dg         = da u sg (1 + g (1 - sg))       (d silu(g) / dg = sg + g sg (1 - sg))
 *   du         = da g sg
 *   dx_t      += dg Wg[e]^T + du Wu[e]^T         (sum over f; the k slots of t added in j order)
 *   dWd[e]    += a^T dy,  dWg[e] += x_t^T dg,  dWu[e] += x_t^T du   (slots in ascending s)
 * Inputs in storage format (float32 or bfloat16; dout in the same format), widened exactly to
 * double; every sum is a double sum in ascending index order.  Outputs double:
 * dx [T, H], dwg / dwu [E, H, F], dwd [E, F, H], dprobs [T, k].  Returns 0, or -1 for a bad id or
 * an unsupported dtype.
 * ---------------------------------------------------------------------------------------------- */
static double sigmoid_d(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Forward and backward quantities of one slot whose weights are decoded (wg, wu [H, F], wd [F, H]):
 * g, u, a (F), da (F) from x row xr and the scaled output gradient dy (H); y (H). */
static void slot_chain(int64_t H, int64_t F, const double* xr, const double* dr, double w,
                       const double* wg, const double* wu, const double* wd, double* g, double* u,
                       double* a, double* y, double* dy, double* da, double* dprob)
{
    for (int64_t f = 0; f < F; ++f) {
        double gs = 0.0, us = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            gs += xr[h] * wg[h * F + f];
            us += xr[h] * wu[h * F + f];
        }
        g[f] = gs;
        u[f] = us;
        a[f] = gs * sigmoid_d(gs) * us;
    }
    double dp = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        double ys = 0.0;
        for (int64_t f = 0; f < F; ++f)
            ys += a[f] * wd[f * H + h];
        y[h] = ys;
        dp += dr[h] * ys;
        dy[h] = w * dr[h];
    }
    *dprob = dp;
    for (int64_t f = 0; f < F; ++f) {
        double s = 0.0;
        for (int64_t h = 0; h < H; ++h)
            s += dy[h] * wd[f * H + h];
        da[f] = s;
    }
}

int oracle_backward(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                    const void* x, const void* w_gate, const void* w_up, const void* w_down,
                    const int32_t* ids, const float* probs, const void* dout, double* dx,
                    double* dwg, double* dwu, double* dwd, double* dprobs)
{
    const int64_t M = T * k;
    const int64_t esz = dtype == O_F32 ? 4 : 2;
    double *xd, *dd, *wg, *wu, *wd, *dxp, *g, *u, *a, *y, *dy, *da, *dg, *du;
    if (dtype != O_F32 && dtype != O_BF16)
        return -1;
    for (int64_t s = 0; s < M; ++s)
        if (ids[s] < 0 || ids[s] >= E)
            return -1;
    xd = (double*)malloc(sizeof(double) * (size_t)(T * H + 1));
    dd = (double*)malloc(sizeof(double) * (size_t)(T * H + 1));
    wg = (double*)malloc(sizeof(double) * (size_t)(H * F));
    wu = (double*)malloc(sizeof(double) * (size_t)(H * F));
    wd = (double*)malloc(sizeof(double) * (size_t)(F * H));
    dxp = (double*)calloc((size_t)(M * H + 1), sizeof(double));
    g = (double*)malloc(sizeof(double) * (size_t)F);
    u = (double*)malloc(sizeof(double) * (size_t)F);
    a = (double*)malloc(sizeof(double) * (size_t)F);
    da = (double*)malloc(sizeof(double) * (size_t)F);
    dg = (double*)malloc(sizeof(double) * (size_t)F);
    du = (double*)malloc(sizeof(double) * (size_t)F);
    y = (double*)malloc(sizeof(double) * (size_t)H);
    dy = (double*)malloc(sizeof(double) * (size_t)H);
    decode_matrix(dtype, x, NULL, T, H, 0, xd);
    decode_matrix(dtype, dout, NULL, T, H, 0, dd);
    for (int64_t e = 0; e < E; ++e) {
        double* gwg = dwg + e * H * F;
        double* gwu = dwu + e * H * F;
        double* gwd = dwd + e * F * H;
        memset(gwg, 0, sizeof(double) * (size_t)(H * F));
        memset(gwu, 0, sizeof(double) * (size_t)(H * F));
        memset(gwd, 0, sizeof(double) * (size_t)(F * H));
        decode_matrix(dtype, (const char*)w_gate + e * H * F * esz, NULL, H, F, 1, wg);
        decode_matrix(dtype, (const char*)w_up + e * H * F * esz, NULL, H, F, 1, wu);
        decode_matrix(dtype, (const char*)w_down + e * F * H * esz, NULL, F, H, 1, wd);
        for (int64_t s = 0; s < M; ++s) {
            if (ids[s] != e)
                continue;
            const double* xr = xd + (s / k) * H;
            slot_chain(H, F, xr, dd + (s / k) * H, (double)probs[s], wg, wu, wd, g, u, a, y, dy,
                       da, &dprobs[s]);
            for (int64_t f = 0; f < F; ++f) {
                const double sg = sigmoid_d(g[f]);
                dg[f] = da[f] * u[f] * sg * (1.0 + g[f] * (1.0 - sg));
                du[f] = da[f] * g[f] * sg;
            }
            for (int64_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int64_t f = 0; f < F; ++f)
                    acc += dg[f] * wg[h * F + f] + du[f] * wu[h * F + f];
                dxp[s * H + h] = acc;
            }
            for (int64_t f = 0; f < F; ++f)
                for (int64_t h = 0; h < H; ++h)
                    gwd[f * H + h] += a[f] * dy[h];
            for (int64_t h = 0; h < H; ++h)
                for (int64_t f = 0; f < F; ++f) {
                    gwg[h * F + f] += xr[h] * dg[f];
                    gwu[h * F + f] += xr[h] * du[f];
                }
        }
    }
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += dxp[(t * k + j) * H + h];
            dx[t * H + h] = acc;
        }
    free(xd); free(dd); free(wg); free(wu); free(wd); free(dxp);
    free(g); free(u); free(a); free(da); free(dg); free(du); free(y); free(dy);
    return 0;
}

/* The same gradients for a list of tokens only: dx[tokens[i]] and dprobs[tokens[i], :], computed
 * per slot exactly as in oracle_backward (used where the whole backward would take too long on a
 * CPU).  Outputs double dx_rows [ntok, H], dprobs_rows [ntok, k]. */
int oracle_backward_tokens(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                           const void* x, const void* w_gate, const void* w_up, const void* w_down,
                           const int32_t* ids, const float* probs, const void* dout,
                           const int32_t* tokens, int64_t ntok, double* dx_rows,
                           double* dprobs_rows)
{
    const int64_t esz = dtype == O_F32 ? 4 : 2;
    int rc = 0;
    int64_t i;
    if (dtype != O_F32 && dtype != O_BF16)
        return -1;
    for (i = 0; i < ntok; ++i) {
        if (tokens[i] < 0 || tokens[i] >= T)
            return -1;
        for (int64_t j = 0; j < k; ++j)
            if (ids[tokens[i] * k + j] < 0 || ids[tokens[i] * k + j] >= E)
                return -1;
    }
#pragma omp parallel for schedule(dynamic)
    for (i = 0; i < ntok; ++i) {
        const int64_t t = tokens[i];
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* dr = (double*)malloc(sizeof(double) * (size_t)H);
        double* wg = (double*)malloc(sizeof(double) * (size_t)(H * F));
        double* wu = (double*)malloc(sizeof(double) * (size_t)(H * F));
        double* wd = (double*)malloc(sizeof(double) * (size_t)(F * H));
        double* g = (double*)malloc(sizeof(double) * (size_t)F);
        double* u = (double*)malloc(sizeof(double) * (size_t)F);
        double* a = (double*)malloc(sizeof(double) * (size_t)F);
        double* da = (double*)malloc(sizeof(double) * (size_t)F);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        double* dy = (double*)malloc(sizeof(double) * (size_t)H);
        double* dxp = (double*)malloc(sizeof(double) * (size_t)(k * H));
        decode_matrix(dtype, (const char*)x + t * H * esz, NULL, 1, H, 0, xr);
        decode_matrix(dtype, (const char*)dout + t * H * esz, NULL, 1, H, 0, dr);
        for (int64_t j = 0; j < k; ++j) {
            const int64_t s = t * k + j, e = ids[s];
            decode_matrix(dtype, (const char*)w_gate + e * H * F * esz, NULL, H, F, 1, wg);
            decode_matrix(dtype, (const char*)w_up + e * H * F * esz, NULL, H, F, 1, wu);
            decode_matrix(dtype, (const char*)w_down + e * F * H * esz, NULL, F, H, 1, wd);
            slot_chain(H, F, xr, dr, (double)probs[s], wg, wu, wd, g, u, a, y, dy, da,
                       &dprobs_rows[i * k + j]);
            for (int64_t h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int64_t f = 0; f < F; ++f) {
                    const double sg = sigmoid_d(g[f]);
                    acc += da[f] * u[f] * sg * (1.0 + g[f] * (1.0 - sg)) * wg[h * F + f] +
                           da[f] * g[f] * sg * wu[h * F + f];
                }
                dxp[j * H + h] = acc;
            }
        }
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += dxp[j * H + h];
            dx_rows[i * H + h] = acc;
        }
        free(xr); free(dr); free(wg); free(wu); free(wd); free(g); free(u); free(a); free(da);
        free(y); free(dy); free(dxp);
    }
    return rc;
}

/* Single entries of the weight gradients: for entry i with (e, f, h) = (ent_e[i], ent_f[i],
 * ent_h[i]), dwg_out[i] = dWg[e][h][f], dwu_out[i] = dWu[e][h][f], dwd_out[i] = dWd[e][f][h], each
 * the sum over the slots of expert e in ascending s, as in oracle_backward, but with only column f
 * of g, u and da evaluated per slot. */
int oracle_wgrad_entries(int dtype, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                         const void* x, const void* w_gate, const void* w_up, const void* w_down,
                         const int32_t* ids, const float* probs, const void* dout, int64_t nent,
                         const int32_t* ent_e, const int32_t* ent_f, const int32_t* ent_h,
                         double* dwg_out, double* dwu_out, double* dwd_out)
{
    const int64_t M = T * k;
    const int64_t esz = dtype == O_F32 ? 4 : 2;
    int64_t i;
    if (dtype != O_F32 && dtype != O_BF16)
        return -1;
    for (i = 0; i < nent; ++i)
        if (ent_e[i] < 0 || ent_e[i] >= E || ent_f[i] < 0 || ent_f[i] >= F || ent_h[i] < 0 ||
            ent_h[i] >= H)
            return -1;
#pragma omp parallel for schedule(dynamic)
    for (i = 0; i < nent; ++i) {
        const int64_t e = ent_e[i], f = ent_f[i], hh = ent_h[i];
        double* wgc = (double*)malloc(sizeof(double) * (size_t)H);   /* column f of Wg[e] */
        double* wuc = (double*)malloc(sizeof(double) * (size_t)H);
        double* wdr = (double*)malloc(sizeof(double) * (size_t)H);   /* row f of Wd[e] */
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* dr = (double*)malloc(sizeof(double) * (size_t)H);
        double sg_acc = 0.0, su_acc = 0.0, sd_acc = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            wgc[h] = dtype == O_F32 ? (double)((const float*)w_gate)[(e * H + h) * F + f]
                                    : oracle_bf16_value(((const uint16_t*)w_gate)[(e * H + h) * F + f]);
            wuc[h] = dtype == O_F32 ? (double)((const float*)w_up)[(e * H + h) * F + f]
                                    : oracle_bf16_value(((const uint16_t*)w_up)[(e * H + h) * F + f]);
            wdr[h] = dtype == O_F32 ? (double)((const float*)w_down)[(e * F + f) * H + h]
                                    : oracle_bf16_value(((const uint16_t*)w_down)[(e * F + f) * H + h]);
        }
        for (int64_t s = 0; s < M; ++s) {
            if (ids[s] != e)
                continue;
            const int64_t t = s / k;
            double g = 0.0, u = 0.0, da = 0.0;
            decode_matrix(dtype, (const char*)x + t * H * esz, NULL, 1, H, 0, xr);
            decode_matrix(dtype, (const char*)dout + t * H * esz, NULL, 1, H, 0, dr);
            for (int64_t h = 0; h < H; ++h) {
                g += xr[h] * wgc[h];
                u += xr[h] * wuc[h];
            }
            const double w = (double)probs[s];
            for (int64_t h = 0; h < H; ++h)
                da += w * dr[h] * wdr[h];
            const double sg = sigmoid_d(g);
            sg_acc += xr[hh] * (da * u * sg * (1.0 + g * (1.0 - sg)));
            su_acc += xr[hh] * (da * g * sg);
            sd_acc += (g * sg * u) * (w * dr[hh]);
        }
        dwg_out[i] = sg_acc;
        dwu_out[i] = su_acc;
        dwd_out[i] = sd_acc;
        free(wgc); free(wuc); free(wdr); free(xr); free(dr);
    }
    return 0;
}
