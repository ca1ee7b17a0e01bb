/*
 * lh_oracle.c - CPU oracle for Local-Hessian NVFP4 weight-scale calibration.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; it exists so that tests, the smoke check and the CPU leg of
 * the benchmark can check the HIP library against a plain, slow, obviously
 * correct evaluation of the same definitions.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Sources (the pages this follows):
 *   [LHG]  "Local-Hessian weight-scale guide", xxmr.cn/news/266017
 *          - "What is Local-Hessian": NVFP4 = 16 weights sharing one FP8 block
 *            scale, values scaled into the E2M1 range [-6, 6]; MSE sweep over
 *            all 126 positive non-zero FP8 scale values.
 *          - "Algorithm principle": Y = WX, X in R^(C_in x N);
 *            Q(W,s) = Cast(W/s)*s, Delta = Q - W;
 *            E(s) = ||Delta X||_F^2 = tr(Delta (X X^T) Delta^T);
 *            block-diagonal approximation E_b(s_b) = Delta_b (X_b X_b^T) Delta_b^T
 *            with W_b in R^(1x16), X_b in R^(16xN); kernel interface: weights
 *            as [N_BLOCKS,16] in (cout, cin//16) order, a global FP32 amax,
 *            per-block Hessians [cin//16,16,16], minimise dw^T H dw over the
 *            126 FP8 E4M3 candidates, output the per-block best amax.
 *          - "Entry API and calibration flow", phase 2: H accumulated as the
 *            sum of X^T X over calibration tokens; phase 3 uses the
 *            normalised per-block Hessian.
 *          - "Combining with GPTQ": the cast rounds to nearest (RTN).
 *   [MOO]  "ModelOpt overview", linlog.top/article/1517, section
 *          "Local-Hessian": 126 candidate FP8 scales per block, blocks
 *          optimised independently.
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes of the repository):
 *   R1  candidate set = the 126 positive finite non-zero OCP E4M3FN values,
 *       codes 0x01..0x7E (max 448); candidate k <-> code k+1.
 *   R2  S_g = fl32(g / 2688) with 2688 = 6 * 448; s_k = fl32(c_k * S_g).
 *   R3  Cast(W/s): x = fl32(|w| / s) by IEEE fp32 division, then the nearest
 *       E2M1 magnitude {0,0.5,1,1.5,2,3,4,6}; ties go to the even code;
 *       x beyond 6 saturates to 6; s == 0 gives 0.  Q = fl32(sign(w) r s),
 *       and -0 is written as +0.
 *   R4  "normalised" Hessian = divided by the token count N (alpha = 1/N).
 *   R5  ties between equal errors go to the lowest candidate index.
 *
 * Arithmetic: Hessian sums and quadratic forms in fp64 from exactly widened
 * inputs; the cast uses exactly the fp32 operations R2/R3 name.
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes used by the Python wrapper: 0 = fp32, 1 = bf16 */
/* layout codes: 0 = channel-major x[c*ld + t], 1 = token-major x[t*ld + c] */

static double widen(const void *p, int dtype, int64_t i)
{
    if (dtype == 0)
        return (double)((const float *)p)[i];
    /* bf16 is the upper half of an IEEE binary32 word */
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float widen_f32(const void *p, int dtype, int64_t i)
{
    return (float)widen(p, dtype, i);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------- */
/* FP8 E4M3 (OCP "FN" variant): 1 sign, 4 exponent (bias 7), 3 mantissa.  */
/* Positive byte e: exponent field E = e >> 3, mantissa m = e & 7.         */
/* E == 0 encodes the subnormals m * 2^-9; otherwise (1 + m/8) * 2^(E-7).  */
/* ---------------------------------------------------------------------- */
double oracle_e4m3_value(int code)
{
    int E = (code >> 3) & 15;
    int m = code & 7;
    if (E == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, E - 7);
}

/* R2: the 126 candidate scales derived from the global amax g. */
void oracle_candidate_scales(float g, float *s_out /* [126] */)
{
    float Sg = g / 2688.0f; /* one fp32 division */
    for (int k = 0; k < 126; ++k) {
        float c = (float)oracle_e4m3_value(k + 1); /* exact in fp32 */
        s_out[k] = c * Sg;                          /* one fp32 multiply */
    }
}

/* ---------------------------------------------------------------------- */
/* E2M1 magnitude grid and the cast (R3).                                 */
/* ---------------------------------------------------------------------- */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Magnitude code (0..7) of the E2M1 value nearest to x >= 0, ties to the
 * even code; anything above the largest grid value saturates to it. */
int oracle_e2m1_code(float x)
{
    if (!(x <= 6.0f))
        return 7; /* saturation (also +inf) */
    int best = 0;
    double bd = fabs((double)x - E2M1_GRID[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs((double)x - E2M1_GRID[c]);
        if (d < bd || (d == bd && (c % 2) == 0)) {
            best = c;
            bd = d;
        }
    }
    return best;
}

double oracle_e2m1_value(int code) { return E2M1_GRID[code & 7]; }

/* Q(w, s) = Cast(w / s) * s for one weight.  Also returns the magnitude code. */
float oracle_quantize(float w, float s, int *code_out)
{
    int code = 0;
    if (s != 0.0f) {
        float a = fabsf(w);
        float x = a / s; /* IEEE fp32 division */
        code = oracle_e2m1_code(x);
    }
    float r = (float)E2M1_GRID[code]; /* exact */
    float q = r * s;                  /* fl32(r * s) */
    if (w < 0.0f)
        q = -q;
    if (q == 0.0f)
        q = 0.0f; /* -0 -> +0 */
    if (code_out)
        *code_out = code;
    return q;
}

/* E_k = dw^T H dw for all 126 candidates of one 16-weight block.
 * w: 16 fp32 weights; H: 16x16 fp32 row-major; g: global amax. */
void oracle_block_errors(const float *w, const float *H, float g, double *E /* [126] */)
{
    float s[126];
    oracle_candidate_scales(g, s);
    for (int k = 0; k < 126; ++k) {
        double dw[16];
        for (int i = 0; i < 16; ++i)
            dw[i] = (double)oracle_quantize(w[i], s[k], 0) - (double)w[i];
        double e = 0.0;
        for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j)
                e += dw[i] * (double)H[i * 16 + j] * dw[j];
        E[k] = e;
    }
}

/* S = sum_ij |H_ij| |dw_i| |dw_j| of one block at candidate k (H NULL: the
 * identity).  Not part of the method: the parity tests use it to size the
 * rounding error that an fp32 evaluation of dw^T H dw may carry. */
static double abs_form_at(const float *w, const float *H, float g, int k)
{
    float s[126];
    oracle_candidate_scales(g, s);
    double dw[16];
    for (int i = 0; i < 16; ++i)
        dw[i] = fabs((double)oracle_quantize(w[i], s[k], 0) - (double)w[i]);
    double acc = 0.0;
    for (int i = 0; i < 16; ++i)
        for (int j = 0; j < 16; ++j) {
            double hij = H ? fabs((double)H[i * 16 + j]) : (i == j ? 1.0 : 0.0);
            acc += dw[i] * hij * dw[j];
        }
    return acc;
}

/* Optional per-block outputs for checking another implementation's pick:
 * the error at a probed candidate (e.g. the one the GPU chose), and the
 * absolute forms S at the probed and at the best candidate. */
static void probe_block(const float *w, const float *H, float g, const double *E, int kb,
                        const int32_t *probe, int64_t n, double *e_probe, double *s_probe,
                        double *s_best)
{
    int kp = probe ? probe[n] : kb;
    if (kp < 0 || kp > 125)
        kp = kb;
    if (e_probe)
        e_probe[n] = E[kp];
    if (s_probe)
        s_probe[n] = abs_form_at(w, H, g, kp);
    if (s_best)
        s_best[n] = abs_form_at(w, H, g, kb);
}

/* Argmin with the lowest index on ties (R5); e2 = best error among k != k*. */
static void argmin126(const double *E, int *k_out, double *e1, double *e2)
{
    int kb = 0;
    for (int k = 1; k < 126; ++k)
        if (E[k] < E[kb])
            kb = k;
    double second = INFINITY;
    for (int k = 0; k < 126; ++k)
        if (k != kb && E[k] < second)
            second = E[k];
    *k_out = kb;
    *e1 = E[kb];
    *e2 = second;
}

/* ---------------------------------------------------------------------- */
/* Global amax per group: g = max |w| over the group's C_out x C_in weights. */
/* ---------------------------------------------------------------------- */
void oracle_absmax(const void *w, int dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                   int64_t n_groups, int64_t gstride_w, float *out)
{
    for (int64_t g = 0; g < n_groups; ++g) {
        double m = 0.0;
        for (int64_t r = 0; r < c_out; ++r)
            for (int64_t c = 0; c < c_in; ++c) {
                double v = fabs(widen(w, dtype, g * gstride_w + r * ld_w + c));
                if (v > m)
                    m = v;
            }
        out[g] = (float)m; /* exact: m is an fp32 value */
    }
}

/* ---------------------------------------------------------------------- */
/* Local Hessians: for the selected (group, block) pairs,                  */
/*   h[g][b][i][j] = beta * h_old + alpha * sum_t x[g][16b+i][t] x[g][16b+j][t] */
/* with every product and the sum in fp64 in token order.  sel lists flat   */
/* indices g * (c_in/16) + b.  h64 (nullable) and h32 are compact:         */
/* entry n of the selection occupies [n*256, n*256+256).  h32 is read for   */
/* beta != 0 and written.                                                   */
/* ---------------------------------------------------------------------- */
void oracle_hessian(const void *x, int dtype, int layout, int64_t c_in, int64_t n_tok,
                    int64_t ld_x, int64_t gstride_x, double alpha, double beta,
                    const int64_t *sel, int64_t n_sel, double *h64, float *h32)
{
    const int64_t nb = c_in / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_sel; ++n) {
        const int64_t g = sel[n] / nb, b = sel[n] % nb;
        for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
                const int64_t ci = 16 * b + i, cj = 16 * b + j;
                double acc = 0.0;
                for (int64_t t = 0; t < n_tok; ++t) {
                    int64_t oi, oj;
                    if (layout == 0) {
                        oi = ci * ld_x + t;
                        oj = cj * ld_x + t;
                    } else {
                        oi = t * ld_x + ci;
                        oj = t * ld_x + cj;
                    }
                    acc += widen(x, dtype, g * gstride_x + oi) * widen(x, dtype, g * gstride_x + oj);
                }
                double v = alpha * acc;
                if (beta != 0.0)
                    v += beta * (double)h32[n * 256 + i * 16 + j];
                if (h64)
                    h64[n * 256 + i * 16 + j] = v;
                h32[n * 256 + i * 16 + j] = (float)v;
            }
    }
}

/* ---------------------------------------------------------------------- */
/* Scale sweep for the selected blocks.  sel lists flat block indices      */
/* (g * c_out + row) * (c_in/16) + b.  H is the full fp32 Hessian tensor    */
/* [g][b][16][16] (group stride gstride_h) that the sweep consumes; amax is */
/* the per-group global amax.  Outputs are compact per selected block.      */
/* ---------------------------------------------------------------------- */
void oracle_sweep(const void *w, int dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                  int64_t gstride_w, const float *H, int64_t gstride_h, const float *amax,
                  const int64_t *sel, int64_t n_sel, int32_t *idx_out, double *e1_out,
                  double *e2_out, float *err_out, float *amax_out, const int32_t *probe,
                  double *e_probe, double *s_probe, double *s_best)
{
    const int64_t nb = c_in / 16;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < n_sel; ++n) {
        const int64_t f = sel[n];
        const int64_t b = f % nb;
        const int64_t row = (f / nb) % c_out;
        const int64_t g = f / (nb * c_out);
        float wb[16];
        for (int i = 0; i < 16; ++i)
            wb[i] = widen_f32(w, dtype, g * gstride_w + row * ld_w + 16 * b + i);
        double E[126];
        const float *Hb = H + g * gstride_h + b * 256;
        oracle_block_errors(wb, Hb, amax[g], E);
        int k;
        double e1, e2;
        argmin126(E, &k, &e1, &e2);
        probe_block(wb, Hb, amax[g], E, k, probe, n, e_probe, s_probe, s_best);
        if (idx_out)
            idx_out[n] = k;
        if (e1_out)
            e1_out[n] = e1;
        if (e2_out)
            e2_out[n] = e2;
        if (err_out)
            err_out[n] = (float)e1;
        if (amax_out) {
            float s[126];
            oracle_candidate_scales(amax[g], s);
            amax_out[n] = 6.0f * s[k]; /* fl32(6 s_k*) */
        }
    }
}

/* ---------------------------------------------------------------------- */
/* NVFP4 fake-quant for the selected blocks with the given candidate index  */
/* per block (idx laid out like the sweep output, full size).  Outputs are  */
/* compact: q[n*16+i], packed[n*8 + i/2] (low nibble = even column; nibble  */
/* = sign bit 3 | magnitude code), code[n] = E4M3 byte idx+1.               */
/* ---------------------------------------------------------------------- */
void oracle_fake_quant(const void *w, int dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                       int64_t gstride_w, const uint8_t *idx, const float *amax,
                       const int64_t *sel, int64_t n_sel, float *q_out, uint8_t *packed_out,
                       uint8_t *code_out)
{
    const int64_t nb = c_in / 16;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_sel; ++n) {
        const int64_t f = sel[n];
        const int64_t b = f % nb;
        const int64_t row = (f / nb) % c_out;
        const int64_t g = f / (nb * c_out);
        float s[126];
        oracle_candidate_scales(amax[g], s);
        const int k = idx[f];
        uint8_t nib[16];
        for (int i = 0; i < 16; ++i) {
            float wv = widen_f32(w, dtype, g * gstride_w + row * ld_w + 16 * b + i);
            int code;
            float q = oracle_quantize(wv, s[k], &code);
            if (q_out)
                q_out[n * 16 + i] = q;
            nib[i] = (uint8_t)(((q < 0.0f) ? 8 : 0) | code);
        }
        if (packed_out)
            for (int i = 0; i < 8; ++i)
                packed_out[n * 8 + i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
        if (code_out)
            code_out[n] = (uint8_t)(k + 1);
    }
}

/* ====================================================================== */
/* Scale-rule variants: the methods [LHG] compares Local-Hessian with.     */
/*   "What is Local-Hessian": max scaling takes the block scale from the   */
/*   largest |w| of the 16 weights; Four-Over-Six picks one of two         */
/*   candidate scales by the in-block error; the MSE method sweeps all 126 */
/*   positive FP8 values by the weight error.                              */
/*   "Entry API and calibration flow": with the 126-value sweep off, the   */
/*   amax is searched from multiplier 0.25 to 4.0 in steps of 0.1.         */
/* Readings:                                                               */
/*   R6  a block scale wanted as the value t (in units of S_g) is stored   */
/*       as the nearest positive finite E4M3 value, ties to the even code; */
/*       values above 448 store 448 and values that round to zero store    */
/*       the smallest candidate 2^-9.                                      */
/*   R7  max scaling: t = fl32(fl32(amax_b / 6) / S_g), amax_b = max |w|   */
/*       over the block.                                                   */
/*   R8  Four-Over-Six: the two candidates map amax_b to 6 (R7) and to 4:  */
/*       t = fl32(fl32(amax_b / 4) / S_g).                                 */
/*   R9  amax search: multipliers m_i = fl32((25 + 10 i) / 100) for        */
/*       i = 0..37 (0.25 .. 3.95; the stop value 4.0 is exclusive);        */
/*       candidate i stores t = fl32(fl32(fl32(m_i amax_b) / 6) / S_g).    */
/*   R10 objective: dw^T H dw with the block's local Hessian when one is   */
/*       given, else the plain weight error sum_i dw_i^2 (H = I).  A rule  */
/*       returns the best of its distinct candidates, lowest index on ties */
/*       (R5); e2 is the best among its other distinct candidates.         */
/*   R11 g = 0 (S_g = 0): every rule returns candidate 0 (all Q are 0).    */
/* ====================================================================== */
enum { ORACLE_RULE_SWEEP = 0, ORACLE_RULE_MAX = 1, ORACLE_RULE_FOUR_OVER_SIX = 2,
       ORACLE_RULE_AMAX_SEARCH = 3 };

/* R6: E4M3 byte (1..126) stored for the wanted scale value t > 0. */
int oracle_e4m3_round_code(float t)
{
    if (!(t > 0.0f))
        return 1;
    int best = 0; /* code 0 is the value zero */
    double bd = (double)t;
    for (int code = 1; code <= 126; ++code) {
        double d = fabs((double)t - oracle_e4m3_value(code));
        if (d < bd || (d == bd && (code % 2) == 0)) {
            best = code;
            bd = d;
        }
    }
    return best == 0 ? 1 : best;
}

/* R9: the i-th amax-search multiplier. */
float oracle_amax_multiplier(int i) { return (float)((25.0 + 10.0 * i) / 100.0); }

/* Distinct candidate indices (ascending) a rule considers for one block;
 * returns their count. */
int oracle_rule_candidates(int rule, const float *w16, float g, int *k_out /* [126] */)
{
    float Sg = g / 2688.0f;
    int n = 0;
    if (rule == ORACLE_RULE_SWEEP) {
        for (int k = 0; k < 126; ++k)
            k_out[n++] = k;
        return n;
    }
    if (Sg == 0.0f) { /* R11 */
        k_out[0] = 0;
        return 1;
    }
    float ab = 0.0f;
    for (int i = 0; i < 16; ++i)
        if (fabsf(w16[i]) > ab)
            ab = fabsf(w16[i]);
    int want[38];
    int nw = 0;
    if (rule == ORACLE_RULE_MAX || rule == ORACLE_RULE_FOUR_OVER_SIX) {
        float t6 = (ab / 6.0f) / Sg;
        want[nw++] = oracle_e4m3_round_code(t6) - 1;
        if (rule == ORACLE_RULE_FOUR_OVER_SIX) {
            float t4 = (ab / 4.0f) / Sg;
            want[nw++] = oracle_e4m3_round_code(t4) - 1;
        }
    } else if (rule == ORACLE_RULE_AMAX_SEARCH) {
        for (int i = 0; i < 38; ++i) {
            float a = oracle_amax_multiplier(i) * ab;
            float t = (a / 6.0f) / Sg;
            want[nw++] = oracle_e4m3_round_code(t) - 1;
        }
    } else {
        return 0;
    }
    /* distinct, ascending */
    for (int k = 0; k < 126; ++k)
        for (int i = 0; i < nw; ++i)
            if (want[i] == k) {
                k_out[n++] = k;
                break;
            }
    return n;
}

/* Errors of all 126 candidates of one block under the R10 objective. */
static void block_errors_objective(const float *w, const float *H, float g, double *E)
{
    if (H) {
        oracle_block_errors(w, H, g, E);
        return;
    }
    float s[126];
    oracle_candidate_scales(g, s);
    for (int k = 0; k < 126; ++k) {
        double e = 0.0;
        for (int i = 0; i < 16; ++i) {
            double dw = (double)oracle_quantize(w[i], s[k], 0) - (double)w[i];
            e += dw * dw;
        }
        E[k] = e;
    }
}

/* Scale selection by rule for the selected blocks (flat indices as in
 * oracle_sweep).  H (nullable) is the fp32 Hessian tensor; outputs compact. */
void oracle_select(int rule, const void *w, int dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                   int64_t gstride_w, const float *H, int64_t gstride_h, const float *amax,
                   const int64_t *sel, int64_t n_sel, int32_t *idx_out, double *e1_out,
                   double *e2_out, float *err_out, float *amax_out, const int32_t *probe,
                   double *e_probe, double *s_probe, double *s_best)
{
    const int64_t nb = c_in / 16;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < n_sel; ++n) {
        const int64_t f = sel[n];
        const int64_t b = f % nb;
        const int64_t row = (f / nb) % c_out;
        const int64_t g = f / (nb * c_out);
        float wb[16];
        for (int i = 0; i < 16; ++i)
            wb[i] = widen_f32(w, dtype, g * gstride_w + row * ld_w + 16 * b + i);
        double E[126];
        const float *Hb = H ? H + g * gstride_h + b * 256 : 0;
        block_errors_objective(wb, Hb, amax[g], E);
        int ks[126];
        int nk = oracle_rule_candidates(rule, wb, amax[g], ks);
        int kb = ks[0];
        for (int i = 1; i < nk; ++i)
            if (E[ks[i]] < E[kb])
                kb = ks[i];
        double second = INFINITY;
        for (int i = 0; i < nk; ++i)
            if (ks[i] != kb && E[ks[i]] < second)
                second = E[ks[i]];
        probe_block(wb, Hb, amax[g], E, kb, probe, n, e_probe, s_probe, s_best);
        if (idx_out)
            idx_out[n] = kb;
        if (e1_out)
            e1_out[n] = E[kb];
        if (e2_out)
            e2_out[n] = second;
        if (err_out)
            err_out[n] = (float)E[kb];
        if (amax_out) {
            float s[126];
            oracle_candidate_scales(amax[g], s);
            amax_out[n] = 6.0f * s[kb];
        }
    }
}

/* ====================================================================== */
/* Ragged / streaming Hessian accumulation ([LHG] "Entry API and          */
/* calibration flow", phase 2: forward hooks capture each linear layer's  */
/* inputs batch by batch and accumulate X^T X per module; MoE experts see  */
/* only the tokens routed to them, so their token counts differ and may   */
/* be zero; phase 3 uses the per-block Hessian normalised by the tokens).  */
/* Readings:                                                               */
/*   R12 x is token-major, rows offsets[g] .. offsets[g+1]-1 belong to     */
/*       group g (expert g); n_g = offsets[g+1] - offsets[g].              */
/*   R13 without counts: H_g = S_g / n_g, S_g = sum over the group's rows   */
/*       of x_t x_t^T (block diagonal); a group with n_g = 0 keeps its old */
/*       H (the caller's fallback, e.g. the identity = plain MSE).         */
/*   R14 with counts (a running mean over batches): n_old = counts[g],     */
/*       H_g = (n_old H_g + S_g) / (n_old + n_g), counts[g] = n_old + n_g; */
/*       unchanged while n_old + n_g = 0.                                  */
/* Outputs are compact per selected flat block g * (c_in/16) + b; h_old    */
/* (compact, fp32) is the previous H of those blocks.  offsets must be     */
/* nondecreasing and within x's rows (callers clamp them first).           */
/* ====================================================================== */
void oracle_hessian_ragged(const void *x, int dtype, int64_t c_in, int64_t ld_x,
                           const int64_t *offsets, int64_t n_groups, const int64_t *counts,
                           const int64_t *sel, int64_t n_sel, const float *h_old, double *h64,
                           float *h32)
{
    const int64_t nb = c_in / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_sel; ++n) {
        const int64_t g = sel[n] / nb, b = sel[n] % nb;
        const int64_t r0 = offsets[g], r1 = offsets[g + 1];
        const int64_t ng = r1 - r0;
        const int64_t nold = counts ? counts[g] : 0;
        for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
                const int64_t ci = 16 * b + i, cj = 16 * b + j;
                double acc = 0.0;
                for (int64_t t = r0; t < r1; ++t)
                    acc += widen(x, dtype, t * ld_x + ci) * widen(x, dtype, t * ld_x + cj);
                const double old = (double)h_old[n * 256 + i * 16 + j];
                double v;
                if (nold + ng == 0 || (!counts && ng == 0))
                    v = old;
                else if (counts)
                    v = ((double)nold * old + acc) / (double)(nold + ng);
                else
                    v = acc / (double)ng;
                if (h64)
                    h64[n * 256 + i * 16 + j] = v;
                h32[n * 256 + i * 16 + j] = (float)v;
            }
    }
}

/* ====================================================================== */
/* Approximation diagnostics ([LHG] "Algorithm principle": the layer's    */
/* output error is E = ||Delta X||_F^2 = tr(Delta X X^T Delta^T); Local-  */
/* Hessian keeps only the 16x16 diagonal blocks of X X^T.  "How scaling   */
/* reshapes the weight distribution": the histogram of W/s, the values    */
/* fed to the E2M1 rounding, per scale rule).                             */
/* Readings:                                                               */
/*   R15 full Hessian H = alpha X X^T (C_in x C_in), alpha = 1/N, so that  */
/*       (q - w) H (q - w)^T summed over rows is ||Delta X||_F^2 / N, the  */
/*       normalisation of the local Hessians.                              */
/*   R16 histogram value x = fl32(|w| / s_k) with the block's chosen k (the */
/*       cast's own quotient); bin = floor(fl32(x * bins_per_unit)), values */
/*       at or past n_bins go to one overflow bin n_bins; s = 0 gives x = 0.*/
/* ====================================================================== */

/* Full Hessian of one group, channel-major x[c * ld_x + t], fp64:
 * h[i * c_in + j] = alpha * sum_t x[i][t] x[j][t]. */
void oracle_full_hessian(const void *x, int dtype, int64_t c_in, int64_t n_tok, int64_t ld_x,
                         double alpha, double *h)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < c_in; ++i)
        for (int64_t j = 0; j < c_in; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < n_tok; ++t)
                acc += widen(x, dtype, i * ld_x + t) * widen(x, dtype, j * ld_x + t);
            h[i * c_in + j] = alpha * acc;
        }
}

/* Output error of the selected rows of one group: e[n] = d H d^T with
 * d = q_row - w_row (fp64 from the fp32 q and the widened w) and the fp32
 * full Hessian h [c_in][c_in]. */
void oracle_output_error(const void *w, int dtype, const float *q, int64_t c_in, int64_t ld_w,
                         int64_t ld_q, const float *h, const int64_t *rows, int64_t n_rows,
                         double *e)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_rows; ++n) {
        const int64_t r = rows[n];
        double acc = 0.0;
        for (int64_t i = 0; i < c_in; ++i) {
            const double di = (double)q[r * ld_q + i] - widen(w, dtype, r * ld_w + i);
            if (di == 0.0)
                continue;
            double row = 0.0;
            for (int64_t j = 0; j < c_in; ++j) {
                const double dj = (double)q[r * ld_q + j] - widen(w, dtype, r * ld_w + j);
                row += (double)h[i * c_in + j] * dj;
            }
            acc += di * row;
        }
        e[n] = acc;
    }
}

/* Histogram of x = fl32(|w| / s_k) over one group's weights with the given
 * per-block candidate indices; counts [n_bins + 1] are added to. */
void oracle_scaled_histogram(const void *w, int dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                             const uint8_t *idx, float g, int32_t n_bins, float bins_per_unit,
                             uint64_t *counts)
{
    float s[126];
    oracle_candidate_scales(g, s);
    const int64_t nb = c_in / 16;
    for (int64_t r = 0; r < c_out; ++r)
        for (int64_t c = 0; c < c_in; ++c) {
            const float sk = s[idx[r * nb + c / 16]];
            const float a = fabsf(widen_f32(w, dtype, r * ld_w + c));
            const float x = (sk == 0.0f) ? 0.0f : a / sk;
            const float y = x * bins_per_unit;
            int64_t bin = (y >= (float)n_bins) ? n_bins : (int64_t)floorf(y);
            counts[bin] += 1;
        }
}

/* ====================================================================== */
/* GPTQ rounding with fixed Local-Hessian scales ([LHG] "Combining with    */
/* GPTQ": Local-Hessian chooses the block scales, GPTQ then replaces the   */
/* round-to-nearest step to minimise the layer output error; the two are   */
/* orthogonal).  The GPTQ steps follow the published method (Frantar et    */
/* al., ICLR 2023): columns are quantised in order and each column's       */
/* rounding error is fed to the not-yet-quantised columns through the      */
/* upper Cholesky factor U of the inverse Hessian (H^-1 = U^T U).          */
/* Readings:                                                               */
/*   R17 H = the full Hessian X X^T / N (any positive factor gives the same */
/*       result), damped: H' = H + 0.01 * mean(diag H) * I, or I when the  */
/*       diagonal is all zero.                                             */
/*   R18 per output row, for i = 0 .. C_in-1: x = w_i (the running value),  */
/*       q_i = Q(x, s) with the block's fixed scale (the cast of R3),       */
/*       e = (x - q_i) / U_ii, and w_j -= e U_ij for j > i.  Each w_j thus  */
/*       receives its updates in increasing i.                              */
/*   R19 precision: the fp32 sweep (the kernel's precision, which decides   */
/*       the codes) takes x, the cast and e in fp32 and each update as one  */
/*       fused multiply-add w_j = fma(-e, U_ij, w_j) in increasing i, with  */
/*       U given as fp32; the fp64 sweep does the same steps in fp64.       */
/* ====================================================================== */

/* U (fp64, upper, row-major n x n) with H'^-1 = U^T U from the fp32 full
 * Hessian h (n x n row-major).  Uses H' = R R^T with R upper (a Cholesky
 * factorisation taken from the last row and column backwards), then
 * U = R^-1.  Returns 0, or -1 if H' is not positive definite. */
int oracle_gptq_u(const float *h, int64_t n, double damp, double *U)
{
    double *Hp = (double *)calloc((size_t)(n * n), sizeof(double));
    double *R = (double *)calloc((size_t)(n * n), sizeof(double));
    if (!Hp || !R) {
        free(Hp);
        free(R);
        return -1;
    }
    double mean = 0.0;
    for (int64_t i = 0; i < n; ++i)
        mean += (double)h[i * n + i];
    mean /= (double)n;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j)
            Hp[i * n + j] = (mean == 0.0) ? (i == j ? 1.0 : 0.0) : (double)h[i * n + j];
    if (mean != 0.0)
        for (int64_t i = 0; i < n; ++i)
            Hp[i * n + i] += damp * mean;
    /* backward Cholesky: H' = R R^T, R upper */
    for (int64_t j = n - 1; j >= 0; --j) {
        double d = Hp[j * n + j];
        for (int64_t k = j + 1; k < n; ++k)
            d -= R[j * n + k] * R[j * n + k];
        if (!(d > 0.0)) {
            free(Hp);
            free(R);
            return -1;
        }
        const double rjj = sqrt(d);
        R[j * n + j] = rjj;
        for (int64_t i = 0; i < j; ++i) {
            double v = Hp[i * n + j];
            for (int64_t k = j + 1; k < n; ++k)
                v -= R[i * n + k] * R[j * n + k];
            R[i * n + j] = v / rjj;
        }
    }
    /* U = R^-1 (upper): solve R U = I column by column, bottom-up */
    memset(U, 0, sizeof(double) * (size_t)(n * n));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < n; ++c)
        for (int64_t i = c; i >= 0; --i) {
            double v = (i == c) ? 1.0 : 0.0;
            for (int64_t k = i + 1; k <= c; ++k)
                v -= R[i * n + k] * U[k * n + c];
            U[i * n + c] = v / R[i * n + i];
        }
    free(Hp);
    free(R);
    return 0;
}

/* GPTQ sweep of the selected rows of one group with fixed per-block
 * candidate indices idx [c_out][c_in/16] and global amax g.  U32 (fp32) is
 * used by the fp32 sweep (precision 32), U64 (fp64) by the fp64 sweep
 * (precision 64).  q_out [n_rows][c_in] fp32. */
void oracle_gptq_sweep(const void *w, int dtype, int64_t c_in, int64_t ld_w, const uint8_t *idx,
                       float g, const float *U32, const double *U64, int precision,
                       const int64_t *rows, int64_t n_rows, float *q_out)
{
    float s[126];
    oracle_candidate_scales(g, s);
    const int64_t nb = c_in / 16;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < n_rows; ++n) {
        const int64_t r = rows[n];
        if (precision == 32) {
            float *wr = (float *)malloc(sizeof(float) * (size_t)c_in);
            for (int64_t i = 0; i < c_in; ++i)
                wr[i] = widen_f32(w, dtype, r * ld_w + i);
            for (int64_t i = 0; i < c_in; ++i) {
                const float x = wr[i];
                const float q = oracle_quantize(x, s[idx[r * nb + i / 16]], 0);
                q_out[n * c_in + i] = q;
                const float e = (x - q) / U32[i * c_in + i];
                for (int64_t j = i + 1; j < c_in; ++j)
                    wr[j] = fmaf(-e, U32[i * c_in + j], wr[j]);
            }
            free(wr);
        } else {
            double *wr = (double *)malloc(sizeof(double) * (size_t)c_in);
            for (int64_t i = 0; i < c_in; ++i)
                wr[i] = widen(w, dtype, r * ld_w + i);
            for (int64_t i = 0; i < c_in; ++i) {
                const float x = (float)wr[i];
                const float q = oracle_quantize(x, s[idx[r * nb + i / 16]], 0);
                q_out[n * c_in + i] = q;
                const double e = (wr[i] - (double)q) / U64[i * c_in + i];
                for (int64_t j = i + 1; j < c_in; ++j)
                    wr[j] -= e * U64[i * c_in + j];
            }
            free(wr);
        }
    }
}
