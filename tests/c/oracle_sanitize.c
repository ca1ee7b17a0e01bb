/* Drives every entry point of the CPU oracle on small ragged inputs under
 * AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure;
 * built and run by tests/test_oracle_sanitize.py).  The oracle source is
 * compiled into this program, so every access it makes is checked: buffer
 * bounds of the strided, grouped and selected layouts, the compact output
 * indexing, the ragged offsets (including clamped and decreasing ones) and
 * the GPTQ factorisation's scratch.  Prints "ok" and a checksum that keeps
 * the results live. */
#include "../../oracle/lh_oracle.c"

#include <stdio.h>

static uint64_t st = 0x2545F4914F6CDD1Dull;
static double uni(void)
{
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 9007199254740992.0;
}
static double gauss(void)
{
    double u = uni() + 1e-12, v = uni();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
/* bf16 bits of a float (truncation is enough for test data) */
static uint16_t bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double sink = 0.0;

static void layer(int dtype, int64_t G, int64_t c_out, int64_t c_in, int64_t n_tok, int64_t pad)
{
    const int64_t nb = c_in / 16, ld_w = c_in + pad, ld_x = n_tok + pad;
    const int64_t gsw = c_out * ld_w, gsx = c_in * ld_x, nblk = G * c_out * nb;
    const size_t es = dtype == 0 ? 4 : 2;
    void *w = malloc((size_t)(G * gsw) * es), *x = malloc((size_t)(G * gsx) * es);
    for (int64_t i = 0; i < G * gsw; ++i) {
        float v = (float)(0.02 * gauss());
        if (dtype == 0) ((float *)w)[i] = v; else ((uint16_t *)w)[i] = bf16(v);
    }
    for (int64_t i = 0; i < G * gsx; ++i) {
        float v = (float)gauss();
        if (dtype == 0) ((float *)x)[i] = v; else ((uint16_t *)x)[i] = bf16(v);
    }
    float *amax = malloc((size_t)G * sizeof(float));
    oracle_absmax(w, dtype, c_out, c_in, ld_w, G, gsw, amax);
    int64_t *hsel = malloc((size_t)(G * nb) * sizeof(int64_t));
    for (int64_t i = 0; i < G * nb; ++i) hsel[i] = i;
    double *h64 = malloc((size_t)(G * nb * 256) * sizeof(double));
    float *h32 = calloc((size_t)(G * nb * 256), sizeof(float));
    oracle_hessian(x, dtype, 0, c_in, n_tok, ld_x, gsx, 1.0 / (double)n_tok, 0.0, hsel, G * nb, h64, h32);
    oracle_hessian(x, dtype, 0, c_in, n_tok, ld_x, gsx, 1.0, 1.0, hsel, G * nb, h64, h32);  /* beta != 0 */
    int64_t *sel = malloc((size_t)nblk * sizeof(int64_t));
    for (int64_t i = 0; i < nblk; ++i) sel[i] = i;
    int32_t *idx = malloc((size_t)nblk * 4), *probe = malloc((size_t)nblk * 4);
    double *e1 = malloc((size_t)nblk * 8), *e2 = malloc((size_t)nblk * 8), *ep = malloc((size_t)nblk * 8);
    double *sp = malloc((size_t)nblk * 8), *sb = malloc((size_t)nblk * 8);
    float *err = malloc((size_t)nblk * 4), *bam = malloc((size_t)nblk * 4);
    for (int64_t i = 0; i < nblk; ++i) probe[i] = (int32_t)(uni() * 126.0);
    oracle_sweep(w, dtype, c_out, c_in, ld_w, gsw, h32, nb * 256, amax, sel, nblk, idx, e1, e2, err, bam, probe,
                 ep, sp, sb);
    oracle_sweep(w, dtype, c_out, c_in, ld_w, gsw, h32, nb * 256, amax, sel, nblk, idx, 0, 0, 0, 0, 0, 0, 0, 0);
    uint8_t *idx8 = malloc((size_t)nblk);
    for (int64_t i = 0; i < nblk; ++i) idx8[i] = (uint8_t)idx[i];
    float *q = malloc((size_t)nblk * 16 * 4);
    uint8_t *packed = malloc((size_t)nblk * 8), *code = malloc((size_t)nblk);
    oracle_fake_quant(w, dtype, c_out, c_in, ld_w, gsw, idx8, amax, sel, nblk, q, packed, code);
    for (int rule = 0; rule < 4; ++rule) {
        oracle_select(rule, w, dtype, c_out, c_in, ld_w, gsw, h32, nb * 256, amax, sel, nblk, idx, e1, e2, err, bam,
                      probe, ep, sp, sb);
        oracle_select(rule, w, dtype, c_out, c_in, ld_w, gsw, 0, 0, amax, sel, nblk, idx, e1, e2, err, bam, 0, ep, 0,
                      sb);
    }
    /* group 0 only: full Hessian, output error, histogram, GPTQ */
    double *hf = malloc((size_t)(c_in * c_in) * 8);
    oracle_full_hessian(x, dtype, c_in, n_tok, ld_x, 1.0 / (double)n_tok, hf);
    float *hf32 = malloc((size_t)(c_in * c_in) * 4);
    for (int64_t i = 0; i < c_in * c_in; ++i) hf32[i] = (float)hf[i];
    int64_t *rows = malloc((size_t)c_out * 8);
    for (int64_t r = 0; r < c_out; ++r) rows[r] = c_out - 1 - r;
    double *oe = malloc((size_t)c_out * 8);
    oracle_output_error(w, dtype, q, c_in, ld_w, c_in, hf32, rows, c_out, oe);
    uint64_t counts[33] = {0};
    oracle_scaled_histogram(w, dtype, c_out, c_in, ld_w, idx8, amax[0], 32, 4.0f, counts);
    double *U = malloc((size_t)(c_in * c_in) * 8);
    float *U32 = malloc((size_t)(c_in * c_in) * 4);
    if (oracle_gptq_u(hf32, c_in, 0.01, U) == 0) {
        for (int64_t i = 0; i < c_in * c_in; ++i) U32[i] = (float)U[i];
        float *gq = malloc((size_t)(c_out * c_in) * 4);
        oracle_gptq_sweep(w, dtype, c_in, ld_w, idx8, amax[0], U32, 0, 32, rows, c_out, gq);
        oracle_gptq_sweep(w, dtype, c_in, ld_w, idx8, amax[0], 0, U, 64, rows, c_out, gq);
        sink += gq[0];
        free(gq);
    }
    for (int64_t i = 0; i < nblk; ++i) sink += e1[i] + err[i] + q[16 * i] + packed[8 * i] + code[i];
    sink += oe[0] + (double)counts[0] + h64[0];
    free(w); free(x); free(amax); free(hsel); free(h64); free(h32); free(sel); free(idx); free(probe);
    free(e1); free(e2); free(ep); free(sp); free(sb); free(err); free(bam); free(idx8); free(q); free(packed);
    free(code); free(hf); free(hf32); free(rows); free(oe); free(U); free(U32);
}

static void ragged(int dtype)
{
    const int64_t c_in = 48, ld_x = 56, n_rows = 40, G = 5;
    const size_t es = dtype == 0 ? 4 : 2;
    void *x = malloc((size_t)(n_rows * ld_x) * es);
    for (int64_t i = 0; i < n_rows * ld_x; ++i) {
        float v = (float)gauss();
        if (dtype == 0) ((float *)x)[i] = v; else ((uint16_t *)x)[i] = bf16(v);
    }
    /* empty groups, a group with one row, the last group to the end (the
     * oracle takes nondecreasing offsets inside the buffer; the tests clamp
     * the library's inputs to that before calling it) */
    int64_t offsets[6] = {0, 7, 7, 30, 31, 40};
    int64_t counts[5] = {0, 3, 0, 9, 1};
    const int64_t nsel = G * (c_in / 16);
    int64_t *sel = malloc((size_t)nsel * 8);
    for (int64_t i = 0; i < nsel; ++i) sel[i] = i;
    float *hold = calloc((size_t)(nsel * 256), 4);
    double *h64 = malloc((size_t)(nsel * 256) * 8);
    float *h32 = malloc((size_t)(nsel * 256) * 4);
    oracle_hessian_ragged(x, dtype, c_in, ld_x, offsets, G, counts, sel, nsel, hold, h64, h32);
    oracle_hessian_ragged(x, dtype, c_in, ld_x, offsets, G, 0, sel, nsel, hold, h64, h32);
    sink += h64[0] + h32[nsel * 256 - 1];
    free(x); free(sel); free(hold); free(h64); free(h32);
}

int main(void)
{
    float s[126];
    oracle_candidate_scales(0.0f, s);
    oracle_candidate_scales(3.5f, s);
    for (int c = 0; c < 128; ++c) sink += oracle_e4m3_value(c);
    for (int i = 0; i < 38; ++i) sink += oracle_amax_multiplier(i);
    sink += oracle_e4m3_round_code(1e-30f) + oracle_e4m3_round_code(1e30f) + oracle_e2m1_code(7.0f);
    int code;
    sink += oracle_quantize(-0.3f, 0.1f, &code) + oracle_quantize(0.3f, 0.0f, &code);
    layer(0, 2, 19, 48, 33, 5);
    layer(1, 3, 7, 64, 17, 3);
    layer(1, 1, 5, 16, 1, 0);
    ragged(0);
    ragged(1);
    printf("ok %g\n", sink);
    return 0;
}
