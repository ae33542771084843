/*
 * NVFP4 block-scaled batched GEMV -- CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load or call this library. The GPU library never links it,
 * includes it or calls it, and this file shares no code, table or header with
 * the GPU library.
 *
 * What is computed (kernelbot NVFP4 GEMV, submission 103289, `cute_kernel`:
 * every k contributes the product a * sfa * b * sfb of the four decoded
 * operands, the products are summed over k for one output row, and the sum is
 * cast to float16):
 *
 *   c[l][m] = fp16( sum_{k<K} e2m1(A[l][m][k]) * e4m3(SFA[l][m][k/16])
 *                            * e2m1(B[l][k])    * e4m3(SFB[l][k/16]) )
 *
 * Every product is exact in binary: e2m1 values are multiples of 2^-1 and
 * e4m3 values multiples of 2^-9, so each product is an integer multiple of
 * 2^-20 below 2^23 in magnitude. The oracle therefore forms the sum exactly,
 * as an int64 count of 2^-20 units (safe for K <= 2^20), and rounds it once to
 * float16 with round-to-nearest-even (IEEE cast semantics, overflow to inf).
 * Alongside it keeps a plain fp64 sum and the fp64 sum of |products|, which
 * the parity tolerance uses.
 *
 * Optional global scale (the per-tensor float32 scale of NVFP4's two-level
 * scaling, mentioned in submission 69575's description of the format and
 * applied nowhere on the pages): c = fp16(alpha * sum). alpha is a finite
 * float32, alpha = ma * 2^ea with a 24-bit integer ma, so alpha * sum is the
 * exact integer |sum| * ma (below 2^87, formed in 128 bits) times a power of
 * two, rounded once. alpha = 1 gives the plain result.
 *
 * Operand formats (the `cute_kernel` module constants name them:
 * Float4E2M1FN elements, Float8E4M3FN scales, 16 elements per scale):
 *   E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf or NaN.
 *   E4M3 "FN": 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
 *   subnormal; 0x7F and 0xFF are NaN; no inf.
 *
 * Scale layouts:
 *   plain   SFA[l][m][kb]  at  (l*M + m)*(K/16) + kb
 *   blocked the 128x4 tiled layout of submission 69953 `to_blocked_batch`
 *           (see nvo_sf_offset_blocked below for the derivation).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decode */

/* E2M1 value of a 4-bit code, from the format definition. */
double nvo_e2m1(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3 (FN) value of an 8-bit code, from the format definition. */
double nvo_e4m3(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

static double g_e2m1[16];
static double g_e4m3[256];
static int64_t g_e2m1_q[16];   /* 2 * e2m1, an integer in [-12, 12]          */
static int64_t g_e4m3_q[256];  /* 512 * e4m3, an integer in [-229376, 229376] */
static pthread_once_t g_once = PTHREAD_ONCE_INIT;

static void init_tables(void)
{
    for (unsigned c = 0; c < 16; ++c) {
        g_e2m1[c] = nvo_e2m1(c);
        g_e2m1_q[c] = (int64_t)(g_e2m1[c] * 2.0);
    }
    for (unsigned c = 0; c < 256; ++c) {
        g_e4m3[c] = nvo_e4m3(c);
        g_e4m3_q[c] = isnan(g_e4m3[c]) ? 0 : (int64_t)(g_e4m3[c] * 512.0);
    }
}

void nvo_tables(double *e2m1_out16, double *e4m3_out256)
{
    pthread_once(&g_once, init_tables);
    if (e2m1_out16)
        memcpy(e2m1_out16, g_e2m1, sizeof g_e2m1);
    if (e4m3_out256)
        memcpy(e4m3_out256, g_e4m3, sizeof g_e4m3);
}

/* ---------------------------------------------------------- scale layout */

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Plain [rows][nkb] scale matrix. */
int64_t nvo_sf_offset_plain(int64_t r, int64_t kb, int64_t rows, int64_t nkb)
{
    (void)rows;
    return r * nkb + kb;
}

/*
 * Blocked layout, from the view chain of submission 69953 `to_blocked_batch`
 * applied to the padded (128*nrb) x (4*ncb) matrix:
 *   view(nrb,128,ncb,4).permute(0,2,1,3)  -> tile t = rb*ncb + cb holds the
 *       128x4 sub-matrix rows rb*128.., columns cb*4..; element (ri, ci)
 *   reshape(-1,4,32,4)                    -> ri = 32*i4 + i32: index (i4,i32,ci)
 *   transpose(1,2).reshape(-1,32,16)      -> (i32, i4, ci): offset i32*16+i4*4+ci
 * so element (r, kb) lands at
 *   (rb*ncb + cb)*512 + (r%32)*16 + ((r%128)/32)*4 + kb%4,
 * with rb = r/128, cb = kb/4.
 */
int64_t nvo_sf_offset_blocked(int64_t r, int64_t kb, int64_t rows, int64_t nkb)
{
    int64_t ncb = cdiv(nkb, 4);
    (void)rows;
    return ((r / 128) * ncb + kb / 4) * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4 + kb % 4;
}

int64_t nvo_sf_batch_bytes(int layout, int64_t rows, int64_t nkb)
{
    if (layout == 0)
        return rows * nkb;
    return cdiv(rows, 128) * cdiv(nkb, 4) * 512;
}

int64_t nvo_sf_offset(int layout, int64_t r, int64_t kb, int64_t rows, int64_t nkb)
{
    return layout == 0 ? nvo_sf_offset_plain(r, kb, rows, nkb)
                       : nvo_sf_offset_blocked(r, kb, rows, nkb);
}

/*
 * Reblock plain scales [L][rows][K/16] into the blocked layout (submission
 * 69953 `to_blocked_batch`, the map above): every scale is written to its
 * blocked byte, every padding byte (row >= rows or column >= K/16) is 0.
 * out holds L * nvo_sf_batch_bytes(1, rows, K/16) bytes. Returns 0, or -1 for
 * invalid arguments.
 */
int nvo_reblock(const uint8_t *plain, int64_t rows, int64_t K, int64_t L, uint8_t *out)
{
    if (!plain || !out || rows < 1 || L < 1 || K < 32 || K % 32 != 0)
        return -1;
    const int64_t nkb = K / 16;
    const int64_t in_batch = rows * nkb, out_batch = nvo_sf_batch_bytes(1, rows, nkb);
    memset(out, 0, (size_t)(L * out_batch));
    for (int64_t l = 0; l < L; ++l)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t kb = 0; kb < nkb; ++kb)
                out[l * out_batch + nvo_sf_offset_blocked(r, kb, rows, nkb)] =
                    plain[l * in_batch + r * nkb + kb];
    return 0;
}

/* ------------------------------------------------------- fp16 rounding */

static int msb64(uint64_t x)
{
    int p = 63;
    while (!(x >> p))
        --p;
    return p;
}

/* mag / 2^sh rounded to nearest, ties to even (sh <= 0 shifts left, exactly). */
static uint64_t rne_shift(uint64_t mag, int sh)
{
    uint64_t q, rem, half;
    if (sh <= 0)
        return mag << (-sh);
    if (sh > 64)
        return 0;
    if (sh == 64)
        return mag > (UINT64_C(1) << 63) ? 1 : 0;
    q = mag >> sh;
    rem = mag & ((UINT64_C(1) << sh) - 1);
    half = UINT64_C(1) << (sh - 1);
    if (rem > half || (rem == half && (q & 1)))
        ++q;
    return q;
}

/*
 * IEEE binary16 bits of (neg ? -1 : 1) * mag * 2^e2, rounded to nearest, ties
 * to even; magnitudes that round to 65536 or more become inf. An exact zero
 * gives a zero of the given sign.
 */
uint16_t nvo_fp16_round(int neg, uint64_t mag, int e2)
{
    uint16_t sign = neg ? 0x8000u : 0u;
    int p, E;
    uint64_t sig;
    if (mag == 0)
        return sign;
    p = msb64(mag);
    E = p + e2;                /* value in [2^E, 2^(E+1)) */
    if (E >= 16)
        return sign | 0x7C00u;
    if (E >= -14) {            /* normal: keep 11 significant bits */
        sig = rne_shift(mag, p - 10);
        if (sig == 2048) {
            sig = 1024;
            ++E;
        }
        if (E >= 16)
            return sign | 0x7C00u;
        return sign | (uint16_t)(((E + 15) << 10) | (sig & 0x3FFu));
    }
    /* subnormal: a count of 2^-24 units; 1024 units is the smallest normal */
    sig = rne_shift(mag, -(e2 + 24));
    return sign | (uint16_t)sig;
}

uint16_t nvo_fp16_from_double(double x)
{
    int e;
    double f;
    uint64_t mag;
    int neg = signbit(x) ? 1 : 0;
    if (isnan(x))
        return 0x7E00u;
    if (isinf(x))
        return (uint16_t)((neg ? 0x8000u : 0u) | 0x7C00u);
    if (x == 0.0)
        return neg ? 0x8000u : 0u;
    f = frexp(fabs(x), &e);                  /* |x| = f * 2^e, f in [0.5, 1) */
    mag = (uint64_t)ldexp(f, 53);            /* exact: 53-bit integer */
    return nvo_fp16_round(neg, mag, e - 53);
}

void nvo_fp16_from_double_n(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = nvo_fp16_from_double(x[i]);
}

double nvo_fp16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 0x3FF;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp(1024.0 + (double)m, e - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------ GEMV */

typedef struct {
    const uint8_t *a, *b, *sfa, *sfb;
    int64_t M, K, L;
    int layout;
    float alpha;
} problem_t;

/* fp16 of alpha * (sum in 2^-20 units), exactly rounded (see the header). */
static uint16_t round_scaled(int64_t exact, float alpha)
{
    int ea;
    const float fa = frexpf(fabsf(alpha), &ea);         /* |alpha| = fa * 2^ea, fa in [0.5, 1) */
    const uint64_t ma = (uint64_t)ldexpf(fa, 24);       /* exact 24-bit integer */
    const int neg = (exact < 0) != (signbit(alpha) != 0);
    const uint64_t mag_s = exact < 0 ? (uint64_t)(-exact) : (uint64_t)exact;
    unsigned __int128 prod = (unsigned __int128)mag_s * ma;
    int e2 = -20 + ea - 24;
    int sh = 0;
    uint64_t mag;
    if (alpha == 0.0f || mag_s == 0)
        return neg ? 0x8000u : 0u;
    /* keep 62 significant bits and a sticky bit: rounding to 11 bits below
       them is unchanged */
    while ((prod >> (62 + sh)) != 0)
        ++sh;
    if (sh > 0) {
        const unsigned __int128 lost = prod & ((((unsigned __int128)1) << sh) - 1);
        mag = (uint64_t)(prod >> sh) | (lost != 0 ? 1u : 0u);
    } else {
        mag = (uint64_t)prod;
    }
    e2 += sh;
    return nvo_fp16_round(neg, mag, e2);
}

typedef struct {
    uint16_t c;
    double s_f64, s_abs;
    int64_t s_exact;
    uint8_t nan;
} row_result_t;

static unsigned nibble(const uint8_t *p, int64_t k)
{
    uint8_t byte = p[k >> 1];
    return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 0xF);
}

static row_result_t gemv_row(const problem_t *pb, int64_t row)
{
    const int64_t M = pb->M, K = pb->K, nkb = K / 16;
    const int64_t l = row / M, m = row % M;
    const uint8_t *arow = pb->a + (l * M + m) * (K / 2);
    const uint8_t *brow = pb->b + l * (K / 2);
    const uint8_t *sfa = pb->sfa + l * nvo_sf_batch_bytes(pb->layout, M, nkb);
    const uint8_t *sfb = pb->sfb + l * nvo_sf_batch_bytes(pb->layout, 1, nkb);
    row_result_t r;
    double s = 0.0, sabs = 0.0;
    int64_t exact = 0;
    int nan = 0;

    for (int64_t k = 0; k < K; ++k) {
        unsigned ac = nibble(arow, k), bc = nibble(brow, k);
        unsigned sa = sfa[nvo_sf_offset(pb->layout, m, k / 16, M, nkb)];
        unsigned sb = sfb[nvo_sf_offset(pb->layout, 0, k / 16, 1, nkb)];
        double t = g_e2m1[ac] * g_e4m3[sa] * g_e2m1[bc] * g_e4m3[sb];
        if (isnan(t)) {
            nan = 1;
            continue;
        }
        s += t;
        sabs += fabs(t);
        exact += g_e2m1_q[ac] * g_e4m3_q[sa] * g_e2m1_q[bc] * g_e4m3_q[sb];
    }
    r.c = nan ? (uint16_t)0x7E00u : round_scaled(exact, pb->alpha);
    r.s_f64 = nan ? NAN : s * (double)pb->alpha;
    r.s_abs = sabs * fabs((double)pb->alpha);
    r.s_exact = exact;
    r.nan = (uint8_t)nan;
    return r;
}

typedef struct {
    problem_t pb;
    const int64_t *rows;          /* NULL: rows row_begin..row_end-1 */
    int64_t begin, end;           /* range of output slots */
    uint16_t *c;
    double *s_f64, *s_abs;
    int64_t *s_exact;
    uint8_t *nan_flag;
} job_t;

static void *gemv_worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    for (int64_t i = j->begin; i < j->end; ++i) {
        row_result_t r = gemv_row(&j->pb, j->rows ? j->rows[i] : i);
        j->c[i] = r.c;
        if (j->s_f64) j->s_f64[i] = r.s_f64;
        if (j->s_abs) j->s_abs[i] = r.s_abs;
        if (j->s_exact) j->s_exact[i] = r.s_exact;
        if (j->nan_flag) j->nan_flag[i] = r.nan;
    }
    return NULL;
}

static int run_jobs(const problem_t *pb, const int64_t *rows, int64_t nout, int nthreads,
                    uint16_t *c, double *s_f64, double *s_abs, int64_t *s_exact, uint8_t *nan_flag)
{
    pthread_t tid[256];
    job_t jobs[256];
    int n = nthreads < 1 ? 1 : (nthreads > 256 ? 256 : nthreads);
    int started = 1;
    if (nout < 1)
        return 0;
    if (n > nout)
        n = (int)nout;
    for (int i = 0; i < n; ++i) {
        job_t *j = &jobs[i];
        j->pb = *pb;
        j->rows = rows;
        j->begin = nout * i / n;
        j->end = nout * (i + 1) / n;
        j->c = c; j->s_f64 = s_f64; j->s_abs = s_abs; j->s_exact = s_exact;
        j->nan_flag = nan_flag;
    }
    for (int i = 1; i < n; ++i) {
        if (pthread_create(&tid[i], NULL, gemv_worker, &jobs[i]) != 0)
            break;                       /* run the rest on this thread */
        ++started;
    }
    gemv_worker(&jobs[0]);
    for (int i = 1; i < started; ++i)
        pthread_join(tid[i], NULL);
    for (int i = started; i < n; ++i)     /* jobs whose thread could not start */
        gemv_worker(&jobs[i]);
    return 0;
}

static int valid(const uint8_t *a, const uint8_t *b, const uint8_t *sfa, const uint8_t *sfb,
                 int64_t M, int64_t K, int64_t L, int layout, float alpha, const uint16_t *c)
{
    return M >= 1 && L >= 1 && K >= 32 && K % 32 == 0 && K <= (INT64_C(1) << 20) &&
           (layout == 0 || layout == 1) && isfinite(alpha) && a && b && sfa && sfb && c;
}

/*
 * Full batched GEMV. Rows (l, m) are split over `nthreads` threads; each row
 * is summed in increasing k, so the result does not depend on the thread
 * count. c, s_f64, s_abs, s_exact and nan_flag hold L*M entries at index
 * l*M + m; all but c may be NULL. s_exact is the exact unscaled sum in units
 * of 2^-20; c, s_f64 and s_abs include the global scale alpha.
 * Returns 0, or -1 for invalid arguments.
 */
int nvo_gemv(const uint8_t *a, const uint8_t *b, const uint8_t *sfa, const uint8_t *sfb,
             int64_t M, int64_t K, int64_t L, int layout, float alpha, int nthreads,
             uint16_t *c, double *s_f64, double *s_abs, int64_t *s_exact, uint8_t *nan_flag)
{
    problem_t pb;
    if (!valid(a, b, sfa, sfb, M, K, L, layout, alpha, c))
        return -1;
    pthread_once(&g_once, init_tables);
    pb.a = a; pb.b = b; pb.sfa = sfa; pb.sfb = sfb;
    pb.M = M; pb.K = K; pb.L = L; pb.layout = layout; pb.alpha = alpha;
    return run_jobs(&pb, NULL, M * L, nthreads, c, s_f64, s_abs, s_exact, nan_flag);
}

/* Selected rows only (spot checks at full size): rows[i] = l*M + m, output slot i. */
int nvo_gemv_rows(const uint8_t *a, const uint8_t *b, const uint8_t *sfa, const uint8_t *sfb,
                  int64_t M, int64_t K, int64_t L, int layout, float alpha, const int64_t *rows,
                  int64_t nrows, int nthreads, uint16_t *c, double *s_f64, double *s_abs,
                  int64_t *s_exact, uint8_t *nan_flag)
{
    problem_t pb;
    if (!valid(a, b, sfa, sfb, M, K, L, layout, alpha, c) || !rows)
        return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M * L)
            return -1;
    pthread_once(&g_once, init_tables);
    pb.a = a; pb.b = b; pb.sfa = sfa; pb.sfb = sfb;
    pb.M = M; pb.K = K; pb.L = L; pb.layout = layout; pb.alpha = alpha;
    return run_jobs(&pb, rows, nrows, nthreads, c, s_f64, s_abs, s_exact, nan_flag);
}
