/*
 * Plain CPU oracle for the MXFP4 dequantize-and-multiply path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library, and it is deliberately slow and literal: every weight is
 * decoded by table lookup, every product is summed in fp64, one term at a
 * time, in column order.
 *
 * Sources (the pages this follows, cited by title and section):
 *   [wgpu]  cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs
 *           - module doc (OCP MX FP4: E2M1 codes, E8M0 scale per 32 columns)
 *           - DECODE shader: mx_e2m1, mx_e8m0
 *           - PEROP shader: MxP uniform, mx_scale, mxfp4_mv / mxfp4_mm
 *           - GLOBAL shader: mxg_bf16, dsv4_global_gate_up_mxfp4,
 *             dsv4_global_down_mxfp4
 *           - matmat (host API): out[t*rows + r] = W[r,:] . xs[t*cols ..]
 *           - tests: reference (f64 dot of the dequantized matrix plus
 *             mag = sum |w*x|), payload / scale_plane
 *   [moe]   cortiq-engine 0.8.77, src/qtensor/moe_fast.rs
 *           - gate_up_block: act = silu(g) * u, silu(g) = g / (1 + e^-g)
 *           - down_block: per pair, down . act
 *   [gguf]  rlx-cpu 0.2.17, src/gguf_matmul.rs
 *           - grouped_moe_sort_plan: counting sort of rows by expert
 *
 * Every function carries "parity pinned by" notes naming the tests that
 * check it against something other than itself.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Format decode                                                            */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes for the low three bits of a code; bit 3 is the sign.
 * [wgpu] DECODE shader, mx_e2m1 (values 0 and 0.5 patched, 1..6 from the
 * exponent construction); the same table is the OCP MX FP4 element format.
 * Parity pinned by: test_oracle_format.py (field decode, the shader's bit
 * construction, golden table). */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1(int code)
{
    double m = E2M1_MAGNITUDE[code & 7];
    return (code & 8) ? -m : m; /* code 8 gives -0.0 */
}

/* E8M0 scale: 2^(k-127); 255 is NaN; 0 is 2^-127 (the format has no zero).
 * [wgpu] DECODE shader, mx_e8m0.  Pinned by test_oracle_format.py. */
double orc_e8m0(int k)
{
    if (k == 255)
        return NAN;
    return ldexp(1.0, k - 127);
}

/* Nibble of element (r, c) of a rows x cols tensor.  The code plane holds
 * cols/2 bytes per row; within a 32-column group the four little-endian
 * words hold 8 nibbles each, nibble j of word q being column 8q + j, so the
 * low nibble of a byte is the earlier column.  [wgpu] PEROP shader,
 * mxfp4_mv (word walk) and MxP (code plane first).  Pinned by the one-hot
 * placement tests in test_oracle_layout.py. */
static int code_at(const uint8_t *w, int64_t cols, int64_t r, int64_t c)
{
    uint8_t byte = w[(r * cols + c) / 2];
    return (c & 1) ? (byte >> 4) : (byte & 15);
}

/* E8M0 byte of element (r, c): the scale plane follows the rows*cols/2 code
 * bytes, one byte per (row, group), row-major.  [wgpu] mx_scale and the
 * scale_plane test helper. */
static int scale_at(const uint8_t *w, int64_t rows, int64_t cols, int64_t r, int64_t c)
{
    const uint8_t *plane = w + rows * cols / 2;
    return plane[r * (cols / 32) + c / 32];
}

/* Exact weight value in fp64 (never rounds, never overflows: |v| <= 6 and
 * the exponent stays inside fp64's range).  NaN for scale byte 255. */
static double weight_f64(const uint8_t *w, int64_t rows, int64_t cols, int64_t r, int64_t c)
{
    int k = scale_at(w, rows, cols, r, c);
    if (k == 255)
        return NAN;
    return ldexp(orc_e2m1(code_at(w, cols, r, c)), k - 127);
}

/* Total bytes of one rows x cols MXFP4 tensor: cols/2 code bytes plus
 * cols/32 scale bytes per row (17/32 byte per weight).  -1 when cols is not
 * a multiple of 32 or a size is negative.  [wgpu] MoeBankCodec::lens and the
 * bank_codec_lengths test. */
int64_t orc_nbytes(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0)
        return -1;
    return rows * cols / 2 + rows * (cols / 32);
}

/* Canonical quiet NaN written for every element of a scale-255 group. */
static float canonical_nan_f32(void)
{
    uint32_t bits = 0x7FC00000u;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* fp32 value of one weight: the exact product rounded once to fp32.  Every
 * finite product is exactly representable (at most two significant bits,
 * smallest magnitude 2^-128), so the only rounding is overflow to +-inf,
 * which happens when |v| * 2^(k-127) >= 2^128. */
float orc_dequant_value_f32(int code, int k)
{
    if (k == 255)
        return canonical_nan_f32();
    double v = ldexp(orc_e2m1(code), k - 127);
    if (fabs(v) >= 0x1p128)
        return (float)copysign(INFINITY, v);
    return (float)v;
}

/* Dequantize a whole tensor to fp32, row-major [rows][cols]. */
void orc_dequant_f32(const uint8_t *w, int64_t rows, int64_t cols, float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] =
                orc_dequant_value_f32(code_at(w, cols, r, c), scale_at(w, rows, cols, r, c));
}

/* Round an fp64 value to bfloat16 (8 significant bits, fp32's exponent
 * range, subnormals down to 2^-133), nearest, ties to even; returns the bit
 * pattern.  NaN gives the canonical 0x7FC0.  The pages round fp32 to bf16 by
 * the same rule ([wgpu] GLOBAL shader, mxg_bf16); here the input is fp64 and
 * rounded once.  Pinned by test_oracle_bf16.py. */
uint16_t orc_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                /* quantum of an 8-bit significand */
    if (q < -133)
        q = -133;                 /* subnormal quantum */
    double n = nearbyint(ldexp(a, -q)); /* default mode: ties to even */
    double r = ldexp(n, q);
    if (r >= 0x1p128)
        return sign | 0x7F80;     /* rounded past the largest finite */
    float f = (float)r;           /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return sign | (uint16_t)(bits >> 16);
}

/* orc_bf16_rne over an array (the same rounding, element by element). */
void orc_bf16_rne_n(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(v[i]);
}

/* Bit pattern of a weight in bf16: the fp32 value is exact with at most two
 * significant bits, so it is its own bf16 rounding. */
void orc_dequant_bf16(const uint8_t *w, int64_t rows, int64_t cols, uint16_t *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int k = scale_at(w, rows, cols, r, c);
            if (k == 255) {
                out[r * cols + c] = 0x7FC0;
                continue;
            }
            out[r * cols + c] = orc_bf16_rne(ldexp(orc_e2m1(code_at(w, cols, r, c)), k - 127));
        }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 activations: the activation side of the block-scaled FP4 x FP8     */
/* product.  [wgpu] module doc: the OCP MX family (a shared E8M0 power-of-  */
/* two scale per 32 elements); here with E4M3 elements, as that family      */
/* defines them.                                                            */
/* ------------------------------------------------------------------------ */

/* E4M3 element: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
 * 2..0; exponent field 0 is subnormal, m * 2^-9; S.1111.111 is NaN; there
 * are no infinities; the largest finite magnitude is 1.75 * 2^8 = 448.
 * Pinned by test_oracle_mx8.py (all 256 codes against the field
 * definition). */
double orc_e4m3(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* The E4M3 code nearest to v: the finite magnitude closest to |v| by exact
 * search over the 127 non-negative finite codes, a tie going to the code
 * with an even mantissa; magnitudes beyond 448 therefore saturate to 448;
 * the sign is kept (-0 for negative values that round to zero); NaN gives
 * 0x7F.  Pinned by test_oracle_mx8.py. */
int orc_e4m3_rne(double v)
{
    if (isnan(v))
        return 0x7F;
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) /* the largest finite magnitude is the nearest */
        return sign | 0x7E;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 0x7F; ++c) {
        double d = fabs(a - orc_e4m3(c));
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return sign | best;
}

/* MXFP8 quantization of x [rows][cols] (cols % 32 == 0) into E4M3 codes
 * q [rows][cols] and E8M0 scale bytes s [rows][cols/32], block by block of
 * 32 elements of a row: with a = the largest magnitude of the block, the
 * shared exponent is E = floor(log2 a) - 8 (8: the exponent of E4M3's
 * largest binade), stored as the byte E + 127 clamped to [0, 254]; each
 * element is the E4M3 code nearest to v / 2^E.  The block's largest then
 * lies in [256, 512) and saturates to 448 when above it (up to 1/8 of its
 * magnitude), as the MX conversion rule has it.  A block whose largest
 * magnitude is 0 takes the byte 0 (2^-127) and zero codes; a block holding
 * NaN or an infinity takes 255 (NaN) and zero codes.  Pinned by
 * test_oracle_mx8.py. */
void orc_mxfp8_quantize(const double *x, int64_t rows, int64_t cols, uint8_t *q, uint8_t *s)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < cols / 32; ++g) {
            const double *v = x + r * cols + g * 32;
            uint8_t *qq = q + r * cols + g * 32;
            double a = 0.0;
            int bad = 0;
            for (int i = 0; i < 32; ++i) {
                if (!isfinite(v[i]))
                    bad = 1;
                else if (fabs(v[i]) > a)
                    a = fabs(v[i]);
            }
            if (bad || a == 0.0) {
                s[r * (cols / 32) + g] = bad ? 255 : 0;
                for (int i = 0; i < 32; ++i)
                    qq[i] = 0;
                continue;
            }
            int e2;
            frexp(a, &e2);       /* a = f * 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1 */
            int E = (e2 - 1) - 8;
            int k = E + 127;
            if (k < 0)
                k = 0;
            if (k > 254)
                k = 254;
            E = k - 127;
            s[r * (cols / 32) + g] = (uint8_t)k;
            for (int i = 0; i < 32; ++i)
                qq[i] = (uint8_t)orc_e4m3_rne(ldexp(v[i], -E));
        }
}

/* ------------------------------------------------------------------------ */
/* Dense product: y[t][r] = sum_c W[r][c] * x[t][c], mag = sum |W x|         */
/* ------------------------------------------------------------------------ */

/* [wgpu] matmat: out[t*rows + r] = W[r,:] . xs[t*cols ..]; the tests'
 * reference(): f64 dot of the dequantized matrix with mag = sum |w*x|.
 * x is given in fp64 (fp32 and bf16 inputs convert exactly). */
typedef struct {
    const uint8_t *w;
    int64_t rows, cols;
    const double *x;
    int64_t b;
    const int64_t *row_list; /* NULL: all rows; else n_rows indices */
    int64_t n_rows;
    double *y, *mag;         /* [b][rows] (all rows) or [b][n_rows] (listed) */
    int tid, nthreads;
} gemm_job;

static void *gemm_worker(void *arg)
{
    gemm_job *j = (gemm_job *)arg;
    double *wrow = (double *)malloc(sizeof(double) * (size_t)j->cols);
    if (!wrow)
        return NULL;
    for (int64_t i = j->tid; i < j->n_rows; i += j->nthreads) {
        int64_t r = j->row_list ? j->row_list[i] : i;
        for (int64_t c = 0; c < j->cols; ++c)
            wrow[c] = weight_f64(j->w, j->rows, j->cols, r, c);
        for (int64_t t = 0; t < j->b; ++t) {
            const double *xt = j->x + t * j->cols;
            double s = 0.0, m = 0.0;
            for (int64_t c = 0; c < j->cols; ++c) {
                double p = wrow[c] * xt[c];
                s += p;
                m += fabs(p);
            }
            j->y[t * j->n_rows + i] = s;
            j->mag[t * j->n_rows + i] = m;
        }
    }
    free(wrow);
    return NULL;
}

static void run_gemm(const uint8_t *w, int64_t rows, int64_t cols, const double *x, int64_t b,
                     const int64_t *row_list, int64_t n_rows, double *y, double *mag, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    gemm_job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (gemm_job){w, rows, cols, x, b, row_list, n_rows, y, mag, i, nthreads};
        if (nthreads == 1) {
            gemm_worker(&jobs[i]);
            return;
        }
        pthread_create(&th[i], NULL, gemm_worker, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        pthread_join(th[i], NULL);
}

void orc_gemm(const uint8_t *w, int64_t rows, int64_t cols, const double *x, int64_t b,
              double *y, double *mag, int nthreads)
{
    run_gemm(w, rows, cols, x, b, NULL, rows, y, mag, nthreads);
}

/* Same product for a list of rows only (sampled checks at full size). */
void orc_gemm_rows(const uint8_t *w, int64_t rows, int64_t cols, const double *x, int64_t b,
                   const int64_t *row_list, int64_t n_rows, double *y, double *mag, int nthreads)
{
    run_gemm(w, rows, cols, x, b, row_list, n_rows, y, mag, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Routed expert bank                                                       */
/* ------------------------------------------------------------------------ */

/* Stable counting sort of the (token, slot) pairs p = t*top_k + k by expert
 * id: counts per expert, exclusive offsets, and the pairs listed in (expert,
 * t, k) order.  slot_of_pair[p] is p's position in that list; a pair whose
 * id is outside [0, n_experts) is left out and gets slot -1.
 * [gguf] grouped_moe_sort_plan (counts -> offsets -> ordered scatter).
 * Pinned by test_oracle_moe.py against Python's stable sort. */
void orc_group(const int32_t *ids, int64_t n_pairs, int64_t n_experts, int32_t *counts,
               int32_t *offsets, int32_t *pair_of_slot, int32_t *slot_of_pair)
{
    for (int64_t e = 0; e < n_experts; ++e)
        counts[e] = 0;
    for (int64_t p = 0; p < n_pairs; ++p)
        if (ids[p] >= 0 && ids[p] < n_experts)
            counts[ids[p]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < n_experts; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)calloc((size_t)(n_experts > 0 ? n_experts : 1), sizeof(int32_t));
    for (int64_t p = 0; p < n_pairs; ++p) {
        int32_t e = ids[p];
        if (e < 0 || e >= n_experts) {
            slot_of_pair[p] = -1;
            continue;
        }
        int32_t s = offsets[e] + fill[e]++;
        pair_of_slot[s] = (int32_t)p;
        slot_of_pair[p] = s;
    }
    free(fill);
}

/* Per-pair work of the expert bank, one pair per job step. */
typedef struct {
    const uint8_t *gate, *up, *down;
    int64_t hidden, inter;
    const double *x;     /* [n_tokens][hidden] */
    const int32_t *ids;  /* [n_pairs] */
    int64_t top_k, n_pairs;
    int round_h_bf16;
    double *g, *u, *h;   /* [n_pairs][inter] */
    double *mag_g, *mag_u;
    const double *h_in;  /* down stage input [n_pairs][inter], or NULL: use h */
    double *y, *mag_y;   /* [n_pairs][hidden] */
    int stage;           /* 1: gate/up, 2: down */
    int tid, nthreads;
} moe_job;

/* silu(g) = g / (1 + e^-g).  [moe] gate_up_block; [wgpu]
 * dsv4_global_gate_up_mxfp4 (without the optional limit). */
static double silu(double g) { return g / (1.0 + exp(-g)); }

static void *moe_worker(void *arg)
{
    moe_job *j = (moe_job *)arg;
    int64_t H = j->hidden, I = j->inter;
    int64_t gu_bytes = orc_nbytes(I, H), dn_bytes = orc_nbytes(H, I);
    double *wrow = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double *wrow2 = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    for (int64_t p = j->tid; p < j->n_pairs; p += j->nthreads) {
        int32_t e = j->ids[p];
        if (e < 0)
            continue;
        int64_t t = p / j->top_k;
        if (j->stage == 1) {
            const uint8_t *wg = j->gate + (int64_t)e * gu_bytes;
            const uint8_t *wu = j->up + (int64_t)e * gu_bytes;
            const double *xt = j->x + t * H;
            for (int64_t r = 0; r < I; ++r) {
                for (int64_t c = 0; c < H; ++c) {
                    wrow[c] = weight_f64(wg, I, H, r, c);
                    wrow2[c] = weight_f64(wu, I, H, r, c);
                }
                double sg = 0, mg = 0, su = 0, mu = 0;
                for (int64_t c = 0; c < H; ++c) {
                    double pg = wrow[c] * xt[c], pu = wrow2[c] * xt[c];
                    sg += pg;
                    mg += fabs(pg);
                    su += pu;
                    mu += fabs(pu);
                }
                double hv = silu(sg) * su;
                if (j->round_h_bf16) {
                    uint32_t bits = (uint32_t)orc_bf16_rne(hv) << 16;
                    float f;
                    memcpy(&f, &bits, 4);
                    hv = f;
                }
                j->g[p * I + r] = sg;
                j->u[p * I + r] = su;
                j->h[p * I + r] = hv;
                j->mag_g[p * I + r] = mg;
                j->mag_u[p * I + r] = mu;
            }
        } else {
            const uint8_t *wd = j->down + (int64_t)e * dn_bytes;
            const double *hp = (j->h_in ? j->h_in : j->h) + p * I;
            for (int64_t r = 0; r < H; ++r) {
                double s = 0, m = 0;
                for (int64_t c = 0; c < I; ++c) {
                    double pr = weight_f64(wd, H, I, r, c) * hp[c];
                    s += pr;
                    m += fabs(pr);
                }
                j->y[p * H + r] = s;
                j->mag_y[p * H + r] = m;
            }
        }
    }
    free(wrow);
    free(wrow2);
    return NULL;
}

static void run_moe(moe_job proto, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    moe_job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].tid = i;
        jobs[i].nthreads = nthreads;
    }
    if (nthreads == 1) {
        moe_worker(&jobs[0]);
        return;
    }
    for (int i = 0; i < nthreads; ++i)
        pthread_create(&th[i], NULL, moe_worker, &jobs[i]);
    for (int i = 0; i < nthreads; ++i)
        pthread_join(th[i], NULL);
}

/* Gate and up products of every pair and the SwiGLU activation
 * h = silu(g) * u (optionally rounded to bf16).  Pairs are indexed
 * p = t*top_k + k; ids[p] < 0 marks a pair to skip.  Weights: n_experts
 * contiguous [inter x hidden] tensors per role. */
void orc_moe_gate_up(const uint8_t *gate, const uint8_t *up, int64_t hidden, int64_t inter,
                     const double *x, const int32_t *ids, int64_t n_pairs, int64_t top_k,
                     int round_h_bf16, double *g, double *u, double *h, double *mag_g,
                     double *mag_u, int nthreads)
{
    moe_job j = {0};
    j.gate = gate;
    j.up = up;
    j.hidden = hidden;
    j.inter = inter;
    j.x = x;
    j.ids = ids;
    j.top_k = top_k;
    j.n_pairs = n_pairs;
    j.round_h_bf16 = round_h_bf16;
    j.g = g;
    j.u = u;
    j.h = h;
    j.mag_g = mag_g;
    j.mag_u = mag_u;
    j.stage = 1;
    run_moe(j, nthreads);
}

/* Down product of every pair: y[p] = W_down[ids[p]] . h[p]. */
void orc_moe_down(const uint8_t *down, int64_t hidden, int64_t inter, const double *h,
                  const int32_t *ids, int64_t n_pairs, int64_t top_k, double *y, double *mag_y,
                  int nthreads)
{
    moe_job j = {0};
    j.down = down;
    j.hidden = hidden;
    j.inter = inter;
    j.ids = ids;
    j.top_k = top_k;
    j.n_pairs = n_pairs;
    j.h_in = h;
    j.y = y;
    j.mag_y = mag_y;
    j.stage = 2;
    run_moe(j, nthreads);
}

/* bf16 value (RNE) of an fp64 number, back as fp64. */
static double bf16_value(double v)
{
    uint32_t bits = (uint32_t)orc_bf16_rne(v) << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* V4.1 expert activation of every pair ("cortiq-engine 0.8.40,
 * src/gpu_wgpu/mxfp4.rs": dsv4_global_gate_up_mxfp4 with its bf16 flag,
 * and the host expert of global_bank_case): gate and up are rounded to
 * bf16; with a limit lim > 0 up is clamped to [-lim, lim] and gate capped
 * at lim (gate has no lower bound); act = silu(gate) * up; the pair's
 * route weight is folded in and the product rounded to bf16:
 * h = bf16(w * act).  g, u: the exact gate/up products [n_pairs][inter];
 * pairs with ids < 0 are skipped (h left untouched).
 * Parity pinned by: test_oracle_v41.py (exact-bf16 gate/up reduce it to the
 * pinned bf16 SwiGLU; limit cases worked by hand; power-of-two route
 * weights scale h exactly; two half-weight slots of one expert equal one
 * full-weight slot; the shared slot equals explicit routing). */
void orc_moe_v41_act(const double *g, const double *u, const double *w, const int32_t *ids,
                     int64_t n_pairs, int64_t inter, double lim, double *h)
{
    for (int64_t p = 0; p < n_pairs; ++p) {
        if (ids[p] < 0)
            continue;
        for (int64_t r = 0; r < inter; ++r) {
            double gb = bf16_value(g[p * inter + r]);
            double ub = bf16_value(u[p * inter + r]);
            if (lim > 0) {
                ub = ub < -lim ? -lim : (ub > lim ? lim : ub);
                gb = gb > lim ? lim : gb;
            }
            h[p * inter + r] = bf16_value(w[p] * (silu(gb) * ub));
        }
    }
}

/* Weighted sum over each token's slots in slot order:
 * out[t] = sum_k w[t][k] * y[t*top_k + k], with the weight applied to the
 * down output ([wgpu] dsv4_global_down_mxfp4, generic f32 weighting), and
 * mag_out[t] = sum_k |w[t][k]| * mag_y[t*top_k + k].  Skipped pairs
 * (ids < 0) contribute nothing. */
void orc_moe_combine(const double *y, const double *mag_y, const double *w, const int32_t *ids,
                     int64_t n_tokens, int64_t top_k, int64_t hidden, double *out,
                     double *mag_out)
{
    for (int64_t t = 0; t < n_tokens; ++t)
        for (int64_t r = 0; r < hidden; ++r) {
            double s = 0, m = 0;
            for (int64_t k = 0; k < top_k; ++k) {
                int64_t p = t * top_k + k;
                if (ids[p] < 0)
                    continue;
                s += w[p] * y[p * hidden + r];
                m += fabs(w[p]) * mag_y[p * hidden + r];
            }
            out[t * hidden + r] = s;
            mag_out[t * hidden + r] = m;
        }
}
