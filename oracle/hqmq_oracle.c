/*
 * hqmq_oracle.c -- plain, slow CPU reference of the HQMQ KV-cache codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; it is written from the method's
 * description, in fp64 wherever the description leaves the precision open,
 * and as brute force wherever the method is defined as an argmax.
 *
 * Sources (cited by page and section; all five pages describe arXiv
 * 2605.27646, "Hurwitz Quaternion Multiplicative Quantization for KV Cache
 * Compression"):
 *   [ABS]    the paper's English abstract, as shown on
 *            paperdance.org/p/2605.27646 ("Abstract (English)") and on
 *            thelatestinai.com/papers/2605.27646.
 *   [NL-M]   gist.science/nl/paper/2605.27646, "Technische Samenvatting",
 *            section "Methodologie" and its subsections 1 (multiplicative
 *            codebook composition), 2 (random initialisation) and
 *            3 (Med3x median-multiplier outlier extraction).
 *   [PT-M]   gist.science/pt/paper/2605.27646, "Resumo Tecnico",
 *            "Metodologia", subsections 1-3 (same content as [NL-M]).
 *   [FR-MEC] signal-ia-rouge.vercel.app article, section "La mecanique :
 *            pourquoi les quaternions de Hurwitz".
 *   [FR-OUT] same article, section "Le probleme des outliers : Med3x".
 *   [NL-LAT] gist.science/nl/paper/2605.27646, "Technische Samenvatting",
 *            "Memory en Latentie" (a fused kernel decodes K/V inside the
 *            attention loop of a decode step).
 *
 * Where the pages leave a step open, the reading used here is stated at the
 * function.  Every reading is also listed in the repository's design notes.
 *
 * Parity status of each function (what pins it is in tests/):
 *   or_qmul, or_t2_element ........ pinned (group axioms, textbook 2T facts,
 *                                   2x2 complex-matrix representation)
 *   or_f16_bits, or_f16_value ..... pinned (numpy float16 conversion)
 *   or_philox4x64_10 .............. pinned (numpy.random.Philox)
 *   or_codebook_value ............. pinned (numpy float16 rounding)
 *   or_make_codebook .............. partially pinned (generator pinned;
 *                                   unit norm, determinism, moments) --
 *                                   the codebook values themselves are a
 *                                   reading: "parity unpinned" for the
 *                                   choice of sampler, see header notes.
 *   or_norm2, or_half_norm_bits ... pinned (exact rational arithmetic)
 *   or_nearest .................... pinned (scipy KD-tree nearest neighbour,
 *                                   codeword inputs, 24-cell deep hole)
 *   or_lower_median, Med3x ........ pinned (numpy partition, designed inputs)
 *   or_pack_row ................... pinned (bit-by-bit unpack in numpy)
 *   or_encode_range/or_decode_range pinned through the above + closed forms
 *   or_compact_norm ............... pinned (brute-force nearest value of the
 *                                   format over every binary16 input; flag,
 *                                   identity at b = 15, error bound)
 *   or_exact_norm ................. pinned (nearest level of the grid by an
 *                                   independent vectorised search over every
 *                                   binary16 input; binade boundaries on the
 *                                   grid; flag; cap)
 *   or_pack_exact_group ........... pinned (an independent unpacker: numpy
 *                                   bit unpacking and base-3 digits; the
 *                                   information bound on the group size;
 *                                   planted slips)
 *   or_attend ..................... pinned (closed forms: uniform scores,
 *                                   one token, dominant key; scipy softmax
 *                                   on random inputs; token permutation)
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC
 * (-ffp-contract=off: every fp32 operation that the declared norm code uses
 * must be rounded on its own, exactly as written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Quaternion algebra.                                                 */
/* ------------------------------------------------------------------ */

/* Hamilton product out = a * b, components (real, i, j, k), with
 * i^2 = j^2 = k^2 = ijk = -1.  The pages write the codeword as the product
 * q_p . q_s with q_p on the left ([ABS]; [NL-M] 1; [FR-MEC] "multiplication
 * a gauche"). */
void or_qmul(const double a[4], const double b[4], double out[4])
{
    double r0 = a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3];
    double r1 = a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2];
    double r2 = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];
    double r3 = a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0];
    out[0] = r0;
    out[1] = r1;
    out[2] = r2;
    out[3] = r3;
}

/* Element p (0..23) of the binary tetrahedral group 2T: the 24 unit Hurwitz
 * quaternions, i.e. the 24 vertices of the 24-cell ([ABS]; [NL-M] 1
 * "Primair Codeboek").  The pages give the set, not an order; the order used
 * here (a reading) is
 *   p = 0..7  : +1, -1, +i, -i, +j, -j, +k, -k
 *   p = 8..23 : (s0, s1, s2, s3)/2 with s_m = -1 exactly when bit m of
 *               (p - 8) is set. */
void or_t2_element(int p, double out[4])
{
    out[0] = out[1] = out[2] = out[3] = 0.0;
    if (p < 8) {
        out[p / 2] = (p % 2 == 0) ? 1.0 : -1.0;
    } else {
        int bits = p - 8;
        for (int m = 0; m < 4; ++m)
            out[m] = ((bits >> m) & 1) ? -0.5 : 0.5;
    }
}

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16, written from the format's definition.            */
/* ------------------------------------------------------------------ */

/* Round a finite or infinite double to binary16 (round to nearest, ties to
 * even) and return its bit pattern. */
uint16_t or_f16_bits(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return 0x7E00u;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 rounds to even: inf */
        return (uint16_t)(sign | 0x7C00u);
    if (a < 0x1p-14) {
        /* subnormal range: the quantum is 2^-24 */
        double r = nearbyint(a * 0x1p24); /* exact scaling, one rounding */
        return (uint16_t)(sign | (uint16_t)r); /* r == 1024 is the smallest normal */
    }
    int e;
    frexp(a, &e);           /* a = f 2^e, f in [0.5, 1) */
    int E = e - 1;          /* a in [2^E, 2^(E+1)) */
    double r = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    unsigned m = (unsigned)r;
    if (m == 2048u) {
        m = 1024u;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (unsigned)((E + 15) << 10) | (m - 1024u));
}

/* Value of a binary16 bit pattern. */
double or_f16_value(uint16_t h)
{
    int s = (h >> 15) & 1;
    int E = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (E == 0)
        v = ldexp((double)m, -24);
    else if (E == 31)
        v = (m == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(m + 1024), E - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Seeded secondary codebook.                                          */
/* ------------------------------------------------------------------ */

/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11): ten rounds of two 64x64->128-bit multiplies with
 * the round keys bumped by the two Weyl constants between rounds. */
static void or_mul128(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo)
{
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void or_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t h0, l0, h1, l1;
        or_mul128(M0, x0, &h0, &l0);
        or_mul128(M1, x2, &h1, &l1);
        uint64_t y0 = h1 ^ x1 ^ k0;
        uint64_t y2 = h0 ^ x3 ^ k1;
        x0 = y0;
        x1 = l1;
        x2 = y2;
        x3 = l0;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* Codebook values are held on the "double binary16" grid: a value q is used
 * as q_eff = h + l with h = binary16(q) and l = binary16(q - h) (q - h is
 * exact in fp32 and fp64).  A reading: the pages fix no precision for the
 * secondary codebook; this one keeps 22 significant bits and lets fp16
 * inputs be multiplied by the two parts exactly in fp32.  Values produced
 * by or_make_codebook are already on the grid (q_eff == q). */
double or_codebook_value(float q)
{
    double h = or_f16_value(or_f16_bits((double)q));
    double l = or_f16_value(or_f16_bits((double)q - h));
    return h + l;
}

/* The S "random unit quaternions" of one (layer, head, role) ([ABS]: a
 * seeded per-(layer, head) codebook; [NL-M] 1 and [PT-M] 1: drawn per
 * (layer, head, role) without calibration).  The pages name no distribution
 * or generator.  Reading (uniform on the 3-sphere, reproducible bit for bit
 * on any IEEE host, no transcendental function):
 *   key  = (seed, layer << 32 | head << 8 | role)
 *   candidate j uses the Philox block of counter (j, 0, 0, 0); its four words
 *   give v_m = (2 (w_m >> 40) - 2^24 + 1) / 2^24, an odd multiple of 2^-24 in
 *   (-1, 1); the candidate is kept when sum v_m^2 <= 1 (exact in fp64);
 *   q = v / sqrt(sum v_m^2) in fp64, rounded to fp32 and then to the double
 *   binary16 grid (or_codebook_value).
 * Candidates are consumed in order until S are kept.
 * out: [layers][heads][S][4] fp32. */
void or_make_codebook(uint64_t seed, int layers, int heads, int role, int S, float *out)
{
    for (int l = 0; l < layers; ++l) {
        for (int h = 0; h < heads; ++h) {
            uint64_t key[2] = {seed, ((uint64_t)l << 32) | ((uint64_t)h << 8) | (uint64_t)role};
            float *dst = out + ((size_t)l * heads + h) * (size_t)S * 4;
            uint64_t j = 0;
            int kept = 0;
            while (kept < S) {
                uint64_t ctr[4] = {j, 0, 0, 0}, w[4];
                ++j;
                or_philox4x64_10(ctr, key, w);
                double v[4], n2 = 0.0;
                for (int m = 0; m < 4; ++m) {
                    v[m] = ldexp(2.0 * (double)(w[m] >> 40) - 16777216.0 + 1.0, -24);
                    n2 += v[m] * v[m];
                }
                if (!(n2 <= 1.0))
                    continue;
                double r = sqrt(n2);
                for (int m = 0; m < 4; ++m)
                    dst[kept * 4 + m] = (float)or_codebook_value((float)(v[m] / r));
                ++kept;
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Per-chunk steps.                                                    */
/* ------------------------------------------------------------------ */

/* Squared chunk norm in declared fp32: s2 = v0 v0, then s2 = fma(v_m, v_m,
 * s2) for m = 1, 2, 3.  The pages define r = ||x|| ([NL-M] "Methodologie");
 * the fp32 operation order is a reading, fixed so that the outlier decision
 * and the stored norm are reproducible bit for bit. */
float or_norm2(const float v[4])
{
    float s2 = v[0] * v[0];
    s2 = fmaf(v[1], v[1], s2);
    s2 = fmaf(v[2], v[2], s2);
    s2 = fmaf(v[3], v[3], s2);
    return s2;
}

/* Stored norm code (a reading; the pages keep the norm r but give no
 * format): binary16 of sqrt(s2) * 0.5, with sqrt correctly rounded in fp32.
 * The decoder uses r^ = 2 * value. */
uint16_t or_half_norm_bits(float s2)
{
    float r = sqrtf(s2);
    float h = r * 0.5f;
    return or_f16_bits((double)h);
}

/* Codeword c_k = a_p * q_s with k = 24 s + p ([ABS]; [NL-M] 1: the
 * effective codebook is {q_p . q_s}). */
void or_codeword(const float *q, int k, double out[4])
{
    int s = k / 24, p = k % 24;
    double a[4], b[4];
    or_t2_element(p, a);
    for (int m = 0; m < 4; ++m)
        b[m] = or_codebook_value(q[4 * s + m]);
    or_qmul(a, b, out);
}

/* Nearest codeword: the unit direction u = x / ||x|| is quantised to the
 * codeword c maximising <u, c> ([NL-M] 1, last sentence; [PT-M] 1).  Brute
 * force over all 24 S explicitly formed codewords, fp64, codewords visited
 * in increasing k, strict '>' so that an exact tie keeps the smallest k.
 * *gap = best score - second best score over the other codewords (0 on an
 * exact tie).  cw: the 24 S codewords [24S][4] in fp64. */
void or_nearest_cw(const float x[4], const double *cw, int S, int32_t *k_out, double *gap_out)
{
    double xd[4], n2 = 0.0;
    for (int m = 0; m < 4; ++m) {
        xd[m] = (double)x[m];
        n2 += xd[m] * xd[m];
    }
    double nrm = sqrt(n2), u[4];
    for (int m = 0; m < 4; ++m)
        u[m] = xd[m] / nrm;
    double best = -INFINITY, second = -INFINITY;
    int32_t kbest = 0;
    for (int k = 0; k < 24 * S; ++k) {
        const double *c = cw + 4 * (size_t)k;
        double sc = u[0] * c[0] + u[1] * c[1] + u[2] * c[2] + u[3] * c[3];
        if (sc > best) {
            second = best;
            best = sc;
            kbest = k;
        } else if (sc > second) {
            second = sc;
        }
    }
    *k_out = kbest;
    *gap_out = best - second;
}

static void or_build_codewords(const float *q, int S, double *cw)
{
    for (int k = 0; k < 24 * S; ++k)
        or_codeword(q, k, cw + 4 * (size_t)k);
}

void or_nearest(const float x[4], const float *q, int S, int32_t *k_out, double *gap_out)
{
    double *cw = (double *)malloc(sizeof(double) * 4 * 24 * (size_t)S);
    or_build_codewords(q, S, cw);
    or_nearest_cw(x, cw, S, k_out, gap_out);
    free(cw);
}

/* ------------------------------------------------------------------ */
/* Med3x.                                                               */
/* ------------------------------------------------------------------ */

static int or_cmp_float(const void *a, const void *b)
{
    float fa = *(const float *)a, fb = *(const float *)b;
    return (fa > fb) - (fa < fb);
}

/* Median of the batch ([NL-M] 3: "the median chunk norm over the current
 * batch").  For an even count the reading is the lower median, an element
 * of the batch: sorted[(n - 1) / 2].  Applied to s2 (monotone in r). */
float or_lower_median(const float *keys, int64_t n)
{
    float *tmp = (float *)malloc(sizeof(float) * (size_t)n);
    memcpy(tmp, keys, sizeof(float) * (size_t)n);
    qsort(tmp, (size_t)n, sizeof(float), or_cmp_float);
    float m = tmp[(n - 1) / 2];
    free(tmp);
    return m;
}

/* Outlier threshold on squared norms: r > C r_med  <=>  s2 > C^2 s2_med, with
 * the right side rounded in fp32 as fl(fl(C C) s2_med) ([NL-M] 3: strict
 * '>' with the fixed constant C = 3). */
float or_med3_threshold(float s2_med, float C)
{
    float cc = C * C;
    return cc * s2_med;
}

/* ------------------------------------------------------------------ */
/* Record packing.                                                     */
/* ------------------------------------------------------------------ */

/* Bits per code: the smallest b with 2^b >= 24 S (a reading: the pages count
 * 24 S codewords, [FR-MEC], but give no storage format). */
int or_code_bits(int S)
{
    int b = 0;
    while ((1L << b) < 24L * S)
        ++b;
    return b;
}

/* Pack the cpt codes of one token row, little-endian, b bits each: bit i of
 * code c is bit (c b + i) of the row, and bit j of the row is bit (j mod 32)
 * of word j / 32.  Written bit by bit. */
void or_pack_row(const int32_t *codes, int cpt, int b, uint32_t *words, int W)
{
    memset(words, 0, sizeof(uint32_t) * (size_t)W);
    for (int c = 0; c < cpt; ++c)
        for (int i = 0; i < b; ++i)
            if ((codes[c] >> i) & 1) {
                long bit = (long)c * b + i;
                words[bit / 32] |= (uint32_t)1u << (bit % 32);
            }
}

void or_unpack_row(const uint32_t *words, int cpt, int b, int32_t *codes)
{
    for (int c = 0; c < cpt; ++c) {
        int32_t v = 0;
        for (int i = 0; i < b; ++i) {
            long bit = (long)c * b + i;
            if ((words[bit / 32] >> (bit % 32)) & 1u)
                v |= (int32_t)1 << i;
        }
        codes[c] = v;
    }
}

/* ------------------------------------------------------------------ */
/* Encode / decode of a token range of one (layer, head, role) slice.   */
/* ------------------------------------------------------------------ */

/*
 * Encode tokens [t0, t0 + T) of one slice.
 *   x        : [T][D] fp32 values (fp16 inputs are passed widened, exactly)
 *   q        : [S][4] fp32 codebook of the slice
 *   B        : Med3x batch length in tokens, 0 = Med3x off.  Batches start
 *              at slice tokens that are multiples of B, so t0 % B must be 0;
 *              a final partial batch is its own batch.
 *   C        : Med3x multiplier (the pages fix C = 3)
 * outputs (per chunk, chunk index n = t cpt + c, cpt = D / 4):
 *   codes    : code k = 24 s + p of the nearest codeword (also for outlier
 *              chunks: the record always holds the nearest codeword)
 *   hnorm    : half-norm binary16 bits, bit 15 set for a Med3x outlier (the
 *              "1-bit flag" of [NL-M] 3; a reading: norms are >= 0 so the
 *              sign bit is free)
 *   gap      : oracle top-2 score gap (INFINITY for an all-zero chunk)
 *   s2       : declared fp32 squared norm
 *   side_pos : slice position (t0 + t) cpt + c of each outlier, in order
 *   side_val : its four values as binary16 bits ("full FP16", [NL-M] 3)
 *   batch_counts : outliers per batch (n_batches = ceil(T / B), or 0 if
 *              B == 0)
 * Returns the number of outliers, or -1 on bad arguments / capacity.
 * Step order follows [NL-M] "Methodologie": chunk, norm and direction,
 * Med3x median per batch, outliers kept in fp16, the bulk quantised to the
 * nearest codeword.  Zero chunks (s2 == 0) take k = 0 and a zero norm.
 */
int64_t or_encode_range(const float *x, int64_t T, int D, int64_t t0,
                        const float *q, int S, int64_t B, float C,
                        int32_t *codes, uint16_t *hnorm, double *gap, float *s2,
                        uint32_t *side_pos, uint16_t *side_val, int64_t side_cap,
                        int64_t *batch_counts)
{
    if (D % 4 != 0 || T < 0 || S < 1 || (B > 0 && t0 % B != 0))
        return -1;
    const int cpt = D / 4;
    const int64_t n = T * cpt;
    double *cw = (double *)malloc(sizeof(double) * 4 * 24 * (size_t)S);
    or_build_codewords(q, S, cw);

    /* chunk -> norm, norm code, nearest codeword */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float *v = x + 4 * i;
        float sq = or_norm2(v);
        s2[i] = sq;
        hnorm[i] = or_half_norm_bits(sq);
        if (sq == 0.0f) {
            codes[i] = 0;
            gap[i] = INFINITY;
        } else {
            or_nearest_cw(v, cw, S, &codes[i], &gap[i]);
        }
    }
    free(cw);

    if (B <= 0)
        return 0;

    /* Med3x per batch */
    int64_t n_out = 0;
    int64_t nb = (T + B - 1) / B;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t c_lo = b * B * cpt;
        int64_t c_hi = ((b + 1) * B < T ? (b + 1) * B : T) * cpt;
        float med = or_lower_median(s2 + c_lo, c_hi - c_lo);
        float thr = or_med3_threshold(med, C);
        int64_t cnt = 0;
        for (int64_t i = c_lo; i < c_hi; ++i) {
            if (s2[i] > thr) {
                if (n_out >= side_cap) {
                    return -1;
                }
                hnorm[i] = (uint16_t)(hnorm[i] | 0x8000u);
                int64_t t = i / cpt, c = i % cpt;
                side_pos[n_out] = (uint32_t)((t0 + t) * cpt + c);
                for (int m = 0; m < 4; ++m)
                    side_val[4 * n_out + m] = or_f16_bits((double)x[4 * i + m]);
                ++n_out;
                ++cnt;
            }
        }
        batch_counts[b] = cnt;
    }
    return n_out;
}

/*
 * Decode tokens [t0, t0 + T) of one slice from unpacked codes and norm codes
 * (the inverse map is implied by the pages, which decode the cache before or
 * inside attention: [NL-M] "Memory en Latentie").
 *   bulk chunk    : y = r^ (a_p * q_s), r^ = 2 value(hnorm), in fp64
 *   outlier chunk : y = the side-list values; the side list is consumed in
 *                   order and its position must match (else -1).
 * y is written as fp64; the caller rounds it to the output type.
 */
int64_t or_decode_range(const int32_t *codes, const uint16_t *hnorm, int64_t T, int D,
                        int64_t t0, const float *q, int S,
                        const uint32_t *side_pos, const uint16_t *side_val, int64_t n_side,
                        double *y)
{
    const int cpt = D / 4;
    const int64_t n = T * cpt;
    int64_t e = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (hnorm[i] & 0x8000u) {
            int64_t t = i / cpt, c = i % cpt;
            if (e >= n_side || side_pos[e] != (uint32_t)((t0 + t) * cpt + c))
                return -1;
            for (int m = 0; m < 4; ++m)
                y[4 * i + m] = or_f16_value(side_val[4 * e + m]);
            ++e;
        } else {
            if (codes[i] < 0 || codes[i] >= 24 * S)
                return -1;
            double c[4];
            or_codeword(q, codes[i], c);
            double r = 2.0 * or_f16_value(hnorm[i]);
            for (int m = 0; m < 4; ++m)
                y[4 * i + m] = r * c[m];
        }
    }
    return e;
}

/* Round fp64 values to fp32 (round to nearest even, the C cast). */
void or_round_f32(const double *y, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)y[i];
}

/* Round fp64 values to binary16 bits. */
void or_round_f16(const double *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_f16_bits(y[i]);
}

/* Compact norm code (reading: the pages' bit figures -- about 3.79 bits
 * per element at S = 8, about 5 at S = 32 [ABS], [FR-MEC] -- are two codes
 * of log2(24 S) bits per 4-element chunk, so the norm gets as many bits as
 * the direction index; the pages do not give its format).  With b the code
 * width and m = b - 5: the binary16 half-norm h16 (outlier flag clear) is
 * rounded to the nearest value of a float with 5 exponent bits (bias 15,
 * subnormals like binary16) and m mantissa bits, a tie going to the even
 * code, capped at that float's largest finite value; the code is the top b bits of the
 * binary16 pattern of the rounded value (its low 10 - m bits are zero).
 * The all-ones code (an infinity of that format) marks a Med3x outlier. */
uint32_t or_compact_norm(uint16_t h16, int b)
{
    const int m = b - 5;
    if (h16 & 0x8000u)
        return (1u << b) - 1u;
    const double v = or_f16_value(h16);
    double q;   /* spacing of the format's values around v */
    if (v < ldexp(1.0, -14)) {
        q = ldexp(1.0, -14 - m);
    } else {
        int e;
        frexp(v, &e);   /* v in [2^(e-1), 2^e) */
        q = ldexp(1.0, e - 1 - m);
    }
    /* the two neighbouring values of the format (v / q is exact), capped at
     * its largest finite value; the nearer one, on a tie the even code */
    const double t = v / q, f = floor(t);
    const double vmax = (2.0 - ldexp(1.0, -m)) * 32768.0;
    const double lo = f * q < vmax ? f * q : vmax;
    const double hi = (f + 1.0) * q < vmax ? (f + 1.0) * q : vmax;
    const uint32_t clo = (uint32_t)or_f16_bits(lo) >> (10 - m);
    const uint32_t chi = (uint32_t)or_f16_bits(hi) >> (10 - m);
    if (t - f < 0.5)
        return clo;
    if (t - f > 0.5)
        return chi;
    return (clo & 1u) ? chi : clo;
}

/* The binary16 half-norm record a compact norm code stands for: the flag
 * (0x8000) for the all-ones code, else the code's binary16 pattern. */
uint16_t or_compact_to_h16(uint32_t c, int b)
{
    if (c == (1u << b) - 1u)
        return 0x8000u;
    return (uint16_t)(c << (15 - b));
}

void or_compact_norms(const uint16_t *h16, int64_t n, int b, uint32_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_compact_norm(h16[i], b);
}

/* ------------------------------------------------------------------ */
/* Exact-rate record (reading).  The pages' rate -- about 3.79 bits per */
/* element at S = 8 and about 5 at S = 32 ([ABS], [FR-MEC]) -- is two   */
/* codes of log2(24 S) bits per 4-element chunk: an index with 24 S     */
/* values and a norm code with as many.  Reading: the norm code has     */
/* R = 24 S levels (the last one is the Med3x flag) and both codes of   */
/* every chunk are stored at that exact rate up to a small packing      */
/* loss.  With S a power of two, R = 3 2^m (m = log2 S + 3): a code is  */
/* m plain bits plus one ternary digit (code = 2^m t + l, t in {0,1,2}), */
/* the digits packed eight to a 13-bit field (3^8 = 6561 <= 2^13).    */
/* ------------------------------------------------------------------ */

/* m with 24 S = 3 2^m, or -1 when S is not a power of two in [1, 1024]. */
int or_exact_m(int S)
{
    int m = 3;
    for (int s = 1; s <= 1024; s *= 2, ++m)
        if (s == S)
            return m;
    return -1;
}

/* binary16 pattern of norm level n (0 <= n < R - 1): the integer nearest to
 * n 2^15 / R, i.e. the levels divide the 32 binades of the binary16
 * pattern range evenly (R / 32 levels per binade, 6 at S = 8, 24 at
 * S = 32).  Levels whose pattern is not finite (>= 0x7C00) are unused. */
uint32_t or_exact_level_pattern(uint32_t n, int S)
{
    const uint64_t R = 24u * (uint64_t)S;
    return (uint32_t)((2u * (uint64_t)n * 32768u + R) / (2u * R));
}

/* Exact-rate norm code of a binary16 half-norm record h16: the flag bit
 * gives R - 1; otherwise the level whose value is nearest to the value of
 * h16, a tie going to the even level, among the levels below R - 1 with
 * finite patterns (so larger norms take the top level).  Brute force over
 * every level. */
uint32_t or_exact_norm(uint16_t h16, int S)
{
    const uint32_t R = 24u * (uint32_t)S;
    if (h16 & 0x8000u)
        return R - 1u;
    const double v = or_f16_value(h16);
    uint32_t best = 0;
    double bd = INFINITY;
    for (uint32_t n = 0; n + 1u < R; ++n) {
        const uint32_t p = or_exact_level_pattern(n, S);
        if (p >= 0x7C00u)
            break;
        const double d = fabs(or_f16_value((uint16_t)p) - v);
        if (d < bd || (d == bd && (n & 1u) == 0u)) {
            bd = d;
            best = n;
        }
    }
    return best;
}

/* The binary16 half-norm record an exact-rate norm code stands for (the
 * flag 0x8000 for R - 1). */
uint16_t or_exact_norm_to_h16(uint32_t n, int S)
{
    if (n == 24u * (uint32_t)S - 1u)
        return 0x8000u;
    return (uint16_t)or_exact_level_pattern(n, S);
}

/* Ternary digits per field and bits per field: 3^8 = 6561 <= 2^13. */
#define OR_DIGITS_PER_FIELD 8
#define OR_FIELD_BITS 13

/* Words of one group of 4 token rows: per row ceil(cpt m / 32) words of
 * index low parts and as many of norm low parts, then the digit area: per
 * row F = 2 ceil(cpt / 8) fields of 13 bits (the index digits' fields, then
 * the norm digits'), rounded up to whole words for the 4 rows. */
int or_exact_group_words(int cpt, int S)
{
    const int m = or_exact_m(S);
    if (m < 0)
        return -1;
    const int wl = (cpt * m + 31) / 32;
    const int F = 2 * ((cpt + OR_DIGITS_PER_FIELD - 1) / OR_DIGITS_PER_FIELD);
    return 8 * wl + (4 * F * OR_FIELD_BITS + 31) / 32;
}

/* Pack rows 0 .. rows-1 (rows <= 4) of a group: codes[r][c] (index) and
 * ncodes[r][c] (norm), both in [0, R), R = 3 2^m; a code is 2^m d + l with
 * d its ternary digit and l its m low bits.  Layout of the group's words
 * (bit j of a stream is bit j % 32 of word j / 32):
 *   [0, 4 wl)      index low parts: row r's stream starts at word r wl; the
 *                  low bits of chunk c are stream bits c m .. c m + m - 1
 *   [4 wl, 8 wl)   norm low parts, the same way
 *   [8 wl, GW)     one stream of digit fields: row r's F fields start at
 *                  bit 13 F r; field f < F / 2 holds the index digits of
 *                  chunks 8 f .. 8 f + 7, field F / 2 + f their norm digits,
 *                  as the 13-bit number sum_i d_i 3^i (d_i of chunk 8 f + i,
 *                  0 past the row's end).
 * Missing rows and unused bits are 0.  Written bit by bit. */
void or_pack_exact_group(const int32_t *codes, const uint32_t *ncodes, int rows, int cpt, int S,
                         uint32_t *words)
{
    const int m = or_exact_m(S);
    const int wl = (cpt * m + 31) / 32;
    const int fh = (cpt + OR_DIGITS_PER_FIELD - 1) / OR_DIGITS_PER_FIELD;   /* fields per plane */
    const int gw = or_exact_group_words(cpt, S);
    memset(words, 0, sizeof(uint32_t) * (size_t)gw);
    uint32_t *digits = words + 8 * wl;
    for (int r = 0; r < rows; ++r) {
        for (int pl = 0; pl < 2; ++pl) {
            const uint32_t *src = pl == 0 ? (const uint32_t *)(codes + r * cpt) : ncodes + r * cpt;
            uint32_t *plane = words + (pl * 4 + r) * wl;
            for (int c = 0; c < cpt; ++c) {
                const uint32_t low = src[c] % (1u << m);
                for (int i = 0; i < m; ++i)
                    if ((low >> i) & 1u) {
                        const long bit = (long)c * m + i;
                        plane[bit / 32] |= 1u << (bit % 32);
                    }
            }
            for (int f = 0; f < fh; ++f) {
                uint32_t value = 0, weight = 1;
                for (int i = 0; i < OR_DIGITS_PER_FIELD; ++i) {
                    const int c = OR_DIGITS_PER_FIELD * f + i;
                    if (c < cpt)
                        value += (src[c] / (1u << m)) * weight;
                    weight *= 3u;
                }
                const long base = (long)OR_FIELD_BITS * (2 * fh * r + pl * fh + f);
                for (int i = 0; i < OR_FIELD_BITS; ++i)
                    if ((value >> i) & 1u)
                        digits[(base + i) / 32] |= 1u << ((base + i) % 32);
            }
        }
    }
}

/* Inverse of or_pack_exact_group for rows 0 .. rows-1. */
void or_unpack_exact_group(const uint32_t *words, int rows, int cpt, int S, int32_t *codes, uint32_t *ncodes)
{
    const int m = or_exact_m(S);
    const int wl = (cpt * m + 31) / 32;
    const int fh = (cpt + OR_DIGITS_PER_FIELD - 1) / OR_DIGITS_PER_FIELD;
    const uint32_t *digits = words + 8 * wl;
    for (int r = 0; r < rows; ++r) {
        for (int pl = 0; pl < 2; ++pl) {
            const uint32_t *plane = words + (pl * 4 + r) * wl;
            for (int c = 0; c < cpt; ++c) {
                uint32_t low = 0;
                for (int i = 0; i < m; ++i) {
                    const long bit = (long)c * m + i;
                    low |= ((plane[bit / 32] >> (bit % 32)) & 1u) << i;
                }
                const long base = (long)OR_FIELD_BITS * (2 * fh * r + pl * fh + c / OR_DIGITS_PER_FIELD);
                uint32_t value = 0;
                for (int i = 0; i < OR_FIELD_BITS; ++i)
                    value |= ((digits[(base + i) / 32] >> ((base + i) % 32)) & 1u) << i;
                for (int i = 0; i < c % OR_DIGITS_PER_FIELD; ++i)
                    value /= 3u;
                const uint32_t code = (value % 3u) * (1u << m) + low;
                if (pl == 0)
                    codes[r * cpt + c] = (int32_t)code;
                else
                    ncodes[r * cpt + c] = code;
            }
        }
    }
}

void or_exact_norms(const uint16_t *h16, int64_t n, int S, uint32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_exact_norm(h16[i], S);
}

/* Decode-step attention of G query rows over T cached tokens ([NL-LAT]):
 * the plain definition, in fp64.  For each query row g:
 *   s_t = scale * <q_g, k_t>,  w_t = exp(s_t) / sum_u exp(s_u),
 *   out_g = sum_t w_t v_t.
 * The largest s_t is subtracted before exp (same w_t, no overflow).  k and v
 * are [T][D] (the decoded cache values), q [G][D], out [G][D]; T = 0 gives
 * zeros. */
void or_attend(const double *k, const double *v, int64_t T, int D, const double *q, int G,
               double scale, double *out)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int g = 0; g < G; ++g) {
        const double *qg = q + (int64_t)g * D;
        double *og = out + (int64_t)g * D;
        for (int d = 0; d < D; ++d)
            og[d] = 0.0;
        if (T == 0)
            continue;
        double smax = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d)
                acc += qg[d] * k[t * D + d];
            s[t] = scale * acc;
            if (s[t] > smax)
                smax = s[t];
        }
        double z = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            s[t] = exp(s[t] - smax);
            z += s[t];
        }
        for (int64_t t = 0; t < T; ++t)
            for (int d = 0; d < D; ++d)
                og[d] += s[t] * v[t * D + d];
        for (int d = 0; d < D; ++d)
            og[d] /= z;
    }
    free(s);
}

int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
