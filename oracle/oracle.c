/*
 * oracle.c -- plain, slow, obviously correct CPU reference of the few-row draft-head
 * vocabulary projection.  TEST INFRASTRUCTURE ONLY: nothing in the product library links,
 * loads or calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the HIP library.
 *
 * Sources (web pages on one inference engine, cited by page title and section):
 *  [TFE]   "dsv41 Zig: the TFE draft head (TF_DS_DRAFTER=eagle), off by default"
 *  [SUPER] "nemotron: Super's MTP drafts on the draft vocabulary's FP8 rows while a stream's
 *           text is covered, same replies"
 *  [METAL] "dsv41 metal: the DSpark drafter on an FP8 head, a concurrent propose and
 *           resident buffers"
 *  [DSV]   "DeepSeek-V4.1: performance hooks and host checks"
 *
 * Floating point: every dot product is accumulated in IEEE double, in increasing h, and
 * rounded once to float.  Build with -O2 -ffp-contract=off and no fast-math, so that the
 * compiler neither fuses nor reorders the sums and NaN/inf follow IEEE rules.
 *
 * Numbering O1..O17 / Q1..Q2 is the oracle's own list of definitions, restated in the
 * comments of each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_BF16 0
#define ORC_FMT_FP8_BLOCK32 1
#define ORC_FMT_FP8_ROW 2

/* ---------------------------------------------------------------- number formats */

/* O1: a bf16 value is the top half of an IEEE binary32; widening is exact. */
double orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* O2: OCP E4M3 ("e4m3" in [TFE] commit notes on FP8 linears, "E4M3 codes" in [METAL]
 * 'FP8 draft head'): sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * Exponent field 0 is subnormal (M/8 * 2^-6).  Exponent 15 with mantissa 7 is NaN; there
 * is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448 -- the divisor of the
 * per-row scale rule in [TFE] 'Update'. */
double orc_e4m3_value(uint8_t c)
{
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* O3: E8M0 block scale ([METAL] 'FP8 draft head': one E8M0 scale per 32x32 block): the
 * byte is a biased power-of-two exponent, 2^(b-127); 255 encodes NaN. */
double orc_e8m0_value(uint8_t b)
{
    if (b == 255)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* O4: the real value of weight (v, h) in each storage format.  Every product here is exact
 * in double: at most 4 significant bits times a power of two or a 24-bit float. */
static double weight_value(int fmt, const void *w, const void *scale, int64_t H, int64_t v,
                           int64_t h)
{
    if (fmt == ORC_FMT_BF16)
        return orc_bf16_value(((const uint16_t *)w)[v * H + h]);
    double q = orc_e4m3_value(((const uint8_t *)w)[v * H + h]);
    if (fmt == ORC_FMT_FP8_BLOCK32) {
        int64_t hb = H / 32;
        return q * orc_e8m0_value(((const uint8_t *)scale)[(v / 32) * hb + h / 32]);
    }
    return q * (double)((const float *)scale)[v];
}

/* ---------------------------------------------------------------- GEMV */

/* O5: logits[r][j] = float( sum over h = 0..H-1 of x[r][h] * w[vids[j]][h] ), the sum taken
 * in double in increasing h.  [TFE] commit notes on the own GEMV: up to 16 activation rows
 * against the head, fp32 output; 'What this changes': fp32 sums.  vids == NULL means every
 * vocabulary row in order (nv must then equal V).  Output layout [R][nv].  Rows are
 * independent, so the OpenMP split over j does not change any result. */
void orc_gemv(int fmt, const void *w, const void *scale, int64_t V, int64_t H,
              const uint16_t *x, int R, const int64_t *vids, int64_t nv, float *out)
{
    (void)V;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nv; j++) {
        int64_t v = vids ? vids[j] : j;
        double acc[64];
        for (int r = 0; r < R; r++)
            acc[r] = 0.0;
        for (int64_t h = 0; h < H; h++) {
            double wv = weight_value(fmt, w, scale, H, v, h);
            for (int r = 0; r < R; r++)
                acc[r] += orc_bf16_value(x[(int64_t)r * H + h]) * wv;
        }
        for (int r = 0; r < R; r++)
            out[(int64_t)r * nv + j] = (float)acc[r];
    }
}

/* O14a: the bf16 encoding of a real number, rounded to nearest with ties to even: 8
 * significant bits, float's exponent range, a quantum of 2^-133 below 2^-126 (subnormals),
 * infinity once the rounded magnitude reaches 2^128; NaN encodes as 0x7fc0.  Taken straight
 * from the double, so there is a single rounding. */
uint16_t orc_bf16_encode(double d)
{
    if (isnan(d))
        return 0x7fc0;
    const uint16_t sign = signbit(d) ? 0x8000 : 0;
    const double a = fabs(d);
    if (isinf(a))
        return sign | 0x7f80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                              /* a in [2^(e-1), 2^e) */
    int q = e - 8;                             /* the quantum of 8 significant bits */
    if (q < -133)
        q = -133;
    const double v = ldexp(nearbyint(ldexp(a, -q)), q);   /* to nearest, ties to even */
    if (v >= ldexp(1.0, 128))
        return sign | 0x7f80;
    const float f = (float)v;                  /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* O14: a linear of the head's own layers through the few-row GEMV ([TFE] commit notes on
 * the own GEMV: fp32 output, bf16 output, or the sum added to a bf16 row, that add rounded
 * once).  With s = sum over k of x[r][k] * w[n][k] in double, increasing k (as O5):
 *   mode 0: out_f32[r][n] = float(s);
 *   mode 1: out_bf16[r][n] = O14a(s);
 *   mode 2: out_bf16[r][n] = O14a(residual[r][n] + s), the add in double.
 * w is [N][K] in any storage format (O4); out is float [R][N] (mode 0) or bf16 bits. */
void orc_linear(int fmt, const void *w, const void *scale, int64_t N, int64_t K,
                const uint16_t *x, int R, int mode, const uint16_t *residual, void *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        double acc[64];
        for (int r = 0; r < R; r++)
            acc[r] = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double wv = weight_value(fmt, w, scale, K, n, k);
            for (int r = 0; r < R; r++)
                acc[r] += orc_bf16_value(x[(int64_t)r * K + k]) * wv;
        }
        for (int r = 0; r < R; r++) {
            const int64_t at = (int64_t)r * N + n;
            if (mode == 0)
                ((float *)out)[at] = (float)acc[r];
            else if (mode == 1)
                ((uint16_t *)out)[at] = orc_bf16_encode(acc[r]);
            else
                ((uint16_t *)out)[at] = orc_bf16_encode(orc_bf16_value(residual[at]) + acc[r]);
        }
    }
}

/* ---------------------------------------------------------------- ordering and top-k */

/* O6: a logit can be picked iff it is neither NaN nor -inf.  [SUPER] commit notes on the
 * few-row router top-k: once the finite scores are used up every later pick is index 0,
 * exactly as repeated argmax over -inf gives; NaN is never the larger of a comparison. */
static int eligible(float l)
{
    return !isnan(l) && l > -INFINITY;
}

/* O7: u beats v iff u is eligible and (v is not, or l_u > l_v, or l_u == l_v and u < v).
 * [SUPER]: higher score first, then lower index; [TFE] 'Update': a tie at the k-th value
 * goes to the lower token id.  Equality is IEEE, so -0 == +0. */
int orc_beats(float lu, int64_t u, float lv, int64_t v)
{
    if (!eligible(lu))
        return 0;
    if (!eligible(lv))
        return 1;
    if (lu > lv)
        return 1;
    if (lu < lv)
        return 0;
    return u < v;
}

struct entry {
    float l;
    int64_t id;
};

static int cmp_entry(const void *a, const void *b)
{
    const struct entry *ea = a, *eb = b;
    if (orc_beats(ea->l, ea->id, eb->l, eb->id))
        return -1;
    if (orc_beats(eb->l, eb->id, ea->l, ea->id))
        return 1;
    return 0;
}

/* O8 + O9: per row, the eligible ids sorted by O7, the first min(k, n_eligible) of them;
 * the remaining slots are (id 0, value -inf) ([SUPER] pad rule).  Slot j holds the entry
 * that exactly j others beat.  ids/vals are [R][k]; the argmax of a row is ids[r][0] (0 for
 * a row with no eligible logit).  Returns 0, or -1 if memory runs out.
 * O13 (idmap != NULL): column v of the logits is token idmap[v] (a subset head, O12); the
 * entries are (logit, idmap[v]) and O7 orders them by that token id ([SUPER] 'What this
 * changes': a level proposes over the subset, and what it proposes are vocabulary ids). */
static int topk_of(const float *logits, int R, int64_t V, int k, const int32_t *idmap,
                   int32_t *ids, float *vals)
{
    struct entry *e = malloc(sizeof *e * (size_t)(V > 0 ? V : 1));
    if (!e)
        return -1;
    for (int r = 0; r < R; r++) {
        const float *row = logits + (int64_t)r * V;
        int64_t n = 0;
        for (int64_t v = 0; v < V; v++)
            if (eligible(row[v])) {
                e[n].l = row[v];
                e[n].id = idmap ? idmap[v] : v;
                n++;
            }
        qsort(e, (size_t)n, sizeof *e, cmp_entry);
        for (int j = 0; j < k; j++) {
            if (j < n) {
                ids[(int64_t)r * k + j] = (int32_t)e[j].id;
                vals[(int64_t)r * k + j] = e[j].l;
            } else {
                ids[(int64_t)r * k + j] = 0;
                vals[(int64_t)r * k + j] = -INFINITY;
            }
        }
    }
    free(e);
    return 0;
}

int orc_topk(const float *logits, int R, int64_t V, int k, int32_t *ids, float *vals)
{
    return topk_of(logits, R, V, k, NULL, ids, vals);
}

int orc_topk_mapped(const float *logits, int R, int64_t V, int k, const int32_t *idmap,
                    int32_t *ids, float *vals)
{
    return topk_of(logits, R, V, k, idmap, ids, vals);
}

/* O16: the softmax statistics of a row ([TFE] commit notes: a top-1 with a confidence, which
 * the pages do not define; read as the softmax probability).  Over the row's eligible logits
 * (O6), with m the largest: z = sum over them of exp(l - m), an entry equal to m counting 1
 * (so with m = +inf each +inf counts 1 and finite entries 0); lse = m + ln z, -inf for a row
 * with no eligible logit; the probability of a kept entry of value l is exp(l - m) / z (1 / z
 * for l == m) and 0 for a pad.  In double, summed in increasing v, rounded once to float.
 * ids/vals as O8; probs [R][k]; lse [R].  Returns 0, or -1 if memory runs out. */
int orc_topk_softmax(const float *logits, int R, int64_t V, int k, int32_t *ids, float *vals,
                     float *probs, float *lse)
{
    if (topk_of(logits, R, V, k, NULL, ids, vals) != 0)
        return -1;
    for (int r = 0; r < R; r++) {
        const float *row = logits + (int64_t)r * V;
        double m = -INFINITY;
        int any = 0;
        for (int64_t v = 0; v < V; v++)
            if (eligible(row[v])) {
                any = 1;
                if (row[v] > m)
                    m = row[v];
            }
        double z = 0.0;
        for (int64_t v = 0; v < V; v++)
            if (eligible(row[v]))
                z += (double)row[v] == m ? 1.0 : exp((double)row[v] - m);
        lse[r] = !any ? -INFINITY : (float)(m + log(z));
        for (int j = 0; j < k; j++) {
            const float l = vals[(int64_t)r * k + j];
            probs[(int64_t)r * k + j] =
                !eligible(l) ? 0.0f : (float)(((double)l == m ? 1.0 : exp((double)l - m)) / z);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- keyed sampling */

/* Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011), from its definition: ten rounds; a round
 * multiplies counter words 0 and 2 by the two round constants into 128-bit products and
 * makes the new counter (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the
 * key is bumped by the two Weyl constants between rounds. */
static void mul128(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo)
{
    const unsigned __int128 p = (unsigned __int128)a * b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void orc_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    uint64_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; round++) {
        if (round) {
            k0 += 0x9E3779B97F4A7C15ull;
            k1 += 0xBB67AE8584CAA73Bull;
        }
        uint64_t h0, l0, h1, l1;
        mul128(0xD2E7470EE14C6C93ull, c[0], &h0, &l0);
        mul128(0xCA5A826395121157ull, c[2], &h1, &l1);
        const uint64_t n0 = h1 ^ c[1] ^ k0, n2 = h0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = l1;
        c[2] = n2;
        c[3] = l0;
    }
    for (int i = 0; i < 4; i++)
        out[i] = c[i];
}

/* The uniform of (seed, position, token id): the first word of Philox4x64-10 with key
 * (seed, 0) and counter (position, id, 0, 0), as (w >> 11 + 1/2) * 2^-53, in (0, 1). */
double orc_keyed_uniform(uint64_t seed, int64_t position, int32_t id)
{
    const uint64_t ctr[4] = {(uint64_t)position, (uint64_t)(uint32_t)id, 0, 0};
    const uint64_t key[2] = {seed, 0};
    uint64_t w[4];
    orc_philox4x64(ctr, key, w);
    return ((double)(w[0] >> 11) + 0.5) * 0x1p-53;
}

/* O17: the keyed pick over a row's top-k candidates ([DSV] commit notes on the serving
 * module's sampler: a window's choices come from the candidates, their nucleus statistics
 * and a pick keyed by seed, position and token id, so a drafted token equals the serial
 * one).  The pages define
 * no formula; the reading: for the eligible candidates j (value v_j > -inf, in the list's
 * order, v_0 the largest) q_j = exp((v_j - v_0) / T) (1 for v_j == v_0); the nucleus keeps
 * j while the mass before it is below top_p * sum(q) (j = 0 always), and min-p drops q_j <
 * min_p; among the kept, the pick maximises (v_j - v_0) / T - ln(-ln u(seed, pos, id_j))
 * (Gumbel-max: the pick has probability q_j / sum of the kept q), the lower id on a tie.
 * T == 0 picks ids[0].  All in double.  token[r] = 0 and kept[r] = 0 for a row with no
 * eligible candidate; score[r][j] is each candidate's score (-inf when not kept). */
void orc_sample(const int32_t *ids, const float *vals, int R, int k, double T, double top_p,
                double min_p, uint64_t seed, const int64_t *pos, int32_t *token, int32_t *kept,
                double *score)
{
    double *q = malloc(sizeof *q * (size_t)(k > 0 ? k : 1));
    for (int r = 0; r < R; r++) {
        const int32_t *ri = ids + (int64_t)r * k;
        const float *rv = vals + (int64_t)r * k;
        double *rs = score + (int64_t)r * k;
        int n = 0;
        while (n < k && rv[n] > -INFINITY)
            n++;
        for (int j = 0; j < k; j++)
            rs[j] = -INFINITY;
        if (n == 0) {
            token[r] = 0;
            kept[r] = 0;
            continue;
        }
        if (T == 0.0) {
            token[r] = ri[0];
            kept[r] = 1;
            rs[0] = 0.0;
            continue;
        }
        const double v0 = rv[0];
        double z = 0.0;
        for (int j = 0; j < n; j++) {
            q[j] = (double)rv[j] == v0 ? 1.0 : exp(((double)rv[j] - v0) / T);
            z += q[j];
        }
        double before = 0.0;
        int m = 0, best = -1;
        for (int j = 0; j < n; j++) {
            const int keep = j == 0 || (before < top_p * z && q[j] >= min_p);
            before += q[j];
            if (!keep)
                continue;
            m++;
            const double d = (double)rv[j] == v0 ? 0.0 : ((double)rv[j] - v0) / T;
            rs[j] = d - log(-log(orc_keyed_uniform(seed, pos[r], ri[j])));
            if (best < 0 || rs[j] > rs[best] || (rs[j] == rs[best] && ri[j] < ri[best]))
                best = j;
        }
        token[r] = ri[best];
        kept[r] = m;
    }
    free(q);
}

/* ---------------------------------------------------------------- draft-vocabulary subset */

/* O12: the subset head of a head for a list of token ids ([SUPER] 'What this changes': the
 * head's FP8 rows of the draft vocabulary's ids are packed into a weight of their own, with
 * the head's scales): row j is row ids[j], its es bytes per element copied as they are, and
 * for per-row FP8 (scale != NULL) scale j is scale[ids[j]].  Reading where the page is
 * silent: an id outside [0, V) gives a row of zero bytes and scale 0. */
void orc_subset_rows(const void *w, const float *scale, int64_t V, int64_t H, int es,
                     const int32_t *ids, int64_t n, void *out, float *out_scale)
{
    const size_t row = (size_t)H * (size_t)es;
    for (int64_t j = 0; j < n; j++) {
        const int64_t id = ids[j];
        const int ok = id >= 0 && id < V;
        if (ok)
            memcpy((char *)out + (size_t)j * row, (const char *)w + (size_t)id * row, row);
        else
            memset((char *)out + (size_t)j * row, 0, row);
        if (scale)
            out_scale[j] = ok ? scale[id] : 0.0f;
    }
}

/* ---------------------------------------------------------------- two-stage rescore */

/* O10: exact[r][j] = float(sum_h x[r][h] * Wd[cand[r][j]][h]) in double, increasing h, from
 * the dense bf16 head ([TFE] 'Update': the two_stage head drafts the argmax of the exact
 * logits of its candidates, taken from a dense bf16 copy of the target's head).
 * Readings where the page is silent:
 *  - a candidate id outside [0, V) is not read; its exact logit is NaN (never drafted);
 *  - if use[r][j] == 0 the slot is a pad of the stage-1 list, not a candidate: it is not
 *    rescored and its exact logit is -inf (use == NULL: every slot is a candidate);
 *  - draft[r] is the candidate token that beats the others under O7 applied to (exact,
 *    token id); 0 when no candidate is eligible. */
void orc_rescore(const uint16_t *Wd, int64_t V, int64_t H, const uint16_t *x, int R,
                 const int32_t *cand, const uint8_t *use, int cand_k, float *exact,
                 int32_t *draft)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < (int64_t)R * cand_k; t++) {
        int r = (int)(t / cand_k);
        int64_t id = cand[t];
        if (use && !use[t]) {
            exact[t] = -INFINITY;
            continue;
        }
        if (id < 0 || id >= V) {
            exact[t] = NAN;
            continue;
        }
        double acc = 0.0;
        for (int64_t h = 0; h < H; h++)
            acc += orc_bf16_value(x[(int64_t)r * H + h]) * orc_bf16_value(Wd[id * H + h]);
        exact[t] = (float)acc;
    }
    for (int r = 0; r < R; r++) {
        int best = -1;
        for (int j = 0; j < cand_k; j++) {
            int64_t t = (int64_t)r * cand_k + j;
            if (!eligible(exact[t]))
                continue;
            if (best < 0 ||
                orc_beats(exact[t], cand[t], exact[(int64_t)r * cand_k + best],
                          cand[(int64_t)r * cand_k + best]))
                best = j;
        }
        draft[r] = best < 0 ? 0 : cand[(int64_t)r * cand_k + best];
    }
}

/* ---------------------------------------------------------------- quantizers (input prep) */

/* E4M3 encode with round-to-nearest-even and saturation to +-448, from a float.
 * NaN maps to the NaN code.  Written from the format definition: find the quantum of the
 * binade the magnitude falls in, divide (exact: a power of two), round half to even. */
uint8_t orc_e4m3_encode(float f)
{
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (isnan(f))
        return sign | 0x7F;
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal binade: quantum 2^-9; m == 8 is the smallest normal, code 0x08 */
        double m = rint(a / ldexp(1.0, -9));
        return sign | (uint8_t)m;
    }
    int e = (int)floor(log2(a));
    /* guard against log2 rounding at exact powers of two */
    while (ldexp(1.0, e) > a)
        e--;
    while (ldexp(1.0, e + 1) <= a)
        e++;
    double m = rint(a / ldexp(1.0, e - 3)); /* in [8, 16] */
    if (m == 16.0) {
        m = 8.0;
        e++;
    }
    return sign | (uint8_t)(((e + 7) << 3) | ((int)m - 8));
}

/* Q1, per-row FP8 ([TFE] commit notes and 'Update' on FP8 linears): from the bf16 weight,
 * s = float(amax_row / 448) and code = E4M3_RNE(float(w / s)).  An all-zero row gets s = 0
 * and all codes 0 (reading: the page leaves a zero row open). */
void orc_quant_row(const uint16_t *w, int64_t V, int64_t H, uint8_t *codes, float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; v++) {
        float amax = 0.0f;
        for (int64_t h = 0; h < H; h++) {
            float a = fabsf((float)orc_bf16_value(w[v * H + h]));
            if (a > amax)
                amax = a;
        }
        float s = amax / 448.0f;
        scale[v] = s;
        for (int64_t h = 0; h < H; h++) {
            if (s == 0.0f) {
                codes[v * H + h] = 0;
                continue;
            }
            float q = (float)orc_bf16_value(w[v * H + h]) / s;
            codes[v * H + h] = orc_e4m3_encode(q);
        }
    }
}

/* Q2, 32x32 block FP8 with E8M0 scales ([METAL] 'FP8 draft head': E4M3 codes, one E8M0
 * scale per 32x32 block, made from the bf16 head at load).  The page gives no rule for the
 * exponent; reading: e is the smallest integer with amax_block <= 448 * 2^e (exact
 * comparison), stored as e + 127 clamped to [0, 254]; an all-zero block stores 127.  Codes
 * are E4M3_RNE(w * 2^-e): one exact scaling and one rounding.  A partial last block (V not
 * a multiple of 32) covers the rows that exist.  Scale layout [ceil(V/32)][H/32]. */
void orc_quant_block32(const uint16_t *w, int64_t V, int64_t H, uint8_t *codes,
                       uint8_t *scales)
{
    int64_t vb = (V + 31) / 32, hb = H / 32;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < vb * hb; b++) {
        int64_t bv = b / hb, bh = b % hb;
        int64_t v1 = bv * 32 + 32 < V ? bv * 32 + 32 : V;
        double amax = 0.0;
        for (int64_t v = bv * 32; v < v1; v++)
            for (int64_t h = bh * 32; h < bh * 32 + 32; h++) {
                double a = fabs(orc_bf16_value(w[v * H + h]));
                if (a > amax)
                    amax = a;
            }
        int e;
        if (amax == 0.0) {
            e = 0;
        } else {
            e = -150;
            while (amax > ldexp(448.0, e))
                e++;
        }
        if (e < -127)
            e = -127;
        if (e > 127)
            e = 127;
        scales[b] = (uint8_t)(e + 127);
        for (int64_t v = bv * 32; v < v1; v++)
            for (int64_t h = bh * 32; h < bh * 32 + 32; h++) {
                double q = ldexp(orc_bf16_value(w[v * H + h]), -e);
                codes[v * H + h] = orc_e4m3_encode((float)q);
            }
    }
}

/* Number of threads OpenMP will use (for reporting the CPU baseline); n > 0 sets it first. */
int orc_threads(int n)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    extern void omp_set_num_threads(int);
    if (n > 0)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
