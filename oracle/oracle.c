/*
 * oracle.c -- plain, slow CPU oracle for SageAttention-style quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file; only the tests, the package's smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the HIP
 * kernels.
 *
 * What it computes (sources: the SageAttention project README on the
 * gittoolsai.com tool page, sections "Current Features", "How to Use",
 * "Available APIs" and the note under "Speed of Kernels"; the qwbw.cn article
 * "SageAttention one-line integration", its paragraphs on tensor layout, GQA,
 * head-dim padding and sm_scale; the trdm.cn 9070XT build blog, section 2.2 on
 * quantising QK^T and compensating the error):
 *
 *   exact mode      O = softmax(sm_scale * Q K^T + M) V in fp64, M = 0 or -inf
 *                   (causal: key j visible to query i iff j <= i + Nkv - Nq, the
 *                   diagonal aligned to the bottom-right corner, so that with
 *                   Nq < Nkv the queries are the last Nq positions of the keys'
 *                   sequence; a row that sees no key at all outputs zeros);
 *   emulation mode  the quantisation scheme step by step:
 *                   K mean smoothing -> INT8 Q / K per 64-token block ->
 *                   exact int32 scores -> dequant -> online exp2 softmax over
 *                   64-key blocks in ascending order -> P rounded to FP16 or
 *                   FP8-e4m3 -> P.V accumulated in fp64 -> normalise.
 *
 * Every floating-point step whose rounding matters for a bit-exact comparison
 * (the K mean, the fp32 subtract, the block scale, the reciprocal, the rounding
 * to int8 / fp16 / e4m3) is spelt out below in the precision it is defined in.
 * Build with -O2 -ffp-contract=off and without -ffast-math.
 *
 * Tensor convention here: every tensor is logical (B, H, N, D) row-major at the
 * TRUE head dim D (no padding); callers convert layouts before calling.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLK 64 /* token block: one quantisation scale per 64 consecutive tokens */

int orc_version(void) { return 4; }

int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * Rounding of a real number to a small binary floating-point format with
 * round-to-nearest, ties-to-even.  p = significand bits including the implicit
 * one, emin = exponent of the smallest normal, maxv = largest finite value.
 *   fp16      p=11 emin=-14  max 65504
 *   bf16      p=8  emin=-126 max (2 - 2^-7) * 2^127
 *   e4m3fn    p=4  emin=-6   max 448 (OCP FP8 E4M3, no infinities)
 *   e2m1      p=2  emin=0    max 6   (OCP FP4 E2M1: +-{0, .5, 1, 1.5, 2, 3, 4, 6})
 * With sat != 0 results beyond maxv clamp to +-maxv; otherwise they become
 * +-inf (fp16/bf16) or NaN (e4m3fn has no infinity).
 * ------------------------------------------------------------------------- */
enum { ORC_FP16 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_E2M1 = 3 };

static void fmt_params(int fmt, int* p, int* emin, double* maxv) {
    switch (fmt) {
    case ORC_FP16: *p = 11; *emin = -14; *maxv = 65504.0; break;
    case ORC_BF16: *p = 8; *emin = -126; *maxv = ldexp(2.0 - ldexp(1.0, -7), 127); break;
    case ORC_E2M1: *p = 2; *emin = 0; *maxv = 6.0; break;
    default: *p = 4; *emin = -6; *maxv = 448.0; break;
    }
}

double orc_round(double x, int fmt, int sat) {
    int p, emin;
    double maxv;
    fmt_params(fmt, &p, &emin, &maxv);
    if (isnan(x) || x == 0.0) return x;
    if (isinf(x)) {
        if (sat) return copysign(maxv, x);
        return fmt == ORC_E4M3 ? NAN : x;
    }
    double ax = fabs(x);
    int e2;
    frexp(ax, &e2);         /* ax = f * 2^e2, f in [0.5, 1): leading bit has exponent e2 - 1 */
    int ex = e2 - 1;
    if (ex < emin) ex = emin; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, ex - (p - 1));
    double r = nearbyint(ax / quantum) * quantum; /* division by a power of two is exact */
    if (r > maxv) {
        if (sat) r = maxv;
        else return fmt == ORC_E4M3 ? NAN : copysign(INFINITY, x);
    }
    return copysign(r, x);
}

void orc_round_array(const double* x, long n, int fmt, int sat, double* out) {
    for (long i = 0; i < n; i++) out[i] = orc_round(x[i], fmt, sat);
}

/* ---------------------------------------------------------------------------
 * K channel mean (the smoothing of K).  For every (b, h, channel c):
 *   part_j = sum over the tokens of 64-token block j, ascending, in fp64;
 *   total  = sum of part_j over blocks, ascending, in fp64;
 *   mean   = fp32(total / N)   (fp64 division, then one rounding to fp32).
 * Subtracting a per-channel constant from every key leaves softmax(q.k) of each
 * query unchanged, because q.mean is the same for all keys of that query.
 * ------------------------------------------------------------------------- */
void orc_k_mean(const float* k, long B, long H, long N, long D, float* mean) {
    long nblk = (N + BLK - 1) / BLK;
#pragma omp parallel for collapse(2) schedule(static)
    for (long b = 0; b < B; b++)
        for (long h = 0; h < H; h++) {
            const float* kb = k + (b * H + h) * N * D;
            for (long c = 0; c < D; c++) {
                double total = 0.0;
                for (long j = 0; j < nblk; j++) {
                    double part = 0.0;
                    long t1 = (j + 1) * BLK < N ? (j + 1) * BLK : N;
                    for (long t = j * BLK; t < t1; t++) part += (double)kb[t * D + c];
                    total += part;
                }
                mean[(b * H + h) * D + c] = (float)(total / (double)N);
            }
        }
}

/* ---------------------------------------------------------------------------
 * Per-block symmetric INT8 quantisation (one fp32 scale per 64 consecutive
 * tokens of one (b, head), covering all D channels).  With mean != NULL the
 * smoothed value y = fp32(x - mean[c]) is quantised instead of x.
 *   amax  = max |y| over the block's real tokens and all channels (exact);
 *   scale = fp32(amax / 127)       (IEEE fp32 division);
 *   inv   = fp32(127 / amax)       (IEEE fp32 division);
 *   q     = clamp(rne(fp32(y * inv)), -127, 127);
 *   amax == 0  ->  scale = 0 and q = 0.
 * ------------------------------------------------------------------------- */
void orc_quant_groups(const float* x, const float* mean, long B, long H, long N, long D, long G,
                      int8_t* xq, float* scale);

void orc_quant_blocks(const float* x, const float* mean, long B, long H, long N, long D,
                      int8_t* xq, float* scale) {
    orc_quant_groups(x, mean, B, H, N, D, BLK, xq, scale);
}

/* The same arithmetic with one scale per G consecutive tokens (G = 64: the blocks
 * above).  Finer groups are the "per-thread" granularity of the SageAttention
 * project README ("Project Updates", v2.0.1: finer quantisation groups that keep
 * the matrix-core path efficient; "Current Features": varying granularities).  On
 * gfx950 that reading is G = 1 for Q (one query column per lane of the score MFMA)
 * and G = 32 for K (the 32 keys one half-wave of lanes holds), so every lane still
 * dequantises a tile with a single factor.  scale: [B][H][ceil(N / G)]. */
void orc_quant_groups(const float* x, const float* mean, long B, long H, long N, long D, long G,
                      int8_t* xq, float* scale) {
    long nblk = (N + G - 1) / G;
#pragma omp parallel for collapse(3) schedule(static)
    for (long b = 0; b < B; b++)
        for (long h = 0; h < H; h++)
            for (long j = 0; j < nblk; j++) {
                const float* xb = x + (b * H + h) * N * D;
                const float* mu = mean ? mean + (b * H + h) * D : NULL;
                int8_t* qb = xq + (b * H + h) * N * D;
                long t0 = j * G, t1 = (j + 1) * G < N ? (j + 1) * G : N;
                float amax = 0.0f;
                for (long t = t0; t < t1; t++)
                    for (long c = 0; c < D; c++) {
                        float y = mu ? xb[t * D + c] - mu[c] : xb[t * D + c];
                        float a = fabsf(y);
                        if (a > amax) amax = a;
                    }
                float* s = scale + (b * H + h) * nblk + j;
                if (amax == 0.0f) {
                    *s = 0.0f;
                    for (long t = t0; t < t1; t++)
                        for (long c = 0; c < D; c++) qb[t * D + c] = 0;
                    continue;
                }
                *s = amax / 127.0f;
                float inv = 127.0f / amax;
                for (long t = t0; t < t1; t++)
                    for (long c = 0; c < D; c++) {
                        float y = mu ? xb[t * D + c] - mu[c] : xb[t * D + c];
                        float r = rintf(y * inv);
                        if (r > 127.0f) r = 127.0f;
                        if (r < -127.0f) r = -127.0f;
                        qb[t * D + c] = (int8_t)r;
                    }
            }
}

/* ---------------------------------------------------------------------------
 * The P.V operand.
 *  pv_fp8 == 0  (FP16 PV): vhat = fp16(v), round-to-nearest-even, saturating
 *               to +-65504; no scale.
 *  pv_fp8 == 1  (FP8 PV):  per (b, h, channel c) over all N tokens:
 *               amax = max |v|; vscale = fp32(amax / 448); inv = fp32(448 / amax);
 *               vhat = e4m3(fp32(v * inv)) with saturating round-to-nearest-even;
 *               amax == 0 -> vscale = 0, vhat = 0.
 * vhat is returned as the exact real value of each code (as float).
 * ------------------------------------------------------------------------- */
void orc_quant_v(const float* v, long B, long H, long N, long D, int pv_fp8, float* vhat, float* vscale) {
#pragma omp parallel for collapse(2) schedule(static)
    for (long b = 0; b < B; b++)
        for (long h = 0; h < H; h++) {
            const float* vb = v + (b * H + h) * N * D;
            float* ob = vhat + (b * H + h) * N * D;
            if (!pv_fp8) {
                for (long i = 0; i < N * D; i++) ob[i] = (float)orc_round((double)vb[i], ORC_FP16, 1);
                continue;
            }
            for (long c = 0; c < D; c++) {
                float amax = 0.0f;
                for (long t = 0; t < N; t++) {
                    float a = fabsf(vb[t * D + c]);
                    if (a > amax) amax = a;
                }
                float* s = vscale + (b * H + h) * D + c;
                if (amax == 0.0f) {
                    *s = 0.0f;
                    for (long t = 0; t < N; t++) ob[t * D + c] = 0.0f;
                    continue;
                }
                *s = amax / 448.0f;
                float inv = 448.0f / amax;
                for (long t = 0; t < N; t++) {
                    float y = vb[t * D + c] * inv;
                    ob[t * D + c] = (float)orc_round((double)y, ORC_E4M3, 1);
                }
            }
        }
}

/* ---------------------------------------------------------------------------
 * INT32 score tiles: out[t][i][j] = sum_c q8[b,h,64*qb+i,c] * k8[b,hk,64*kb+j,c]
 * (exact integers), zero where the row or column lies beyond the sequence.
 * tiles holds T quadruples (b, h, qb, kb); hk = h / (Hq / Hkv).
 * ------------------------------------------------------------------------- */
void orc_scores_i32(const int8_t* q8, const int8_t* k8, long B, long Hq, long Hkv, long Nq, long Nkv,
                    long D, const int64_t* tiles, long T, int32_t* out) {
    long group = Hq / Hkv;
    (void)B;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < T; t++) {
        long b = tiles[4 * t], h = tiles[4 * t + 1], qb = tiles[4 * t + 2], kb = tiles[4 * t + 3];
        long hk = h / group;
        for (long i = 0; i < BLK; i++)
            for (long j = 0; j < BLK; j++) {
                long qi = qb * BLK + i, kj = kb * BLK + j;
                int64_t s = 0;
                if (qi < Nq && kj < Nkv)
                    for (long c = 0; c < D; c++)
                        s += (int64_t)q8[((b * Hq + h) * Nq + qi) * D + c] *
                             (int64_t)k8[((b * Hkv + hk) * Nkv + kj) * D + c];
                out[(t * BLK + i) * BLK + j] = (int32_t)s;
            }
    }
}

/* ---------------------------------------------------------------------------
 * Emulation-mode attention for selected query rows.  rows holds R triples
 * (b, h, i); out is [R, D] in fp64 (before the cast to the output dtype).
 *
 * Precision of the softmax.  The pages name fp32 as the precision of the scheme's
 * floating-point side (SageAttention README, "Available APIs": pv_accum_dtype
 * "fp32"; the qwbw.cn integration article calls the fp32 accumulation the most
 * stable setting) and fix no other; the block scales the quantiser produces are
 * fp32 numbers.  The dequantised scores and the online softmax are therefore
 * evaluated in fp32, each operation rounded once (round to nearest even):
 *   c    = fp32( fp32(sq * sk) * fp32(sm_scale * log2(e)) )     dequant factor
 *   S2   = fp32( S32 * c )                                       (S32 exact in fp32)
 *   m    = running max of S2 over the row (fp32), -inf while empty
 *   p    = fp32( 2^fp32(S2 - m) )                               (correctly rounded)
 *   p^   = fp16(p)  or  e4m3(fp32(p * 448))                     (RNE, saturating)
 * and everything else in fp64.  For each row, for each 64-key block in ascending
 * order (blocks whose keys all lie beyond i + Nkv - Nq are skipped when causal):
 *   masked keys (causal j > i + Nkv - Nq) take no part;
 *   alpha = 2^(m_old - m_new)   (0 when the row was empty)
 *   l     = alpha * l + sum_j p_j                     (unrounded p, fp64 sum)
 *   acc   = alpha * acc + sum_j p^_j * vhat_j         (fp64)
 * Finally o = acc / l, times vscale[c] / 448 in FP8 mode; o = 0 for a row with no
 * visible key (l = 0).
 * Both PV accumulation modes (single-level fp32 and two-level) are modelled by the
 * same fp64 accumulation: they differ only in how the hardware rounds.
 *
 * amb (optional, [R, D]): a rounding of p to FP16 / e4m3 is an integer-like decision
 * taken on an fp32 value.  Another fp32 evaluation of the same formula (t formed with
 * one rounding instead of two, a faithfully rounded exp2, 448 folded into the
 * exponent) lands within a relative 2^-14 of this p whenever every score that can
 * still produce a nonzero code has |S2| < 2^10: the difference is then at most one
 * half ulp of 2^10 (2^-15) in t plus a few fp32 ulps, i.e. below 0.4 * 2^-14 in p.
 * So a p within a relative 2^-14 of a rounding tie may legitimately round either way;
 * for each such p, amb adds the output change that flipping that single decision
 * causes, |code_hi - code_lo| * |vhat| / l (rescaled like acc).  The margin is a fixed
 * constant and depends on nothing but the formula above.  A row in which a score with
 * t > -32 (p > 2^-32, the only ones that can round to a nonzero code) or the running
 * max reaches |S2| >= 2^10 lies outside the range where the margin holds: the return
 * value counts such rows, and the caller treats a nonzero count as an error when it
 * asked for amb.
 * ------------------------------------------------------------------------- */
static const double AMB_REL = 1.0 / 16384.0;
static const float SCORE_RANGE = 1024.0f; /* |S2| below which AMB_REL covers every fp32 evaluation */

/* quantum of the format at x (> 0): spacing of representable values around x */
static double fmt_quantum(double x, int fmt) {
    int p, emin;
    double maxv;
    fmt_params(fmt, &p, &emin, &maxv);
    int e2;
    frexp(x, &e2);
    int ex = e2 - 1;
    if (ex < emin) ex = emin;
    return ldexp(1.0, ex - (p - 1));
}

/* |code_hi - code_lo| when x (> 0) lies within AMB_REL * x of a rounding tie
 * (the midpoint of two neighbouring codes), else 0 */
double orc_tie_flip(double x, int fmt) {
    if (!(x > 0.0)) return 0.0;
    double q = fmt_quantum(x, fmt);
    double lo = floor(x / q) * q;
    double mid = lo + 0.5 * q;
    return fabs(x - mid) <= AMB_REL * x ? q : 0.0;
}
static double tie_flip(double x, int fmt) { return orc_tie_flip(x, fmt); }

/* 1 when a score s2 (with running max m, t = s2 - m) can produce a nonzero code and
 * lies outside the range where AMB_REL covers every fp32 evaluation */
static int out_of_range(float s2, float m, float t) {
    return t > -32.0f && (fabsf(s2) >= SCORE_RANGE || fabsf(m) >= SCORE_RANGE);
}

long orc_attn_emulate_g(const int8_t* q8, const float* sq, const int8_t* k8, const float* sk,
                        const float* vhat, const float* vscale, int pv_fp8, long B, long Hq, long Hkv,
                        long Nq, long Nkv, long D, long qg, long kg, int causal, double sm_scale,
                        const int64_t* rows, long R, double* out, double* amb);

long orc_attn_emulate(const int8_t* q8, const float* sq, const int8_t* k8, const float* sk,
                      const float* vhat, const float* vscale, int pv_fp8, long B, long Hq, long Hkv,
                      long Nq, long Nkv, long D, int causal, double sm_scale, const int64_t* rows,
                      long R, double* out, double* amb) {
    return orc_attn_emulate_g(q8, sq, k8, sk, vhat, vscale, pv_fp8, B, Hq, Hkv, Nq, Nkv, D, BLK, BLK, causal, sm_scale,
                       rows, R, out, amb);
}

/* The same with Q scales per qg tokens and K scales per kg keys (orc_quant_groups):
 * the dequantisation factor c of a score takes the scale of its query's group and
 * of its key's group.  The online softmax still advances in 64-key blocks. */
long orc_attn_emulate_g(const int8_t* q8, const float* sq, const int8_t* k8, const float* sk,
                        const float* vhat, const float* vscale, int pv_fp8, long B, long Hq, long Hkv,
                        long Nq, long Nkv, long D, long qg, long kg, int causal, double sm_scale,
                        const int64_t* rows, long R, double* out, double* amb) {
    const float scale2 = (float)sm_scale * 1.44269504088896341f; /* fp32(sm_scale * log2 e) */
    const int fmt = pv_fp8 ? ORC_E4M3 : ORC_FP16;
    long group = Hq / Hkv;
    long nqg = (Nq + qg - 1) / qg, nkg = (Nkv + kg - 1) / kg, nkb = (Nkv + BLK - 1) / BLK;
    const long off = Nkv - Nq; /* causal: key j visible to query i iff j <= i + off */
    long bad_rows = 0;
    (void)B;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : bad_rows)
    for (long r = 0; r < R; r++) {
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        long hk = h / group;
        const int8_t* qrow = q8 + ((b * Hq + h) * Nq + i) * D;
        float sqi = sq[(b * Hq + h) * nqg + i / qg];
        double* acc = (double*)calloc((size_t)D, sizeof(double));
        double* aacc = (double*)calloc((size_t)D, sizeof(double));
        int bad = 0;
        float s2[BLK];
        int vis[BLK];
        double pj[BLK], flip[BLK];
        float m = -INFINITY;
        double l = 0.0;
        for (long kb = 0; kb < nkb; kb++) {
            long j0 = kb * BLK;
            if (causal && j0 > i + off) break;
            long j1 = j0 + BLK < Nkv ? j0 + BLK : Nkv;
            float bmax = -INFINITY;
            for (long j = j0; j < j1; j++) {
                vis[j - j0] = !(causal && j > i + off);
                if (!vis[j - j0]) continue;
                const float c = (sqi * sk[(b * Hkv + hk) * nkg + j / kg]) * scale2;
                const int8_t* krow = k8 + ((b * Hkv + hk) * Nkv + j) * D;
                int64_t s32 = 0;
                for (long d = 0; d < D; d++) s32 += (int64_t)qrow[d] * (int64_t)krow[d];
                float v = (float)s32 * c;
                s2[j - j0] = v;
                if (v > bmax) bmax = v;
            }
            float mnew = m > bmax ? m : bmax;
            double alpha = (m == -INFINITY) ? 0.0 : exp2((double)m - (double)mnew);
            double psum = 0.0;
            for (long j = j0; j < j1; j++) {
                pj[j - j0] = 0.0;
                flip[j - j0] = 0.0;
                if (!vis[j - j0]) continue;
                float t = s2[j - j0] - mnew;
                float p = (float)exp2((double)t);
                psum += (double)p;
                double x = pv_fp8 ? (double)(p * 448.0f) : (double)p;
                pj[j - j0] = orc_round(x, fmt, 1);
                flip[j - j0] = tie_flip(x, fmt);
                bad |= out_of_range(s2[j - j0], mnew, t);
            }
            l = alpha * l + psum;
            for (long d = 0; d < D; d++) {
                double a = 0.0, fa = 0.0;
                for (long j = j0; j < j1; j++) {
                    double vv = (double)vhat[((b * Hkv + hk) * Nkv + j) * D + d];
                    a += pj[j - j0] * vv;
                    fa += flip[j - j0] * fabs(vv);
                }
                acc[d] = alpha * acc[d] + a;
                aacc[d] = alpha * aacc[d] + fa;
            }
            m = mnew;
        }
        for (long d = 0; d < D; d++) {
            double o = l > 0.0 ? acc[d] / l : 0.0, ao = l > 0.0 ? aacc[d] / l : 0.0;
            if (pv_fp8) {
                o *= (double)vscale[(b * Hkv + hk) * D + d] / 448.0;
                ao *= (double)vscale[(b * Hkv + hk) * D + d] / 448.0;
            }
            out[r * D + d] = o;
            if (amb) amb[r * D + d] = ao;
        }
        free(acc);
        free(aacc);
        bad_rows += bad;
    }
    return bad_rows;
}

/* ---------------------------------------------------------------------------
 * Exact attention for selected rows, in fp64 from the exactly upcast inputs:
 *   s_j = sm_scale * sum_c q_c k_jc  (-inf where masked),  w_j = exp(s_j - max s),
 *   o   = sum_j w_j v_j / sum_j w_j   (0 for a row with no visible key).
 * ------------------------------------------------------------------------- */
void orc_attn_exact(const float* q, const float* k, const float* v, long B, long Hq, long Hkv, long Nq,
                    long Nkv, long D, int causal, double sm_scale, const int64_t* rows, long R,
                    double* out) {
    long group = Hq / Hkv;
    const long off = Nkv - Nq; /* causal: key j visible to query i iff j <= i + off */
    (void)B;
#pragma omp parallel for schedule(dynamic, 4)
    for (long r = 0; r < R; r++) {
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        long hk = h / group;
        const float* qrow = q + ((b * Hq + h) * Nq + i) * D;
        double* s = (double*)malloc((size_t)Nkv * sizeof(double));
        double smax = -INFINITY;
        for (long j = 0; j < Nkv; j++) {
            if (causal && j > i + off) {
                s[j] = -INFINITY;
                continue;
            }
            const float* krow = k + ((b * Hkv + hk) * Nkv + j) * D;
            double d = 0.0;
            for (long c = 0; c < D; c++) d += (double)qrow[c] * (double)krow[c];
            s[j] = sm_scale * d;
            if (s[j] > smax) smax = s[j];
        }
        double wsum = 0.0;
        for (long c = 0; c < D; c++) out[r * D + c] = 0.0;
        for (long j = 0; j < Nkv; j++) {
            if (s[j] == -INFINITY) continue;
            double w = exp(s[j] - smax);
            wsum += w;
            const float* vrow = v + ((b * Hkv + hk) * Nkv + j) * D;
            for (long c = 0; c < D; c++) out[r * D + c] += w * (double)vrow[c];
        }
        for (long c = 0; c < D; c++) out[r * D + c] = wsum > 0.0 ? out[r * D + c] / wsum : 0.0;
        free(s);
    }
}

/* ---------------------------------------------------------------------------
 * Microscaling FP4.  The SageAttention README (gittoolsai.com tool page, "Project
 * Updates" and the citation list) names a microscaling FP4 attention for inference
 * (SageAttention3) and gives nothing past that title.  Reading: the OCP Microscaling
 * Formats (MX) v1.0 MXFP4 format, which is what gfx950's scaled matrix instructions
 * consume, applied to both products of the scheme above:
 *   block    32 consecutive elements along the contraction axis share one scale:
 *            Q and the smoothed K per token along the channels, V per channel along
 *            the tokens, P per query along 32 consecutive keys of a 64-key block;
 *   scale    X = 2^E with E = floor(log2 amax) - 2 (2 is the largest E2M1 exponent),
 *            held to [-126, 127]; a block with amax = 0 takes E = -126 and codes of
 *            zero (with the sign of each zero);
 *   element  e2m1(x / X): round to nearest, ties to even, saturating at 6 (so a block's
 *            largest element may clip from [6, 8) X to 6 X); the sign is kept, also
 *            for values that round to zero;
 *   code     4 bits, sign bit 8 | index of the magnitude in {0, .5, 1, 1.5, 2, 3, 4, 6}.
 * The attention itself is the scheme above with S = sum of dequantised Q * K products,
 * P quantised per 32-key half block after the online-softmax step, and
 * P.V = sum of dequantised P * V products.
 * ------------------------------------------------------------------------- */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int orc_mx_exp(double amax) {
    if (!(amax > 0.0)) return -126;
    int e2;
    frexp(amax, &e2); /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
    int E = e2 - 1 - 2;
    if (E < -126) E = -126;
    if (E > 127) E = 127;
    return E;
}

double orc_e2m1_value(int code) { return (code & 8 ? -1.0 : 1.0) * E2M1_MAG[code & 7]; }

/* code of an E2M1 value (already rounded); the sign bit follows the sign of v, -0 included */
int orc_e2m1_code(double v) {
    double a = fabs(v);
    int idx = 0;
    for (int i = 0; i < 8; i++)
        if (E2M1_MAG[i] == a) idx = i;
    return (signbit(v) ? 8 : 0) | idx;
}

/* one block of n (<= 32) values: exponent and codes */
static int mx_block(const double* x, long n, uint8_t* code) {
    double amax = 0.0;
    for (long i = 0; i < n; i++)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    int E = orc_mx_exp(amax);
    for (long i = 0; i < n; i++) {
        double y = amax > 0.0 ? ldexp(x[i], -E) : x[i]; /* exact: a power-of-two scaling */
        code[i] = (uint8_t)orc_e2m1_code(orc_round(y, ORC_E2M1, 1));
    }
    return E;
}

/* Q or K (B, H, N, D): blocks of 32 channels of each token; mean (B, H, D) or NULL is
 * subtracted first in fp32.  code [B, H, N, D], E [B, H, N, ceil(D/32)]. */
void orc_quant_mxfp4_rows(const float* x, const float* mean, long B, long H, long N, long D, uint8_t* code,
                          int32_t* E) {
    long nb = (D + 31) / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (long b = 0; b < B; b++)
        for (long h = 0; h < H; h++) {
            double buf[32];
            for (long t = 0; t < N; t++) {
                const float* row = x + ((b * H + h) * N + t) * D;
                for (long c0 = 0; c0 < D; c0 += 32) {
                    long n = D - c0 < 32 ? D - c0 : 32;
                    for (long i = 0; i < n; i++) {
                        float v = row[c0 + i];
                        if (mean) v = v - mean[(b * H + h) * D + c0 + i]; /* fp32 subtract */
                        buf[i] = (double)v;
                    }
                    E[((b * H + h) * N + t) * nb + c0 / 32] =
                        mx_block(buf, n, code + ((b * H + h) * N + t) * D + c0);
                }
            }
        }
}

/* V (B, H, N, D): blocks of 32 tokens of each channel.  code [B, H, D, N] (channel
 * major), E [B, H, D, ceil(N/32)]. */
void orc_quant_mxfp4_tokens(const float* v, long B, long H, long N, long D, uint8_t* code, int32_t* E) {
    long nb = (N + 31) / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (long b = 0; b < B; b++)
        for (long h = 0; h < H; h++) {
            double buf[32];
            for (long c = 0; c < D; c++)
                for (long t0 = 0; t0 < N; t0 += 32) {
                    long n = N - t0 < 32 ? N - t0 : 32;
                    for (long i = 0; i < n; i++) buf[i] = (double)v[((b * H + h) * N + t0 + i) * D + c];
                    E[((b * H + h) * D + c) * nb + t0 / 32] = mx_block(buf, n, code + ((b * H + h) * D + c) * N + t0);
                }
        }
}

/* P of one half block (n <= 32 values p = 2^t >= 0): the dequantised values ph, and
 * for the ambiguity: per element the change that a different rounding decision would
 * make when p / X sits within 2^-14 of a tie, or when the block maximum sits within
 * 2^-14 of a power of two without being one exactly (another fp32 evaluation of p,
 * within 2^-14 of this one, may then pick the neighbouring exponent), the change the
 * other exponent makes.  A maximum from an integer t (the row maximum itself, t = 0)
 * is an exact power of two in any faithful evaluation of 2^t. */
void orc_mx_p_block(const double* p, const float* t, const int* vis, long n, double* ph, double* flip) {
    double pmax = 0.0;
    float tmax = -INFINITY;
    for (long i = 0; i < n; i++) {
        if (vis[i] && p[i] > pmax) pmax = p[i];
        if (vis[i] && t[i] > tmax) tmax = t[i];
    }
    int E = orc_mx_exp(pmax);
    int Ealt = E;
    if (pmax > 0.0 && tmax != floorf(tmax)) {
        int e2;
        double f = frexp(pmax, &e2); /* f in [0.5, 1) */
        if (f - 0.5 <= AMB_REL * pmax / ldexp(1.0, e2)) Ealt = E - 1;       /* just above 2^(e2-1) */
        else if (1.0 - f <= AMB_REL) Ealt = E + 1;                         /* just below 2^e2 */
        if (Ealt < -126 || Ealt > 127) Ealt = E;
    }
    for (long i = 0; i < n; i++) {
        ph[i] = 0.0;
        flip[i] = 0.0;
        if (!vis[i] || pmax == 0.0) continue;
        double y = ldexp(p[i], -E);
        ph[i] = ldexp(orc_round(y, ORC_E2M1, 1), E);
        flip[i] = ldexp(tie_flip(y, ORC_E2M1), E);
        if (Ealt != E) {
            double alt = ldexp(orc_round(ldexp(p[i], -Ealt), ORC_E2M1, 1), Ealt);
            flip[i] += fabs(alt - ph[i]);
        }
    }
}

/* Emulation of the microscaling FP4 scheme for selected rows (b, h, i).
 *   qc, kc: codes [B, H, N, D] with exponents qE, kE [B, H, N, ceil(D/32)];
 *   vc: codes [B, Hkv, D, Nkv] with vE [B, Hkv, D, ceil(Nkv/32)].
 * Scores: S = sum_d q * k over the dequantised values (fp64, exact for these
 * operands), then, as for INT8, s2 = fp32(S) * fp32(sm_scale * log2 e) in fp32, the
 * running max over 64-key blocks, p = fp32(2^(s2 - m)), l += p (unquantised),
 * p quantised per 32-key half block, acc = alpha * acc + sum ph * v (fp64). */
long orc_attn_emulate_mxfp4(const uint8_t* qc, const int32_t* qE, const uint8_t* kc, const int32_t* kE,
                            const uint8_t* vc, const int32_t* vE, long B, long Hq, long Hkv, long Nq, long Nkv,
                            long D, int causal, double sm_scale, const int64_t* rows, long R, double* out,
                            double* amb) {
    const float scale2 = (float)sm_scale * 1.44269504088896341f;
    long group = Hq / Hkv, nbd = (D + 31) / 32, nbt = (Nkv + 31) / 32, nkb = (Nkv + BLK - 1) / BLK;
    const long off = Nkv - Nq;
    long bad_rows = 0;
    (void)B;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : bad_rows)
    for (long r = 0; r < R; r++) {
        int bad = 0;
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        long hk = h / group;
        double* qd = (double*)malloc((size_t)D * sizeof(double));
        double* acc = (double*)calloc((size_t)D, sizeof(double));
        double* aacc = (double*)calloc((size_t)D, sizeof(double));
        for (long d = 0; d < D; d++)
            qd[d] = ldexp(orc_e2m1_value(qc[((b * Hq + h) * Nq + i) * D + d]), qE[((b * Hq + h) * Nq + i) * nbd + d / 32]);
        float s2[BLK];
        int vis[BLK];
        double pj[BLK], ph[BLK], flip[BLK];
        float tj[BLK];
        float m = -INFINITY;
        double l = 0.0;
        for (long kb = 0; kb < nkb; kb++) {
            long j0 = kb * BLK;
            if (causal && j0 > i + off) break;
            long j1 = j0 + BLK < Nkv ? j0 + BLK : Nkv;
            float bmax = -INFINITY;
            for (long j = j0; j < j1; j++) {
                vis[j - j0] = !(causal && j > i + off);
                if (!vis[j - j0]) continue;
                const uint8_t* krow = kc + ((b * Hkv + hk) * Nkv + j) * D;
                const int32_t* ke = kE + ((b * Hkv + hk) * Nkv + j) * nbd;
                double S = 0.0;
                for (long d = 0; d < D; d++) S += qd[d] * ldexp(orc_e2m1_value(krow[d]), ke[d / 32]);
                float v = (float)S * scale2;
                s2[j - j0] = v;
                if (v > bmax) bmax = v;
            }
            float mnew = m > bmax ? m : bmax;
            double alpha = (m == -INFINITY) ? 0.0 : exp2((double)m - (double)mnew);
            double psum = 0.0;
            for (long j = j0; j < j1; j++) {
                pj[j - j0] = 0.0;
                tj[j - j0] = -INFINITY;
                if (!vis[j - j0]) continue;
                float t = s2[j - j0] - mnew;
                float p = (float)exp2((double)t);
                psum += (double)p;
                pj[j - j0] = (double)p;
                tj[j - j0] = t;
                bad |= out_of_range(s2[j - j0], mnew, t);
            }
            for (long h0 = j0; h0 < j1; h0 += 32) {
                long n = j1 - h0 < 32 ? j1 - h0 : 32;
                orc_mx_p_block(pj + (h0 - j0), tj + (h0 - j0), vis + (h0 - j0), n, ph + (h0 - j0), flip + (h0 - j0));
            }
            l = alpha * l + psum;
            for (long d = 0; d < D; d++) {
                const uint8_t* vrow = vc + ((b * Hkv + hk) * D + d) * Nkv;
                const int32_t* ve = vE + ((b * Hkv + hk) * D + d) * nbt;
                double a = 0.0, fa = 0.0;
                for (long j = j0; j < j1; j++) {
                    double vv = ldexp(orc_e2m1_value(vrow[j]), ve[j / 32]);
                    a += ph[j - j0] * vv;
                    fa += flip[j - j0] * fabs(vv);
                }
                acc[d] = alpha * acc[d] + a;
                aacc[d] = alpha * aacc[d] + fa;
            }
            m = mnew;
        }
        for (long d = 0; d < D; d++) {
            out[r * D + d] = l > 0.0 ? acc[d] / l : 0.0;
            if (amb) amb[r * D + d] = l > 0.0 ? aacc[d] / l : 0.0;
        }
        free(qd);
        free(acc);
        free(aacc);
        bad_rows += bad;
    }
    return bad_rows;
}

/* ---------------------------------------------------------------------------
 * Error breakdown of the scheme: the attention of selected rows with each of its
 * three approximations switched on or off independently (parts, a bit set):
 *   bit 0  scores from the INT8 codes and block scales, S2 = S32 sq sk sm_scale log2 e
 *          (else exact scores sm_scale log2 e q.k from the unquantised q and k);
 *   bit 1  P rounded to its P.V format: fp16(p), or e4m3(448 p) / 448
 *          (else the unrounded p);
 *   bit 2  V as the quantised operand: fp16(v), or the e4m3 code times v_scale
 *          (v_scale = amax / 448) (else the exact v).
 * Everything is fp64; the online softmax walks 64-key blocks in ascending order with
 * the running maximum (so P is rounded relative to it, as in the emulation), and l sums
 * the unrounded p.  parts = 0 is exact attention; parts = 7 is the emulation's
 * arithmetic with its fp32 score and softmax steps taken in fp64 instead.
 * q, k, v: the exact inputs (B, H, N, D); q8/sq/k8/sk/vhat/vscale: as orc_attn_emulate.
 * ------------------------------------------------------------------------- */
void orc_attn_breakdown(const float* q, const float* k, const float* v, const int8_t* q8, const float* sq,
                        const int8_t* k8, const float* sk, const float* vhat, const float* vscale, int pv_fp8, long B,
                        long Hq, long Hkv, long Nq, long Nkv, long D, int causal, double sm_scale,
                        const int64_t* rows, long R, int parts, double* out) {
    const double LOG2E = 1.4426950408889634074;
    const int fmt = pv_fp8 ? ORC_E4M3 : ORC_FP16;
    long group = Hq / Hkv;
    long nqb = (Nq + BLK - 1) / BLK, nkb = (Nkv + BLK - 1) / BLK;
    const long off = Nkv - Nq;
    (void)B;
#pragma omp parallel for schedule(dynamic, 4)
    for (long r = 0; r < R; r++) {
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        long hk = h / group;
        double* acc = (double*)calloc((size_t)D, sizeof(double));
        double s2[BLK], pj[BLK];
        int vis[BLK];
        double m = -INFINITY, l = 0.0;
        for (long kb = 0; kb < nkb; kb++) {
            long j0 = kb * BLK;
            if (causal && j0 > i + off) break;
            long j1 = j0 + BLK < Nkv ? j0 + BLK : Nkv;
            double bmax = -INFINITY;
            for (long j = j0; j < j1; j++) {
                vis[j - j0] = !(causal && j > i + off);
                if (!vis[j - j0]) continue;
                double sc = 0.0;
                if (parts & 1) {
                    const int8_t* qr = q8 + ((b * Hq + h) * Nq + i) * D;
                    const int8_t* kr = k8 + ((b * Hkv + hk) * Nkv + j) * D;
                    int64_t s32 = 0;
                    for (long d = 0; d < D; d++) s32 += (int64_t)qr[d] * (int64_t)kr[d];
                    sc = (double)s32 * (double)sq[(b * Hq + h) * nqb + i / BLK] *
                         (double)sk[(b * Hkv + hk) * nkb + kb] * sm_scale * LOG2E;
                } else {
                    const float* qr = q + ((b * Hq + h) * Nq + i) * D;
                    const float* kr = k + ((b * Hkv + hk) * Nkv + j) * D;
                    for (long d = 0; d < D; d++) sc += (double)qr[d] * (double)kr[d];
                    sc *= sm_scale * LOG2E;
                }
                s2[j - j0] = sc;
                if (sc > bmax) bmax = sc;
            }
            double mnew = m > bmax ? m : bmax;
            double alpha = (m == -INFINITY) ? 0.0 : exp2(m - mnew);
            double psum = 0.0;
            for (long j = j0; j < j1; j++) {
                pj[j - j0] = 0.0;
                if (!vis[j - j0]) continue;
                double p = exp2(s2[j - j0] - mnew);
                psum += p;
                pj[j - j0] = (parts & 2) ? (pv_fp8 ? orc_round(p * 448.0, fmt, 1) / 448.0 : orc_round(p, fmt, 1)) : p;
            }
            l = alpha * l + psum;
            for (long d = 0; d < D; d++) {
                double a = 0.0;
                for (long j = j0; j < j1; j++) {
                    double vv;
                    if (parts & 4) {
                        vv = (double)vhat[((b * Hkv + hk) * Nkv + j) * D + d];
                        if (pv_fp8) vv *= (double)vscale[(b * Hkv + hk) * D + d]; /* v = code * amax / 448 */
                    } else {
                        vv = (double)v[((b * Hkv + hk) * Nkv + j) * D + d];
                    }
                    a += pj[j - j0] * vv;
                }
                acc[d] = alpha * acc[d] + a;
            }
            m = mnew;
        }
        for (long d = 0; d < D; d++) out[r * D + d] = l > 0.0 ? acc[d] / l : 0.0;
        free(acc);
    }
}
