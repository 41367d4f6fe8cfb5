/*
 * mac_oracle.c -- fp64 CPU reference of the MAC-Attention decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library under kv_reuse_amd/.
 *
 * Source: "MAC-Attention: a Match-Amend-Complete scheme for fast and accurate
 * attention computation" (arXiv 2604.00235), paper card at thelatestinai.com:
 *   abstract ........ match on pre-RoPE queries by L2 over a short window,
 *                     amend by recomputing a band near the match boundary,
 *                     complete by merging with fresh attention on the tail
 *   Figure 2 (a) .... match: nearest ring entry, threshold, fetch AS_{1:p-r}
 *   Figure 2 (b) .... complete: attend [p-r+1, m] with the post-RoPE query,
 *                     log-domain merge with the fetched summary
 *   Figure 2 (c) .... amend: remove the last-r band, insert (q~_m, AS_{1:m-r})
 * Prior art named by the pages: online softmax (Milakov & Gimelshein),
 * FlashAttention, RoFormer (rotary embedding).
 *
 * Every function is written straight from its definition: no blocking, no
 * fusion, fp64 arithmetic throughout, no fast-math.  Positions are 0-based
 * (the pages write 1-based ranges; "all keys of the matched query except its
 * last r" is the same set in both indexings).
 *
 * Attention summary layout (d+2 doubles): s[0..d-1] = o (normalised output),
 * s[d] = M (reference max of the logits), s[d+1] = l (sum of exp(logit - M)).
 * EMPTY = (o = 0, M = -inf, l = 0).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F_DISABLE_REUSE 1u
#define ORC_F_RING_BF16 2u      /* ring keeps pre-RoPE queries rounded to bfloat16 */
/* Stale-by-one ring: the match of call t sees only entries inserted by calls
 * up to t-2.  The pages update the cache asynchronously (Figure 2 (c)); with
 * this reading the amend of call t-1 may still be writing its slot while call
 * t matches, so that slot takes no part in call t's match or override. */
#define ORC_F_STALE_RING 4u

/* ---------------------------------------------------------------- values */

/* x rounded to the nearest bfloat16 (ties to even), returned as a float:
 * bfloat16 is the top 16 bits of an IEEE-754 single, so rounding adds half of
 * the dropped 16-bit unit (less one when the kept part is even) and clears
 * the low half.  NaN stays NaN; overflow rounds to infinity.  The ring keeps
 * its queries in this form when ORC_F_RING_BF16 is set (the pages' Table 7
 * puts the auxiliary memory at ~6x a token's KV per ring entry, which fits a
 * 16-bit query plus an fp32 summary per head). */
float orc_round_bf16(float x)
{
    if (isnan(x))
        return x;
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    float y;
    memcpy(&y, &u, sizeof y);
    return y;
}

/* bfloat16 bit pattern -> double; exact (bf16 is the top half of a float). */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element idx of a key/value row block stored as fp32 (kv_fp32 != 0) or bf16. */
static double kv_at(const void *base, int kv_fp32, int64_t idx)
{
    if (kv_fp32)
        return (double)((const float *)base)[idx];
    return bf16_bits_to_double(((const uint16_t *)base)[idx]);
}

/* ------------------------------------------------------------------ RoPE */

/* Rotary embedding, rotate-half convention (RoFormer): for i < d/2 the pair
 * (x_i, x_{i+d/2}) is rotated by the angle m * theta^(-2i/d).  The angle is
 * formed in fp64 (at m ~ 1.3e5 an fp32 angle is off by ~3e-3 rad). */
void orc_rope(const float *x, int d, int64_t m, double theta, double *out)
{
    int h = d / 2;
    for (int i = 0; i < h; i++) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
        double phi = (double)m * inv_freq;
        double c = cos(phi), s = sin(phi);
        double a = (double)x[i], b = (double)x[i + h];
        out[i] = a * c - b * s;
        out[i + h] = b * c + a * s;
    }
}

/* ------------------------------------------------------- summaries, merge */

void orc_empty(int d, double *s)
{
    for (int j = 0; j < d; j++)
        s[j] = 0.0;
    s[d] = -INFINITY;
    s[d + 1] = 0.0;
}

int orc_is_empty(int d, const double *s)
{
    return !(s[d + 1] > 0.0);
}

/* A(q, [a, b]): softmax attention of q over keys a..b (inclusive) of one KV
 * head.  k and v point at that head's rows, row i at offset i*d.  Logit
 * s_i = scale * <q, k_i>.  Two passes: the max, then the weights. */
void orc_attend(const double *q, const void *k, const void *v, int kv_fp32,
                int d, int64_t a, int64_t b, double scale, double *out)
{
    if (a < 0)
        a = 0;
    if (b < a) {
        orc_empty(d, out);
        return;
    }
    int64_t n = b - a + 1;
    double *logit = (double *)malloc((size_t)n * sizeof(double));
    double M = -INFINITY;
    for (int64_t i = 0; i < n; i++) {
        double acc = 0.0;
        int64_t row = (a + i) * (int64_t)d;
        for (int j = 0; j < d; j++)
            acc += q[j] * kv_at(k, kv_fp32, row + j);
        logit[i] = scale * acc;
        if (logit[i] > M)
            M = logit[i];
    }
    double l = 0.0;
    for (int j = 0; j < d; j++)
        out[j] = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double w = exp(logit[i] - M);
        int64_t row = (a + i) * (int64_t)d;
        l += w;
        for (int j = 0; j < d; j++)
            out[j] += w * kv_at(v, kv_fp32, row + j);
    }
    for (int j = 0; j < d; j++)
        out[j] /= l;
    out[d] = M;
    out[d + 1] = l;
    free(logit);
}

/* X (+) Y: log-domain merge of two summaries over disjoint key sets
 * (Figure 2 (b); the online-softmax combination rule). */
void orc_merge(const double *x, const double *y, int d, double *z)
{
    double tmp[d + 2];
    if (orc_is_empty(d, x)) {
        memcpy(tmp, y, sizeof tmp);
    } else if (orc_is_empty(d, y)) {
        memcpy(tmp, x, sizeof tmp);
    } else {
        double M = x[d] > y[d] ? x[d] : y[d];
        double a = x[d + 1] * exp(x[d] - M);
        double b = y[d + 1] * exp(y[d] - M);
        double l = a + b;
        for (int j = 0; j < d; j++)
            tmp[j] = (a * x[j] + b * y[j]) / l;
        tmp[d] = M;
        tmp[d + 1] = l;
    }
    memcpy(z, tmp, sizeof tmp);
}

/* Z (-) Y: log-domain removal of a sub-summary Y (same query, Y's keys a
 * subset of Z's) from Z (Figure 2 (c), "online subtraction").  Z's reference
 * max is kept as the stabiliser.  When the remainder is at or below 2^-24 of
 * Z's normaliser nothing meaningful is left and the result is EMPTY. */
void orc_remove(const double *z, const double *y, int d, double *x)
{
    double tmp[d + 2];
    if (orc_is_empty(d, y)) {
        memcpy(tmp, z, sizeof tmp);
    } else {
        double c = y[d + 1] * exp(y[d] - z[d]);
        double l = z[d + 1] - c;
        if (!(l > ldexp(z[d + 1], -24))) {
            orc_empty(d, tmp);
        } else {
            for (int j = 0; j < d; j++)
                tmp[j] = (z[d + 1] * z[j] - c * y[j]) / l;
            tmp[d] = z[d];
            tmp[d + 1] = l;
        }
    }
    memcpy(x, tmp, sizeof tmp);
}

/* ----------------------------------------------------------------- match */

/* Squared L2 distance between two fp32 vectors, in fp64. */
static double sqdist(const float *a, const float *b, int d)
{
    double acc = 0.0;
    for (int j = 0; j < d; j++) {
        double t = (double)a[j] - (double)b[j];
        acc += t * t;
    }
    return acc;
}

/* Nearest ring entry to the pre-RoPE query qt (Figure 2 (a)).
 * ring_q: [W][d] pre-RoPE queries; ring_pos: [W] stored positions (-1 = empty).
 * Valid entries hold a position in [0, m].  Smallest distance wins; equal
 * distances go to the most recent entry (largest position), then to the
 * larger slot.  Returns the slot or -1 when no entry is valid; *d1 and *d2
 * receive the best and second-best distances (+inf when missing). */
int orc_nearest(const float *qt, const float *ring_q, const int32_t *ring_pos,
                int W, int d, int64_t m, double *d1, double *d2)
{
    int best = -1;
    double b1 = INFINITY, b2 = INFINITY;
    for (int j = 0; j < W; j++) {
        if (ring_pos[j] < 0 || ring_pos[j] > m)
            continue;
        double D = sqdist(qt, ring_q + (int64_t)j * d, d);
        /* j only grows, so >= also sends an exact duplicate (same distance and
         * position) to the larger slot */
        if (best < 0 || D < b1 || (D == b1 && ring_pos[j] >= ring_pos[best])) {
            if (best >= 0)
                b2 = b1;
            b1 = D;
            best = j;
        } else if (D < b2) {
            b2 = D;
        }
    }
    *d1 = b1;
    *d2 = b2;
    return best;
}

/* Threads of the batched decode call (OpenMP over (request, head)); returns
 * the count in use before.  Timing only: results do not depend on it. */
int orc_set_threads(int n)
{
    int before = omp_get_max_threads();
    if (n > 0)
        omp_set_num_threads(n);
    return before;
}

/* ------------------------------------------------------------ the policy */

typedef struct {
    int B, Hq, Hkv, d, W, r;
    double tau, theta, scale;
    int kv_fp32;
    unsigned flags;
    int64_t calls;    /* decode calls so far; the next insert goes to slot calls % W */
    int32_t *band;    /* [Hq] band r of each query head (r for all unless set) */
    int32_t *pos;     /* [B][Hq][W] stored positions, -1 = empty */
    float *ring_q;    /* [B][Hq][W][d] pre-RoPE queries */
    double *ring_s;   /* [B][Hq][W][d+2] stored summaries AS_{1:pos-r} */
} orc_ctx;

orc_ctx *orc_create(int B, int Hq, int Hkv, int d, int W, int r, double tau,
                    double theta, double scale, int kv_fp32, unsigned flags)
{
    orc_ctx *c = (orc_ctx *)calloc(1, sizeof *c);
    c->B = B; c->Hq = Hq; c->Hkv = Hkv; c->d = d; c->W = W; c->r = r;
    c->tau = tau; c->theta = theta; c->scale = scale; c->kv_fp32 = kv_fp32;
    c->flags = flags;
    size_t nslot = (size_t)B * Hq * W;
    c->pos = (int32_t *)malloc(nslot * sizeof(int32_t));
    c->band = (int32_t *)malloc((size_t)Hq * sizeof(int32_t));
    for (int h = 0; h < Hq; h++)
        c->band[h] = r;
    c->ring_q = (float *)calloc(nslot * d, sizeof(float));
    c->ring_s = (double *)calloc(nslot * (d + 2), sizeof(double));
    for (size_t i = 0; i < nslot; i++)
        c->pos[i] = -1;
    c->calls = 0;
    return c;
}

void orc_destroy(orc_ctx *c)
{
    if (!c)
        return;
    free(c->pos);
    free(c->band);
    free(c->ring_q);
    free(c->ring_s);
    free(c);
}

/* Per-head bands (Figure 3 (b): the band size r varies by head): query head
 * h, in every request, uses band[h] >= 1 for its hit span [p - r_h + 1, m]
 * and for the amend band [m - r_h + 1, m]. */
void orc_set_bands(orc_ctx *c, const int32_t *band)
{
    for (int h = 0; h < c->Hq; h++)
        c->band[h] = band[h];
}

/* Empty every ring; the next call misses everywhere. */
void orc_reset(orc_ctx *c)
{
    size_t nslot = (size_t)c->B * c->Hq * c->W;
    for (size_t i = 0; i < nslot; i++)
        c->pos[i] = -1;
    c->calls = 0;
}

/* Read-only views of one stored ring entry (for tests). */
void orc_ring_entry(const orc_ctx *c, int b, int h, int slot, int32_t *pos,
                    float *q, double *s)
{
    size_t e = ((size_t)b * c->Hq + h) * c->W + slot;
    *pos = c->pos[e];
    if (q)
        memcpy(q, c->ring_q + e * c->d, (size_t)c->d * sizeof(float));
    if (s)
        memcpy(s, c->ring_s + e * (c->d + 2), (size_t)(c->d + 2) * sizeof(double));
}

/* One decode call over the whole batch.
 *
 * k_grp / v_grp: [B*Hkv] pointers; entry b*Hkv+g is request b's KV head g, its
 *   logical rows [seq][d] (fp32 or bf16 bits per kv_fp32).  A NULL entry is
 *   allowed when no head of that group is in `track`.
 * seq_lens: [B]; the query position is m = seq_lens[b]-1 and its own K/V row
 *   is already present.  seq_lens[b] <= 0 marks an idle request: no output,
 *   no ring insert.
 * q_pre: [B*Hq*d] pre-RoPE queries (fp32).
 * override: NULL or [B*Hq]: -2 no override, -1 force a miss, p >= 0 force a
 *   hit on the entry stored at position p (a miss if no such entry).
 * track: NULL (all) or [B*Hq] flags; attention is evaluated only for tracked
 *   heads.  Untracked heads still take decisions and store their query; their
 *   stored summaries are NaN.  A head must stay tracked or untracked for the
 *   whole run.
 * Outputs (all [B*Hq] unless noted; any may be NULL):
 *   out [B*Hq*d]      the MAC output o (tracked heads; zeros otherwise)
 *   full [B*Hq*d]     plain full attention A(q,[0,m]).o (tracked heads)
 *   hit, p            decision and matched position (-1 on a miss)
 *   rel               ||q~_m - q~_p|| / ||q~_m|| for the nearest entry (NaN if none)
 *   near_tau          |rel - tau| < 1e-4
 *   near_tie          second-best distance within a relative 1e-5 of the best
 *   start             first key of the head's span: max(p-r+1,0) on a hit, 0 on a miss
 *   kv_tokens [B*Hkv] keys a GQA group streams on the critical path:
 *                     m - min_h start_h + 1 (0 for an idle request)
 * Returns the number of overrides that named no stored entry. */
int orc_step(orc_ctx *c, const void *const *k_grp, const void *const *v_grp,
             const int32_t *seq_lens, const float *q_pre, const int32_t *override,
             const uint8_t *track, double *out, double *full, uint8_t *hit,
             int32_t *p_out, double *rel, uint8_t *near_tau, uint8_t *near_tie,
             int32_t *start, int64_t *kv_tokens)
{
    const int B = c->B, Hq = c->Hq, Hkv = c->Hkv, d = c->d, W = c->W;
    const int G = Hq / Hkv;
    const int slot_new = (int)(c->calls % W);
    const int reuse = !(c->flags & ORC_F_DISABLE_REUSE) && c->tau >= 0.0;
    int invalid_total = 0;
    int32_t *start_all = (int32_t *)malloc((size_t)B * Hq * sizeof(int32_t));

    #pragma omp parallel for schedule(dynamic, 1) reduction(+ : invalid_total)
    for (int bh = 0; bh < B * Hq; bh++) {
        int b = bh / Hq, h = bh % Hq, g = h / G;
        const int r = c->band[h];
        int64_t m = (int64_t)seq_lens[b] - 1;
        const float *qt = q_pre + (size_t)bh * d;
        int32_t *pos = c->pos + (size_t)bh * W;
        float *rq = c->ring_q + (size_t)bh * W * d;
        double *rs = c->ring_s + (size_t)bh * W * (d + 2);
        int tracked = track ? track[bh] != 0 : 1;

        if (hit) hit[bh] = 0;
        if (p_out) p_out[bh] = -1;
        if (rel) rel[bh] = NAN;
        if (near_tau) near_tau[bh] = 0;
        if (near_tie) near_tie[bh] = 0;
        start_all[bh] = 0;
        if (out) memset(out + (size_t)bh * d, 0, (size_t)d * sizeof(double));
        if (full) memset(full + (size_t)bh * d, 0, (size_t)d * sizeof(double));
        if (m < 0)
            continue;

        /* Figure 2 (a): match on the pre-RoPE query, over the entries this
         * call may see. */
        int32_t *vis = (int32_t *)malloc((size_t)W * sizeof(int32_t));
        memcpy(vis, pos, (size_t)W * sizeof(int32_t));
        if ((c->flags & ORC_F_STALE_RING) && c->calls > 0)
            vis[(c->calls - 1) % W] = -1;
        int slot = -1;
        if (reuse) {
            double d1, d2;
            int j = orc_nearest(qt, rq, vis, W, d, m, &d1, &d2);
            if (j >= 0) {
                double qn2 = 0.0;
                for (int e = 0; e < d; e++)
                    qn2 += (double)qt[e] * (double)qt[e];
                double rr = qn2 > 0.0 ? sqrt(d1 / qn2) : (d1 == 0.0 ? 0.0 : INFINITY);
                if (rel) rel[bh] = rr;
                if (near_tau) near_tau[bh] = fabs(rr - c->tau) < 1e-4;
                if (near_tie) near_tie[bh] = (d2 - d1) <= 1e-5 * d1;
                /* relative-L2 test, compared squared: hit iff D <= tau^2 * ||q~||^2 */
                if (d1 <= c->tau * c->tau * qn2)
                    slot = j;
            }
            if (override && override[bh] != -2) {
                slot = -1;
                if (override[bh] >= 0) {
                    for (int e = 0; e < W; e++)
                        if (vis[e] >= 0 && vis[e] == override[bh] && vis[e] <= m)
                            slot = e;
                    if (slot < 0)
                        invalid_total += 1;
                }
            }
        }
        free(vis);
        int32_t p = slot >= 0 ? pos[slot] : -1;
        int64_t st = slot >= 0 ? (int64_t)p - r + 1 : 0;
        if (st < 0)
            st = 0;
        if (hit) hit[bh] = slot >= 0;
        if (p_out) p_out[bh] = p;
        start_all[bh] = (int32_t)st;

        double *q = (double *)malloc((size_t)d * sizeof(double));
        double *O = (double *)malloc((size_t)(d + 2) * sizeof(double));
        double *tmp = (double *)malloc((size_t)(d + 2) * sizeof(double));
        double *Sm = (double *)malloc((size_t)(d + 2) * sizeof(double));
        orc_rope(qt, d, m, c->theta, q);

        if (tracked) {
            const void *kg = k_grp[b * Hkv + g], *vg = v_grp[b * Hkv + g];
            /* Figure 2 (b): complete.  A hit attends only [p-r+1, m] and
             * merges with the stored AS_{1:p-r}; a miss attends [0, m]. */
            orc_attend(q, kg, vg, c->kv_fp32, d, st, m, c->scale, tmp);
            if (slot >= 0)
                orc_merge(rs + (size_t)slot * (d + 2), tmp, d, O);
            else
                memcpy(O, tmp, (size_t)(d + 2) * sizeof(double));
            if (out)
                memcpy(out + (size_t)bh * d, O, (size_t)d * sizeof(double));
            if (full) {
                orc_attend(q, kg, vg, c->kv_fp32, d, 0, m, c->scale, tmp);
                memcpy(full + (size_t)bh * d, tmp, (size_t)d * sizeof(double));
            }
            /* Figure 2 (c): amend.  AS_{1:m-r} = AS_{1:m} (-) A(q, [m-r+1, m]);
             * nothing is left when m-r < 0. */
            if (m - r < 0) {
                orc_empty(d, Sm);
            } else {
                orc_attend(q, kg, vg, c->kv_fp32, d, m - r + 1, m, c->scale, tmp);
                orc_remove(O, tmp, d, Sm);
            }
        } else {
            for (int e = 0; e < d + 2; e++)
                Sm[e] = NAN;
        }
        if (reuse) {
            pos[slot_new] = (int32_t)m;
            float *dst = rq + (size_t)slot_new * d;
            for (int i = 0; i < d; i++)
                dst[i] = (c->flags & ORC_F_RING_BF16) ? orc_round_bf16(qt[i]) : qt[i];
            memcpy(rs + (size_t)slot_new * (d + 2), Sm, (size_t)(d + 2) * sizeof(double));
        }
        free(q); free(O); free(tmp); free(Sm);
    }

    for (int b = 0; b < B; b++) {
        int64_t m = (int64_t)seq_lens[b] - 1;
        for (int g = 0; g < Hkv; g++) {
            int64_t lo = m + 1;
            for (int i = 0; i < G; i++) {
                int32_t s = start_all[b * Hq + g * G + i];
                if (s < lo)
                    lo = s;
            }
            if (kv_tokens)
                kv_tokens[b * Hkv + g] = m < 0 ? 0 : m - lo + 1;
        }
    }
    if (start)
        memcpy(start, start_all, (size_t)B * Hq * sizeof(int32_t));
    free(start_all);
    c->calls += 1;
    return invalid_total;
}
