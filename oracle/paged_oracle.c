/*
 * paged_oracle.c -- plain fp64 CPU oracle for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the plain definition, no blocking, no fusion, no
 * reordering beyond the definition):
 *
 *   boostr 0.2.0-beta.2, attention/flash_standard.rs, `standard_attention_fwd`:
 *     out = softmax(scale * Q K^T + mask) V, and the natural-log logsumexp of
 *     the masked, scaled scores per query row.
 *   ...with the mask of `build_attention_mask` (same page): a key is hidden
 *     when causal and it lies after the query, or when a window W > 0 is set and
 *     key + W <= query; W = 0 means unlimited.
 *   ...with GQA as in `expand_kv` (same page): query head h reads KV head
 *     floor(h / (Hq / Hkv)).
 *   ruDNN 0.1.107, paged_attention/mod.rs, `DevicePlan::attention`: Q packed
 *     [queries, Hq, D]; K [pages, page_size, Hkv, D]; V [pages, page_size,
 *     Hkv, Dv]; causal masking compares absolute positions taken from the plan,
 *     prefill chunks included.  The logical key index t of a sequence IS its
 *     absolute position; it lives in page block_table[s][t / page_size], slot
 *     t % page_size.
 *   ruDNN, `DevicePlan::mla`: absorbed Q [queries, H, R], position Q
 *     [queries, H, P], latent [pages, page_size, 1, R] used as both key and
 *     value, rotated position cache [pages, page_size, 1, P]; the score adds
 *     the latent dot product and the position dot product before scaling.
 *
 * Keys that are not visible to a query row are never read.  Inputs are f32,
 * bf16 or IEEE binary16 (both as raw 16-bit patterns; ruDNN's tensor check
 * admits all three types) and are widened exactly to double.  All arithmetic
 * is double precision with libm exp/log.
 *
 * Rows run in parallel on POSIX threads; each (query, head) row is computed by
 * one thread in one fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { PO_F32 = 0, PO_BF16 = 1, PO_F16 = 2 };

/* IEEE 754 binary16 bits -> double (exact): 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits; exponent 0 holds zero and the subnormals
 * m * 2^-24, exponent 31 infinities and NaN. */
static double po_half(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* Exact widening of one stored element to double. */
static double po_load(int dtype, const void *base, int64_t idx)
{
    if (dtype == PO_F32)
        return (double)((const float *)base)[idx];
    if (dtype == PO_F16)
        return po_half(((const uint16_t *)base)[idx]);
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The widening above, exported for tests: out[i] = element i of base. */
int po_widen(int dtype, const void *base, int64_t n, double *out)
{
    if (dtype != PO_F32 && dtype != PO_BF16 && dtype != PO_F16)
        return -4;
    for (int64_t i = 0; i < n; ++i)
        out[i] = po_load(dtype, base, i);
    return 0;
}

typedef struct {
    /* geometry */
    int dtype;
    int num_seqs, table_width, page_size, num_pages;
    const int32_t *seq_lens, *cu_q, *q_pos, *block_table;
    int num_queries;
    int hq, hkv, d, dv;          /* MLA: hkv = 1, d = R (latent rank), dv = R */
    int p;                       /* MLA position width; 0 for plain attention */
    double scale;
    int causal, window;
    /* tensors */
    const void *q, *k, *v;       /* MLA: k = v = latent */
    const void *qp, *kp;         /* MLA only */
    /* block-sparse attention only: keys of block t / block_size count for
     * (query i, KV head h) iff that block is among sel[(i * hkv + h) * sel_k
     * .. + sel_k) (-1 entries unused); NULL = every visible key */
    const int32_t *sel;
    int sel_k, block_size;
    /* rows to evaluate: NULL = every (query, head) in order */
    const int64_t *rows;
    int64_t num_rows;
    double *out, *lse;
    /* work distribution */
    int nthreads;
    int status;
} po_job;

typedef struct { po_job *job; int tid; } po_thread_arg;

/* Sequence that owns packed query i: cu_q[s] <= i < cu_q[s + 1]. */
static int po_seq_of(const po_job *j, int i)
{
    for (int s = 0; s < j->num_seqs; ++s)
        if (j->cu_q[s] <= i && i < j->cu_q[s + 1])
            return s;
    return -1;
}

/* Visibility of key t for a query at absolute position pos in a sequence of
 * length len (the mask predicate above, on absolute positions). */
static int po_visible(const po_job *j, int t, int pos, int len)
{
    if (t < 0 || t >= len) return 0;
    if (j->causal && t > pos) return 0;
    if (j->window > 0 && (int64_t)t + j->window <= pos) return 0;
    return 1;
}

/* Key t of a visible row counts: every visible key, or for block-sparse
 * attention the visible keys of the selected blocks. */
static int po_used(const po_job *j, int i, int kvh, int t, int pos, int len)
{
    if (!po_visible(j, t, pos, len)) return 0;
    if (!j->sel) return 1;
    const int32_t *row = j->sel + ((int64_t)i * j->hkv + kvh) * j->sel_k;
    for (int e = 0; e < j->sel_k; ++e)
        if (row[e] >= 0 && row[e] == t / j->block_size) return 1;
    return 0;
}

/* Element offset of (key t, kv head kvh, component c) in a pool whose rows are
 * `width` wide and that has `heads` heads per slot. */
static int64_t po_pool_offset(const po_job *j, int s, int t, int kvh, int heads, int width, int c,
                              int *bad)
{
    int page = j->block_table[(int64_t)s * j->table_width + t / j->page_size];
    if (page < 0 || page >= j->num_pages) { *bad = 1; return 0; }
    int slot = t % j->page_size;
    return (((int64_t)page * j->page_size + slot) * heads + kvh) * width + c;
}

/* One (query i, head h) row: out_row[0..dv), *lse_row. */
static int po_row(const po_job *j, int i, int h, double *sc, double *out_row, double *lse_row)
{
    int s = po_seq_of(j, i);
    if (s < 0) return -1;
    int len = j->seq_lens[s];
    int pos = j->q_pos[i];
    int group = j->hq / j->hkv;
    int kvh = h / group;
    int bad = 0;

    /* scores of the visible keys; invisible keys are skipped, never read */
    double m = -INFINITY;
    int count = 0;
    for (int t = 0; t < len; ++t) {
        if (!po_used(j, i, kvh, t, pos, len)) { sc[t] = -INFINITY; continue; }
        double dot = 0.0;
        for (int c = 0; c < j->d; ++c) {
            double qv = po_load(j->dtype, j->q, ((int64_t)i * j->hq + h) * j->d + c);
            double kv = po_load(j->dtype, j->k, po_pool_offset(j, s, t, kvh, j->hkv, j->d, c, &bad));
            dot += qv * kv;
        }
        for (int c = 0; c < j->p; ++c) {
            double qv = po_load(j->dtype, j->qp, ((int64_t)i * j->hq + h) * j->p + c);
            double kv = po_load(j->dtype, j->kp, po_pool_offset(j, s, t, 0, 1, j->p, c, &bad));
            dot += qv * kv;
        }
        if (bad) return -2;
        sc[t] = j->scale * dot;
        if (sc[t] > m) m = sc[t];
        ++count;
    }
    if (count == 0) {
        /* softmax over an empty set is undefined */
        for (int c = 0; c < j->dv; ++c) out_row[c] = NAN;
        *lse_row = -INFINITY;
        return 0;
    }

    /* softmax weights and their sum */
    double l = 0.0;
    for (int t = 0; t < len; ++t) {
        if (sc[t] == -INFINITY) continue;
        sc[t] = exp(sc[t] - m);
        l += sc[t];
    }
    /* weighted sum of the visible value rows, keys in increasing order */
    for (int c = 0; c < j->dv; ++c) out_row[c] = 0.0;
    for (int t = 0; t < len; ++t) {
        if (!po_used(j, i, kvh, t, pos, len)) continue;
        for (int c = 0; c < j->dv; ++c)
            out_row[c] += sc[t] * po_load(j->dtype, j->v, po_pool_offset(j, s, t, kvh, j->hkv, j->dv, c, &bad));
    }
    for (int c = 0; c < j->dv; ++c) out_row[c] /= l;
    if (bad) return -2;
    *lse_row = m + log(l);
    return 0;
}

static void *po_worker(void *arg)
{
    po_thread_arg *a = (po_thread_arg *)arg;
    po_job *j = a->job;
    int max_len = 1;
    for (int s = 0; s < j->num_seqs; ++s)
        if (j->seq_lens[s] > max_len) max_len = j->seq_lens[s];
    double *sc = (double *)malloc(sizeof(double) * (size_t)max_len);
    if (!sc) { j->status = -3; return NULL; }
    int64_t total = j->rows ? j->num_rows : (int64_t)j->num_queries * j->hq;
    for (int64_t r = a->tid; r < total; r += j->nthreads) {
        int64_t flat = j->rows ? j->rows[r] : r;
        int i = (int)(flat / j->hq), h = (int)(flat % j->hq);
        int rc = po_row(j, i, h, sc, j->out + r * j->dv, j->lse + r);
        if (rc) j->status = rc;
    }
    free(sc);
    return NULL;
}

static int po_run(po_job *j)
{
    if (j->hq <= 0 || j->hkv <= 0 || j->hq % j->hkv != 0 || j->page_size <= 0) return -4;
    if (j->dtype != PO_F32 && j->dtype != PO_BF16 && j->dtype != PO_F16) return -4;
    if (j->rows) {
        for (int64_t r = 0; r < j->num_rows; ++r)
            if (j->rows[r] < 0 || j->rows[r] >= (int64_t)j->num_queries * j->hq) return -4;
    }
    int n = j->nthreads > 0 ? j->nthreads : 1;
    j->nthreads = n;
    j->status = 0;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n);
    po_thread_arg *args = (po_thread_arg *)malloc(sizeof(po_thread_arg) * (size_t)n);
    if (!th || !args) { free(th); free(args); return -3; }
    for (int t = 0; t < n; ++t) {
        args[t].job = j;
        args[t].tid = t;
        pthread_create(&th[t], NULL, po_worker, &args[t]);
    }
    for (int t = 0; t < n; ++t) pthread_join(th[t], NULL);
    free(th);
    free(args);
    return j->status;
}

/*
 * Paged GQA/MHA attention.  Returns 0, or a negative code: -1 query outside
 * every sequence, -2 block-table entry outside the pool, -3 out of memory,
 * -4 bad geometry.  out is [rows, dv] (all rows: [queries, hq, dv]) and lse
 * is [rows] natural-log logsumexp of the scaled, masked scores.
 */
int po_attention(int dtype, const void *q, const void *k, const void *v,
                 int num_seqs, const int32_t *seq_lens, const int32_t *cu_q, const int32_t *q_pos,
                 const int32_t *block_table, int table_width, int page_size, int num_pages,
                 int hq, int hkv, int d, int dv, double scale, int causal, int window,
                 const int64_t *rows, int64_t num_rows, double *out, double *lse, int nthreads)
{
    po_job j;
    memset(&j, 0, sizeof j);
    j.dtype = dtype;
    j.num_seqs = num_seqs; j.table_width = table_width; j.page_size = page_size; j.num_pages = num_pages;
    j.seq_lens = seq_lens; j.cu_q = cu_q; j.q_pos = q_pos; j.block_table = block_table;
    j.num_queries = num_seqs > 0 ? cu_q[num_seqs] : 0;
    j.hq = hq; j.hkv = hkv; j.d = d; j.dv = dv; j.p = 0;
    j.scale = scale; j.causal = causal; j.window = window;
    j.q = q; j.k = k; j.v = v;
    j.rows = rows; j.num_rows = num_rows; j.out = out; j.lse = lse; j.nthreads = nthreads;
    return po_run(&j);
}

/*
 * Absorbed MLA: one shared latent head used as key and value, plus a rotated
 * position cache that only enters the score.  Same return codes and output
 * layout as po_attention, with dv = r.
 */
int po_mla(int dtype, const void *q_abs, const void *q_rope, const void *latent, const void *kpos,
           int num_seqs, const int32_t *seq_lens, const int32_t *cu_q, const int32_t *q_pos,
           const int32_t *block_table, int table_width, int page_size, int num_pages,
           int heads, int r, int p, double scale, int causal, int window,
           const int64_t *rows, int64_t num_rows, double *out, double *lse, int nthreads)
{
    po_job j;
    memset(&j, 0, sizeof j);
    j.dtype = dtype;
    j.num_seqs = num_seqs; j.table_width = table_width; j.page_size = page_size; j.num_pages = num_pages;
    j.seq_lens = seq_lens; j.cu_q = cu_q; j.q_pos = q_pos; j.block_table = block_table;
    j.num_queries = num_seqs > 0 ? cu_q[num_seqs] : 0;
    j.hq = heads; j.hkv = 1; j.d = r; j.dv = r; j.p = p;
    j.scale = scale; j.causal = causal; j.window = window;
    j.q = q_abs; j.k = latent; j.v = latent; j.qp = q_rope; j.kp = kpos;
    j.rows = rows; j.num_rows = num_rows; j.out = out; j.lse = lse; j.nthreads = nthreads;
    return po_run(&j);
}

/* ------------------------------------------------------------------------
 * Backward (ruDNN paged_attention `attention_backward`, `mla_backward`:
 * first-order gradients of the forward above, recomputing the scores from
 * Q and K), written out from the standard attention backward of boostr
 * attention/flash_standard.rs (`standard_attention_bwd`): with P the softmax
 * weights of a row and dO its output gradient,
 *   dV_t += P_t dO,   dP_t = dO . V_t,   D = dO . O,   dS_t = P_t (dP_t - D),
 *   dQ = scale sum_t dS_t K_t,   dK_t += scale dS_t Q,
 * with the GQA head map summing the gradients of the G query heads that share
 * a KV head (`sum_gqa_grads`).  MLA: the latent is key and value, so its
 * gradient receives both the dK and the dV terms; the position query and
 * cache receive the dQ / dK terms of the position dot product.
 *
 * Single pass per KV head (threads own disjoint KV heads, so the history
 * gradients of one head are summed by one thread in a fixed order: sequences,
 * queries, query heads, keys ascending); pool rows no visible key names keep
 * gradient zero.
 * ---------------------------------------------------------------------- */
typedef struct {
    po_job *job;
    const void *dout;            /* [queries, hq, dv], storage dtype */
    double *dq, *dqp;            /* [queries, hq, d] / [queries, hq, p] */
    double *dk, *dv, *dkp;       /* pool shaped; MLA: dk == dv (latent), dkp [pages, ps, 1, p] */
    int kvh0, kvh_step;
    int status;
} po_bwd_arg;

static void *po_bwd_worker(void *arg)
{
    po_bwd_arg *a = (po_bwd_arg *)arg;
    po_job *j = a->job;
    const int group = j->hq / j->hkv;
    int max_len = 1;
    for (int s = 0; s < j->num_seqs; ++s)
        if (j->seq_lens[s] > max_len) max_len = j->seq_lens[s];
    double *pw = (double *)malloc(sizeof(double) * (size_t)max_len);  /* P_t */
    double *ds = (double *)malloc(sizeof(double) * (size_t)max_len);  /* dS_t */
    double *o = (double *)malloc(sizeof(double) * (size_t)j->dv);
    if (!pw || !ds || !o) { free(pw); free(ds); free(o); a->status = -3; return NULL; }
    for (int kvh = a->kvh0; kvh < j->hkv; kvh += a->kvh_step) {
        for (int s = 0; s < j->num_seqs; ++s) {
            const int len = j->seq_lens[s];
            for (int i = j->cu_q[s]; i < j->cu_q[s + 1]; ++i) {
                const int pos = j->q_pos[i];
                for (int h = kvh * group; h < (kvh + 1) * group; ++h) {
                    const int64_t row = (int64_t)i * j->hq + h;
                    int bad = 0, count = 0;
                    double m = -INFINITY;
                    /* scores of the visible keys */
                    for (int t = 0; t < len; ++t) {
                        if (!po_visible(j, t, pos, len)) { pw[t] = -INFINITY; continue; }
                        double dot = 0.0;
                        for (int c = 0; c < j->d; ++c)
                            dot += po_load(j->dtype, j->q, row * j->d + c) *
                                   po_load(j->dtype, j->k, po_pool_offset(j, s, t, kvh, j->hkv, j->d, c, &bad));
                        for (int c = 0; c < j->p; ++c)
                            dot += po_load(j->dtype, j->qp, row * j->p + c) *
                                   po_load(j->dtype, j->kp, po_pool_offset(j, s, t, 0, 1, j->p, c, &bad));
                        if (bad) { a->status = -2; goto done; }
                        pw[t] = j->scale * dot;
                        if (pw[t] > m) m = pw[t];
                        ++count;
                    }
                    if (count == 0) { a->status = -1; goto done; }
                    /* softmax weights P_t and the row output O */
                    double l = 0.0;
                    for (int t = 0; t < len; ++t) {
                        if (pw[t] == -INFINITY) continue;
                        pw[t] = exp(pw[t] - m);
                        l += pw[t];
                    }
                    for (int c = 0; c < j->dv; ++c) o[c] = 0.0;
                    for (int t = 0; t < len; ++t) {
                        if (pw[t] == -INFINITY) continue;
                        pw[t] /= l;
                        for (int c = 0; c < j->dv; ++c)
                            o[c] += pw[t] * po_load(j->dtype, j->v, po_pool_offset(j, s, t, kvh, j->hkv, j->dv, c, &bad));
                    }
                    /* D = dO . O, then dP_t, dS_t and dV_t */
                    double dd = 0.0;
                    for (int c = 0; c < j->dv; ++c) dd += po_load(j->dtype, a->dout, row * j->dv + c) * o[c];
                    for (int t = 0; t < len; ++t) {
                        if (pw[t] == -INFINITY) { ds[t] = 0.0; continue; }
                        double dp = 0.0;
                        for (int c = 0; c < j->dv; ++c) {
                            const double g = po_load(j->dtype, a->dout, row * j->dv + c);
                            const int64_t off = po_pool_offset(j, s, t, kvh, j->hkv, j->dv, c, &bad);
                            dp += g * po_load(j->dtype, j->v, off);
                            a->dv[off] += pw[t] * g;
                        }
                        ds[t] = pw[t] * (dp - dd);
                    }
                    /* dQ (and the position query) from dS and K; dK_t from dS_t and Q */
                    for (int c = 0; c < j->d; ++c) a->dq[row * j->d + c] = 0.0;
                    for (int c = 0; c < j->p; ++c) a->dqp[row * j->p + c] = 0.0;
                    for (int t = 0; t < len; ++t) {
                        if (pw[t] == -INFINITY) continue;
                        for (int c = 0; c < j->d; ++c) {
                            const int64_t off = po_pool_offset(j, s, t, kvh, j->hkv, j->d, c, &bad);
                            a->dq[row * j->d + c] += j->scale * ds[t] * po_load(j->dtype, j->k, off);
                            a->dk[off] += j->scale * ds[t] * po_load(j->dtype, j->q, row * j->d + c);
                        }
                        for (int c = 0; c < j->p; ++c) {
                            const int64_t off = po_pool_offset(j, s, t, 0, 1, j->p, c, &bad);
                            a->dqp[row * j->p + c] += j->scale * ds[t] * po_load(j->dtype, j->kp, off);
                            a->dkp[off] += j->scale * ds[t] * po_load(j->dtype, j->qp, row * j->p + c);
                        }
                    }
                    if (bad) { a->status = -2; goto done; }
                }
            }
        }
    }
done:
    free(pw);
    free(ds);
    free(o);
    return NULL;
}

static int po_bwd_run(po_job *j, const void *dout, double *dq, double *dqp, double *dk, double *dv, double *dkp,
                      int64_t k_elems, int64_t v_elems, int64_t kp_elems)
{
    if (j->hq <= 0 || j->hkv <= 0 || j->hq % j->hkv != 0 || j->page_size <= 0) return -4;
    if (j->dtype != PO_F32 && j->dtype != PO_BF16 && j->dtype != PO_F16) return -4;
    /* history gradients start at zero (MLA: dk and dv are the same array) */
    for (int64_t e = 0; e < k_elems; ++e) dk[e] = 0.0;
    if (dv != dk)
        for (int64_t e = 0; e < v_elems; ++e) dv[e] = 0.0;
    for (int64_t e = 0; e < kp_elems; ++e) dkp[e] = 0.0;
    int n = j->nthreads > 0 ? j->nthreads : 1;
    if (n > j->hkv) n = j->hkv;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n);
    po_bwd_arg *args = (po_bwd_arg *)malloc(sizeof(po_bwd_arg) * (size_t)n);
    if (!th || !args) { free(th); free(args); return -3; }
    for (int t = 0; t < n; ++t) {
        po_bwd_arg init = {j, dout, dq, dqp, dk, dv, dkp, t, n, 0};
        args[t] = init;
        pthread_create(&th[t], NULL, po_bwd_worker, &args[t]);
    }
    int status = 0;
    for (int t = 0; t < n; ++t) {
        pthread_join(th[t], NULL);
        if (args[t].status) status = args[t].status;
    }
    free(th);
    free(args);
    return status;
}

/*
 * Paged GQA/MHA backward: dq [queries, hq, d]; dk, dv pool shaped ([pages,
 * page_size, hkv, d] / [.., dv]), zero where no visible key lands.  dout has
 * the storage dtype.  Return codes as po_attention.
 */
int po_attention_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout,
                     int num_seqs, const int32_t *seq_lens, const int32_t *cu_q, const int32_t *q_pos,
                     const int32_t *block_table, int table_width, int page_size, int num_pages,
                     int hq, int hkv, int d, int dv, double scale, int causal, int window,
                     double *dq, double *dk, double *dvv, int nthreads)
{
    po_job j;
    memset(&j, 0, sizeof j);
    j.dtype = dtype;
    j.num_seqs = num_seqs; j.table_width = table_width; j.page_size = page_size; j.num_pages = num_pages;
    j.seq_lens = seq_lens; j.cu_q = cu_q; j.q_pos = q_pos; j.block_table = block_table;
    j.num_queries = num_seqs > 0 ? cu_q[num_seqs] : 0;
    j.hq = hq; j.hkv = hkv; j.d = d; j.dv = dv; j.p = 0;
    j.scale = scale; j.causal = causal; j.window = window;
    j.q = q; j.k = k; j.v = v;
    j.nthreads = nthreads;
    const int64_t slots = (int64_t)num_pages * page_size * hkv;
    return po_bwd_run(&j, dout, dq, NULL, dk, dvv, NULL, slots * d, slots * dv, 0);
}

/*
 * Absorbed-MLA backward: dq_abs [queries, heads, r], dq_rope [queries, heads,
 * p], dlatent [pages, page_size, 1, r] (key and value terms), dkpos [pages,
 * page_size, 1, p].  Return codes as po_attention.
 */
int po_mla_bwd(int dtype, const void *q_abs, const void *q_rope, const void *latent, const void *kpos,
               const void *dout, int num_seqs, const int32_t *seq_lens, const int32_t *cu_q,
               const int32_t *q_pos, const int32_t *block_table, int table_width, int page_size,
               int num_pages, int heads, int r, int p, double scale, int causal, int window,
               double *dq_abs, double *dq_rope, double *dlatent, double *dkpos, int nthreads)
{
    po_job j;
    memset(&j, 0, sizeof j);
    j.dtype = dtype;
    j.num_seqs = num_seqs; j.table_width = table_width; j.page_size = page_size; j.num_pages = num_pages;
    j.seq_lens = seq_lens; j.cu_q = cu_q; j.q_pos = q_pos; j.block_table = block_table;
    j.num_queries = num_seqs > 0 ? cu_q[num_seqs] : 0;
    j.hq = heads; j.hkv = 1; j.d = r; j.dv = r; j.p = p;
    j.scale = scale; j.causal = causal; j.window = window;
    j.q = q_abs; j.k = latent; j.v = latent; j.qp = q_rope; j.kp = kpos;
    j.nthreads = nthreads;
    const int64_t slots = (int64_t)num_pages * page_size;
    return po_bwd_run(&j, dout, dq_abs, dq_rope, dlatent, dlatent, dkpos, slots * r, slots * r, slots * p);
}

/* ------------------------------------------------------------------------
 * Block-sparse top-k attention (alice-llm 2.0.0, sparse_attention/
 * llama3_bridge.rs, `llama3_sparse_attention`): keys are grouped in blocks
 * of block_size consecutive positions; for each (query, KV head) a proxy
 * scores every block by the largest dot product between the first query
 * head of the group and the block's keys (`compute_proxy_block_max_scores`,
 * the cheap proxy "first Q lane of each KV head"), the top-k blocks are kept
 * (`sparse_topk_select_batch`) and attention runs over the keys of the kept
 * blocks only, its per-block partials merged by log-sum-exp
 * (`kvouter_forward`, `lse_combine`) -- the same value as one softmax over
 * the union of those keys, which is what po_sparse_attention computes.
 *
 * The page runs the proxy in f32 on the CPU.  The proxy here is the f32
 * product sum taken in increasing dimension order, each step one fused
 * multiply-add (for 16-bit inputs the products are exact in f32, so a plain
 * multiply then add gives the same bits); a block's score is the largest
 * score of its visible keys, -inf for a block with none.
 * ---------------------------------------------------------------------- */

/* Exact widening of one stored element to float (f32 data as is). */
static float po_loadf(int dtype, const void *base, int64_t idx)
{
    if (dtype == PO_F32)
        return ((const float *)base)[idx];
    return (float)po_load(dtype, base, idx);
}

typedef struct {
    const po_job *job;
    float *scores;      /* [queries, hkv, nblk] */
    int nblk, tid, nthreads, status;
} po_proxy_arg;

static void *po_proxy_worker(void *arg)
{
    po_proxy_arg *a = (po_proxy_arg *)arg;
    const po_job *j = a->job;
    const int64_t rows = (int64_t)j->num_queries * j->hkv;
    const int group = j->hq / j->hkv;
    for (int64_t row = a->tid; row < rows; row += a->nthreads) {
        const int i = (int)(row / j->hkv), kvh = (int)(row % j->hkv);
        float *out = a->scores + row * a->nblk;
        for (int r = 0; r < a->nblk; ++r) out[r] = -INFINITY;
        const int s = po_seq_of(j, i);
        if (s < 0) { a->status = -1; continue; }
        const int len = j->seq_lens[s], pos = j->q_pos[i];
        const int64_t qbase = ((int64_t)i * j->hq + (int64_t)kvh * group) * j->d; /* first head of the group */
        for (int t = 0; t < len; ++t) {
            if (!po_visible(j, t, pos, len)) continue;
            int bad = 0;
            float acc = 0.f;
            for (int c = 0; c < j->d; ++c) {
                const float qv = po_loadf(j->dtype, j->q, qbase + c);
                const float kv = po_loadf(j->dtype, j->k, po_pool_offset(j, s, t, kvh, j->hkv, j->d, c, &bad));
                acc = j->dtype == PO_F32 ? fmaf(qv, kv, acc) : acc + qv * kv;
            }
            if (bad) { a->status = -2; break; }
            const int r = t / j->block_size;
            if (r < a->nblk && acc > out[r]) out[r] = acc;
        }
    }
    return NULL;
}

/*
 * Proxy block scores of every (query, KV head) row: scores [queries, hkv,
 * nblk] float, block r covering key positions [r * block_size, (r + 1) *
 * block_size).  Return codes as po_attention.
 */
int po_sparse_proxy(int dtype, const void *q, const void *k, int num_seqs, const int32_t *seq_lens,
                    const int32_t *cu_q, const int32_t *q_pos, const int32_t *block_table, int table_width,
                    int page_size, int num_pages, int hq, int hkv, int d, int causal, int window, int block_size,
                    float *scores, int nblk, int nthreads)
{
    po_job j;
    memset(&j, 0, sizeof j);
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || page_size <= 0 || block_size <= 0 || nblk < 0) return -4;
    if (dtype != PO_F32 && dtype != PO_BF16 && dtype != PO_F16) return -4;
    j.dtype = dtype;
    j.num_seqs = num_seqs; j.table_width = table_width; j.page_size = page_size; j.num_pages = num_pages;
    j.seq_lens = seq_lens; j.cu_q = cu_q; j.q_pos = q_pos; j.block_table = block_table;
    j.num_queries = num_seqs > 0 ? cu_q[num_seqs] : 0;
    j.hq = hq; j.hkv = hkv; j.d = d; j.dv = d;
    j.causal = causal; j.window = window; j.block_size = block_size;
    j.q = q; j.k = k;
    int n = nthreads > 0 ? nthreads : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n);
    po_proxy_arg *args = (po_proxy_arg *)malloc(sizeof(po_proxy_arg) * (size_t)n);
    if (!th || !args) { free(th); free(args); return -3; }
    for (int t = 0; t < n; ++t) {
        po_proxy_arg init = {&j, scores, nblk, t, n, 0};
        args[t] = init;
        pthread_create(&th[t], NULL, po_proxy_worker, &args[t]);
    }
    int status = 0;
    for (int t = 0; t < n; ++t) {
        pthread_join(th[t], NULL);
        if (args[t].status) status = args[t].status;
    }
    free(th);
    free(args);
    return status;
}

/*
 * Attention over the visible keys of the selected blocks: sel [queries, hkv,
 * sel_k] block indices (-1 = none); otherwise as po_attention.  With every
 * block of a row selected the row is exactly po_attention's.
 */
int po_sparse_attention(int dtype, const void *q, const void *k, const void *v,
                        int num_seqs, const int32_t *seq_lens, const int32_t *cu_q, const int32_t *q_pos,
                        const int32_t *block_table, int table_width, int page_size, int num_pages,
                        int hq, int hkv, int d, int dv, double scale, int causal, int window,
                        const int32_t *sel, int sel_k, int block_size,
                        double *out, double *lse, int nthreads)
{
    po_job j;
    memset(&j, 0, sizeof j);
    if (!sel || sel_k <= 0 || block_size <= 0) return -4;
    j.dtype = dtype;
    j.num_seqs = num_seqs; j.table_width = table_width; j.page_size = page_size; j.num_pages = num_pages;
    j.seq_lens = seq_lens; j.cu_q = cu_q; j.q_pos = q_pos; j.block_table = block_table;
    j.num_queries = num_seqs > 0 ? cu_q[num_seqs] : 0;
    j.hq = hq; j.hkv = hkv; j.d = d; j.dv = dv; j.p = 0;
    j.scale = scale; j.causal = causal; j.window = window;
    j.q = q; j.k = k; j.v = v;
    j.sel = sel; j.sel_k = sel_k; j.block_size = block_size;
    j.out = out; j.lse = lse; j.nthreads = nthreads;
    return po_run(&j);
}
