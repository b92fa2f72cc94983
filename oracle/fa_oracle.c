/*
 * fa_oracle.c -- the attention oracle: a plain, slow, fp64, two-pass CPU implementation of the
 * forward pass and (at the end of this file) of its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
 * may load this library.  It shares no code, header or constant with the HIP library and includes
 * nothing from it.
 *
 * What it computes (for every requested query row i of head (b, h)):
 *
 *   Attention(Q, K, V) = Softmax(Q K^T / sqrt(d)) V, with the 1/sqrt(d) factor generalised to a
 *   caller-given scale.  Source: page "FlashAttention：让长文本推理不再"卡显存"" (ai6s.net,
 *   6a0d42d8...), section "Attention 的显存黑洞" (the formula and its three steps: scores,
 *   softmax, product with V); the same three steps as code on page ai6s.net/6a0d3bfb... section
 *   "为什么传统attention会卡住？" and in the precision check of page hwcomputing.csdn.net/6a0d4444...
 *
 *   Causal: key j is visible to query i iff j <= i.  Source: page ai6s.net/6a0d3bfb..., the
 *   causal-mask section, where the mask tensor marks entries strictly above the diagonal
 *   (torch.triu(..., diagonal=1)) as hidden; page hwcomputing.csdn.net/6a0d4681..., section
 *   "Causal Mask的实现差异" (each position sees only earlier tokens).
 *
 *   lse_i = ln sum_{j visible} exp(s_ij), the natural-log log-sum-exp of the scaled logits, one fp
 *   value per (b, h, i).  Source: page ai6s.net/6a140d07..., section "第二层：数值稳定性增强" (the
 *   lse accumulator of shape [B, H, block_i], built with torch.log / torch.exp).
 *
 * Generalised rows (fa_oracle_rows_ex).  Query row i of an Nq-row Q sits at sequence position
 * q_offset + i; key row j of an Nk-row K/V at position j.  A call covers the key chunk
 * [kv_start, kv_start + kv_len), so that one long key sequence can be processed in pieces whose
 * partial (O, lse) are combined exactly afterwards through their lse: page ai6s.net/6a0d3bfb...,
 * section "ops-transformer仓库里还有什么？" (Ring Attention and block-wise attention for long
 * sequences) and page ai6s.net/6a140d07..., sections "第二层：数值稳定性增强" (combining two partial
 * log-sum-exps, shifted by their maximum) and "多卡并行" (a 64K sequence split into 8K pieces).
 * Visible keys of row i (qpos = q_offset + i):
 *     j in [kv_start, kv_start + kv_len),
 *     j <= qpos                if causal,
 *     j >= qpos - window       if window >= 0 (a sliding window of `window` earlier keys plus the
 *                              query's own position; page ai6s.net/6a140d07..., section
 *                              "与其他优化方法对比", lists sliding-window attention; only with causal).
 * A row with no visible key has O = 0 and lse = -inf (the identity of the lse combination).
 * Q/O are [B][H][Nq][D] or [B][Nq][H][D]; K/V [B][H][Nk][D] or [B][Nk][H][D].
 *
 * Steps, per row, in this order (nothing is tiled, fused or reordered):
 *   1. widen the stored q, k, v elements exactly to double;
 *   2. pass 1: s_j = scale * sum_d q_d k_jd (d ascending) for every visible j; m = max_j s_j;
 *   3. pass 2: e_j = exp(s_j - m); l = sum_j e_j (j ascending); o_d = (sum_j e_j v_jd) / l;
 *   4. lse = m + log(l).
 *
 * Element addressing (packed, contiguous tensors):
 *   layout 0, BHSD = [B][H][N][D]:  ((b*H + h)*N + i)*D + d
 *   layout 1, BSND = [B][N][H][D]:  ((b*N + i)*H + h)*D + d
 * Input element types: 0 = IEEE binary32, 1 = IEEE binary16, 2 = bfloat16, 3 = IEEE binary64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_F64 3

/* binary16 -> double, exactly: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double orc_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* zero or subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16 -> double, exactly: bfloat16 is the upper half of a binary32. */
static double orc_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double orc_load(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_F16: return orc_half_to_double(((const uint16_t*)base)[idx]);
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[idx]);
    default: return ((const double*)base)[idx];
    }
}

typedef struct {
    const void *q, *k, *v;
    int dtype, layout, causal;
    int64_t B, H, Nq, Nk, D;
    int64_t window, q_offset, kv_start, kv_len;
    double scale;
    const int64_t* rows; /* nrows triples (b, h, i) */
    int64_t nrows;
    double* o;   /* nrows * D */
    double* lse; /* nrows */
    int64_t first, last;
    int status;
} orc_job;

/* element index of row i of a tensor with N rows per (b, h) */
static int64_t orc_index(const orc_job* J, int64_t N, int64_t b, int64_t h, int64_t i, int64_t d) {
    if (J->layout == 0) return ((b * J->H + h) * N + i) * J->D + d;
    return ((b * N + i) * J->H + h) * J->D + d;
}

static void* orc_worker(void* arg) {
    orc_job* J = (orc_job*)arg;
    const int64_t Nq = J->Nq, Nk = J->Nk, D = J->D;
    double* srow = (double*)malloc(sizeof(double) * (size_t)(J->kv_len > 0 ? J->kv_len : 1));
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!srow || !qrow) {
        free(srow);
        free(qrow);
        J->status = -1;
        return NULL;
    }
    for (int64_t r = J->first; r < J->last; ++r) {
        const int64_t b = J->rows[3 * r], h = J->rows[3 * r + 1], i = J->rows[3 * r + 2];
        /* visible keys: jbeg .. jend-1 */
        const int64_t qpos = J->q_offset + i;
        int64_t jbeg = J->kv_start, jend = J->kv_start + J->kv_len;
        if (J->causal && qpos + 1 < jend) jend = qpos + 1;
        if (J->window >= 0 && qpos - J->window > jbeg) jbeg = qpos - J->window;
        double* o = J->o + r * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (jend <= jbeg) { /* no visible key */
            J->lse[r] = -INFINITY;
            continue;
        }
        for (int64_t d = 0; d < D; ++d) qrow[d] = orc_load(J->q, J->dtype, orc_index(J, Nq, b, h, i, d));

        /* pass 1: scaled scores and their maximum */
        double m = -INFINITY;
        for (int64_t j = jbeg; j < jend; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qrow[d] * orc_load(J->k, J->dtype, orc_index(J, Nk, b, h, j, d));
            srow[j - jbeg] = J->scale * dot;
            if (srow[j - jbeg] > m) m = srow[j - jbeg];
        }

        /* pass 2: exponentials relative to the maximum, their sum, and the weighted sum of V rows */
        double l = 0.0;
        for (int64_t j = jbeg; j < jend; ++j) {
            const double e = exp(srow[j - jbeg] - m);
            l += e;
            for (int64_t d = 0; d < D; ++d) o[d] += e * orc_load(J->v, J->dtype, orc_index(J, Nk, b, h, j, d));
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= l;
        J->lse[r] = m + log(l);
    }
    free(srow);
    free(qrow);
    return NULL;
}

/*
 * Computes O (nrows x D, fp64, row r for triple r) and lse (nrows, fp64) for the requested
 * (b, h, i) triples, i < Nq, under the generalised visibility rule above.  nthreads >= 1 workers
 * take contiguous slices of the triple list.  Returns 0 on success, -2 on a bad argument, -1 if
 * memory for the row buffers ran out.
 */
int fa_oracle_rows_ex(const void* q, const void* k, const void* v, int dtype, int layout, int64_t B,
                      int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, int64_t window,
                      int64_t q_offset, int64_t kv_start, int64_t kv_len, double scale,
                      const int64_t* rows, int64_t nrows, double* o_out, double* lse_out, int nthreads) {
    if (!q || !k || !v || !rows || !o_out || !lse_out) return -2;
    if (dtype < 0 || dtype > 3 || layout < 0 || layout > 1) return -2;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1 || nrows < 0) return -2;
    if (kv_start < 0 || kv_len < 0 || kv_start + kv_len > Nk) return -2;
    if (window >= 0 && !causal) return -2;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Nq) return -2;
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    if (nrows < nthreads) nthreads = nrows > 0 ? (int)nrows : 1;

    orc_job* jobs = (orc_job*)calloc((size_t)nthreads, sizeof(orc_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    char* running = (char*)calloc((size_t)nthreads, 1);
    if (!jobs || !tids || !running) {
        free(jobs);
        free(tids);
        free(running);
        return -1;
    }
    int status = 0;
    for (int t = 0; t < nthreads; ++t) {
        orc_job* J = &jobs[t];
        J->q = q; J->k = k; J->v = v;
        J->dtype = dtype; J->layout = layout; J->causal = causal ? 1 : 0;
        J->B = B; J->H = H; J->Nq = Nq; J->Nk = Nk; J->D = D;
        J->window = window < 0 ? -1 : window;
        J->q_offset = q_offset; J->kv_start = kv_start; J->kv_len = kv_len;
        J->scale = scale;
        J->rows = rows; J->nrows = nrows;
        J->o = o_out; J->lse = lse_out;
        J->first = nrows * t / nthreads;
        J->last = nrows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) {
        /* a worker that cannot be started has its slice done on this thread instead */
        if (pthread_create(&tids[t], NULL, orc_worker, &jobs[t]) == 0)
            running[t] = 1;
        else
            orc_worker(&jobs[t]);
    }
    orc_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (running[t]) pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) status = jobs[t].status;
    free(jobs);
    free(tids);
    free(running);
    return status;
}

/* The plain case: Nq = Nk = N, every key, query i at position i. */
int fa_oracle_rows(const void* q, const void* k, const void* v, int dtype, int layout, int64_t B,
                   int64_t H, int64_t N, int64_t D, int causal, double scale, const int64_t* rows,
                   int64_t nrows, double* o_out, double* lse_out, int nthreads) {
    return fa_oracle_rows_ex(q, k, v, dtype, layout, B, H, N, N, D, causal, -1, 0, 0, N, scale, rows, nrows,
                             o_out, lse_out, nthreads);
}

/*
 * ---------------------------------------------------------------------------------------------
 * Backward pass (gradients of the attention forward above, plain case Nq = Nk = N).
 *
 * Page ai6s.net/6a0d3bfb..., section "FlashAttention在昇腾NPU上怎么跑？" (item 3, recomputation
 * instead of storage) says the backward pass needs the forward's intermediate results and that
 * FlashAttention recomputes them rather than storing the N x N matrices; page
 * hwcomputing.csdn.net/6a0d4681..., section "反向传播的特殊处理", names the backward's extra
 * `deterministic` switch.  Neither page prints the gradient formulas, so this oracle writes out
 * the plain definition: with the upstream gradient dO (same shape as O), it returns the
 * vector-Jacobian product of O = Softmax(scale Q K^T [+ causal mask]) V, i.e. the gradients of
 * L = sum_{i,d} dO_id O_id with respect to Q, K and V.  By the chain rule, per row i:
 *
 *   s_ij  = scale * q_i . k_j            (visible j only; hidden pairs contribute nothing)
 *   P_ij  = exp(s_ij - m_i) / l_i        (two-pass softmax, as in the forward)
 *   dV_j += P_ij dO_i                    (O_i = sum_j P_ij v_j)
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)           (softmax Jacobian dP_ij/ds_ik = P_ij (delta_jk - P_ik))
 *   dQ_i += scale * dS_ij k_j
 *   dK_j += scale * dS_ij q_i
 *
 * Everything is in double.  D_i is taken from P and dP as the chain rule gives it (not from O).
 * Rows are split among the workers; each worker keeps its own dK and dV accumulators, which are
 * added in worker order at the end.
 *
 * Generalised rows (fa_oracle_bwd_head_ex), matching fa_oracle_rows_ex: query row i of an Nq-row Q
 * sits at position q_offset + i and sees the keys j of [0, Nk) with j <= q_offset + i (causal) and
 * j >= q_offset + i - window (window >= 0, causal only); P and D are those of this full softmax.  A
 * key chunk [kv_start, kv_start + kv_len) restricts what is returned: dQ_i sums dS_ij k_j over the
 * chunk's keys only, and dK, dV are accumulated for the chunk's rows only (other rows are 0).  Summed
 * over disjoint chunks covering [0, Nk), the partial dQ give the full dQ: the backward of attention
 * computed in key chunks whose partial results were merged through their lse (page ai6s.net/
 * 6a0d3bfb..., section "ops-transformer仓库里还有什么？", ring / block-wise attention).
 *
 * Term magnitudes (fa_oracle_bwd_head_mag_ex; test infrastructure for per-element error bounds, not part
 * of the gradient): next to each gradient element, the sum of the absolute values of the terms of its
 * defining sum above, where every dS_ij is counted with the size of what D_i is made of --
 * D_i = sum_d dO_id O_id = sum_d sum_j dO_id P_ij v_jd has the magnitude A_i = sum_d |dO_id| sum_j P_ij |v_jd|,
 * so a relative perturbation of the stored O moves dS_ij by at most P_ij A_i times that size:
 *
 *   MdQ_id = |scale| sum_j |k_jd| (|dS_ij| + P_ij A_i)
 *   MdK_jd = |scale| sum_i |q_id| (|dS_ij| + P_ij A_i)
 *   MdV_jd = sum_i P_ij |dO_id|
 *
 * over the same (i, j) pairs as the gradients.  Each is at least the absolute value of its gradient.
 * ---------------------------------------------------------------------------------------------
 */
typedef struct {
    const void *q, *k, *v, *dout;
    int dtype, layout, causal;
    int64_t B, H, Nq, Nk, D, b, h;
    int64_t window, q_offset, kv_start, kv_len;
    double scale;
    double *dq, *dk, *dv; /* dq: Nq x D shared (rows are disjoint); dk, dv: this worker's Nk x D */
    double *mq, *mk, *mv; /* the term magnitudes, laid out as dq, dk, dv; all NULL when not asked for */
    int64_t first, last;
    int status;
} orc_bwd_job;

/* element index of row i of a tensor with N rows per (b, h) */
static int64_t orc_bwd_index(const orc_bwd_job* J, int64_t N, int64_t i, int64_t d) {
    if (J->layout == 0) return ((J->b * J->H + J->h) * N + i) * J->D + d;
    return ((J->b * N + i) * J->H + J->h) * J->D + d;
}

static void* orc_bwd_worker(void* arg) {
    orc_bwd_job* J = (orc_bwd_job*)arg;
    const int64_t Nq = J->Nq, Nk = J->Nk, D = J->D;
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    double* dorow = (double*)malloc(sizeof(double) * (size_t)D);
    double* p = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* pv = (double*)malloc(sizeof(double) * (size_t)D); /* sum_j P_ij |v_jd| (magnitudes only) */
    if (!qrow || !dorow || !p || !dp || !pv) {
        free(qrow); free(dorow); free(p); free(dp); free(pv);
        J->status = -1;
        return NULL;
    }
    const int mags = J->mq != NULL;
    const int64_t c0 = J->kv_start, c1 = J->kv_start + J->kv_len; /* the chunk */
    for (int64_t i = J->first; i < J->last; ++i) {
        double* dqi = J->dq + i * D;
        for (int64_t d = 0; d < D; ++d) dqi[d] = 0.0;
        if (mags)
            for (int64_t d = 0; d < D; ++d) J->mq[i * D + d] = 0.0;
        /* visible keys jbeg .. jend-1 of the full softmax */
        const int64_t qpos = i + J->q_offset;
        int64_t jbeg = 0, jend = Nk;
        if (J->causal && jend > qpos + 1) jend = qpos + 1;
        if (J->window >= 0 && jbeg < qpos - J->window) jbeg = qpos - J->window;
        if (jend <= jbeg) continue; /* no visible key: O is constant 0, every gradient from this row is 0 */
        for (int64_t d = 0; d < D; ++d) {
            qrow[d] = orc_load(J->q, J->dtype, orc_bwd_index(J, Nq, i, d));
            dorow[d] = orc_load(J->dout, J->dtype, orc_bwd_index(J, Nq, i, d));
        }
        /* softmax row, two passes */
        double m = -INFINITY;
        for (int64_t j = jbeg; j < jend; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qrow[d] * orc_load(J->k, J->dtype, orc_bwd_index(J, Nk, j, d));
            p[j] = J->scale * dot;
            if (p[j] > m) m = p[j];
        }
        double l = 0.0;
        for (int64_t j = jbeg; j < jend; ++j) {
            p[j] = exp(p[j] - m);
            l += p[j];
        }
        for (int64_t j = jbeg; j < jend; ++j) p[j] /= l;
        /* dP and D */
        double Di = 0.0;
        for (int64_t j = jbeg; j < jend; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += dorow[d] * orc_load(J->v, J->dtype, orc_bwd_index(J, Nk, j, d));
            dp[j] = dot;
            Di += p[j] * dp[j];
        }
        /* magnitude of D_i's expansion: A_i = sum_d |dO_id| sum_j P_ij |v_jd| */
        double Ai = 0.0;
        if (mags) {
            for (int64_t d = 0; d < D; ++d) pv[d] = 0.0;
            for (int64_t j = jbeg; j < jend; ++j)
                for (int64_t d = 0; d < D; ++d) pv[d] += p[j] * fabs(orc_load(J->v, J->dtype, orc_bwd_index(J, Nk, j, d)));
            for (int64_t d = 0; d < D; ++d) Ai += fabs(dorow[d]) * pv[d];
        }
        /* dS and the three gradients, over the visible keys of the chunk */
        const int64_t kb = jbeg > c0 ? jbeg : c0, ke = jend < c1 ? jend : c1;
        for (int64_t j = kb; j < ke; ++j) {
            const double ds = p[j] * (dp[j] - Di);
            double* dkj = J->dk + j * D;
            double* dvj = J->dv + j * D;
            for (int64_t d = 0; d < D; ++d) {
                dqi[d] += J->scale * ds * orc_load(J->k, J->dtype, orc_bwd_index(J, Nk, j, d));
                dkj[d] += J->scale * ds * qrow[d];
                dvj[d] += p[j] * dorow[d];
            }
            if (mags) {
                const double w = fabs(J->scale) * (fabs(ds) + p[j] * Ai);
                double* mqi = J->mq + i * D;
                double* mkj = J->mk + j * D;
                double* mvj = J->mv + j * D;
                for (int64_t d = 0; d < D; ++d) {
                    mqi[d] += w * fabs(orc_load(J->k, J->dtype, orc_bwd_index(J, Nk, j, d)));
                    mkj[d] += w * fabs(qrow[d]);
                    mvj[d] += p[j] * fabs(dorow[d]);
                }
            }
        }
    }
    free(qrow); free(dorow); free(p); free(dp); free(pv);
    return NULL;
}

/*
 * Generalised gradients of head (b, h): dq (Nq x D), dk and dv (Nk x D; rows outside the chunk 0),
 * row-major fp64, under the rule described above, and, when mq, mk, mv are all given, the term
 * magnitudes laid out the same way (all three NULL: not computed).  q, dout: [B][H][Nq][D] or
 * [B][Nq][H][D]; k, v: [B][H][Nk][D] or [B][Nk][H][D].  Returns 0 on success, -2 on a bad argument, -1
 * if memory ran out.
 */
int fa_oracle_bwd_head_mag_ex(const void* q, const void* k, const void* v, const void* dout, int dtype, int layout,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, int64_t window,
                              int64_t q_offset, int64_t kv_start, int64_t kv_len, double scale, int64_t b, int64_t h,
                              double* dq, double* dk, double* dv, double* mq, double* mk, double* mv, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -2;
    const int mags = mq != NULL;
    if ((mk != NULL) != mags || (mv != NULL) != mags) return -2;
    if (dtype < 0 || dtype > 3 || layout < 0 || layout > 1) return -2;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1 || b < 0 || b >= B || h < 0 || h >= H) return -2;
    if (kv_start < 0 || kv_len < 0 || kv_start + kv_len > Nk) return -2;
    if (window >= 0 && !causal) return -2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    if (Nq < nthreads) nthreads = (int)Nq;
    orc_bwd_job* jobs = (orc_bwd_job*)calloc((size_t)nthreads, sizeof(orc_bwd_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    char* running = (char*)calloc((size_t)nthreads, 1);
    const int nparts = mags ? 4 : 2; /* per worker: dk, dv (and mk, mv) */
    double* part = (double*)calloc((size_t)nthreads * nparts * (size_t)(Nk * D), sizeof(double));
    if (!jobs || !tids || !running || !part) {
        free(jobs); free(tids); free(running); free(part);
        return -1;
    }
    for (int t = 0; t < nthreads; ++t) {
        orc_bwd_job* J = &jobs[t];
        J->q = q; J->k = k; J->v = v; J->dout = dout;
        J->dtype = dtype; J->layout = layout; J->causal = causal ? 1 : 0;
        J->B = B; J->H = H; J->Nq = Nq; J->Nk = Nk; J->D = D; J->b = b; J->h = h;
        J->window = window < 0 ? -1 : window;
        J->q_offset = q_offset; J->kv_start = kv_start; J->kv_len = kv_len;
        J->scale = scale;
        J->dq = dq;
        J->dk = part + (size_t)(nparts * t) * (size_t)(Nk * D);
        J->dv = part + (size_t)(nparts * t + 1) * (size_t)(Nk * D);
        if (mags) {
            J->mq = mq;
            J->mk = part + (size_t)(nparts * t + 2) * (size_t)(Nk * D);
            J->mv = part + (size_t)(nparts * t + 3) * (size_t)(Nk * D);
        }
        J->first = Nq * t / nthreads;
        J->last = Nq * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, orc_bwd_worker, &jobs[t]) == 0)
            running[t] = 1;
        else
            orc_bwd_worker(&jobs[t]);
    }
    orc_bwd_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (running[t]) pthread_join(tids[t], NULL);
    int status = 0;
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status) status = jobs[t].status;
    for (int64_t e = 0; e < Nk * D; ++e) {
        double sk = 0.0, sv = 0.0;
        for (int t = 0; t < nthreads; ++t) {
            sk += jobs[t].dk[e];
            sv += jobs[t].dv[e];
        }
        dk[e] = sk;
        dv[e] = sv;
        if (mags) {
            double mks = 0.0, mvs = 0.0;
            for (int t = 0; t < nthreads; ++t) {
                mks += jobs[t].mk[e];
                mvs += jobs[t].mv[e];
            }
            mk[e] = mks;
            mv[e] = mvs;
        }
    }
    free(jobs); free(tids); free(running); free(part);
    return status;
}

int fa_oracle_bwd_head_ex(const void* q, const void* k, const void* v, const void* dout, int dtype, int layout,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, int64_t window,
                          int64_t q_offset, int64_t kv_start, int64_t kv_len, double scale, int64_t b, int64_t h,
                          double* dq, double* dk, double* dv, int nthreads) {
    return fa_oracle_bwd_head_mag_ex(q, k, v, dout, dtype, layout, B, H, Nq, Nk, D, causal, window, q_offset, kv_start,
                                     kv_len, scale, b, h, dq, dk, dv, NULL, NULL, NULL, nthreads);
}

/*
 * Gradients dQ, dK, dV (each N x D, row-major, fp64) of head (b, h) for upstream gradient `dout`
 * (same dtype and layout as q): the plain case Nq = Nk = N, every key.  Returns 0 on success, -2 on a
 * bad argument, -1 if memory ran out.
 */
int fa_oracle_bwd_head(const void* q, const void* k, const void* v, const void* dout, int dtype, int layout,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal, double scale, int64_t b,
                       int64_t h, double* dq, double* dk, double* dv, int nthreads) {
    return fa_oracle_bwd_head_ex(q, k, v, dout, dtype, layout, B, H, N, N, D, causal, -1, 0, 0, N, scale, b, h,
                                 dq, dk, dv, nthreads);
}
