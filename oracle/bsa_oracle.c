/*
 * Plain CPU oracle for the block-sparse tiled attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library shares no
 * code, header, table or helper with it, and nothing here is ever used as a
 * fallback for the GPU path.
 *
 * What it computes (FastVideo fastvideo-kernel commit list, page 3: the
 * 128-token sm_121a forward commit, which gives the binding
 * block_sparse_sm121_blk128_fwd(q, k, v, q2k_idx, q2k_num, variable_block_sizes)
 * -> {out}, a forward without log-sum-exp; and the hardening commit's kernel bullets
 * on the softmax-sum rule, empty selections and padding keys):
 *
 *   For batch b, head h, query tile i and row r of that tile
 *     - rows at or past the tile's valid length vbs[i] are padding: out = +0;
 *     - the key set is, in list order, every valid row c < vbs[j] of every
 *       listed key tile j = q2k_idx[b,h,i,n], n < q2k_num[b,h,i]; padding
 *       key rows (c >= vbs[j]) are never read;
 *     - an empty key set gives out = +0 (rows without keys stay zero);
 *     - otherwise out = sum_key p_key * v_key / l with s_key = scale * q.k,
 *       m = max s, p_key = exp(s_key - m), l = sum p_key, and the division
 *       happens only when l != 0 (so a NaN softmax sum yields a NaN row).
 *
 * This is the plain definition of softmax attention restricted to a block
 * mask: no tiling, no online rescaling, no reduced precision for P.  The pages'
 * kernel tests compare against binary32 results, so every floating-point step is
 * IEEE binary32 with contraction off, in the order written above (dot
 * products over d ascending, sums over keys in list order).  The softmax
 * scale, which the binding does not take as an argument, is 1/sqrt(D)
 * rounded to binary32.
 *
 * Tensors: q, k, v are bf16 bit patterns, [B, H, NT*T, D] row-major; q2k_idx
 * is int32 [B, H, NT, MS]; q2k_num is int32 [B, H, NT]; vbs is int32 [NT],
 * shared by query and key tiles (self-attention).  Invalid contents (an
 * index outside [0, NT), a count outside [0, MS], a length outside [0, T])
 * are rejected with a negative return code before any output is written.
 *
 * The layout step (the fused token-to-tile scatter) is a pure permutation
 * with zero padding; its oracle is a NumPy gather in oracle/__init__.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1
#define ORACLE_ERR_INDEX -2
#define ORACLE_ERR_COUNT -3
#define ORACLE_ERR_LENGTH -4
#define ORACLE_ERR_NOMEM -5

/* bf16 is the upper half of a binary32; widening is exact. */
static float widen_bf16(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

typedef struct {
  const uint16_t *q, *k, *v;
  const int32_t *q2k_idx, *q2k_num, *vbs;
  int64_t B, H, NT, T, D, MS;
  float scale;
} problem_t;

/* Output row of query `r` in tile `i` of batch-head `bh`, into dst[0..D). */
static void attend_row(const problem_t *p, int64_t bh, int64_t i, int64_t r,
                       float *scores, float *acc, float *dst) {
  const int64_t D = p->D, T = p->T, S = p->NT * p->T;
  int64_t d, n;
  for (d = 0; d < D; ++d) dst[d] = 0.0f;
  if (r >= p->vbs[i]) return; /* padding query row */

  const uint16_t *qrow = p->q + (bh * S + i * T + r) * D;
  const int32_t *list = p->q2k_idx + (bh * p->NT + i) * p->MS;
  const int64_t count = p->q2k_num[bh * p->NT + i];

  /* scores over the key set, in list order */
  int64_t nkeys = 0;
  for (n = 0; n < count; ++n) {
    const int64_t j = list[n];
    const int64_t vk = p->vbs[j];
    int64_t c;
    for (c = 0; c < vk; ++c) {
      const uint16_t *krow = p->k + (bh * S + j * T + c) * D;
      float dot = 0.0f;
      for (d = 0; d < D; ++d) dot = dot + widen_bf16(qrow[d]) * widen_bf16(krow[d]);
      scores[nkeys++] = p->scale * dot;
    }
  }
  if (nkeys == 0) return; /* no selected keys: the row stays zero */

  float m = -INFINITY;
  int64_t key;
  for (key = 0; key < nkeys; ++key)
    if (scores[key] > m) m = scores[key];

  float l = 0.0f;
  for (d = 0; d < D; ++d) acc[d] = 0.0f;
  key = 0;
  for (n = 0; n < count; ++n) {
    const int64_t j = list[n];
    const int64_t vk = p->vbs[j];
    int64_t c;
    for (c = 0; c < vk; ++c, ++key) {
      const float pk = expf(scores[key] - m);
      const uint16_t *vrow = p->v + (bh * S + j * T + c) * D;
      l = l + pk;
      for (d = 0; d < D; ++d) acc[d] = acc[d] + pk * widen_bf16(vrow[d]);
    }
  }
  if (l != 0.0f)
    for (d = 0; d < D; ++d) dst[d] = acc[d] / l;
}

static int check_problem(const problem_t *p) {
  int64_t bh, i, n, j;
  if (p->B < 0 || p->H < 0 || p->NT < 0 || p->T <= 0 || p->D <= 0 || p->MS < 0)
    return ORACLE_ERR_ARG;
  for (i = 0; i < p->NT; ++i)
    if (p->vbs[i] < 0 || p->vbs[i] > p->T) return ORACLE_ERR_LENGTH;
  for (bh = 0; bh < p->B * p->H; ++bh)
    for (i = 0; i < p->NT; ++i) {
      const int64_t count = p->q2k_num[bh * p->NT + i];
      if (count < 0 || count > p->MS) return ORACLE_ERR_COUNT;
      for (n = 0; n < count; ++n) {
        j = p->q2k_idx[(bh * p->NT + i) * p->MS + n];
        if (j < 0 || j >= p->NT) return ORACLE_ERR_INDEX;
      }
    }
  return ORACLE_OK;
}

typedef struct {
  const problem_t *p;
  const int64_t *rows; /* NULL: every row of the problem */
  int64_t nrows;
  float *out;
  int tid, nthreads;
  int failed;
} job_t;

static void *worker(void *arg) {
  job_t *job = (job_t *)arg;
  const problem_t *p = job->p;
  float *scores = (float *)malloc(sizeof(float) * (size_t)(p->MS * p->T + 1));
  float *acc = (float *)malloc(sizeof(float) * (size_t)p->D);
  if (!scores || !acc) {
    job->failed = 1;
    free(scores);
    free(acc);
    return NULL;
  }
  const int64_t S = p->NT * p->T;
  int64_t w;
  for (w = job->tid; w < job->nrows; w += job->nthreads) {
    const int64_t flat = job->rows ? job->rows[w] : w; /* (b*H + h)*S + t */
    const int64_t bh = flat / S, t = flat % S;
    attend_row(p, bh, t / p->T, t % p->T, scores, acc, job->out + w * p->D);
  }
  free(scores);
  free(acc);
  return NULL;
}

static int run(const problem_t *p, const int64_t *rows, int64_t nrows, float *out,
               int nthreads) {
  int rc = check_problem(p);
  if (rc != ORACLE_OK) return rc;
  if (nthreads < 1) nthreads = 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
  if (!th || !jobs) {
    free(th);
    free(jobs);
    return ORACLE_ERR_NOMEM;
  }
  int t, failed = 0;
  for (t = 0; t < nthreads; ++t) {
    jobs[t].p = p;
    jobs[t].rows = rows;
    jobs[t].nrows = nrows;
    jobs[t].out = out;
    jobs[t].tid = t;
    jobs[t].nthreads = nthreads;
    jobs[t].failed = 0;
  }
  int started = 1; /* threads 1..started-1 run concurrently */
  while (started < nthreads &&
         pthread_create(&th[started], NULL, worker, &jobs[started]) == 0)
    ++started;
  /* shares whose thread could not start run here, after share 0 */
  for (t = started; t < nthreads; ++t) worker(&jobs[t]);
  worker(&jobs[0]);
  for (t = 1; t < started; ++t) pthread_join(th[t], NULL);
  for (t = 0; t < nthreads; ++t) failed |= jobs[t].failed;
  free(th);
  free(jobs);
  return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

static void fill_problem(problem_t *p, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const int32_t *q2k_idx,
                         const int32_t *q2k_num, const int32_t *vbs, int64_t B,
                         int64_t H, int64_t NT, int64_t T, int64_t D, int64_t MS) {
  p->q = q;
  p->k = k;
  p->v = v;
  p->q2k_idx = q2k_idx;
  p->q2k_num = q2k_num;
  p->vbs = vbs;
  p->B = B;
  p->H = H;
  p->NT = NT;
  p->T = T;
  p->D = D;
  p->MS = MS;
  p->scale = (float)(1.0 / sqrt((double)D));
}

/* Every output row: out is float32 [B, H, NT*T, D]. */
int oracle_bsa_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const int32_t *q2k_idx, const int32_t *q2k_num, const int32_t *vbs,
                   int64_t B, int64_t H, int64_t NT, int64_t T, int64_t D, int64_t MS,
                   float *out, int nthreads) {
  problem_t p;
  fill_problem(&p, q, k, v, q2k_idx, q2k_num, vbs, B, H, NT, T, D, MS);
  return run(&p, NULL, B * H * NT * T, out, nthreads);
}

/* Selected rows only: rows[n] = (b*H + h)*(NT*T) + t; out is float32 [nrows, D]. */
int oracle_bsa_fwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const int32_t *q2k_idx, const int32_t *q2k_num,
                        const int32_t *vbs, int64_t B, int64_t H, int64_t NT, int64_t T,
                        int64_t D, int64_t MS, const int64_t *rows, int64_t nrows,
                        float *out, int nthreads) {
  problem_t p;
  int64_t n;
  fill_problem(&p, q, k, v, q2k_idx, q2k_num, vbs, B, H, NT, T, D, MS);
  for (n = 0; n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= B * H * NT * T) return ORACLE_ERR_ARG;
  return run(&p, rows, nrows, out, nthreads);
}

/* The binary32 softmax scale the oracle uses for head dimension D. */
float oracle_softmax_scale(int64_t D) { return (float)(1.0 / sqrt((double)D)); }

/*
 * Coarse stage: tile selection (the q2k_idx lists) and the coarse output.
 *
 * The pages call the block-sparse kernel the "fine" attention (hardening
 * commit: the fine-attention override; fused-layout commit: the gate scattered
 * with Q, K and V) but never say how a query tile's key tiles are chosen.  The
 * definition adopted is the coarse stage of Video Sparse Attention (Zhang et
 * al., 2025), written out plainly:
 *
 *   pooling   every tile t with vbs[t] > 0 becomes one token, the mean of its
 *             valid rows: xm[t][d] = (sum over s < vbs[t], ascending, of
 *             x[t*T + s][d]) / vbs[t], binary32 sums and one division;
 *   logits    g[i][j] = sum over d ascending of qm[i][d] * km[j][d], one fused
 *             multiply-add per term (fmaf: the product and the sum rounded once);
 *   selection for a query tile i with vbs[i] > 0, the candidates are the key
 *             tiles j with vbs[j] > 0, ranked by g[i][j] descending (a NaN
 *             logit ranks as -inf, -0 as +0), equal logits by ascending j; the
 *             first k = min(topk, candidates) are kept and listed in
 *             q2k_idx[i][0..k) by ascending j, q2k_num[i] = k; the other
 *             entries are -1.  A query tile with vbs[i] = 0 keeps nothing;
 *   coarse    oc[i] = sum over candidates j (ascending) of p_j * vm[j] / l,
 *   output    p_j = exp(scale*g[i][j] - m), m = the largest scale*g[i][j],
 *             l = sum p_j, divided only when l != 0 (as the fine stage);
 *             0 for a query tile with vbs[i] = 0 or without candidates.
 *
 * Everything is binary32 with contraction off (the one fused step is the
 * explicit fmaf), so the lists are a fixed function of the inputs.
 */

/* xm [B*H, NT, D]: the mean of each tile's valid rows (0 for empty tiles). */
int oracle_coarse_pool(const uint16_t *x, const int32_t *vbs, int64_t BH, int64_t NT,
                       int64_t T, int64_t D, float *xm) {
  int64_t bh, t, s, d;
  if (BH < 0 || NT < 0 || T <= 0 || D <= 0) return ORACLE_ERR_ARG;
  for (t = 0; t < NT; ++t)
    if (vbs[t] < 0 || vbs[t] > T) return ORACLE_ERR_LENGTH;
  for (bh = 0; bh < BH; ++bh)
    for (t = 0; t < NT; ++t)
      for (d = 0; d < D; ++d) {
        float acc = 0.0f;
        const int64_t n = vbs[t];
        for (s = 0; s < n; ++s) acc = acc + widen_bf16(x[((bh * NT + t) * T + s) * D + d]);
        xm[(bh * NT + t) * D + d] = n > 0 ? acc / (float)n : 0.0f;
      }
  return ORACLE_OK;
}

/* Ranking key of a logit: NaN as -inf, -0 as +0. */
static float rank_key(float g) {
  if (g != g) return -INFINITY;
  return g == 0.0f ? 0.0f : g;
}

typedef struct {
  float key;
  int64_t j;
} ranked_t;

/* Ranked order: larger key first, equal keys by ascending tile index (a total
 * order, so any sort gives the same sequence). */
static int rank_cmp(const void *pa, const void *pb) {
  const ranked_t *a = (const ranked_t *)pa, *b = (const ranked_t *)pb;
  if (a->key > b->key) return -1;
  if (a->key < b->key) return 1;
  return a->j < b->j ? -1 : (a->j > b->j ? 1 : 0);
}

/*
 * From the pooled tensors: q2k_idx [B*H, NT, MS], q2k_num [B*H, NT], and the
 * coarse output oc [B*H, NT, D] (float32).  topk >= 0, MS >= topk.
 */
int oracle_coarse_select(const float *qm, const float *km, const float *vm, const int32_t *vbs,
                         int64_t BH, int64_t NT, int64_t D, int64_t topk, int64_t MS,
                         int32_t *q2k_idx, int32_t *q2k_num, float *oc) {
  int64_t bh, i, j, d, n;
  if (BH < 0 || NT < 0 || D <= 0 || topk < 0 || MS < topk) return ORACLE_ERR_ARG;
  for (j = 0; j < NT; ++j)
    if (vbs[j] < 0) return ORACLE_ERR_LENGTH;
  const size_t nt1 = (size_t)(NT > 0 ? NT : 1);
  float *g = (float *)malloc(sizeof(float) * nt1);
  ranked_t *order = (ranked_t *)malloc(sizeof(ranked_t) * nt1);
  char *keep = (char *)malloc(nt1);
  float *acc = (float *)malloc(sizeof(float) * (size_t)D);
  if (!g || !order || !keep || !acc) {
    free(g);
    free(order);
    free(keep);
    free(acc);
    return ORACLE_ERR_NOMEM;
  }
  const float scale = (float)(1.0 / sqrt((double)D));
  for (bh = 0; bh < BH; ++bh)
    for (i = 0; i < NT; ++i) {
      int32_t *list = q2k_idx + (bh * NT + i) * MS;
      float *o = oc + (bh * NT + i) * D;
      for (n = 0; n < MS; ++n) list[n] = -1;
      for (d = 0; d < D; ++d) o[d] = 0.0f;
      q2k_num[bh * NT + i] = 0;
      if (vbs[i] <= 0) continue;
      /* logits of the candidates, ascending j */
      int64_t cand = 0;
      for (j = 0; j < NT; ++j) {
        keep[j] = 0;
        if (vbs[j] <= 0) continue;
        float dot = 0.0f;
        for (d = 0; d < D; ++d) dot = fmaf(qm[(bh * NT + i) * D + d], km[(bh * NT + j) * D + d], dot);
        g[j] = dot;
        order[cand].key = rank_key(dot);
        order[cand].j = j;
        ++cand;
      }
      if (cand == 0) continue;
      qsort(order, (size_t)cand, sizeof(ranked_t), rank_cmp);
      const int64_t k = topk < cand ? topk : cand;
      for (n = 0; n < k; ++n) keep[order[n].j] = 1;
      int64_t w = 0;
      for (j = 0; j < NT; ++j)
        if (vbs[j] > 0 && keep[j]) list[w++] = (int32_t)j;
      q2k_num[bh * NT + i] = (int32_t)k;
      /* coarse output over every candidate, ascending j */
      float mx = -INFINITY;
      for (j = 0; j < NT; ++j)
        if (vbs[j] > 0 && scale * g[j] > mx) mx = scale * g[j];
      float l = 0.0f;
      for (d = 0; d < D; ++d) acc[d] = 0.0f;
      for (j = 0; j < NT; ++j) {
        if (vbs[j] <= 0) continue;
        const float p = expf(scale * g[j] - mx);
        l = l + p;
        for (d = 0; d < D; ++d) acc[d] = acc[d] + p * vm[(bh * NT + j) * D + d];
      }
      if (l != 0.0f)
        for (d = 0; d < D; ++d) o[d] = acc[d] / l;
    }
  free(g);
  free(order);
  free(keep);
  free(acc);
  return ORACLE_OK;
}
