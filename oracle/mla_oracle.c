/*
 * CPU oracle for the absorbed MLA decode path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package's smoke check and the benchmark's CPU
 * baseline leg may load this library.  It shares no code, header or table
 * with the HIP library: every index rule and every formula below is written
 * out again from the pages.
 *
 * Everything is computed in IEEE double from the exact values of the bf16
 * inputs (a bf16 bit pattern widened by a 16-bit shift is exact in double).
 * No GPU rounding (bf16 q_lat, bf16 probabilities) is emulated.
 *
 * Sources (page title, section):
 *  - "MLA in full detail" (mlinterviewnotes), "Step 1 - what the naive path
 *    does": read the latents, up-project keys and values per head through
 *    W_UK / W_UV, append the shared rope key, run ordinary attention with
 *    192-wide keys and 128-wide values.
 *  - Same page, "Step 2 - fold W_UK into the query" and "Step 4 - fold W_UV
 *    into the output": the absorbed form, q~ = W_UK^T q_nope, out = W_UV * latent.
 *  - "M5.8 - Multi-Head Latent Attention", 0x04 "Batched absorption trace":
 *    W_UK [H, d_N, d_c], W_UV [H, d_V, d_c]; softmax over the key axis only;
 *    latent output kept per head.
 *  - M5.8, 0x05 "Paged and ragged address translation": physical row of
 *    logical token j is block_table[b, j / P] * P + j % P; a negative page
 *    entry is an error; one visible length per request.
 *  - M5.8, 0x05 "Exact phase algorithms and commit state": a query at
 *    position p sees visible_length = p + 1 rows (causal rule for T > 1).
 *  - M5.8, 0x0C (sequence-split attention): the exact merge of partial
 *    (max, denominator, numerator) states; averaging is wrong.
 *  - mlxcel "MLA absorbed decode", Stage 2: partials are normalised by their
 *    own denominator and carry an LSE; this oracle keeps natural-log units.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - softmax scale 1/sqrt(d_nope + d_rope) = 1/sqrt(192) for the absorbed
 *    and the normal form alike (both "MLA in full detail" and zdszero state
 *    the scale stays that of the original 192-wide key);
 *  - seqlens count the T current rows, which are already in the cache; query
 *    t of a sequence of length L sees keys j <= L - T + t;
 *  - a split of a sequence of length L into S chunks cuts contiguous chunks of
 *    ceil(ceil(L / S) / P) * P tokens; trailing chunks may be empty and then
 *    carry lse = -inf and a zero numerator.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MLAO_OK 0
#define MLAO_ERR_ARG (-1)
#define MLAO_ERR_INDEX (-2)
#define MLAO_ERR_MEM (-3)

static double bf16_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Physical row of logical token j of sequence b; -1 when the page entry is
 * negative or past num_blocks (M5.8 0x05 asserts physical_page >= 0). */
static long long phys_row(const int32_t *block_table, int max_blocks, int b,
                          int j, int page_size, int num_blocks) {
  int page = j / page_size;
  int off = j % page_size;
  if (page >= max_blocks) return -1;
  int32_t physical_page = block_table[(size_t)b * max_blocks + page];
  if (physical_page < 0 || physical_page >= num_blocks) return -1;
  return (long long)physical_page * page_size + off;
}

/* ------------------------------------------------------------------ */
/* a tiny thread pool: items 0..n-1 are handed out one at a time        */

typedef void (*item_fn)(void *ctx, int item, double *scratch);

typedef struct {
  item_fn fn;
  void *ctx;
  int n;
  int next;
  pthread_mutex_t lock;
  size_t scratch_doubles;
  int failed;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  double *scratch = NULL;
  if (p->scratch_doubles) {
    scratch = (double *)malloc(p->scratch_doubles * sizeof(double));
    if (!scratch) {
      pthread_mutex_lock(&p->lock);
      p->failed = 1;
      pthread_mutex_unlock(&p->lock);
      return NULL;
    }
  }
  for (;;) {
    pthread_mutex_lock(&p->lock);
    int i = p->next++;
    pthread_mutex_unlock(&p->lock);
    if (i >= p->n) break;
    p->fn(p->ctx, i, scratch);
  }
  free(scratch);
  return NULL;
}

static int run_pool(item_fn fn, void *ctx, int n, int nthreads,
                    size_t scratch_doubles) {
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n = n;
  p.next = 0;
  p.scratch_doubles = scratch_doubles;
  p.failed = 0;
  pthread_mutex_init(&p.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = n > 0 ? n : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return MLAO_ERR_MEM;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, pool_worker, &p) != 0) break;
    started++;
  }
  if (started == 0) pool_worker(&p);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&p.lock);
  return p.failed ? MLAO_ERR_MEM : MLAO_OK;
}

static double *widen(const uint16_t *src, size_t n) {
  double *d = (double *)malloc(n * sizeof(double));
  if (!d) return NULL;
  for (size_t i = 0; i < n; ++i) d[i] = bf16_to_double(src[i]);
  return d;
}

/* ------------------------------------------------------------------ */
/* Normal ("naive", decompressed) path: MHA over up-projected K and V.  */

typedef struct {
  const uint16_t *q_nope, *q_pe, *kv_cache;
  const double *w_uk, *w_uv; /* widened [H,dn,r], [H,dv,r] */
  const int32_t *block_table, *seqlens, *pairs;
  int num_blocks, page_size, max_blocks;
  int B, T, H, dn, dr, dv, r, max_len;
  double scale;
  double *out, *lse;
  int bad_index;
} normal_ctx;

static void normal_item(void *vctx, int item, double *scratch) {
  normal_ctx *c = (normal_ctx *)vctx;
  int b = c->pairs[2 * item], h = c->pairs[2 * item + 1];
  int T = c->T, H = c->H, dn = c->dn, dr = c->dr, dv = c->dv, r = c->r;
  int L = c->seqlens[b];
  int row_w = r + dr;
  double *s = scratch;                       /* [T][max_len] scores */
  double *lat = s + (size_t)T * c->max_len;  /* [r] latent c_j */
  double *k_nope = lat + r;                  /* [dn] */
  double *v = k_nope + dn;                   /* [dv] */
  double *acc = v + dv;                      /* [T][dv] */
  double *m = acc + (size_t)T * dv;          /* [T] */
  double *l = m + T;                         /* [T] */
  const double *Wk = c->w_uk + (size_t)h * dn * r;
  const double *Wv = c->w_uv + (size_t)h * dv * r;

  /* Pass 1: keys.  K_j = [W_UK[h] c_j || k_pe_j] (192 wide). */
  for (int j = 0; j < L; ++j) {
    long long pr = phys_row(c->block_table, c->max_blocks, b, j, c->page_size,
                            c->num_blocks);
    if (pr < 0) { c->bad_index = 1; return; }
    const uint16_t *row = c->kv_cache + (size_t)pr * row_w;
    for (int i = 0; i < r; ++i) lat[i] = bf16_to_double(row[i]);
    for (int n = 0; n < dn; ++n) {
      double a = 0.0;
      for (int i = 0; i < r; ++i) a += Wk[(size_t)n * r + i] * lat[i];
      k_nope[n] = a;
    }
    for (int t = 0; t < T; ++t) {
      int vis = L - T + t + 1;
      if (j >= vis) continue;
      const uint16_t *qn = c->q_nope + (((size_t)b * T + t) * H + h) * dn;
      const uint16_t *qp = c->q_pe + (((size_t)b * T + t) * H + h) * dr;
      double dot = 0.0;
      for (int n = 0; n < dn; ++n) dot += bf16_to_double(qn[n]) * k_nope[n];
      for (int i = 0; i < dr; ++i) dot += bf16_to_double(qp[i]) * bf16_to_double(row[r + i]);
      s[(size_t)t * c->max_len + j] = dot * c->scale;
    }
  }
  /* Softmax over the visible keys of each query row. */
  for (int t = 0; t < T; ++t) {
    int vis = L - T + t + 1;
    double mx = -INFINITY;
    for (int j = 0; j < vis; ++j) {
      double x = s[(size_t)t * c->max_len + j];
      if (x > mx) mx = x;
    }
    double sum = 0.0;
    for (int j = 0; j < vis; ++j) sum += exp(s[(size_t)t * c->max_len + j] - mx);
    m[t] = mx;
    l[t] = sum;
    for (int k = 0; k < dv; ++k) acc[(size_t)t * dv + k] = 0.0;
  }
  /* Pass 2: values.  V_j = W_UV[h] c_j (128 wide); out = sum_j p_j V_j. */
  for (int j = 0; j < L; ++j) {
    long long pr = phys_row(c->block_table, c->max_blocks, b, j, c->page_size,
                            c->num_blocks);
    const uint16_t *row = c->kv_cache + (size_t)pr * row_w;
    for (int i = 0; i < r; ++i) lat[i] = bf16_to_double(row[i]);
    for (int k = 0; k < dv; ++k) {
      double a = 0.0;
      for (int i = 0; i < r; ++i) a += Wv[(size_t)k * r + i] * lat[i];
      v[k] = a;
    }
    for (int t = 0; t < T; ++t) {
      int vis = L - T + t + 1;
      if (j >= vis) continue;
      double p = exp(s[(size_t)t * c->max_len + j] - m[t]) / l[t];
      for (int k = 0; k < dv; ++k) acc[(size_t)t * dv + k] += p * v[k];
    }
  }
  for (int t = 0; t < T; ++t) {
    size_t o = ((size_t)b * T + t) * H + h;
    for (int k = 0; k < dv; ++k) c->out[o * dv + k] = acc[(size_t)t * dv + k];
    if (c->lse) c->lse[o] = m[t] + log(l[t]);
  }
}

static int check_common(int B, int T, int H, int r, int dr, int page_size,
                        int max_blocks, int num_blocks, const int32_t *seqlens) {
  if (B < 1 || T < 1 || H < 1 || r < 1 || dr < 0 || page_size < 1 ||
      max_blocks < 1 || num_blocks < 1)
    return MLAO_ERR_ARG;
  for (int b = 0; b < B; ++b) {
    if (seqlens[b] < T) return MLAO_ERR_ARG;
    if ((long long)seqlens[b] > (long long)max_blocks * page_size) return MLAO_ERR_INDEX;
  }
  return MLAO_OK;
}

static int32_t *all_pairs(int B, int H) {
  int32_t *p = (int32_t *)malloc(sizeof(int32_t) * 2 * (size_t)B * H);
  if (!p) return NULL;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      p[2 * ((size_t)b * H + h)] = b;
      p[2 * ((size_t)b * H + h) + 1] = h;
    }
  return p;
}

/* Normal-path decode for the (b, h) pairs listed in `pairs` (n_pairs of them;
 * NULL = every pair).  Writes out[b,t,h,:dv] and lse[b,t,h] (natural log) for
 * the listed pairs only.  scale <= 0 selects 1/sqrt(dn + dr). */
int mlao_normal_decode(const uint16_t *q_nope, const uint16_t *q_pe,
                       const uint16_t *w_uk, const uint16_t *w_uv,
                       const uint16_t *kv_cache, int num_blocks, int page_size,
                       const int32_t *block_table, int max_blocks,
                       const int32_t *seqlens, int B, int T, int H, int dn,
                       int dr, int dv, int r, double scale,
                       const int32_t *pairs, int n_pairs, double *out,
                       double *lse, int nthreads) {
  int st = check_common(B, T, H, r, dr, page_size, max_blocks, num_blocks, seqlens);
  if (st) return st;
  if (dn < 1 || dv < 1) return MLAO_ERR_ARG;
  normal_ctx c;
  memset(&c, 0, sizeof c);
  c.q_nope = q_nope; c.q_pe = q_pe; c.kv_cache = kv_cache;
  c.block_table = block_table; c.seqlens = seqlens;
  c.num_blocks = num_blocks; c.page_size = page_size; c.max_blocks = max_blocks;
  c.B = B; c.T = T; c.H = H; c.dn = dn; c.dr = dr; c.dv = dv; c.r = r;
  c.scale = scale > 0 ? scale : 1.0 / sqrt((double)(dn + dr));
  c.out = out; c.lse = lse;
  int max_len = 0;
  for (int b = 0; b < B; ++b) if (seqlens[b] > max_len) max_len = seqlens[b];
  c.max_len = max_len;
  double *wk = widen(w_uk, (size_t)H * dn * r);
  double *wv = widen(w_uv, (size_t)H * dv * r);
  int32_t *own = NULL;
  if (!pairs) {
    own = all_pairs(B, H);
    pairs = own;
    n_pairs = B * H;
  }
  if (!wk || !wv || !pairs) { free(wk); free(wv); free(own); return MLAO_ERR_MEM; }
  for (int i = 0; i < n_pairs; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= B || pairs[2 * i + 1] < 0 || pairs[2 * i + 1] >= H) {
      free(wk); free(wv); free(own); return MLAO_ERR_ARG;
    }
  c.w_uk = wk; c.w_uv = wv; c.pairs = pairs;
  size_t scratch = (size_t)T * max_len + r + dn + dv + (size_t)T * dv + 2 * (size_t)T;
  st = run_pool(normal_item, &c, n_pairs, nthreads, scratch);
  free(wk); free(wv); free(own);
  if (st) return st;
  return c.bad_index ? MLAO_ERR_INDEX : MLAO_OK;
}

/* ------------------------------------------------------------------ */
/* Absorbed mirror, stage by stage.                                     */

/* q_lat[b,t,h,c] = sum_n q_nope[b,t,h,n] * W_UK[h,n,c]  ("fold W_UK into the
 * query"; M5.8 0x04 einsum bhqn,hnc->bhqc). */
int mlao_absorb(const uint16_t *q_nope, const uint16_t *w_uk, int B, int T,
                int H, int dn, int r, double *q_lat) {
  if (B < 1 || T < 1 || H < 1 || dn < 1 || r < 1) return MLAO_ERR_ARG;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) {
        const uint16_t *q = q_nope + (((size_t)b * T + t) * H + h) * dn;
        double *o = q_lat + (((size_t)b * T + t) * H + h) * r;
        for (int c = 0; c < r; ++c) o[c] = 0.0;
        for (int n = 0; n < dn; ++n) {
          double qn = bf16_to_double(q[n]);
          const uint16_t *w = w_uk + ((size_t)h * dn + n) * r;
          for (int c = 0; c < r; ++c) o[c] += qn * bf16_to_double(w[c]);
        }
      }
  return MLAO_OK;
}

/* out[b,t,h,v] = sum_c latent[b,t,h,c] * W_UV[h,v,c]  ("fold W_UV into the
 * output"; M5.8 0x04 einsum bhqc,hvc->bhqv). */
int mlao_unabsorb(const double *latent, const uint16_t *w_uv, int B, int T,
                  int H, int r, int dv, double *out) {
  if (B < 1 || T < 1 || H < 1 || dv < 1 || r < 1) return MLAO_ERR_ARG;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) {
        const double *x = latent + (((size_t)b * T + t) * H + h) * r;
        double *o = out + (((size_t)b * T + t) * H + h) * dv;
        for (int v = 0; v < dv; ++v) {
          const uint16_t *w = w_uv + ((size_t)h * dv + v) * r;
          double a = 0.0;
          for (int c = 0; c < r; ++c) a += x[c] * bf16_to_double(w[c]);
          o[v] = a;
        }
      }
  return MLAO_OK;
}

/* Split plan for a uniform split count S >= 1: sequence b is cut into S
 * contiguous chunks of ceil(ceil(L_b / S) / P) * P tokens.  Writes
 * split_indptr[B+1] (= b * S) and, for every split k, its token range
 * [begin[k], end[k]) (begin == end for an empty trailing chunk). */
int mlao_split_plan(const int32_t *seqlens, int B, int S, int page_size,
                    int32_t *split_indptr, int32_t *begin, int32_t *end) {
  if (B < 1 || S < 1 || page_size < 1) return MLAO_ERR_ARG;
  split_indptr[0] = 0;
  for (int b = 0; b < B; ++b) {
    int L = seqlens[b];
    int per = (L + S - 1) / S;
    int chunk = ((per + page_size - 1) / page_size) * page_size;
    for (int s = 0; s < S; ++s) {
      long long j0 = (long long)s * chunk, j1 = j0 + chunk;
      if (j0 > L) j0 = L;
      if (j1 > L) j1 = L;
      begin[(size_t)b * S + s] = (int32_t)j0;
      end[(size_t)b * S + s] = (int32_t)j1;
    }
    split_indptr[b + 1] = (b + 1) * S;
  }
  return MLAO_OK;
}

typedef struct {
  const double *q_lat;
  const uint16_t *q_pe, *kv_cache;
  const int32_t *block_table, *seqlens, *pairs;
  const int32_t *split_indptr, *begin, *end; /* NULL: one split = whole sequence */
  int num_blocks, page_size, max_blocks;
  int B, T, H, dr, r;
  double scale;
  double *lat_out, *lse_out; /* [n_rows_out, T, H, r], [n_rows_out, T, H] */
  int bad_index;
} latent_ctx;

/* Attention of one (b, h) pair over the latent rows in [j0, j1), for every
 * query row t (keys j < L - T + t + 1 only).  Scores are
 * (q~ . c_j + q_pe . k_pe_j) * scale; the output is the softmax-weighted sum
 * of the 512-wide latents c_j; lse in natural log.  An empty range gives
 * lse = -inf and a zero output. */
static void latent_range(latent_ctx *c, int b, int h, int j0, int j1,
                         size_t out_row, double *scratch) {
  int T = c->T, H = c->H, r = c->r, dr = c->dr, L = c->seqlens[b];
  int row_w = r + dr;
  int n = j1 - j0;
  double *s = scratch; /* [T][n] */
  for (int t = 0; t < T; ++t) {
    int vis = L - T + t + 1;
    const double *ql = c->q_lat + (((size_t)b * T + t) * H + h) * r;
    const uint16_t *qp = c->q_pe + (((size_t)b * T + t) * H + h) * dr;
    double *o = c->lat_out + ((out_row * T + t) * H + h) * (size_t)r;
    for (int i = 0; i < r; ++i) o[i] = 0.0;
    int hi = j1 < vis ? j1 : vis;
    double mx = -INFINITY;
    for (int j = j0; j < hi; ++j) {
      long long pr = phys_row(c->block_table, c->max_blocks, b, j, c->page_size,
                              c->num_blocks);
      if (pr < 0) { c->bad_index = 1; return; }
      const uint16_t *row = c->kv_cache + (size_t)pr * row_w;
      double dot = 0.0;
      for (int i = 0; i < r; ++i) dot += ql[i] * bf16_to_double(row[i]);
      for (int i = 0; i < dr; ++i) dot += bf16_to_double(qp[i]) * bf16_to_double(row[r + i]);
      s[(size_t)t * n + (j - j0)] = dot * c->scale;
      if (s[(size_t)t * n + (j - j0)] > mx) mx = s[(size_t)t * n + (j - j0)];
    }
    double *lse = c->lse_out + (out_row * T + t) * H + h;
    if (hi <= j0) { *lse = -INFINITY; continue; }
    double sum = 0.0;
    for (int j = j0; j < hi; ++j) sum += exp(s[(size_t)t * n + (j - j0)] - mx);
    for (int j = j0; j < hi; ++j) {
      long long pr = phys_row(c->block_table, c->max_blocks, b, j, c->page_size,
                              c->num_blocks);
      const uint16_t *row = c->kv_cache + (size_t)pr * row_w;
      double p = exp(s[(size_t)t * n + (j - j0)] - mx) / sum;
      for (int i = 0; i < r; ++i) o[i] += p * bf16_to_double(row[i]);
    }
    *lse = mx + log(sum);
  }
}

static void latent_item(void *vctx, int item, double *scratch) {
  latent_ctx *c = (latent_ctx *)vctx;
  int b = c->pairs[2 * item], h = c->pairs[2 * item + 1];
  if (!c->split_indptr) {
    latent_range(c, b, h, 0, c->seqlens[b], (size_t)b, scratch);
    return;
  }
  for (int k = c->split_indptr[b]; k < c->split_indptr[b + 1]; ++k)
    latent_range(c, b, h, c->begin[k], c->end[k], (size_t)k, scratch);
}

/* Absorbed latent attention ("attend against the latent directly"; M5.8 0x04
 * einsums bhqc,bkc->bhqk and bhqk,bkc->bhqc).  q_lat is [B,T,H,r] double;
 * scale must be given (the absorbed form keeps the 192-wide key's scale).
 * With split_indptr == NULL: latent_out [B,T,H,r], lse [B,T,H] over each
 * whole sequence.  Otherwise partial states per split k (ranges from
 * mlao_split_plan): latent_out [n_splits,T,H,r] normalised by the split's own
 * denominator, lse [n_splits,T,H]. */
int mlao_latent_attention(const double *q_lat, const uint16_t *q_pe,
                          const uint16_t *kv_cache, int num_blocks,
                          int page_size, const int32_t *block_table,
                          int max_blocks, const int32_t *seqlens, int B, int T,
                          int H, int dr, int r, double scale,
                          const int32_t *split_indptr, const int32_t *begin,
                          const int32_t *end, const int32_t *pairs,
                          int n_pairs, double *latent_out, double *lse,
                          int nthreads) {
  int st = check_common(B, T, H, r, dr, page_size, max_blocks, num_blocks, seqlens);
  if (st) return st;
  latent_ctx c;
  memset(&c, 0, sizeof c);
  c.q_lat = q_lat; c.q_pe = q_pe; c.kv_cache = kv_cache;
  c.block_table = block_table; c.seqlens = seqlens;
  c.split_indptr = split_indptr; c.begin = begin; c.end = end;
  c.num_blocks = num_blocks; c.page_size = page_size; c.max_blocks = max_blocks;
  c.B = B; c.T = T; c.H = H; c.dr = dr; c.r = r;
  if (!(scale > 0)) return MLAO_ERR_ARG;
  c.scale = scale;
  c.lat_out = latent_out; c.lse_out = lse;
  int max_len = 0;
  for (int b = 0; b < B; ++b) if (seqlens[b] > max_len) max_len = seqlens[b];
  int32_t *own = NULL;
  if (!pairs) {
    own = all_pairs(B, H);
    if (!own) return MLAO_ERR_MEM;
    pairs = own;
    n_pairs = B * H;
  }
  c.pairs = pairs;
  st = run_pool(latent_item, &c, n_pairs, nthreads, (size_t)T * (max_len + 1));
  free(own);
  if (st) return st;
  return c.bad_index ? MLAO_ERR_INDEX : MLAO_OK;
}

/* Exact merge of split partial states (M5.8 0x0C): for each (b,t,h) over the
 * splits k of sequence b, M = max_k lse_k, w_k = exp(lse_k - M),
 * lse = M + log(sum w_k), out = sum w_k o_k / sum w_k.  Splits with
 * lse = -inf carry no weight.  part_out [n_splits,T,H,r] holds numerators
 * already divided by their own denominators (mlxcel Stage 2 contract). */
int mlao_merge(const double *part_out, const double *part_lse,
               const int32_t *split_indptr, int B, int T, int H, int r,
               double *out, double *lse) {
  if (B < 1 || T < 1 || H < 1 || r < 1) return MLAO_ERR_ARG;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h) {
        double M = -INFINITY;
        for (int k = split_indptr[b]; k < split_indptr[b + 1]; ++k) {
          double x = part_lse[((size_t)k * T + t) * H + h];
          if (x > M) M = x;
        }
        double *o = out + (((size_t)b * T + t) * H + h) * r;
        for (int i = 0; i < r; ++i) o[i] = 0.0;
        size_t lo = ((size_t)b * T + t) * H + h;
        if (M == -INFINITY) {
          if (lse) lse[lo] = -INFINITY;
          continue;
        }
        double wsum = 0.0;
        for (int k = split_indptr[b]; k < split_indptr[b + 1]; ++k) {
          double x = part_lse[((size_t)k * T + t) * H + h];
          if (x == -INFINITY) continue;
          double w = exp(x - M);
          wsum += w;
          const double *po = part_out + (((size_t)k * T + t) * H + h) * r;
          for (int i = 0; i < r; ++i) o[i] += w * po[i];
        }
        for (int i = 0; i < r; ++i) o[i] /= wsum;
        if (lse) lse[lo] = M + log(wsum);
      }
  return MLAO_OK;
}

/* Physical row lookup exposed for the addressing tests. */
long long mlao_phys_row(const int32_t *block_table, int max_blocks, int b,
                        int j, int page_size, int num_blocks) {
  return phys_row(block_table, max_blocks, b, j, page_size, num_blocks);
}
