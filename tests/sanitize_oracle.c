/* Drives every entry point of the C oracle on a small ragged, paged, split
 * case, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (test infrastructure: tests/test_sanitize_oracle.py compiles and runs it).
 * Buffers are allocated at their exact sizes, so any access past them is
 * reported.  Also checks two facts the oracle must satisfy: the absorbed
 * mirror equals the Normal path (associativity) and merging the split
 * partials gives the unsplit result. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mlao_normal_decode(const uint16_t *, const uint16_t *, const uint16_t *, const uint16_t *,
                       const uint16_t *, int, int, const int32_t *, int, const int32_t *, int, int, int,
                       int, int, int, int, double, const int32_t *, int, double *, double *, int);
int mlao_absorb(const uint16_t *, const uint16_t *, int, int, int, int, int, double *);
int mlao_unabsorb(const double *, const uint16_t *, int, int, int, int, int, double *);
int mlao_split_plan(const int32_t *, int, int, int, int32_t *, int32_t *, int32_t *);
int mlao_latent_attention(const double *, const uint16_t *, const uint16_t *, int, int, const int32_t *,
                          int, const int32_t *, int, int, int, int, int, double, const int32_t *,
                          const int32_t *, const int32_t *, const int32_t *, int, double *, double *, int);
int mlao_merge(const double *, const double *, const int32_t *, int, int, int, int, double *, double *);
long long mlao_phys_row(const int32_t *, int, int, int, int, int);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 11);
}
/* a bf16 value of magnitude in [2^-4, 2^1), random sign and mantissa */
static uint16_t rand_bf16(void) {
  uint32_t u = next_u32();
  uint16_t exp = (uint16_t)(123 + (u % 5));
  return (uint16_t)(((u >> 8) & 1u) << 15 | exp << 7 | ((u >> 9) & 0x7Fu));
}
static uint16_t *bf16_array(size_t n) {
  uint16_t *p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) p[i] = rand_bf16();
  return p;
}
static int fail(const char *what) {
  printf("FAIL %s\n", what);
  return 1;
}

int main(void) {
  enum { B = 3, T = 2, H = 4, DN = 8, DR = 4, DV = 6, R = 16, P = 8, S = 3 };
  const int32_t seqlens[B] = {37, 2, 20};
  int pages = 0, max_blocks = 0;
  for (int b = 0; b < B; ++b) {
    int n = (seqlens[b] + P - 1) / P;
    pages += n;
    if (n > max_blocks) max_blocks = n;
  }
  const int num_blocks = pages + 2; /* two blocks nobody maps */
  int32_t *bt = malloc(sizeof(int32_t) * B * max_blocks);
  int next = num_blocks - 1; /* pages handed out from the top */
  for (int b = 0; b < B; ++b)
    for (int k = 0; k < max_blocks; ++k) bt[b * max_blocks + k] = k * P < seqlens[b] ? next-- : -1;
  uint16_t *q_nope = bf16_array((size_t)B * T * H * DN), *q_pe = bf16_array((size_t)B * T * H * DR);
  uint16_t *w_uk = bf16_array((size_t)H * DN * R), *w_uv = bf16_array((size_t)H * DV * R);
  uint16_t *kv = bf16_array((size_t)num_blocks * P * (R + DR));
  const double scale = 1.0 / sqrt((double)(DN + DR));

  double *out_n = malloc(sizeof(double) * B * T * H * DV), *lse_n = malloc(sizeof(double) * B * T * H);
  if (mlao_normal_decode(q_nope, q_pe, w_uk, w_uv, kv, num_blocks, P, bt, max_blocks, seqlens, B, T, H, DN,
                         DR, DV, R, 0.0, NULL, 0, out_n, lse_n, 3))
    return fail("normal_decode");

  double *q_lat = malloc(sizeof(double) * B * T * H * R);
  if (mlao_absorb(q_nope, w_uk, B, T, H, DN, R, q_lat)) return fail("absorb");
  double *lat = malloc(sizeof(double) * B * T * H * R), *lse = malloc(sizeof(double) * B * T * H);
  if (mlao_latent_attention(q_lat, q_pe, kv, num_blocks, P, bt, max_blocks, seqlens, B, T, H, DR, R, scale,
                            NULL, NULL, NULL, NULL, 0, lat, lse, 2))
    return fail("latent_attention");
  double *out_a = malloc(sizeof(double) * B * T * H * DV);
  if (mlao_unabsorb(lat, w_uv, B, T, H, R, DV, out_a)) return fail("unabsorb");

  int32_t ind[B + 1], beg[B * S], end[B * S];
  if (mlao_split_plan(seqlens, B, S, P, ind, beg, end)) return fail("split_plan");
  double *po = malloc(sizeof(double) * B * S * T * H * R), *pl = malloc(sizeof(double) * B * S * T * H);
  if (mlao_latent_attention(q_lat, q_pe, kv, num_blocks, P, bt, max_blocks, seqlens, B, T, H, DR, R, scale, ind,
                            beg, end, NULL, 0, po, pl, 4))
    return fail("latent_attention (splits)");
  double *lat_m = malloc(sizeof(double) * B * T * H * R), *lse_m = malloc(sizeof(double) * B * T * H);
  if (mlao_merge(po, pl, ind, B, T, H, R, lat_m, lse_m)) return fail("merge");

  double scale_out = 0, err_assoc = 0, err_merge = 0, scale_lat = 0;
  for (int i = 0; i < B * T * H * DV; ++i) {
    if (!isfinite(out_n[i]) || !isfinite(out_a[i])) return fail("non-finite output");
    scale_out = fmax(scale_out, fabs(out_n[i]));
    err_assoc = fmax(err_assoc, fabs(out_n[i] - out_a[i]));
  }
  for (int i = 0; i < B * T * H * R; ++i) {
    scale_lat = fmax(scale_lat, fabs(lat[i]));
    err_merge = fmax(err_merge, fabs(lat[i] - lat_m[i]));
  }
  for (int i = 0; i < B * T * H; ++i)
    if (fabs(lse[i] - lse_m[i]) > 1e-12 * fmax(1.0, fabs(lse[i])) || fabs(lse[i] - lse_n[i]) > 1e-9)
      return fail("lse");
  if (err_assoc > 1e-9 * scale_out) return fail("absorbed vs normal");
  if (err_merge > 1e-12 * scale_lat) return fail("merge vs unsplit");
  /* the paged address of the last token of sequence 0, and of an unmapped page */
  const int j = seqlens[0] - 1;
  if (mlao_phys_row(bt, max_blocks, 0, j, P, num_blocks) != (long long)bt[j / P] * P + j % P)
    return fail("phys_row");
  free(bt); free(q_nope); free(q_pe); free(w_uk); free(w_uv); free(kv); free(out_n); free(lse_n);
  free(q_lat); free(lat); free(lse); free(out_a); free(po); free(pl); free(lat_m); free(lse_m);
  printf("ok\n");
  return 0;
}
