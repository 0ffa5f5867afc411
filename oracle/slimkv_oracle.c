/*
 * slimkv_oracle.c -- plain fp64 CPU oracle for SlimKV latent decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header or constant with the HIP library it checks.
 *
 * What it computes (page "Can SlimKV compress KV cache jointly across tokens
 * and features", section "Latent-space attention removes the rebuild step";
 * the abstract on page "SlimKV: Joint Token-Feature KV Cache Compression with
 * Reconstruction-Free Beacon Attention"): for one decode query per sequence,
 * attention over a cache made of
 *   - N_b beacon rows held as low-rank latents C_K (rank r_K) and C_V
 *     (rank r_V) whose keys carry no rotary position, and
 *   - W raw-token rows K_raw, V_raw at full head dimension d whose keys are
 *     stored already rotated;
 * the query keeps its rotation.  Beacon scores are taken in latent space as
 * (q' U_K) . C_K[j], beacon values are summed in latent space as sum_j a_j
 * C_V[j] and lifted once by U_V; beacon and raw rows share one softmax.
 *
 * Every step is done in double precision, in the order the section lists
 * it, per query head:
 *   1. q' = RoPE(q, q_pos)           rotate-half pairs (i, i + d/2),
 *                                      angle q_pos * theta^(-2i/d)
 *   2. qh = U_K^T q'                   query in the head's latent key space
 *   3. s_j = scale * qh . C_K[j]       (j < N_b, no rotation on C_K)
 *      s_{N_b+t} = scale * q' . K_raw[t]
 *   4. a = softmax(s) over all N_b + W rows jointly
 *   5. o_lat = sum_j a_j C_V[j],  o_raw = sum_t a_{N_b+t} V_raw[t]
 *   6. out = U_V o_lat + o_raw,     lse = max(s) + log(sum exp(s - max(s)))
 * Query head g reads KV head floor(g / G), G = H_q / H_kv.
 *
 * Inputs are read in their storage format (fp64, fp32, or bf16 as the top
 * 16 bits of an IEEE binary32) and widened exactly to double.
 *
 * slimkv_oracle_decode_ragged adds what a serving decode step needs around
 * that computation: per-sequence numbers of live beacon and raw rows in
 * capacity-sized arrays, and the step's new token, whose key is rotated at
 * the query position and attended as one more raw row (see oracle_unit).
 * slimkv_oracle_decode_chunk takes a chunk of several query tokens per
 * sequence, each attending causally to the chunk's new tokens (see
 * oracle_chunk_unit).  slimkv_oracle_decode_alibi is the ALiBi variant (no
 * rotation, a linear distance bias on every score; see oracle_alibi_unit),
 * and slimkv_oracle_decode_chunk_alibi its serving form (ragged lengths, new
 * tokens, several query tokens; see oracle_alibi_chunk_unit).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

enum {
  ORACLE_OK = 0,
  ORACLE_BAD_SHAPE = 1,
  ORACLE_BAD_DTYPE = 2,
  ORACLE_NO_MEMORY = 3,
};

typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t num_beacons;
  int32_t rank_k;
  int32_t rank_v;
  int32_t raw_window;
  double scale;
  double rope_theta;
  int32_t dtype;
} oracle_problem;

static double widen(const void* base, int dtype, size_t i) {
  if (dtype == ORACLE_F64) return ((const double*)base)[i];
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * One (b, kv head) unit: all G query heads of the group, in the steps above.
 *
 * Ragged batches with an optional new token (one decode step with append):
 * the cache arrays keep the capacities of the problem as their row strides
 * (N_cap = num_beacons, W_cap = raw_window); sequence b uses the first
 * nb_b = clamp(num_beacons_b[b], 0, N_cap) beacon rows and the first
 * w_b = clamp(raw_len[b], 0, W_cap) raw rows.  With k_new / v_new
 * ([B, H_kv, d], the new token's key before rotation and its value), the
 * token's key is rotated at its own position q_pos[b] (the decode token
 * attends to itself), rounded to the storage precision as a cache row is,
 * and takes part in the softmax as one more raw row after the w_b others;
 * when w_b < W_cap it is also the row the cache would store at index w_b,
 * and k_app (if given) receives that rounded key.  A sequence with no rows
 * at all gets out = 0 and lse = -inf.  With nb_len = raw_len = NULL and no
 * new token this is the plain call: every capacity row is live.
 *
 * bpos (the reconstruction variant that keeps beacon-key rotation): beacon
 * j's key is rebuilt at full dimension, U_K C_K[j], and rotated at position
 * bpos[j] before it is scored against the rotated query; values are as in
 * the latent path (sum_j a_j U_V C_V[j] = U_V sum_j a_j C_V[j]).  NULL: the
 * latent scores of step 3.
 */

/* Round to the storage precision, to nearest with ties to even. */
static double narrow(double x, int dtype) {
  if (dtype == ORACLE_F64) return x;
  if (dtype == ORACLE_F32) return (double)(float)x;
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  const double m = frexp(x, &e); /* x = m 2^e, 1/2 <= |m| < 1 */
  return ldexp(nearbyint(ldexp(m, 8)), e - 8); /* 8 significant bits */
}

static void oracle_unit(const oracle_problem* p, int b, int h, const void* q,
                        const int32_t* q_pos, const void* U_K, const void* U_V,
                        const void* C_K, const void* C_V, const void* K_raw,
                        const void* V_raw, const int32_t* nb_len,
                        const int32_t* raw_len, const void* k_new,
                        const void* v_new, const int32_t* bpos, double* out,
                        double* lse, double* k_app, double* work) {
  const int d = p->head_dim, half = p->head_dim / 2;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int ncap = p->num_beacons, wcap = p->raw_window;
  const int rk = p->rank_k, rv = p->rank_v;
  const int dt = p->dtype;
  int nb = nb_len ? nb_len[b] : ncap, w = raw_len ? raw_len[b] : wcap;
  nb = nb < 0 ? 0 : (nb > ncap ? ncap : nb);
  w = w < 0 ? 0 : (w > wcap ? wcap : w);
  const int app = k_new != NULL;
  const size_t n = (size_t)nb + (size_t)w + (size_t)app;

  double* qr = work;          /* [d]   rotated query          */
  double* ka = qr + d;        /* [d]   rotated new key        */
  double* qh = ka + d;        /* [rk]  latent query           */
  double* s = qh + rk;        /* [n]   scores, then weights   */
  double* olat = s + n;       /* [rv]  latent value sum       */
  double* oraw = olat + rv;   /* [d]   raw value sum          */
  double* kb = oraw + d;      /* [d]   rebuilt beacon key (bpos) */

  const size_t unit = (size_t)b * p->num_kv_heads + h;
  const size_t ck0 = unit * (size_t)ncap * rk, cv0 = unit * (size_t)ncap * rv;
  const size_t kr0 = unit * (size_t)wcap * d;
  const size_t uk0 = (size_t)h * d * rk, uv0 = (size_t)h * d * rv;

  /* the new token's key: rotated at q_pos[b], rounded like a cache row */
  if (app) {
    for (int i = 0; i < half; ++i) {
      double inv_freq = pow(p->rope_theta, -2.0 * (double)i / (double)d);
      double ang = (double)q_pos[b] * inv_freq;
      double c = cos(ang), sn = sin(ang);
      double x1 = widen(k_new, dt, unit * d + i), x2 = widen(k_new, dt, unit * d + i + half);
      ka[i] = narrow(x1 * c - x2 * sn, dt);
      ka[i + half] = narrow(x2 * c + x1 * sn, dt);
    }
    if (k_app)
      for (int i = 0; i < d; ++i) k_app[unit * d + i] = ka[i];
  }

  for (int g = 0; g < G; ++g) {
    const int hq = h * G + g;
    const size_t q0 = ((size_t)b * p->num_q_heads + hq) * d;
    if (n == 0) {
      for (int i = 0; i < d; ++i) out[q0 + i] = 0.0;
      if (lse) lse[(size_t)b * p->num_q_heads + hq] = -INFINITY;
      continue;
    }

    /* 1. rotary embedding of the query at its own position */
    for (int i = 0; i < half; ++i) {
      double inv_freq = pow(p->rope_theta, -2.0 * (double)i / (double)d);
      double ang = (double)q_pos[b] * inv_freq;
      double c = cos(ang), sn = sin(ang);
      double x1 = widen(q, dt, q0 + i), x2 = widen(q, dt, q0 + i + half);
      qr[i] = x1 * c - x2 * sn;
      qr[i + half] = x2 * c + x1 * sn;
    }
    /* 2. projection into the beacon latent key space: qh = U_K^T q' */
    for (int k = 0; k < rk; ++k) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += qr[i] * widen(U_K, dt, uk0 + (size_t)i * rk + k);
      qh[k] = acc;
    }

    /* 3. scores: live latent beacons, live rotated raw keys, the new token */
    for (int j = 0; j < nb && !bpos; ++j) {
      double acc = 0.0;
      for (int k = 0; k < rk; ++k) acc += qh[k] * widen(C_K, dt, ck0 + (size_t)j * rk + k);
      s[j] = p->scale * acc;
    }
    for (int j = 0; j < nb && bpos; ++j) {
      /* the reconstruction variant: rebuild the key, rotate it at bpos[j] */
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int k = 0; k < rk; ++k)
          acc += widen(U_K, dt, uk0 + (size_t)i * rk + k) * widen(C_K, dt, ck0 + (size_t)j * rk + k);
        kb[i] = acc;
      }
      double acc = 0.0;
      for (int i = 0; i < half; ++i) {
        double inv_freq = pow(p->rope_theta, -2.0 * (double)i / (double)d);
        double ang = (double)bpos[j] * inv_freq;
        double c = cos(ang), sn = sin(ang);
        acc += qr[i] * (kb[i] * c - kb[i + half] * sn) + qr[i + half] * (kb[i + half] * c + kb[i] * sn);
      }
      s[j] = p->scale * acc;
    }
    for (int t = 0; t < w; ++t) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += qr[i] * widen(K_raw, dt, kr0 + (size_t)t * d + i);
      s[nb + t] = p->scale * acc;
    }
    if (app) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += qr[i] * ka[i];
      s[nb + w] = p->scale * acc;
    }

    /* 4. one softmax over beacon and raw rows together */
    double m = -INFINITY;
    for (size_t j = 0; j < n; ++j) m = s[j] > m ? s[j] : m;
    double l = 0.0;
    for (size_t j = 0; j < n; ++j) {
      s[j] = exp(s[j] - m);
      l += s[j];
    }
    for (size_t j = 0; j < n; ++j) s[j] /= l;

    /* 5. value sums: latent for beacons, full width for raw rows */
    for (int k = 0; k < rv; ++k) olat[k] = 0.0;
    for (int j = 0; j < nb; ++j)
      for (int k = 0; k < rv; ++k) olat[k] += s[j] * widen(C_V, dt, cv0 + (size_t)j * rv + k);
    for (int i = 0; i < d; ++i) oraw[i] = 0.0;
    for (int t = 0; t < w; ++t)
      for (int i = 0; i < d; ++i) oraw[i] += s[nb + t] * widen(V_raw, dt, kr0 + (size_t)t * d + i);
    if (app)
      for (int i = 0; i < d; ++i) oraw[i] += s[nb + w] * widen(v_new, dt, unit * d + i);

    /* 6. lift the latent value sum once: out = U_V o_lat + o_raw */
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int k = 0; k < rv; ++k) acc += widen(U_V, dt, uv0 + (size_t)i * rv + k) * olat[k];
      out[q0 + i] = acc + oraw[i];
    }
    if (lse) lse[(size_t)b * p->num_q_heads + hq] = m + log(l);
  }
}

/*
 * Compute the units listed in `units` (pairs b, h; NULL means every unit).
 * out: [B, H_q, d] doubles, lse: [B, H_q] doubles or NULL; entries of units
 * not listed are left untouched.  threads <= 0 uses the OpenMP default.
 */
static int decode_units(const oracle_problem* p, const void* q, const int32_t* q_pos,
                        const void* U_K, const void* U_V, const void* C_K, const void* C_V,
                        const void* K_raw, const void* V_raw, const int32_t* bpos,
                        const int32_t* units, int64_t n_units, double* out, double* lse,
                        int threads) {
  if (!p || !q || !q_pos || !out) return ORACLE_BAD_SHAPE;
  if (p->dtype != ORACLE_F64 && p->dtype != ORACLE_F32 && p->dtype != ORACLE_BF16)
    return ORACLE_BAD_DTYPE;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 ||
      p->num_q_heads % p->num_kv_heads != 0 || p->head_dim < 2 || p->head_dim % 2 ||
      p->num_beacons < 0 || p->raw_window < 0 ||
      (int64_t)p->num_beacons + p->raw_window < 1)
    return ORACLE_BAD_SHAPE;
  if (p->num_beacons > 0 && (p->rank_k < 1 || p->rank_v < 1 || !U_K || !U_V || !C_K || !C_V))
    return ORACLE_BAD_SHAPE;
  if (p->raw_window > 0 && (!K_raw || !V_raw)) return ORACLE_BAD_SHAPE;

  const int64_t all = (int64_t)p->batch * p->num_kv_heads;
  const int64_t count = units ? n_units : all;
  const int rk = p->num_beacons > 0 ? p->rank_k : 0;
  const int rv = p->num_beacons > 0 ? p->rank_v : 0;
  const size_t work_len =
      4 * (size_t)p->head_dim + rk + rv + (size_t)p->num_beacons + p->raw_window + 1;
  oracle_problem pp = *p;
  pp.rank_k = rk;
  pp.rank_v = rv;

  int failed = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel
  {
    double* work = (double*)malloc(work_len * sizeof(double));
    if (!work) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < count; ++u) {
      if (!work) continue;
      int b = units ? units[2 * u] : (int)(u / p->num_kv_heads);
      int h = units ? units[2 * u + 1] : (int)(u % p->num_kv_heads);
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_kv_heads) {
#pragma omp atomic write
        failed = 2;
        continue;
      }
      oracle_unit(&pp, b, h, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, NULL, NULL, NULL, NULL,
                  bpos, out, lse, NULL, work);
    }
    free(work);
  }
  if (failed == 1) return ORACLE_NO_MEMORY;
  if (failed == 2) return ORACLE_BAD_SHAPE;
  return ORACLE_OK;
}

int slimkv_oracle_decode(const oracle_problem* p, const void* q,
                         const int32_t* q_pos, const void* U_K,
                         const void* U_V, const void* C_K, const void* C_V,
                         const void* K_raw, const void* V_raw,
                         const int32_t* units, int64_t n_units, double* out,
                         double* lse, int threads) {
  return decode_units(p, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, NULL, units, n_units, out,
                      lse, threads);
}

/*
 * The reconstruction variant that keeps beacon-key rotation (page "Can
 * SlimKV compress KV cache jointly across tokens and features", section
 * "Speedups are real, but memory is set by the ratio"): as
 * slimkv_oracle_decode, but beacon j's key is rebuilt as U_K C_K[j] and
 * rotated at bpos[j] ([N_b] int32, the same for every sequence) before it
 * is scored.
 */
int slimkv_oracle_decode_beacon_rope(const oracle_problem* p, const void* q,
                                     const int32_t* q_pos, const void* U_K,
                                     const void* U_V, const void* C_K,
                                     const void* C_V, const void* K_raw,
                                     const void* V_raw, const int32_t* bpos,
                                     const int32_t* units, int64_t n_units,
                                     double* out, double* lse, int threads) {
  if (p && p->num_beacons > 0 && !bpos) return ORACLE_BAD_SHAPE;
  return decode_units(p, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, bpos, units, n_units, out,
                      lse, threads);
}

/*
 * Ragged counterpart of slimkv_oracle_decode (see oracle_unit).
 * num_beacons_b, raw_len: [B] live rows per sequence (NULL: the capacity);
 * k_new, v_new: [B, H_kv, d] in the storage dtype, both or neither;
 * k_app: [B, H_kv, d] doubles receiving the rounded new keys, or NULL.
 */
int slimkv_oracle_decode_ragged(const oracle_problem* p, const void* q,
                                const int32_t* q_pos, const void* U_K,
                                const void* U_V, const void* C_K, const void* C_V,
                                const void* K_raw, const void* V_raw,
                                const int32_t* num_beacons_b, const int32_t* raw_len,
                                const void* k_new, const void* v_new,
                                const int32_t* units, int64_t n_units, double* out,
                                double* lse, double* k_app, int threads) {
  if (!p || !q || !q_pos || !out) return ORACLE_BAD_SHAPE;
  if (p->dtype != ORACLE_F64 && p->dtype != ORACLE_F32 && p->dtype != ORACLE_BF16)
    return ORACLE_BAD_DTYPE;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 ||
      p->num_q_heads % p->num_kv_heads != 0 || p->head_dim < 2 || p->head_dim % 2 ||
      p->num_beacons < 0 || p->raw_window < 0)
    return ORACLE_BAD_SHAPE;
  if (p->num_beacons > 0 && (p->rank_k < 1 || p->rank_v < 1 || !U_K || !U_V || !C_K || !C_V))
    return ORACLE_BAD_SHAPE;
  if (p->raw_window > 0 && (!K_raw || !V_raw)) return ORACLE_BAD_SHAPE;
  if ((k_new == NULL) != (v_new == NULL)) return ORACLE_BAD_SHAPE;

  const int64_t all = (int64_t)p->batch * p->num_kv_heads;
  const int64_t count = units ? n_units : all;
  const int rk = p->num_beacons > 0 ? p->rank_k : 0;
  const int rv = p->num_beacons > 0 ? p->rank_v : 0;
  const size_t work_len =
      4 * (size_t)p->head_dim + rk + rv + (size_t)p->num_beacons + p->raw_window + 1;
  oracle_problem pp = *p;
  pp.rank_k = rk;
  pp.rank_v = rv;

  int failed = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel
  {
    double* work = (double*)malloc(work_len * sizeof(double));
    if (!work) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < count; ++u) {
      if (!work) continue;
      int b = units ? units[2 * u] : (int)(u / p->num_kv_heads);
      int h = units ? units[2 * u + 1] : (int)(u % p->num_kv_heads);
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_kv_heads) {
#pragma omp atomic write
        failed = 2;
        continue;
      }
      oracle_unit(&pp, b, h, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, num_beacons_b, raw_len,
                  k_new, v_new, NULL, out, lse, k_app, work);
    }
    free(work);
  }
  if (failed == 1) return ORACLE_NO_MEMORY;
  if (failed == 2) return ORACLE_BAD_SHAPE;
  return ORACLE_OK;
}

/*
 * The ALiBi variant (page "Can SlimKV compress KV cache jointly across
 * tokens and features": ALiBi adds its positional bias after the query-key
 * product, so it composes with the latent scores).  An ALiBi backbone has
 * no rotary embedding: neither the query nor any key is rotated, and every
 * score gets the bias -slope[hq] * (q_pos - k_pos) added after the scaled
 * product, with the query head's slope.  Key positions: beacon j at
 * bpos[j]; raw row t at q_pos[b] - W + 1 + t (the window ends at the
 * query's position).  Otherwise the steps of oracle_unit: project the
 * query, score latent beacons and raw keys, one softmax, latent value sum
 * lifted once.
 */
static void oracle_alibi_unit(const oracle_problem* p, int b, int h, const void* q,
                              const int32_t* q_pos, const void* U_K, const void* U_V,
                              const void* C_K, const void* C_V, const void* K_raw,
                              const void* V_raw, const int32_t* bpos, const double* slope,
                              double* out, double* lse, double* work) {
  const int d = p->head_dim;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int nb = p->num_beacons, w = p->raw_window;
  const int rk = p->rank_k, rv = p->rank_v;
  const int dt = p->dtype;
  const size_t n = (size_t)nb + (size_t)w;
  double* qv = work;        /* [d]  the query (no rotation)  */
  double* qh = qv + d;      /* [rk] latent query             */
  double* s = qh + rk;      /* [n]  scores, then weights     */
  double* olat = s + n;     /* [rv] latent value sum         */
  double* oraw = olat + rv; /* [d]  raw value sum            */
  const size_t unit = (size_t)b * p->num_kv_heads + h;
  const size_t ck0 = unit * (size_t)nb * rk, cv0 = unit * (size_t)nb * rv;
  const size_t kr0 = unit * (size_t)w * d;
  const size_t uk0 = (size_t)h * d * rk, uv0 = (size_t)h * d * rv;
  const double qp = (double)q_pos[b];
  for (int g = 0; g < G; ++g) {
    const int hq = h * G + g;
    const size_t q0 = ((size_t)b * p->num_q_heads + hq) * d;
    const double m_h = slope[hq];
    for (int i = 0; i < d; ++i) qv[i] = widen(q, dt, q0 + i);
    for (int k = 0; k < rk; ++k) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += qv[i] * widen(U_K, dt, uk0 + (size_t)i * rk + k);
      qh[k] = acc;
    }
    for (int j = 0; j < nb; ++j) {
      double acc = 0.0;
      for (int k = 0; k < rk; ++k) acc += qh[k] * widen(C_K, dt, ck0 + (size_t)j * rk + k);
      s[j] = p->scale * acc - m_h * (qp - (double)bpos[j]);
    }
    for (int t = 0; t < w; ++t) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += qv[i] * widen(K_raw, dt, kr0 + (size_t)t * d + i);
      const double kpos = qp - (double)w + 1.0 + (double)t;
      s[nb + t] = p->scale * acc - m_h * (qp - kpos);
    }
    double mx = -INFINITY;
    for (size_t j = 0; j < n; ++j) mx = s[j] > mx ? s[j] : mx;
    double den = 0.0;
    for (size_t j = 0; j < n; ++j) {
      s[j] = exp(s[j] - mx);
      den += s[j];
    }
    for (size_t j = 0; j < n; ++j) s[j] /= den;
    for (int k = 0; k < rv; ++k) olat[k] = 0.0;
    for (int j = 0; j < nb; ++j)
      for (int k = 0; k < rv; ++k) olat[k] += s[j] * widen(C_V, dt, cv0 + (size_t)j * rv + k);
    for (int i = 0; i < d; ++i) oraw[i] = 0.0;
    for (int t = 0; t < w; ++t)
      for (int i = 0; i < d; ++i) oraw[i] += s[nb + t] * widen(V_raw, dt, kr0 + (size_t)t * d + i);
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int k = 0; k < rv; ++k) acc += widen(U_V, dt, uv0 + (size_t)i * rv + k) * olat[k];
      out[q0 + i] = acc + oraw[i];
    }
    if (lse) lse[(size_t)b * p->num_q_heads + hq] = mx + log(den);
  }
}

/*
 * ALiBi counterpart of slimkv_oracle_decode (see oracle_alibi_unit):
 * bpos [N_b] int32 beacon positions (the same for every sequence), slope
 * [H_q] doubles.
 */
int slimkv_oracle_decode_alibi(const oracle_problem* p, const void* q, const int32_t* q_pos,
                               const void* U_K, const void* U_V, const void* C_K,
                               const void* C_V, const void* K_raw, const void* V_raw,
                               const int32_t* bpos, const double* slope, const int32_t* units,
                               int64_t n_units, double* out, double* lse, int threads) {
  if (!p || !q || !q_pos || !out || !slope) return ORACLE_BAD_SHAPE;
  if (p->dtype != ORACLE_F64 && p->dtype != ORACLE_F32 && p->dtype != ORACLE_BF16)
    return ORACLE_BAD_DTYPE;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 ||
      p->num_q_heads % p->num_kv_heads != 0 || p->head_dim < 1 || p->num_beacons < 0 ||
      p->raw_window < 0 || (int64_t)p->num_beacons + p->raw_window < 1)
    return ORACLE_BAD_SHAPE;
  if (p->num_beacons > 0 &&
      (p->rank_k < 1 || p->rank_v < 1 || !U_K || !U_V || !C_K || !C_V || !bpos))
    return ORACLE_BAD_SHAPE;
  if (p->raw_window > 0 && (!K_raw || !V_raw)) return ORACLE_BAD_SHAPE;
  const int64_t all = (int64_t)p->batch * p->num_kv_heads;
  const int64_t count = units ? n_units : all;
  const int rk = p->num_beacons > 0 ? p->rank_k : 0;
  const int rv = p->num_beacons > 0 ? p->rank_v : 0;
  const size_t work_len = 2 * (size_t)p->head_dim + rk + rv + (size_t)p->num_beacons + p->raw_window;
  oracle_problem pp = *p;
  pp.rank_k = rk;
  pp.rank_v = rv;
  int failed = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel
  {
    double* work = (double*)malloc(work_len * sizeof(double));
    if (!work) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < count; ++u) {
      if (!work) continue;
      int b = units ? units[2 * u] : (int)(u / p->num_kv_heads);
      int h = units ? units[2 * u + 1] : (int)(u % p->num_kv_heads);
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_kv_heads) {
#pragma omp atomic write
        failed = 2;
        continue;
      }
      oracle_alibi_unit(&pp, b, h, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw, bpos, slope, out,
                        lse, work);
    }
    free(work);
  }
  if (failed == 1) return ORACLE_NO_MEMORY;
  if (failed == 2) return ORACLE_BAD_SHAPE;
  return ORACLE_OK;
}

/*
 * Multi-token queries against the compressed cache: a chunk of Q tokens per
 * sequence, as when speculative decoding checks several drafted tokens in
 * one pass or a prompt is fed Q tokens at a time (the query side of the
 * same attention; page "Can SlimKV compress KV cache jointly across tokens
 * and features", section "Latent-space attention removes the rebuild
 * step").  Token t of sequence b sits at position q_pos[b] + t.  Each of
 * its G query heads is rotated at that position and attends, under one
 * softmax, over the live beacon rows, the live raw rows and the chunk's new
 * tokens 0 .. t -- token u's key rotated at its own position q_pos[b] + u
 * and rounded like a cache row -- but not over the chunk's later tokens.
 * Without new tokens every query of the chunk attends over the cache rows
 * only.  Lengths are clamped as in oracle_unit.  k_app (if given) receives
 * token u's rounded key, the row the cache would store at w_b + u.
 * Layouts: q, out [B, Q, H_q, d]; lse [B, Q, H_q]; k_new, v_new, k_app
 * [B, Q, H_kv, d].  With Q = 1 this is oracle_unit's computation.
 */
static void oracle_chunk_unit(const oracle_problem* p, int ntok, int b, int h, const void* q,
                              const int32_t* q_pos, const void* U_K, const void* U_V,
                              const void* C_K, const void* C_V, const void* K_raw,
                              const void* V_raw, const int32_t* nb_len, const int32_t* raw_len,
                              const void* k_new, const void* v_new, double* out, double* lse,
                              double* k_app, double* work) {
  const int d = p->head_dim, half = p->head_dim / 2;
  const int H = p->num_kv_heads, Hq = p->num_q_heads, G = Hq / H;
  const int ncap = p->num_beacons, wcap = p->raw_window;
  const int rk = p->rank_k, rv = p->rank_v;
  const int dt = p->dtype;
  int nb = nb_len ? nb_len[b] : ncap, w = raw_len ? raw_len[b] : wcap;
  nb = nb < 0 ? 0 : (nb > ncap ? ncap : nb);
  w = w < 0 ? 0 : (w > wcap ? wcap : w);
  const int app = k_new != NULL;

  double* qrot = work;                       /* [d]             rotated query     */
  double* qlat = qrot + d;                   /* [rk]            latent query      */
  double* sc = qlat + rk;                    /* [nb + w + Q]    scores, weights   */
  double* vl = sc + (size_t)nb + w + ntok;   /* [rv]            latent value sum  */
  double* vr = vl + rv;                      /* [d]             raw value sum     */
  double* kt = vr + d;                       /* [Q * d]         rotated new keys  */

  const size_t unit = (size_t)b * H + h;
  const size_t ck0 = unit * (size_t)ncap * rk, cv0 = unit * (size_t)ncap * rv;
  const size_t kr0 = unit * (size_t)wcap * d;
  const size_t uk0 = (size_t)h * d * rk, uv0 = (size_t)h * d * rv;

  /* the chunk's new keys, token u rotated at q_pos[b] + u and rounded */
  for (int u = 0; u < ntok && app; ++u) {
    const size_t k0 = (((size_t)b * ntok + u) * H + h) * d;
    const double tpos = (double)q_pos[b] + (double)u;
    for (int i = 0; i < half; ++i) {
      const double ang = tpos * pow(p->rope_theta, -2.0 * (double)i / (double)d);
      const double c = cos(ang), sn = sin(ang);
      const double x1 = widen(k_new, dt, k0 + i), x2 = widen(k_new, dt, k0 + i + half);
      kt[(size_t)u * d + i] = narrow(x1 * c - x2 * sn, dt);
      kt[(size_t)u * d + i + half] = narrow(x2 * c + x1 * sn, dt);
    }
    if (k_app)
      for (int i = 0; i < d; ++i) k_app[k0 + i] = kt[(size_t)u * d + i];
  }

  for (int t = 0; t < ntok; ++t) {
    const double qpos = (double)q_pos[b] + (double)t;
    const int seen = app ? t + 1 : 0; /* new tokens this query attends to */
    const size_t n = (size_t)nb + (size_t)w + (size_t)seen;
    for (int g = 0; g < G; ++g) {
      const int hq = h * G + g;
      const size_t row = ((size_t)b * ntok + t) * Hq + hq;
      const size_t q0 = row * d;
      if (n == 0) {
        for (int i = 0; i < d; ++i) out[q0 + i] = 0.0;
        if (lse) lse[row] = -INFINITY;
        continue;
      }
      /* rotate the query at its token's position, then project it */
      for (int i = 0; i < half; ++i) {
        const double ang = qpos * pow(p->rope_theta, -2.0 * (double)i / (double)d);
        const double c = cos(ang), sn = sin(ang);
        const double x1 = widen(q, dt, q0 + i), x2 = widen(q, dt, q0 + i + half);
        qrot[i] = x1 * c - x2 * sn;
        qrot[i + half] = x2 * c + x1 * sn;
      }
      for (int k = 0; k < rk; ++k) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qrot[i] * widen(U_K, dt, uk0 + (size_t)i * rk + k);
        qlat[k] = acc;
      }
      /* scores: latent beacons, rotated raw keys, new tokens 0 .. t */
      for (int j = 0; j < nb; ++j) {
        double acc = 0.0;
        for (int k = 0; k < rk; ++k) acc += qlat[k] * widen(C_K, dt, ck0 + (size_t)j * rk + k);
        sc[j] = p->scale * acc;
      }
      for (int j = 0; j < w; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qrot[i] * widen(K_raw, dt, kr0 + (size_t)j * d + i);
        sc[nb + j] = p->scale * acc;
      }
      for (int u = 0; u < seen; ++u) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qrot[i] * kt[(size_t)u * d + i];
        sc[nb + w + u] = p->scale * acc;
      }
      /* one softmax over all of them */
      double mx = -INFINITY;
      for (size_t j = 0; j < n; ++j) mx = sc[j] > mx ? sc[j] : mx;
      double den = 0.0;
      for (size_t j = 0; j < n; ++j) {
        sc[j] = exp(sc[j] - mx);
        den += sc[j];
      }
      for (size_t j = 0; j < n; ++j) sc[j] /= den;
      /* value sums (latent for beacons), then the lift */
      for (int k = 0; k < rv; ++k) vl[k] = 0.0;
      for (int j = 0; j < nb; ++j)
        for (int k = 0; k < rv; ++k) vl[k] += sc[j] * widen(C_V, dt, cv0 + (size_t)j * rv + k);
      for (int i = 0; i < d; ++i) vr[i] = 0.0;
      for (int j = 0; j < w; ++j)
        for (int i = 0; i < d; ++i) vr[i] += sc[nb + j] * widen(V_raw, dt, kr0 + (size_t)j * d + i);
      for (int u = 0; u < seen; ++u) {
        const size_t v0 = (((size_t)b * ntok + u) * H + h) * d;
        for (int i = 0; i < d; ++i) vr[i] += sc[nb + w + u] * widen(v_new, dt, v0 + i);
      }
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int k = 0; k < rv; ++k) acc += widen(U_V, dt, uv0 + (size_t)i * rv + k) * vl[k];
        out[q0 + i] = acc + vr[i];
      }
      if (lse) lse[row] = mx + log(den);
    }
  }
}

/*
 * Multi-token counterpart of slimkv_oracle_decode_ragged (see
 * oracle_chunk_unit): num_tokens = Q >= 1 query tokens per sequence.
 */
int slimkv_oracle_decode_chunk(const oracle_problem* p, int num_tokens, const void* q,
                               const int32_t* q_pos, const void* U_K, const void* U_V,
                               const void* C_K, const void* C_V, const void* K_raw,
                               const void* V_raw, const int32_t* num_beacons_b,
                               const int32_t* raw_len, const void* k_new, const void* v_new,
                               const int32_t* units, int64_t n_units, double* out, double* lse,
                               double* k_app, int threads) {
  if (!p || !q || !q_pos || !out || num_tokens < 1) return ORACLE_BAD_SHAPE;
  if (p->dtype != ORACLE_F64 && p->dtype != ORACLE_F32 && p->dtype != ORACLE_BF16)
    return ORACLE_BAD_DTYPE;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 ||
      p->num_q_heads % p->num_kv_heads != 0 || p->head_dim < 2 || p->head_dim % 2 ||
      p->num_beacons < 0 || p->raw_window < 0)
    return ORACLE_BAD_SHAPE;
  if (p->num_beacons > 0 && (p->rank_k < 1 || p->rank_v < 1 || !U_K || !U_V || !C_K || !C_V))
    return ORACLE_BAD_SHAPE;
  if (p->raw_window > 0 && (!K_raw || !V_raw)) return ORACLE_BAD_SHAPE;
  if ((k_new == NULL) != (v_new == NULL)) return ORACLE_BAD_SHAPE;

  const int64_t all = (int64_t)p->batch * p->num_kv_heads;
  const int64_t count = units ? n_units : all;
  const int rk = p->num_beacons > 0 ? p->rank_k : 0;
  const int rv = p->num_beacons > 0 ? p->rank_v : 0;
  const size_t work_len = (3 + (size_t)num_tokens) * (size_t)p->head_dim + rk + rv +
                          (size_t)p->num_beacons + p->raw_window + num_tokens;
  oracle_problem pp = *p;
  pp.rank_k = rk;
  pp.rank_v = rv;

  int failed = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel
  {
    double* work = (double*)malloc(work_len * sizeof(double));
    if (!work) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < count; ++u) {
      if (!work) continue;
      int b = units ? units[2 * u] : (int)(u / p->num_kv_heads);
      int h = units ? units[2 * u + 1] : (int)(u % p->num_kv_heads);
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_kv_heads) {
#pragma omp atomic write
        failed = 2;
        continue;
      }
      oracle_chunk_unit(&pp, num_tokens, b, h, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                        num_beacons_b, raw_len, k_new, v_new, out, lse, k_app, work);
    }
    free(work);
  }
  if (failed == 1) return ORACLE_NO_MEMORY;
  if (failed == 2) return ORACLE_BAD_SHAPE;
  return ORACLE_OK;
}

/*
 * The ALiBi variant of a serving step: ragged lengths, optional new tokens,
 * and Q >= 1 query tokens per sequence (Q = 1: one decode step; the
 * uniform variant above is the case of full lengths, no new tokens and
 * Q = 1).  As in oracle_alibi_unit nothing is rotated and every score gets
 * -slope[hq] * (q_pos_t - k_pos) after the scaled product.  Positions, the
 * reading of a window that ends at the newest token:
 *   query token t        q_pos[b] + t
 *   beacon j             bpos[j]
 *   new token u          q_pos[b] + u
 *   live raw row i < w   q_pos[b] - w + i with new tokens (they follow the
 *                        raw rows), q_pos[b] - w + 1 + i without (the first
 *                        query's own token is the last raw row)
 * Query token t attends over the live beacon rows, the live raw rows and
 * the new tokens 0 .. t; new keys are stored as given (no rotation), so
 * k_app (if given) receives them widened.  Lengths are clamped as in
 * oracle_unit.  Layouts as in oracle_chunk_unit.
 */
static void oracle_alibi_chunk_unit(const oracle_problem* p, int ntok, int b, int h,
                                    const void* q, const int32_t* q_pos, const void* U_K,
                                    const void* U_V, const void* C_K, const void* C_V,
                                    const void* K_raw, const void* V_raw, const int32_t* nb_len,
                                    const int32_t* raw_len, const void* k_new, const void* v_new,
                                    const int32_t* bpos, const double* slope, double* out,
                                    double* lse, double* k_app, double* work) {
  const int d = p->head_dim;
  const int H = p->num_kv_heads, Hq = p->num_q_heads, G = Hq / H;
  const int ncap = p->num_beacons, wcap = p->raw_window;
  const int rk = p->rank_k, rv = p->rank_v;
  const int dt = p->dtype;
  int nb = nb_len ? nb_len[b] : ncap, w = raw_len ? raw_len[b] : wcap;
  nb = nb < 0 ? 0 : (nb > ncap ? ncap : nb);
  w = w < 0 ? 0 : (w > wcap ? wcap : w);
  const int app = k_new != NULL;

  double* qv = work;                         /* [d]           the query (unrotated) */
  double* qlat = qv + d;                     /* [rk]          latent query          */
  double* sc = qlat + rk;                    /* [nb + w + Q]  scores, weights       */
  double* vl = sc + (size_t)nb + w + ntok;   /* [rv]          latent value sum      */
  double* vr = vl + rv;                      /* [d]           raw value sum         */

  const size_t unit = (size_t)b * H + h;
  const size_t ck0 = unit * (size_t)ncap * rk, cv0 = unit * (size_t)ncap * rv;
  const size_t kr0 = unit * (size_t)wcap * d;
  const size_t uk0 = (size_t)h * d * rk, uv0 = (size_t)h * d * rv;
  const double qp0 = (double)q_pos[b];
  const double raw0 = qp0 - (double)w + (app ? 0.0 : 1.0); /* position of raw row 0 */

  for (int u = 0; u < ntok && app && k_app; ++u) {
    const size_t k0 = (((size_t)b * ntok + u) * H + h) * d;
    for (int i = 0; i < d; ++i) k_app[k0 + i] = widen(k_new, dt, k0 + i);
  }

  for (int t = 0; t < ntok; ++t) {
    const double qpos = qp0 + (double)t;
    const int seen = app ? t + 1 : 0;
    const size_t n = (size_t)nb + (size_t)w + (size_t)seen;
    for (int g = 0; g < G; ++g) {
      const int hq = h * G + g;
      const double m_h = slope[hq];
      const size_t row = ((size_t)b * ntok + t) * Hq + hq;
      const size_t q0 = row * d;
      if (n == 0) {
        for (int i = 0; i < d; ++i) out[q0 + i] = 0.0;
        if (lse) lse[row] = -INFINITY;
        continue;
      }
      for (int i = 0; i < d; ++i) qv[i] = widen(q, dt, q0 + i);
      for (int k = 0; k < rk; ++k) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qv[i] * widen(U_K, dt, uk0 + (size_t)i * rk + k);
        qlat[k] = acc;
      }
      for (int j = 0; j < nb; ++j) {
        double acc = 0.0;
        for (int k = 0; k < rk; ++k) acc += qlat[k] * widen(C_K, dt, ck0 + (size_t)j * rk + k);
        sc[j] = p->scale * acc - m_h * (qpos - (double)bpos[j]);
      }
      for (int j = 0; j < w; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qv[i] * widen(K_raw, dt, kr0 + (size_t)j * d + i);
        sc[nb + j] = p->scale * acc - m_h * (qpos - (raw0 + (double)j));
      }
      for (int u = 0; u < seen; ++u) {
        const size_t k0 = (((size_t)b * ntok + u) * H + h) * d;
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qv[i] * widen(k_new, dt, k0 + i);
        sc[nb + w + u] = p->scale * acc - m_h * (qpos - (qp0 + (double)u));
      }
      double mx = -INFINITY;
      for (size_t j = 0; j < n; ++j) mx = sc[j] > mx ? sc[j] : mx;
      double den = 0.0;
      for (size_t j = 0; j < n; ++j) {
        sc[j] = exp(sc[j] - mx);
        den += sc[j];
      }
      for (size_t j = 0; j < n; ++j) sc[j] /= den;
      for (int k = 0; k < rv; ++k) vl[k] = 0.0;
      for (int j = 0; j < nb; ++j)
        for (int k = 0; k < rv; ++k) vl[k] += sc[j] * widen(C_V, dt, cv0 + (size_t)j * rv + k);
      for (int i = 0; i < d; ++i) vr[i] = 0.0;
      for (int j = 0; j < w; ++j)
        for (int i = 0; i < d; ++i) vr[i] += sc[nb + j] * widen(V_raw, dt, kr0 + (size_t)j * d + i);
      for (int u = 0; u < seen; ++u) {
        const size_t v0 = (((size_t)b * ntok + u) * H + h) * d;
        for (int i = 0; i < d; ++i) vr[i] += sc[nb + w + u] * widen(v_new, dt, v0 + i);
      }
      for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int k = 0; k < rv; ++k) acc += widen(U_V, dt, uv0 + (size_t)i * rv + k) * vl[k];
        out[q0 + i] = acc + vr[i];
      }
      if (lse) lse[row] = mx + log(den);
    }
  }
}

/*
 * ALiBi counterpart of slimkv_oracle_decode_chunk (see
 * oracle_alibi_chunk_unit): bpos [N_b] int32 beacon positions, slope [H_q]
 * doubles; num_tokens = Q >= 1.
 */
int slimkv_oracle_decode_chunk_alibi(const oracle_problem* p, int num_tokens, const void* q,
                                     const int32_t* q_pos, const void* U_K, const void* U_V,
                                     const void* C_K, const void* C_V, const void* K_raw,
                                     const void* V_raw, const int32_t* num_beacons_b,
                                     const int32_t* raw_len, const void* k_new,
                                     const void* v_new, const int32_t* bpos,
                                     const double* slope, const int32_t* units, int64_t n_units,
                                     double* out, double* lse, double* k_app, int threads) {
  if (!p || !q || !q_pos || !out || !slope || num_tokens < 1) return ORACLE_BAD_SHAPE;
  if (p->dtype != ORACLE_F64 && p->dtype != ORACLE_F32 && p->dtype != ORACLE_BF16)
    return ORACLE_BAD_DTYPE;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 ||
      p->num_q_heads % p->num_kv_heads != 0 || p->head_dim < 1 || p->num_beacons < 0 ||
      p->raw_window < 0)
    return ORACLE_BAD_SHAPE;
  if (p->num_beacons > 0 &&
      (p->rank_k < 1 || p->rank_v < 1 || !U_K || !U_V || !C_K || !C_V || !bpos))
    return ORACLE_BAD_SHAPE;
  if (p->raw_window > 0 && (!K_raw || !V_raw)) return ORACLE_BAD_SHAPE;
  if ((k_new == NULL) != (v_new == NULL)) return ORACLE_BAD_SHAPE;

  const int64_t all = (int64_t)p->batch * p->num_kv_heads;
  const int64_t count = units ? n_units : all;
  const int rk = p->num_beacons > 0 ? p->rank_k : 0;
  const int rv = p->num_beacons > 0 ? p->rank_v : 0;
  const size_t work_len = 2 * (size_t)p->head_dim + rk + rv + (size_t)p->num_beacons +
                          p->raw_window + num_tokens;
  oracle_problem pp = *p;
  pp.rank_k = rk;
  pp.rank_v = rv;

  int failed = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel
  {
    double* work = (double*)malloc(work_len * sizeof(double));
    if (!work) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < count; ++u) {
      if (!work) continue;
      int b = units ? units[2 * u] : (int)(u / p->num_kv_heads);
      int h = units ? units[2 * u + 1] : (int)(u % p->num_kv_heads);
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_kv_heads) {
#pragma omp atomic write
        failed = 2;
        continue;
      }
      oracle_alibi_chunk_unit(&pp, num_tokens, b, h, q, q_pos, U_K, U_V, C_K, C_V, K_raw, V_raw,
                              num_beacons_b, raw_len, k_new, v_new, bpos, slope, out, lse, k_app,
                              work);
    }
    free(work);
  }
  if (failed == 1) return ORACLE_NO_MEMORY;
  if (failed == 2) return ORACLE_BAD_SHAPE;
  return ORACLE_OK;
}

/* Threads an OpenMP parallel region would use (for reporting). */
int slimkv_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
