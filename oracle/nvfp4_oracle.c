/*
 * nvfp4_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for the two operations of the
 * NVFP4 paged-KV hot path:
 *   (1) quantize new K/V rows to NVFP4 and append them into a paged cache
 *       through a slot mapping, and
 *   (2) batched causal prefill attention that reads those NVFP4 pages.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this file's library.  It shares no code, header, table or helper with the
 * HIP implementation under nvfp4_paged_kv_amd/csrc; each side was written on
 * its own from the same readings of the source pages.
 *
 * Sources (FlashInfer pull-request analysis pages):
 *   - PR #6204 page (NVFP4 KV cache append: host sync removed), sections on
 *     `_as_float32_scalar_tensors` and on the append function's docstring:
 *     a global decode scale per tensor, positive and finite, checked only
 *     when there are rows to write.
 *   - PR #4769 page (NVFP4 KV tile repack), introduction and code analysis:
 *     NVFP4 = E2M1 elements with E4M3 scale factors; the attention reads the
 *     dequantized values.
 *   - PR #3575 page (FP8 causal attention), introduction: causal attention,
 *     the key range a query sees grows with its position.
 * Where the pages are silent (block size 16, the E2M1 grid, round-to-nearest-
 * even, the exact fp32 operation order of the block scale, nibble order,
 * cache layout, slot meaning, GQA grouping, causal alignment) this file
 * follows the readings listed in the design notes; each function says which.
 *
 * Precision: the codecs and the block quantizer work in IEEE fp32 exactly as
 * the quantizer's readings pin them (this decides integer codes, so both
 * sides take the decision in fp32); the attention works in fp64.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 *        -pthread nvfp4_oracle.c -o liboracle.so -lm
 * (-ffp-contract=off: no a*b+c fusion, every fp32 step rounds on its own.)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Error bits the oracle reports (same meaning as the library's device flag). */
#define ORACLE_BAD_K_SCALE 1u
#define ORACLE_BAD_V_SCALE 2u
#define ORACLE_SLOT_OOB 4u
#define ORACLE_PAGE_OOB 8u

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32: a bf16 is the upper half of an fp32 bit pattern.     */
/* ------------------------------------------------------------------ */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------ */
/* E2M1 (FP4) element codec.                                            */
/* 4-bit code: bit 3 = sign, bits 2..1 = exponent (bias 1), bit 0 =     */
/* mantissa.  Exponent field 0 is subnormal (value m * 0.5).  The       */
/* magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}.                         */
/* ------------------------------------------------------------------ */
double oracle_e2m1_value(int code) {
  int e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return (code & 8) ? -mag : mag;
}

/* Magnitude code (0..7) of |y| rounded to the nearest E2M1 magnitude;
 * an exact tie goes to the even code (round-to-nearest-even); anything
 * beyond 6, infinity included, saturates to 6 (code 7); NaN gives 0
 * (reading: a NaN element carries no magnitude). */
int oracle_e2m1_encode_mag(float y) {
  if (isnan(y)) return 0;
  double a = fabs((double)y);
  if (isinf(a) || a >= 6.0) return 7;
  int best = 0;
  double best_d = a; /* distance to code 0 (value 0) */
  for (int c = 1; c < 8; ++c) {
    double d = fabs(oracle_e2m1_value(c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return best;
}

/* ------------------------------------------------------------------ */
/* E4M3 (OCP E4M3FN) scale-factor codec.                                */
/* 8-bit code: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0       */
/* mantissa.  Exponent 0 is subnormal (m * 2^-9).  0x7F/0xFF are NaN,   */
/* there is no infinity, the largest finite value is 448 (0x7E).        */
/* ------------------------------------------------------------------ */
double oracle_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Unsigned E4M3 encode of a block scale s (s is >= 0 by construction):
 * nearest finite non-negative code, ties to the even code; values at or
 * above 448 (infinity included) saturate to 448 (code 0x7E); zero, NaN and
 * anything not > 0 give code 0.  The finite non-negative codes 0..0x7E are
 * increasing in value, so "nearest" is found by locating the last code not
 * above s and comparing with its successor. */
int oracle_e4m3_encode(float s_f) {
  double s = (double)s_f;
  if (!(s > 0.0)) return 0;
  if (s >= 448.0) return 0x7E;
  int lo = 0, hi = 0x7E; /* invariant: value(lo) <= s < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_value(mid) <= s) lo = mid; else hi = mid;
  }
  double dl = s - oracle_e4m3_value(lo), dh = oracle_e4m3_value(hi) - s;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) ? hi : lo; /* exact tie: even code */
}

/* Bulk helpers used by the pins (exhaustive sweeps over fp32 patterns);
 * the array is split over threads, each element is encoded on its own. */
typedef struct { const float* in; uint8_t* out; int64_t n; int kind; } bulk_job;

static void* bulk_worker(void* arg) {
  bulk_job* J = (bulk_job*)arg;
  for (int64_t i = 0; i < J->n; ++i) {
    float v = J->in[i];
    J->out[i] = (uint8_t)(J->kind == 0 ? ((signbit(v) ? 8 : 0) | oracle_e2m1_encode_mag(v))
                                       : oracle_e4m3_encode(v));
  }
  return NULL;
}

static void bulk_run(const float* in, int64_t n, uint8_t* out, int kind) {
  enum { NT = 8 };
  bulk_job jobs[NT];
  pthread_t th[NT];
  int64_t per = (n + NT - 1) / NT;
  for (int i = 0; i < NT; ++i) {
    int64_t lo = i * per < n ? i * per : n, hi = (i + 1) * per < n ? (i + 1) * per : n;
    jobs[i] = (bulk_job){in + lo, out + lo, hi - lo, kind};
    pthread_create(&th[i], NULL, bulk_worker, &jobs[i]);
  }
  for (int i = 0; i < NT; ++i) pthread_join(th[i], NULL);
}

void oracle_e2m1_encode_array(const float* y, int64_t n, uint8_t* codes) { bulk_run(y, n, codes, 0); }
void oracle_e4m3_encode_array(const float* s, int64_t n, uint8_t* codes) { bulk_run(s, n, codes, 1); }

/* ------------------------------------------------------------------ */
/* Global decode scale check (PR #6204 page, docstring section: a       */
/* scale must be a positive finite fp32 value).                         */
/* ------------------------------------------------------------------ */
int oracle_scale_ok(float g) { return (g > 0.0f) && isfinite(g); }

/* ------------------------------------------------------------------ */
/* One NVFP4 block: 16 consecutive head_dim elements of one (token,      */
/* head), a global decode scale g, out: 8 packed bytes + 1 scale byte.   */
/* Steps (readings of the NVFP4 format; decode is x ~ e2m1 * S * g):     */
/*   O1 a   = max |x_i|            (NaN elements are ignored)            */
/*   O2 s   = fl32(a / fl32(6 g))  (6 = largest E2M1 magnitude)          */
/*   O3 sf  = E4M3 encode of s,  S = its exact value                     */
/*   O4 r   = 0 if sf == 0, else fl32(1 / fl32(S g))                     */
/*   O5 y_i = fl32(x_i r); code_i = sign(x_i) | E2M1 magnitude of y_i    */
/*   O6 byte_j = code_{2j} | code_{2j+1} << 4   (even element low)       */
/* ------------------------------------------------------------------ */
void oracle_quantize_block(const uint16_t* xb, float g, uint8_t* packed, uint8_t* sf_out) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = bf16_bits_to_float(xb[i]);
  float a = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float m = fabsf(x[i]);
    if (m > a) a = m; /* false for NaN: NaN is skipped */
  }
  float d6 = 6.0f * g;
  float s = a / d6;
  int sf = oracle_e4m3_encode(s);
  float S = (float)oracle_e4m3_value(sf); /* exact in fp32 */
  float den = S * g;
  float r = (sf == 0) ? 0.0f : 1.0f / den;
  uint8_t code[16];
  for (int i = 0; i < 16; ++i) {
    float y = x[i] * r;
    code[i] = (uint8_t)((signbit(x[i]) ? 8 : 0) | oracle_e2m1_encode_mag(y));
  }
  for (int j = 0; j < 8; ++j) packed[j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
  *sf_out = (uint8_t)sf;
}

/* ------------------------------------------------------------------ */
/* Append (PR #6204 page: quantize the new rows and write them to the   */
/* cache positions the slot mapping names).                             */
/* Layout (reading): cache [num_pages][page_size][H_kv][D/2] bytes,      */
/* scale factors [num_pages][page_size][H_kv][D/16] bytes.               */
/* slot -> page = slot / page_size, offset = slot % page_size.           */
/* slot < 0: padding, skipped.  slot >= num_pages*page_size: skipped and */
/* reported.  T == 0: nothing is written and nothing is checked.  A bad  */
/* scale (either one): nothing at all is written.                        */
/* ------------------------------------------------------------------ */
typedef struct {
  const uint16_t *k, *v;
  const int64_t* slots;
  int64_t t0, t1;
  float gk, gv;
  uint8_t *kc, *vc, *ksf, *vsf;
  int64_t num_slots;
  int ps, H, D;
  uint32_t err;
} append_job;

static void* append_worker(void* arg) {
  append_job* J = (append_job*)arg;
  const int nb = J->D / 16;
  for (int64_t t = J->t0; t < J->t1; ++t) {
    int64_t slot = J->slots[t];
    if (slot < 0) continue;
    if (slot >= J->num_slots) { J->err |= ORACLE_SLOT_OOB; continue; }
    int64_t page = slot / J->ps, off = slot % J->ps;
    for (int h = 0; h < J->H; ++h) {
      int64_t row = (page * J->ps + off) * J->H + h;
      const uint16_t* kin = J->k + (t * J->H + h) * (int64_t)J->D;
      const uint16_t* vin = J->v + (t * J->H + h) * (int64_t)J->D;
      for (int b = 0; b < nb; ++b) {
        oracle_quantize_block(kin + 16 * b, J->gk, J->kc + row * (J->D / 2) + 8 * b,
                              J->ksf + row * nb + b);
        oracle_quantize_block(vin + 16 * b, J->gv, J->vc + row * (J->D / 2) + 8 * b,
                              J->vsf + row * nb + b);
      }
    }
  }
  return NULL;
}

uint32_t oracle_append(const uint16_t* k, const uint16_t* v, const int64_t* slots, int64_t T,
                       float k_scale, float v_scale, uint8_t* k_cache, uint8_t* v_cache,
                       uint8_t* k_sf, uint8_t* v_sf, int64_t num_pages, int page_size, int H_kv,
                       int head_dim, int nthreads) {
  if (T <= 0) return 0;
  uint32_t err = 0;
  if (!oracle_scale_ok(k_scale)) err |= ORACLE_BAD_K_SCALE;
  if (!oracle_scale_ok(v_scale)) err |= ORACLE_BAD_V_SCALE;
  if (err) return err;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  append_job jobs[256];
  pthread_t th[256];
  int64_t per = (T + nthreads - 1) / nthreads;
  for (int i = 0; i < nthreads; ++i) {
    append_job J = {k, v, slots, i * per, (i + 1) * per < T ? (i + 1) * per : T, k_scale, v_scale,
                    k_cache, v_cache, k_sf, v_sf, num_pages * page_size, page_size, H_kv,
                    head_dim, 0};
    if (J.t0 > T) J.t0 = T;
    jobs[i] = J;
    pthread_create(&th[i], NULL, append_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) {
    pthread_join(th[i], NULL);
    err |= jobs[i].err;
  }
  return err;
}

/* Dequantized value of element d of cache row `row` (fp64, exact):
 * e2m1(code) * S(sf) * g. */
static double dequant_elem(const uint8_t* cache, const uint8_t* sf, int64_t row, int D, int d,
                           double g) {
  uint8_t byte = cache[row * (D / 2) + d / 2];
  int code = (d & 1) ? (byte >> 4) : (byte & 15);
  return oracle_e2m1_value(code) * oracle_e4m3_value(sf[row * (D / 16) + d / 16]) * g;
}

/* Dequantize `n` cache rows (row index = (page*page_size + off)*H_kv + h)
 * into out[n][D] (fp64). */
void oracle_dequant_rows(const uint8_t* cache, const uint8_t* sf, const int64_t* rows, int64_t n,
                         int head_dim, double g, double* out) {
  for (int64_t i = 0; i < n; ++i)
    for (int d = 0; d < head_dim; ++d)
      out[i * head_dim + d] = dequant_elem(cache, sf, rows[i], head_dim, d, g);
}

/* ------------------------------------------------------------------ */
/* Causal paged prefill, the plain definition (fp64).                   */
/* Request r: Lq = qo_indptr[r+1]-qo_indptr[r], Lk = kv_lens[r], Lq<=Lk. */
/* Query row i sits at absolute position Lk-Lq+i (bottom-right causal   */
/* alignment, the chunked-prefill reading) and sees keys 0..Lk-Lq+i.    */
/* Q head hq reads KV head hq / (H_q/H_kv) (contiguous GQA groups).     */
/* Key j of request r lives in page page_table[kv_indptr[r] + j/ps] at   */
/* offset j % ps.                                                        */
/*   s_j = sm_scale * sum_d q[d] khat[j][d]                              */
/*   p_j = exp(s_j - max s) / sum_j' exp(s_j' - max s)                   */
/*   o   = sum_j p_j vhat[j]                                              */
/* ------------------------------------------------------------------ */
typedef struct {
  const uint16_t* q;
  const int32_t *qo, *kvp, *pt, *kvl;
  const uint8_t *kc, *vc, *ksf, *vsf;
  int64_t num_pages;
  int ps, Hq, Hk, D;
  double gk, gv, sm;
  const int32_t* reqs;
  int nreq;
  double* out;
  int next; /* work counter: (request index, kv head) pairs */
  pthread_mutex_t mu;
  uint32_t err;
} prefill_ctx;

static void* prefill_worker(void* arg) {
  prefill_ctx* C = (prefill_ctx*)arg;
  const int D = C->D, G = C->Hq / C->Hk;
  double* kh = NULL; double* vh = NULL; double* s = NULL;
  int64_t cap = 0;
  for (;;) {
    pthread_mutex_lock(&C->mu);
    int w = C->next++;
    pthread_mutex_unlock(&C->mu);
    if (w >= C->nreq * C->Hk) break;
    int r = C->reqs[w / C->Hk], hk = w % C->Hk;
    int Lq = C->qo[r + 1] - C->qo[r], Lk = C->kvl[r];
    if (Lq > Lk || Lq < 0) { pthread_mutex_lock(&C->mu); C->err |= 16; pthread_mutex_unlock(&C->mu); continue; }
    if (Lk > cap) {
      cap = Lk;
      kh = realloc(kh, sizeof(double) * cap * D);
      vh = realloc(vh, sizeof(double) * cap * D);
      s = realloc(s, sizeof(double) * cap);
    }
    int bad = 0;
    for (int j = 0; j < Lk; ++j) {
      int32_t page = C->pt[C->kvp[r] + j / C->ps];
      if (page < 0 || page >= C->num_pages) { bad = 1; break; }
      int64_t row = ((int64_t)page * C->ps + j % C->ps) * C->Hk + hk;
      for (int d = 0; d < D; ++d) {
        kh[(int64_t)j * D + d] = dequant_elem(C->kc, C->ksf, row, D, d, C->gk);
        vh[(int64_t)j * D + d] = dequant_elem(C->vc, C->vsf, row, D, d, C->gv);
      }
    }
    if (bad) { pthread_mutex_lock(&C->mu); C->err |= ORACLE_PAGE_OOB; pthread_mutex_unlock(&C->mu); continue; }
    for (int g = 0; g < G; ++g) {
      int hq = hk * G + g;
      for (int i = 0; i < Lq; ++i) {
        const uint16_t* qrow = C->q + ((int64_t)(C->qo[r] + i) * C->Hq + hq) * D;
        double qd[512];
        for (int d = 0; d < D; ++d) qd[d] = (double)bf16_bits_to_float(qrow[d]);
        int n = Lk - Lq + i + 1;
        double mx = -INFINITY;
        for (int j = 0; j < n; ++j) {
          double acc = 0.0;
          for (int d = 0; d < D; ++d) acc += qd[d] * kh[(int64_t)j * D + d];
          s[j] = C->sm * acc;
          if (s[j] > mx) mx = s[j];
        }
        double den = 0.0;
        for (int j = 0; j < n; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
        double* o = C->out + ((int64_t)(C->qo[r] + i) * C->Hq + hq) * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int j = 0; j < n; ++j) {
          double p = s[j] / den;
          for (int d = 0; d < D; ++d) o[d] += p * vh[(int64_t)j * D + d];
        }
      }
    }
  }
  free(kh); free(vh); free(s);
  return NULL;
}

/* requests == NULL: every request.  Output rows of requests not computed
 * are left untouched.  Returns 0, or error bits (16: q_len > kv_len,
 * ORACLE_PAGE_OOB: a page id outside the pool). */
uint32_t oracle_prefill(const uint16_t* q, const int32_t* qo_indptr, const int32_t* kv_indptr,
                        const int32_t* page_table, const int32_t* kv_lens, int batch,
                        const uint8_t* k_cache, const uint8_t* v_cache, const uint8_t* k_sf,
                        const uint8_t* v_sf, int64_t num_pages, int page_size, float k_scale,
                        float v_scale, int H_q, int H_kv, int head_dim, double sm_scale,
                        const int32_t* requests, int n_requests, double* out, int nthreads) {
  if (head_dim > 512 || head_dim % 16 || H_kv <= 0 || H_q % H_kv) return 32;
  int32_t* all = NULL;
  if (!requests) {
    all = malloc(sizeof(int32_t) * (batch > 0 ? batch : 1));
    for (int i = 0; i < batch; ++i) all[i] = i;
    requests = all;
    n_requests = batch;
  }
  prefill_ctx C = {q, qo_indptr, kv_indptr, page_table, kv_lens, k_cache, v_cache, k_sf, v_sf,
                   num_pages, page_size, H_q, H_kv, head_dim, (double)k_scale, (double)v_scale,
                   sm_scale, requests, n_requests, out, 0, PTHREAD_MUTEX_INITIALIZER, 0};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, prefill_worker, &C);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(all);
  return C.err;
}
