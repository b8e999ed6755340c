/*
 * A decode loop through the C ABI of libkvz alone: no Python and no torch. Device memory comes
 * from hipMalloc and every call goes to one HIP stream, as a serving engine written in C or C++
 * would drive the library. For a multi-head and a grouped-query shape it
 *   - compresses the full pages of every request (kvz_compress_pages),
 *   - runs decode steps that append one token per request (kvz_append_token, crossing page fills)
 *     and attend over the compressed cache (kvz_decode_attention), checking every step's BF16
 *     and fp32 outputs against the fp64 oracle (libkvz_oracle, test infrastructure) at the
 *     library's tolerances: |out - o| <= max(2e-2, 2^-7 |o|), max_d |out32 - o| <= 1e-4 max_d |o|;
 *   - on the last step, runs the uncompressed baseline (kvz_decode_attention_dense) and the
 *     allocation-free call (kvz_decode_attention_noalloc, which must match bit for bit);
 *   - rebuilds every full page through the kernels' decode routes (kvz_decompress_pages) and
 *     compares them with the source bits.
 * Prints one line per shape and exits 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvz.h"

/* the fp64 oracle over dense pages (oracle/c/kvz_oracle.c) */
void kvzo_dense_attention_rows(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages,
                               const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                               int Hq, int Hkv, int D, int P, double scale, const int32_t* rows,
                               int nrows, double* out);

#define CHECK_HIP(x)                                                                  \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));      \
      exit(2);                                                                        \
    }                                                                                 \
  } while (0)
#define CHECK_KVZ(x)                                                                  \
  do {                                                                                \
    int r_ = (x);                                                                     \
    if (r_ != KVZ_OK) {                                                               \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #x, kvz_strerror(r_)); \
      exit(3);                                                                        \
    }                                                                                 \
  } while (0)

/* ---- inputs: xorshift64*, Box-Muller, round to BF16 (nearest even) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rng_next(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
static double rng_uniform(void) { return ((rng_next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
static double rng_normal(void) {
  return sqrt(-2.0 * log(rng_uniform())) * cos(6.283185307179586 * rng_uniform());
}
static uint16_t bf16_of(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static double f64_of_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void* dalloc(size_t n) {
  void* p = NULL;
  CHECK_HIP(hipMalloc(&p, n ? n : 16));
  CHECK_HIP(hipMemset(p, 0, n ? n : 16));
  return p;
}
static void h2d(void* d, const void* h, size_t n) { CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice)); }
static void d2h(void* h, const void* d, size_t n) { CHECK_HIP(hipMemcpy(h, d, n, hipMemcpyDeviceToHost)); }

static int failures = 0;

/* out16 [n][D] BF16 and out32 [n][D] against ref [n][D] */
static void check_rows(const char* what, const uint16_t* out16, const float* out32, const double* ref, int n, int D) {
  double worst16 = 0, worst32 = 0;
  for (int i = 0; i < n; ++i) {
    double nrm = 0, e32 = 0;
    for (int d = 0; d < D; ++d) {
      const double o = ref[(size_t)i * D + d];
      const double e = fabs(f64_of_bf16(out16[(size_t)i * D + d]) - o);
      const double tol = fmax(2e-2, ldexp(fabs(o), -7));
      if (e > tol) ++failures;
      if (e / tol > worst16) worst16 = e / tol;
      nrm = fmax(nrm, fabs(o));
      if (out32) e32 = fmax(e32, fabs((double)out32[(size_t)i * D + d] - o));
    }
    if (out32) {
      if (e32 > 1e-4 * nrm) ++failures;
      if (nrm > 0 && e32 / nrm > worst32) worst32 = e32 / nrm;
    }
  }
  if (failures) fprintf(stderr, "%s: out of tolerance (worst bf16 error / tolerance %.3g)\n", what, worst16);
}

static void run_shape(int B, int Hq, int H, int steps) {
  const int D = 128, P = 16;
  const int L0[3] = {37, 100, 16};
  int Lmax = 0;
  for (int r = 0; r < B; ++r) Lmax = L0[r] + steps > Lmax ? L0[r] + steps : Lmax;
  const int max_pages = (Lmax + P - 1) / P;
  /* pages of every request up to its final length; physical ids shuffled */
  int npr[3], num_pages = 0;
  for (int r = 0; r < B; ++r) num_pages += npr[r] = (L0[r] + steps + P - 1) / P;
  int32_t* perm = malloc(sizeof(int32_t) * num_pages);
  for (int i = 0; i < num_pages; ++i) perm[i] = i;
  for (int i = num_pages - 1; i > 0; --i) {
    const int j = (int)(rng_next() % (uint64_t)(i + 1));
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  int32_t* table = malloc(sizeof(int32_t) * B * max_pages);
  for (int i = 0; i < B * max_pages; ++i) table[i] = -1;
  for (int r = 0, pos = 0; r < B; ++r)
    for (int i = 0; i < npr[r]; ++i) table[r * max_pages + i] = perm[pos++];
  /* K with four x20 channels per head (escapes), V plain; a few exact zeros */
  const size_t pv = (size_t)H * P * D, nvals = (size_t)num_pages * pv;
  uint16_t* kp = malloc(2 * nvals);
  uint16_t* vp = malloc(2 * nvals);
  for (size_t i = 0; i < nvals; ++i) {
    const int d = (int)(i % D), h = (int)(i / (P * D) % H);
    const float s = (d % 32 == (7 * h) % 32) ? 20.f : 1.f;
    kp[i] = bf16_of((float)rng_normal() * s);
    vp[i] = rng_uniform() < 0.01 ? 0 : bf16_of((float)rng_normal());
  }
  uint16_t* q = malloc(2 * (size_t)B * Hq * D);
  for (size_t i = 0; i < (size_t)B * Hq * D; ++i) q[i] = bf16_of((float)rng_normal());
  const float scale = 1.0f / sqrtf((float)D);

  /* device cache */
  const size_t U = kvz_unit_bytes(P, D);
  kvz_cache c;
  memset(&c, 0, sizeof c);
  c.page_size = P;
  c.num_kv_heads = H;
  c.head_dim = D;
  c.num_pages = num_pages;
  c.max_batch = B;
  c.format = KVZ_FORMAT_ESCAPE;
  c.units = dalloc((size_t)num_pages * H * U);
  c.esc_capacity = (int64_t)nvals;   /* room for every value */
  c.esc_pool = dalloc(2 * (size_t)c.esc_capacity);
  c.esc_cursor = dalloc(8);
  c.k_tail = dalloc(2 * (size_t)B * pv);
  c.v_tail = dalloc(2 * (size_t)B * pv);
  c.status = dalloc(4);
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  /* full pages of the initial lengths, compressed into their slots; partial pages into the tails */
  int nfull = 0;
  for (int r = 0; r < B; ++r) nfull += L0[r] / P;
  int32_t* ids = malloc(sizeof(int32_t) * (nfull ? nfull : 1));
  uint16_t* ksrc = malloc(2 * (size_t)(nfull ? nfull : 1) * pv);
  uint16_t* vsrc = malloc(2 * (size_t)(nfull ? nfull : 1) * pv);
  for (int r = 0, n = 0; r < B; ++r)
    for (int i = 0; i < L0[r] / P; ++i, ++n) {
      ids[n] = table[r * max_pages + i];
      memcpy(ksrc + n * pv, kp + (size_t)ids[n] * pv, 2 * pv);
      memcpy(vsrc + n * pv, vp + (size_t)ids[n] * pv, 2 * pv);
    }
  int32_t* d_ids = dalloc(4 * (size_t)nfull);
  uint16_t* d_ksrc = dalloc(2 * (size_t)nfull * pv);
  uint16_t* d_vsrc = dalloc(2 * (size_t)nfull * pv);
  h2d(d_ids, ids, 4 * (size_t)nfull);
  h2d(d_ksrc, ksrc, 2 * (size_t)nfull * pv);
  h2d(d_vsrc, vsrc, 2 * (size_t)nfull * pv);
  CHECK_KVZ(kvz_compress_pages(&c, d_ksrc, d_vsrc, d_ids, nfull, stream));
  uint16_t* tk = calloc((size_t)B * pv, 2);
  uint16_t* tv = calloc((size_t)B * pv, 2);
  for (int r = 0; r < B; ++r)
    if (L0[r] % P) {
      const size_t src = (size_t)table[r * max_pages + L0[r] / P] * pv;
      memcpy(tk + (size_t)r * pv, kp + src, 2 * pv);
      memcpy(tv + (size_t)r * pv, vp + src, 2 * pv);
    }
  CHECK_HIP(hipStreamSynchronize(stream));
  h2d(c.k_tail, tk, 2 * (size_t)B * pv);
  h2d(c.v_tail, tv, 2 * (size_t)B * pv);

  int32_t lens[3];
  for (int r = 0; r < B; ++r) lens[r] = L0[r];
  int32_t* d_lens = dalloc(4 * (size_t)B);
  int32_t* d_table = dalloc(4 * (size_t)B * max_pages);
  uint16_t* d_q = dalloc(2 * (size_t)B * Hq * D);
  uint16_t* d_new_k = dalloc(2 * (size_t)B * H * D);
  uint16_t* d_new_v = dalloc(2 * (size_t)B * H * D);
  uint16_t* d_out = dalloc(2 * (size_t)B * Hq * D);
  float* d_out32 = dalloc(4 * (size_t)B * Hq * D);
  h2d(d_lens, lens, 4 * (size_t)B);
  h2d(d_table, table, 4 * (size_t)B * max_pages);
  h2d(d_q, q, 2 * (size_t)B * Hq * D);
  const size_t ws_bytes = kvz_workspace_bytes(B, Hq, H, D, P, max_pages, 0);
  void* d_ws = dalloc(ws_bytes);

  uint16_t* new_k = malloc(2 * (size_t)B * H * D);
  uint16_t* new_v = malloc(2 * (size_t)B * H * D);
  uint16_t* out16 = malloc(2 * (size_t)B * Hq * D);
  float* out32 = malloc(4 * (size_t)B * Hq * D);
  int32_t* rows = malloc(sizeof(int32_t) * 2 * B * Hq);
  for (int r = 0; r < B; ++r)
    for (int h = 0; h < Hq; ++h) {
      rows[2 * (r * Hq + h)] = r;
      rows[2 * (r * Hq + h) + 1] = h;
    }
  double* ref = malloc(sizeof(double) * (size_t)B * Hq * D);
  for (int s = 0; s < steps; ++s) {
    /* the token at position lens[r] of every request, from its page */
    for (int r = 0; r < B; ++r) {
      const size_t page = (size_t)table[r * max_pages + lens[r] / P];
      for (int h = 0; h < H; ++h) {
        const size_t src = ((page * H + h) * P + lens[r] % P) * D;
        memcpy(new_k + ((size_t)r * H + h) * D, kp + src, 2 * (size_t)D);
        memcpy(new_v + ((size_t)r * H + h) * D, vp + src, 2 * (size_t)D);
      }
    }
    h2d(d_new_k, new_k, 2 * (size_t)B * H * D);
    h2d(d_new_v, new_v, 2 * (size_t)B * H * D);
    CHECK_KVZ(kvz_append_token(&c, d_new_k, d_new_v, d_table, max_pages, d_lens, B, stream));
    CHECK_KVZ(kvz_decode_attention(d_q, &c, d_table, max_pages, d_lens, B, Hq, scale, 0, d_out, d_out32, d_ws, ws_bytes,
                                   stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    for (int r = 0; r < B; ++r) ++lens[r];
    d2h(out16, d_out, 2 * (size_t)B * Hq * D);
    d2h(out32, d_out32, 4 * (size_t)B * Hq * D);
    kvzo_dense_attention_rows(q, kp, vp, table, max_pages, lens, Hq, H, D, P, scale, rows, B * Hq, ref);
    check_rows("decode step", out16, out32, ref, B * Hq, D);
  }
  int32_t dev_lens[3];
  d2h(dev_lens, d_lens, 4 * (size_t)B);
  for (int r = 0; r < B; ++r)
    if (dev_lens[r] != lens[r]) ++failures;

  /* the allocation-free call: the same bits as the workspace call */
  uint16_t* d_out_na = dalloc(2 * (size_t)B * Hq * D);
  float* d_out32_na = dalloc(4 * (size_t)B * Hq * D);
  CHECK_KVZ(kvz_decode_attention_noalloc(d_q, &c, d_table, max_pages, d_lens, B, Hq, scale, 0, d_out_na, d_out32_na,
                                         stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  uint16_t* na16 = malloc(2 * (size_t)B * Hq * D);
  float* na32 = malloc(4 * (size_t)B * Hq * D);
  d2h(na16, d_out_na, 2 * (size_t)B * Hq * D);
  d2h(na32, d_out32_na, 4 * (size_t)B * Hq * D);
  if (memcmp(na16, out16, 2 * (size_t)B * Hq * D) || memcmp(na32, out32, 4 * (size_t)B * Hq * D)) {
    fprintf(stderr, "allocation-free call differs from the workspace call\n");
    ++failures;
  }

  /* the uncompressed baseline over the same tokens */
  uint16_t* d_kp = dalloc(2 * nvals);
  uint16_t* d_vp = dalloc(2 * nvals);
  h2d(d_kp, kp, 2 * nvals);
  h2d(d_vp, vp, 2 * nvals);
  uint32_t* d_dstatus = dalloc(4);
  CHECK_KVZ(kvz_decode_attention_dense(d_q, d_kp, d_vp, num_pages, H, D, P, d_table, max_pages, d_lens, B, Hq, scale, 0,
                                       d_out, d_out32, d_ws, ws_bytes, d_dstatus, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  d2h(out16, d_out, 2 * (size_t)B * Hq * D);
  d2h(out32, d_out32, 4 * (size_t)B * Hq * D);
  check_rows("uncompressed baseline", out16, out32, ref, B * Hq, D);

  /* every full page rebuilt bit for bit on every decode route */
  int nf = 0;
  for (int r = 0; r < B; ++r) nf += lens[r] / P;
  int32_t* fids = malloc(sizeof(int32_t) * nf);
  for (int r = 0, n = 0; r < B; ++r)
    for (int i = 0; i < lens[r] / P; ++i) fids[n++] = table[r * max_pages + i];
  int32_t* d_fids = dalloc(4 * (size_t)nf);
  h2d(d_fids, fids, 4 * (size_t)nf);
  uint16_t* d_kd = dalloc(2 * (size_t)nf * pv);
  uint16_t* d_vd = dalloc(2 * (size_t)nf * pv);
  uint16_t* kd = malloc(2 * (size_t)nf * pv);
  uint16_t* vd = malloc(2 * (size_t)nf * pv);
  for (int lane_map = 0; lane_map < 4; ++lane_map) {
    CHECK_KVZ(kvz_decompress_pages(&c, d_fids, nf, lane_map, d_kd, d_vd, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    d2h(kd, d_kd, 2 * (size_t)nf * pv);
    d2h(vd, d_vd, 2 * (size_t)nf * pv);
    for (int n = 0; n < nf; ++n)
      if (memcmp(kd + n * pv, kp + (size_t)fids[n] * pv, 2 * pv) || memcmp(vd + n * pv, vp + (size_t)fids[n] * pv, 2 * pv)) {
        fprintf(stderr, "page %d not rebuilt bit for bit on lane map %d\n", fids[n], lane_map);
        ++failures;
        break;
      }
  }
  uint32_t status = 0, dstatus = 0;
  d2h(&status, c.status, 4);
  d2h(&dstatus, d_dstatus, 4);
  if (status || dstatus) {
    fprintf(stderr, "status bits %u / %u\n", status, dstatus);
    ++failures;
  }
  uint64_t cursor = 0;
  d2h(&cursor, c.esc_cursor, 8);
  printf("%d requests, %d/%d heads, %d decode steps, %d full pages, %llu pool escapes: %s\n", B, Hq, H, steps, nf,
         (unsigned long long)cursor, failures ? "FAILED" : "ok");
  fflush(stdout);

  CHECK_HIP(hipStreamDestroy(stream));
  void* dev_bufs[] = {c.units, c.esc_pool, c.esc_cursor, c.k_tail, c.v_tail, c.status, d_ids, d_ksrc, d_vsrc,
                      d_lens, d_table, d_q, d_new_k, d_new_v, d_out, d_out32, d_ws, d_out_na, d_out32_na,
                      d_kp, d_vp, d_dstatus, d_fids, d_kd, d_vd};
  for (size_t i = 0; i < sizeof dev_bufs / sizeof dev_bufs[0]; ++i) CHECK_HIP(hipFree(dev_bufs[i]));
  void* host_bufs[] = {perm, table, kp, vp, q, ids, ksrc, vsrc, tk, tv, new_k, new_v, out16, out32, rows, ref,
                       na16, na32, fids, kd, vd};
  for (size_t i = 0; i < sizeof host_bufs / sizeof host_bufs[0]; ++i) free(host_bufs[i]);
}

int main(void) {
  run_shape(3, 4, 4, 20);   /* multi-head */
  run_shape(3, 8, 2, 20);   /* grouped queries, 4 per KV head */
  return failures ? 1 : 0;
}
