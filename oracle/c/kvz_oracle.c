/*
 * CPU oracle of the lossless BF16 KV-cache format and of fp64 decode attention, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
 * load this library; the HIP library never does. It shares no header, constant or helper
 * with the HIP path and restates the layout from its definition:
 *
 *  - BF16 = 1 sign, 8 exponent, 7 fraction bits; lossless means every bit pattern comes back
 *    (ZipFusion summary, §II.A "KV Cache and BF16"; §III.B "Lossless KV Cache Format").
 *  - group = 64 values of one token row of one head; sm byte = (sign << 7) | mantissa;
 *    base = the group exponent with the most exponents in [base, base + 14], smallest on
 *    ties; offset = e - base in 0..14, or 15 = escape with the raw value in the block's
 *    escape list, in storage order.
 *  - storage order inside a 16-token tile: K token-major (tok*D + d), V dim-major (d*16 + tok);
 *    a tile is 16*D sm bytes then 2*D u32 offset words, word w holding position 8w+2k in bits
 *    4k..4k+3 and 8w+2k+1 in bits 16+4k..16+4k+3.
 *  - unit (page, head) = meta region (K bases, V bases in [tile][group][tok] order, u32 K
 *    escape count, u32 V escape count, u64 pool offset or all ones when inline, then, when
 *    inline, one u32 per escape = value | (storage position in its block << 16); rounded up to
 *    128 bytes), then the K block, then the V block.
 *  - attention: s_t = scale * q.k_t; o = sum_t exp(s_t - max) v_t / sum_t exp(s_t - max), over
 *    the full pages of the page table then the uncompressed tail rows (§III.D: partially filled
 *    pages stay uncompressed); query head h reads KV head h / (Hq / Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GRP 64
#define TILE_T 16
#define ESC_CODE 15
#define ALL_ONES 0xFFFFFFFFFFFFFFFFull

static int expo(uint16_t x) { return (x >> 7) & 0xFF; }
static uint8_t smb(uint16_t x) { return (uint8_t)(((x >> 8) & 0x80) | (x & 0x7F)); }
static uint16_t rebuild(uint8_t sm, int e) {
  return (uint16_t)(((sm & 0x80) << 8) | ((e & 0xFF) << 7) | (sm & 0x7F));
}

size_t kvzo_meta_bytes(int P, int D) {
  size_t used = 2 * (size_t)P * (D / GRP) + 16;
  return (used + 127) / 128 * 128;
}
size_t kvzo_block_bytes(int P, int D) { return (size_t)P * D + (size_t)P * D / 2; }
size_t kvzo_unit_bytes(int P, int D) { return kvzo_meta_bytes(P, D) + 2 * kvzo_block_bytes(P, D); }
int kvzo_inline_capacity(int P, int D) {
  return (int)((kvzo_meta_bytes(P, D) - 2 * (size_t)P * (D / GRP) - 16) / 4);
}

/* base of one group of 64 exponents: largest coverage, smallest exponent on ties */
int kvzo_group_base(const int* e) {
  int best_b = 256, best_c = -1;
  for (int i = 0; i < GRP; i++) {
    int c = 0;
    for (int j = 0; j < GRP; j++) {
      int d = e[j] - e[i];
      if (d >= 0 && d <= 14) c++;
    }
    if (c > best_c || (c == best_c && e[i] < best_b)) { best_c = c; best_b = e[i]; }
  }
  return best_b;
}

/* token-major flat index (tok*D + d) of storage position s of a block */
static int pos_to_index(int s, int D, int is_v) {
  int t = s / (TILE_T * D), r = s % (TILE_T * D);
  int tok, d;
  if (!is_v) { tok = r / D; d = r % D; } else { d = r / TILE_T; tok = r % TILE_T; }
  return (t * TILE_T + tok) * D + d;
}

/* one block: writes bases (P*G bytes), payload, escapes; returns the escape count */
static int encode_block(const uint16_t* X, int P, int D, int is_v, uint8_t* bases,
                        uint8_t* payload, uint16_t* esc, uint32_t* pos) {
  int G = D / GRP, n = 0;
  int* base = (int*)malloc(sizeof(int) * P * G);
  int e[GRP];
  for (int tok = 0; tok < P; tok++)
    for (int g = 0; g < G; g++) {
      for (int j = 0; j < GRP; j++) e[j] = expo(X[tok * D + g * GRP + j]);
      base[tok * G + g] = kvzo_group_base(e);
    }
  for (int tok = 0; tok < P; tok++)
    for (int g = 0; g < G; g++)
      bases[(tok / TILE_T) * TILE_T * G + g * TILE_T + tok % TILE_T] = (uint8_t)base[tok * G + g];
  size_t per_tile = (size_t)TILE_T * D;
  for (int s = 0; s < P * D; s++) {
    int idx = pos_to_index(s, D, is_v);
    int tok = idx / D, d = idx % D;
    uint16_t x = X[idx];
    int off = expo(x) - base[tok * G + d / GRP];
    if (off < 0 || off > 14) { off = ESC_CODE; pos[n] = (uint32_t)s; esc[n++] = x; }
    size_t t = s / per_tile, r = s % per_tile;
    uint8_t* tile = payload + t * (per_tile + per_tile / 2);
    tile[r] = smb(x);
    uint8_t* words = tile + per_tile;
    size_t w = r / 8, k = r % 8;
    int bit = (k % 2 == 0) ? 4 * (int)(k / 2) : 16 + 4 * (int)(k / 2);
    uint32_t word;
    memcpy(&word, words + 4 * w, 4);
    word = (word & ~(0xFu << bit)) | ((uint32_t)off << bit);
    memcpy(words + 4 * w, &word, 4);
  }
  free(base);
  return n;
}

static void decode_block(const uint8_t* bases, const uint8_t* payload, const uint16_t* esc, int P,
                         int D, int is_v, uint16_t* X) {
  int G = D / GRP, n = 0;
  size_t per_tile = (size_t)TILE_T * D;
  for (int s = 0; s < P * D; s++) {
    int idx = pos_to_index(s, D, is_v);
    int tok = idx / D, d = idx % D;
    size_t t = s / per_tile, r = s % per_tile;
    const uint8_t* tile = payload + t * (per_tile + per_tile / 2);
    uint32_t word;
    memcpy(&word, tile + per_tile + 4 * (r / 8), 4);
    size_t k = r % 8;
    int bit = (k % 2 == 0) ? 4 * (int)(k / 2) : 16 + 4 * (int)(k / 2);
    int off = (word >> bit) & 0xF;
    int b = bases[(tok / TILE_T) * TILE_T * G + (d / GRP) * TILE_T + tok % TILE_T];
    X[idx] = (off == ESC_CODE) ? esc[n++] : rebuild(tile[r], b + off);
  }
}

/* One unit. Returns how many escapes go to the pool (0 when they fit inline); those are
   written to pool_esc (room for 2*P*D). */
int64_t kvzo_encode_unit(const uint16_t* K, const uint16_t* V, int P, int D, uint64_t pool_offset,
                         uint8_t* unit, uint16_t* pool_esc) {
  int G = D / GRP;
  size_t mb = kvzo_meta_bytes(P, D), bb = kvzo_block_bytes(P, D);
  uint16_t* esc = (uint16_t*)malloc(sizeof(uint16_t) * 2 * (size_t)P * D);
  uint32_t* pos = (uint32_t*)malloc(sizeof(uint32_t) * 2 * (size_t)P * D);
  memset(unit, 0, kvzo_unit_bytes(P, D));
  int kc = encode_block(K, P, D, 0, unit, unit + mb, esc, pos);
  int vc = encode_block(V, P, D, 1, unit + (size_t)P * G, unit + mb + bb, esc + kc, pos + kc);
  uint8_t* h = unit + 2 * (size_t)P * G;
  uint32_t c[2] = {(uint32_t)kc, (uint32_t)vc};
  memcpy(h, c, 8);
  int64_t ret = 0;
  if (kc + vc <= kvzo_inline_capacity(P, D)) {
    uint64_t o = ALL_ONES;
    memcpy(h + 8, &o, 8);
    for (int i = 0; i < kc + vc; i++) {
      uint32_t e = (uint32_t)esc[i] | (pos[i] << 16);
      memcpy(h + 16 + 4 * (size_t)i, &e, 4);
    }
  } else {
    memcpy(h + 8, &pool_offset, 8);
    memcpy(pool_esc, esc, 2 * (size_t)(kc + vc));
    ret = kc + vc;
  }
  free(esc);
  free(pos);
  return ret;
}

/* Encodes pages [n][H][P][D] into units [n][H][U]; pool escapes are placed in unit order from
   pool_start. Returns the new pool end, or -1 when the pool capacity would be exceeded. */
int64_t kvzo_encode_pages(const uint16_t* K, const uint16_t* V, int64_t n, int H, int P, int D,
                          uint8_t* units, uint16_t* pool, int64_t pool_start, int64_t pool_cap) {
  size_t U = kvzo_unit_bytes(P, D), blk = (size_t)P * D;
  int64_t m = n * H;
  int64_t* cnt = (int64_t*)calloc(m, sizeof(int64_t));
  uint16_t** tmp = (uint16_t**)calloc(m, sizeof(uint16_t*));
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < m; i++) {
    tmp[i] = (uint16_t*)malloc(sizeof(uint16_t) * 2 * blk);
    cnt[i] = kvzo_encode_unit(K + i * blk, V + i * blk, P, D, 0, units + i * U, tmp[i]);
  }
  int64_t cur = pool_start, ok = 1;
  for (int64_t i = 0; i < m; i++) {
    if (cnt[i] > 0) {
      if (cur + cnt[i] > pool_cap) { ok = 0; break; }
      uint64_t o = (uint64_t)cur;
      memcpy(units + i * U + 2 * (size_t)P * (D / GRP) + 8, &o, 8);
      memcpy(pool + cur, tmp[i], 2 * (size_t)cnt[i]);
      cur += cnt[i];
    }
  }
  for (int64_t i = 0; i < m; i++) free(tmp[i]);
  free(tmp);
  free(cnt);
  return ok ? cur : -1;
}

void kvzo_decode_unit(const uint8_t* unit, const uint16_t* pool, int P, int D, uint16_t* K,
                      uint16_t* V) {
  int G = D / GRP;
  size_t mb = kvzo_meta_bytes(P, D), bb = kvzo_block_bytes(P, D);
  const uint8_t* h = unit + 2 * (size_t)P * G;
  uint32_t c[2];
  uint64_t off;
  memcpy(c, h, 8);
  memcpy(&off, h + 8, 8);
  uint16_t* esc = (uint16_t*)malloc(sizeof(uint16_t) * (c[0] + c[1] + 1));
  if (off == ALL_ONES) {
    for (uint32_t i = 0; i < c[0] + c[1]; i++) {
      uint32_t e;
      memcpy(&e, h + 16 + 4 * (size_t)i, 4);
      esc[i] = (uint16_t)(e & 0xFFFF);
    }
  } else {
    memcpy(esc, pool + off, 2 * (size_t)(c[0] + c[1]));
  }
  decode_block(unit, unit + mb, esc, P, D, 0, K);
  decode_block(unit + (size_t)P * G, unit + mb + bb, esc + c[0], P, D, 1, V);
  free(esc);
}

void kvzo_decode_pages(const uint8_t* units, const uint16_t* pool, const int32_t* ids, int64_t n,
                       int H, int P, int D, uint16_t* K, uint16_t* V) {
  size_t U = kvzo_unit_bytes(P, D), blk = (size_t)P * D;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < n * H; i++) {
    int64_t p = ids[i / H], h = i % H;
    kvzo_decode_unit(units + (p * H + h) * U, pool, P, D, K + i * blk, V + i * blk);
  }
}

static double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* fp64 attention of one query row over L rows of K/V (row stride D) */
static void attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int L, int D,
                   double scale, double* out) {
  for (int d = 0; d < D; d++) out[d] = 0.0;
  if (L == 0) return;
  double* s = (double*)malloc(sizeof(double) * L);
  double mx = -INFINITY;
  for (int t = 0; t < L; t++) {
    double a = 0.0;
    for (int d = 0; d < D; d++) a += bf(q[d]) * bf(K[(size_t)t * D + d]);
    s[t] = scale * a;
    if (s[t] > mx) mx = s[t];
  }
  double den = 0.0;
  for (int t = 0; t < L; t++) {
    double w = exp(s[t] - mx);
    den += w;
    for (int d = 0; d < D; d++) out[d] += w * bf(V[(size_t)t * D + d]);
  }
  for (int d = 0; d < D; d++) out[d] /= den;
  free(s);
}

/* rows of one (request, KV head) from compressed units and the tail -> K, V [L][D] */
static void gather_compressed(const uint8_t* units, const uint16_t* pool, const int32_t* ids,
                              const uint16_t* tk, const uint16_t* tv, int L, int H, int h, int P,
                              int D, uint16_t* K, uint16_t* V) {
  size_t U = kvzo_unit_bytes(P, D), blk = (size_t)P * D;
  uint16_t* k = (uint16_t*)malloc(2 * blk);
  uint16_t* v = (uint16_t*)malloc(2 * blk);
  int full = L / P;
  for (int i = 0; i < full; i++) {
    kvzo_decode_unit(units + ((size_t)ids[i] * H + h) * U, pool, P, D, k, v);
    memcpy(K + (size_t)i * blk, k, 2 * blk);
    memcpy(V + (size_t)i * blk, v, 2 * blk);
  }
  int rest = L - full * P;
  memcpy(K + (size_t)full * blk, tk, 2 * (size_t)rest * D);
  memcpy(V + (size_t)full * blk, tv, 2 * (size_t)rest * D);
  free(k);
  free(v);
}

/* out[i][D] for the (request, query head) pairs rows[2i], rows[2i+1] */
void kvzo_decode_attention_rows(const uint16_t* q, const uint8_t* units, const uint16_t* pool,
                                const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                const uint16_t* tail_k, const uint16_t* tail_v, int Hq, int Hkv,
                                int D, int P, double scale, const int32_t* rows, int nrows,
                                double* out) {
  int grp = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < nrows; i++) {
    int r = rows[2 * i], hq = rows[2 * i + 1], h = hq / grp, L = seq_lens[r];
    uint16_t* K = (uint16_t*)malloc(2 * (size_t)(L + 1) * D);
    uint16_t* V = (uint16_t*)malloc(2 * (size_t)(L + 1) * D);
    size_t toff = ((size_t)r * Hkv + h) * P * D;
    gather_compressed(units, pool, page_table + (size_t)r * max_pages, tail_k + toff, tail_v + toff,
                      L, Hkv, h, P, D, K, V);
    attend(q + ((size_t)r * Hq + hq) * D, K, V, L, D, scale, out + (size_t)i * D);
    free(K);
    free(V);
  }
}

/* Same over dense pages [num_pages][Hkv][P][D]; the request's first ceil(L/P) pages. */
void kvzo_dense_attention_rows(const uint16_t* q, const uint16_t* k_pages, const uint16_t* v_pages,
                               const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                               int Hq, int Hkv, int D, int P, double scale, const int32_t* rows,
                               int nrows, double* out) {
  int grp = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < nrows; i++) {
    int r = rows[2 * i], hq = rows[2 * i + 1], h = hq / grp, L = seq_lens[r];
    uint16_t* K = (uint16_t*)malloc(2 * (size_t)(L + 1) * D);
    uint16_t* V = (uint16_t*)malloc(2 * (size_t)(L + 1) * D);
    for (int t = 0; t < L; t++) {
      size_t pid = (size_t)page_table[(size_t)r * max_pages + t / P];
      size_t src = ((pid * Hkv + h) * P + t % P) * D;
      memcpy(K + (size_t)t * D, k_pages + src, 2 * (size_t)D);
      memcpy(V + (size_t)t * D, v_pages + src, 2 * (size_t)D);
    }
    attend(q + ((size_t)r * Hq + hq) * D, K, V, L, D, scale, out + (size_t)i * D);
    free(K);
    free(V);
  }
}

/* threads the parallel loops use from now on (n <= 0: the OpenMP default) */
void kvzo_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int kvzo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
