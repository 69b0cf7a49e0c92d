/*
 * CPU oracle for low-bit MLA KV caching and decode: plain loops, fp64
 * attention. TEST INFRASTRUCTURE ONLY (see oracle.h): the product path never
 * uses this file.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no contraction and no fast-math, so every fp32 step of the quantizer is one
 * IEEE-754 operation rounded to nearest-even).
 *
 * Readings of the pages (QuantMLA, newx.sg summary page and thelatestinai.com
 * cards page) where they leave a step open:
 *  Q1 Quantizer: per token and per group of `group` contiguous channels
 *     (32 in the workloads; 64 and 128 as variants; a group never spans the
 *     content / RoPE boundary, and a vector narrower than the group, the
 *     64-channel RoPE key at group 128, is one group of its own width),
 *     asymmetric min-max round-to-nearest (the RTN baseline row of Table 1 is
 *     the plain quantizer; QuantMLA's learned transforms are fused into the
 *     weights offline per the abstract, so the runtime writer sees
 *     already-transformed values). lo = min, hi = max; scale = (hi-lo)/(2^b-1)
 *     in fp32, stored as fp16; zero = lo stored as fp16; dequant x = q*s + z.
 *  Q2 Rounding: fp32 subtraction and correctly rounded fp32 division, RNE
 *     rint, RNE fp32->fp16. Ties go to the even code.
 *  Q3 A group whose fp16 scale is zero gets all-zero codes.
 *  Q4 Code order (the pages give none; chosen so that one 128-bit load hands
 *     a GPU lane the same 8-channel sub-block of several blocks). It is
 *     defined on blocks of 32 channels, whatever the quantization group: a
 *     vector of n_g blocks at b bits is cut into chunks of u = min(n_g, 16/b)
 *     blocks; chunk (ld, j) lies at byte u*b*(4*ld + j) and holds sub-block j
 *     (channels 8j..8j+7 of each block) of blocks u*ld .. u*ld+u-1. Inside a
 *     chunk, block u*ld + gi sits in 32-bit little-endian word gi / (4/b),
 *     code block e = gi mod (4/b); channel 8j + 2i + k of the block sits at bit
 *     16k + b*(4e + i): even channels fill the low half-word, odd ones the high.
 *     With 32-channel groups a block is a group.
 *  Q5 Page layout: page_size token slots, four token-major regions: content
 *     codes, RoPE codes, content (scale, zero) fp16 pairs (one per content
 *     group), RoPE pairs (one per RoPE group).
 *  Q6 Protection (sink4/local128 of Figure 5 and Table 9; Figure 8): token p
 *     of a sequence of length L is read from the sink buffer if p < n_sink,
 *     else from the local ring (slot p mod n_local) if p >= L - n_local, else
 *     from its packed copy. The recent window includes the newest token.
 *  Q7 Every token gets a packed copy, protected ones included (Figure 8: a
 *     packed copy for every incoming token; a token leaving the window reuses
 *     it without re-quantization).
 *  Q8 Attention: score = scale * (q_lat . c + q_rope . k_rope), softmax over
 *     all valid tokens at once, out = sum_p P_p * c_p (the value is the
 *     content latent: absorbed form, GQLA card), lse = natural log of the sum
 *     of exp(score). Dequantized values are exact in fp64.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_check_cfg(const orc_cfg* c) {
  if (!c) return -1;
  if (c->c_bits != 2 && c->c_bits != 4) return -1;
  if (c->r_bits != 2 && c->r_bits != 4) return -1;
  if (c->group != 32 && c->group != 64 && c->group != 128) return -1;
  /* the code order works in 32-channel blocks of 8-channel sub-blocks */
  if (c->d_c <= 0 || c->d_c % 32 != 0 || c->d_c % c->group != 0) return -1;
  if (c->d_r <= 0 || c->d_r % 32 != 0) return -1;
  if (c->d_r % (c->group < c->d_r ? c->group : c->d_r) != 0) return -1;
  /* a chunk must hold at least one whole 32-bit word */
  if ((c->d_c / 32) * c->c_bits < 4 && c->c_bits == 2) return -1;
  if ((c->d_r / 32) * c->r_bits < 4 && c->r_bits == 2) return -1;
  if (c->page_size <= 0 || c->n_sink < 0 || c->n_local < 0) return -1;
  return 0;
}

/* ---------------- number formats (IEEE-754 binary16, bfloat16) ---------------- */

uint16_t orc_f32_to_f16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t exp = (u >> 23) & 0xffu;
  uint32_t man = u & 0x7fffffu;
  if (exp == 0xffu) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));
  if (exp >= 143u) return (uint16_t)(sign | 0x7c00u); /* >= 2^16: overflow */
  if (exp >= 113u) {
    /* normal binary16: exponent exp-112, keep 10 mantissa bits, RNE on 13 */
    uint32_t h = ((exp - 112u) << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++; /* carry may reach inf */
    return (uint16_t)(sign | h);
  }
  if (exp == 0u) return (uint16_t)sign; /* binary32 subnormal: far below 2^-25 */
  /* subnormal binary16: value / 2^-24 = (2^23 + man) * 2^(exp - 126) */
  uint32_t v = 0x800000u | man;
  int s = 126 - (int)exp; /* >= 14 */
  if (s >= 32) return (uint16_t)sign;
  uint32_t q = v >> s;
  uint32_t rem = v & ((1u << s) - 1u);
  uint32_t half = 1u << (s - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;
  return (uint16_t)(sign | q); /* q == 0x400 is the smallest normal */
}

double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (exp == 0)
    v = ldexp((double)man, -24);
  else if (exp == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + man), exp - 25);
  return sign ? -v : v;
}

float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t orc_f64_to_bf16(double x) {
  /* round fp64 to the nearest bf16: through the exact fp32 neighbours would
   * double-round, so round on the fp64 bits directly. */
  if (isnan(x)) return 0x7fc0;
  uint64_t u;
  memcpy(&u, &x, 8);
  uint64_t sign = (u >> 48) & 0x8000u;
  double a = fabs(x);
  if (a == 0.0) return (uint16_t)sign;
  int e;
  (void)frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  /* bf16: 8 significant bits for normals (exponent >= -126); subnormals have
   * spacing 2^-133 */
  int unb = e - 1; /* a = 1.f * 2^unb */
  double spacing = unb >= -126 ? ldexp(1.0, unb - 7) : ldexp(1.0, -133);
  double q = a / spacing; /* exact: power-of-two scaling */
  double fl = floor(q);
  double r = q - fl;
  if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  double y = fl * spacing;
  float f = (float)y; /* exact: y has at most 8 significant bits */
  if (y >= 3.4028236692093846e38) f = INFINITY;
  uint32_t fu;
  memcpy(&fu, &f, 4);
  return (uint16_t)(sign | ((fu >> 16) & 0x7fffu));
}

/* ---------------- quantizer (readings Q1-Q3) ---------------- */

void orc_quantize_group(const float* x, int n, int bits, uint16_t* s16, uint16_t* z16,
                        uint8_t* codes) {
  float lo = x[0], hi = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  const float qmax = (float)((1 << bits) - 1);
  volatile float range = hi - lo; /* one fp32 subtraction */
  volatile float s32 = range / qmax; /* one correctly rounded fp32 division */
  *s16 = orc_f32_to_f16(s32);
  *z16 = orc_f32_to_f16(lo);
  const float s = (float)orc_f16_to_f64(*s16);
  const float z = (float)orc_f16_to_f64(*z16);
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    volatile float d = x[i] - z;
    volatile float t = d / s;
    float r = rintf(t); /* default rounding mode: nearest-even */
    if (r < 0.0f) r = 0.0f;
    if (r > qmax) r = qmax;
    codes[i] = (uint8_t)r;
  }
}

/* ---------------- page layout (readings Q4-Q5) ---------------- */

static size_t code_bytes(int d, int bits) { return (size_t)d * (size_t)bits / 8u; }

/* Channels per quantization group of a d-channel vector (reading Q1). */
static int group_of(const orc_cfg* c, int d) { return c->group < d ? c->group : d; }

/* (scale, zero) bytes per token of a d-channel vector. */
static size_t sz_bytes(const orc_cfg* c, int d) { return (size_t)(d / group_of(c, d)) * 4u; }

void orc_page_regions(const orc_cfg* c, size_t off[4]) {
  size_t P = (size_t)c->page_size;
  size_t cc = code_bytes(c->d_c, c->c_bits);
  size_t rc = code_bytes(c->d_r, c->r_bits);
  size_t cs = sz_bytes(c, c->d_c);
  off[0] = 0;
  off[1] = P * cc;
  off[2] = P * (cc + rc);
  off[3] = P * (cc + rc + cs);
}

size_t orc_page_bytes(const orc_cfg* c) {
  size_t P = (size_t)c->page_size;
  return P * (code_bytes(c->d_c, c->c_bits) + code_bytes(c->d_r, c->r_bits) +
              sz_bytes(c, c->d_c) + sz_bytes(c, c->d_r));
}

/* Byte offset of the 32-bit word and bit offset inside it of channel ch of a
 * vector of n_g blocks of 32 channels stored at `bits` bits (reading Q4). */
static void code_position(int n_g, int bits, int ch, int* byte_off, int* bit_off) {
  int g = ch / 32, c = ch % 32;
  int j = c / 8, i = (c % 8) / 2, k = c % 2;
  int u = n_g < 16 / bits ? n_g : 16 / bits; /* blocks per chunk */
  int ld = g / u, gi = g % u;
  int per_word = 4 / bits; /* blocks sharing one word */
  int w = gi / per_word, e = gi % per_word;
  *byte_off = u * bits * (4 * ld + j) + 4 * w;
  *bit_off = 16 * k + bits * (4 * e + i);
}

static void put_u32(uint8_t* p, uint32_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
  p[2] = (uint8_t)(v >> 16);
  p[3] = (uint8_t)(v >> 24);
}

static uint32_t get_u32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static void put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
}

static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Quantize d channels (bf16 input) and store codes + (scale, zero) pairs. */
static void pack_vector(const uint16_t* in, int d, int bits, int group, uint8_t* code_dst,
                        uint8_t* sz_dst) {
  float x[1024];
  uint8_t q[1024];
  for (int g = 0; g < d / group; ++g) {
    uint16_t s16, z16;
    for (int i = 0; i < group; ++i) x[i] = orc_bf16_to_f32(in[g * group + i]);
    orc_quantize_group(x, group, bits, &s16, &z16, q + g * group);
    put_u16(sz_dst + 4 * g, s16);
    put_u16(sz_dst + 4 * g + 2, z16);
  }
  for (int w = 0; w < d * bits / 32; ++w) put_u32(code_dst + 4 * w, 0u);
  for (int ch = 0; ch < d; ++ch) {
    int byte_off, bit_off;
    code_position(d / 32, bits, ch, &byte_off, &bit_off);
    uint32_t word = get_u32(code_dst + byte_off);
    word |= (uint32_t)q[ch] << bit_off;
    put_u32(code_dst + byte_off, word);
  }
}

/* ---------------- fused writer (reading Q6-Q7) ---------------- */

int orc_token_source(const orc_cfg* c, int p, int L) {
  if (p < c->n_sink) return 0;
  if (p >= L - c->n_local) return 1;
  return 2;
}

int orc_write(const orc_cfg* c, int n, const uint16_t* c_kv, const uint16_t* k_rope,
              const int32_t* seq_idx, const int32_t* pos, const int32_t* seq_lens,
              const int32_t* page_table, int B, int max_pages, uint8_t* pages, int64_t num_pages,
              uint16_t* sink, uint16_t* local) {
  if (orc_check_cfg(c)) return -1;
  if (c->d_c > 1024 || c->d_r > 1024) return -1;
  size_t off[4];
  orc_page_regions(c, off);
  const size_t pb = orc_page_bytes(c);
  const size_t cc = code_bytes(c->d_c, c->c_bits), rc = code_bytes(c->d_r, c->r_bits);
  const size_t cs = sz_bytes(c, c->d_c), rs = sz_bytes(c, c->d_r);
  const int D = c->d_c + c->d_r;
  /* validate every index first, then write (tokens are independent: each
   * (sequence, position) appears once, so no two tokens share a slot) */
  for (int t = 0; t < n; ++t) {
    int b = seq_idx[t], p = pos[t];
    if (b < 0 || b >= B) return -1;
    int L = seq_lens[b];
    if (p < 0 || p >= L || p / c->page_size >= max_pages) return -1;
    int64_t page = page_table[(size_t)b * max_pages + p / c->page_size];
    if (page < 0 || page >= num_pages) return -1;
  }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < n; ++t) {
    int b = seq_idx[t], p = pos[t];
    int L = seq_lens[b];
    int64_t page = page_table[(size_t)b * max_pages + p / c->page_size];
    int slot = p % c->page_size;
    uint8_t* base = pages + (size_t)page * pb;
    const uint16_t* xc = c_kv + (size_t)t * c->d_c;
    const uint16_t* xr = k_rope + (size_t)t * c->d_r;
    pack_vector(xc, c->d_c, c->c_bits, group_of(c, c->d_c), base + off[0] + slot * cc,
                base + off[2] + slot * cs);
    pack_vector(xr, c->d_r, c->r_bits, group_of(c, c->d_r), base + off[1] + slot * rc,
                base + off[3] + slot * rs);
    uint16_t* dst = NULL;
    int src = orc_token_source(c, p, L);
    if (src == 0)
      dst = sink + ((size_t)b * c->n_sink + p) * D;
    else if (src == 1)
      dst = local + ((size_t)b * c->n_local + p % c->n_local) * D;
    if (dst) {
      for (int i = 0; i < c->d_c; ++i) dst[i] = xc[i];
      for (int i = 0; i < c->d_r; ++i) dst[c->d_c + i] = xr[i];
    }
  }
  return 0;
}

/* ---------------- decode (reading Q8) ---------------- */

static void unpack_vector(const uint8_t* code_src, const uint8_t* sz_src, int d, int bits,
                          int group, double* out) {
  uint32_t mask = (1u << bits) - 1u;
  for (int i = 0; i < d; ++i) {
    int byte_off, bit_off;
    code_position(d / 32, bits, i, &byte_off, &bit_off);
    uint32_t q = (get_u32(code_src + byte_off) >> bit_off) & mask;
    int g = i / group;
    double s = orc_f16_to_f64(get_u16(sz_src + 4 * g));
    double z = orc_f16_to_f64(get_u16(sz_src + 4 * g + 2));
    out[i] = (double)q * s + z; /* exact in fp64 */
  }
}

int orc_token_values(const orc_cfg* c, int b, int p, const uint8_t* pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const uint16_t* sink, const uint16_t* local, double* kc, double* kr) {
  int L = seq_lens[b];
  if (p < 0 || p >= L) return -1;
  const int D = c->d_c + c->d_r;
  int src = orc_token_source(c, p, L);
  if (src != 2) {
    const uint16_t* v = src == 0 ? sink + ((size_t)b * c->n_sink + p) * D
                                 : local + ((size_t)b * c->n_local + p % c->n_local) * D;
    for (int i = 0; i < c->d_c; ++i) kc[i] = orc_bf16_to_f32(v[i]);
    for (int i = 0; i < c->d_r; ++i) kr[i] = orc_bf16_to_f32(v[c->d_c + i]);
    return 0;
  }
  size_t off[4];
  orc_page_regions(c, off);
  const size_t pb = orc_page_bytes(c);
  const size_t cc = code_bytes(c->d_c, c->c_bits), rc = code_bytes(c->d_r, c->r_bits);
  const size_t cs = sz_bytes(c, c->d_c), rs = sz_bytes(c, c->d_r);
  int64_t page = page_table[(size_t)b * max_pages + p / c->page_size];
  int slot = p % c->page_size;
  const uint8_t* base = pages + (size_t)page * pb;
  unpack_vector(base + off[0] + slot * cc, base + off[2] + slot * cs, c->d_c, c->c_bits,
                group_of(c, c->d_c), kc);
  unpack_vector(base + off[1] + slot * rc, base + off[3] + slot * rs, c->d_r, c->r_bits,
                group_of(c, c->d_r), kr);
  return 0;
}

/* Attention of one head over the rows [0, n) of a gathered key matrix
 * (kc: n x d_c, kr: n x d_r). */
static void attend(int n, int d_c, int d_r, double scale, const double* ql, const double* qr,
                   const double* kc, const double* kr, double* score, double* out,
                   double* lse) {
  for (int i = 0; i < d_c; ++i) out[i] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int p = 0; p < n; ++p) {
    double a = 0.0, r = 0.0;
    for (int i = 0; i < d_c; ++i) a += ql[i] * kc[(size_t)p * d_c + i];
    for (int i = 0; i < d_r; ++i) r += qr[i] * kr[(size_t)p * d_r + i];
    score[p] = scale * (a + r);
    if (score[p] > m) m = score[p];
  }
  double l = 0.0;
  for (int p = 0; p < n; ++p) {
    double e = exp(score[p] - m);
    l += e;
    for (int i = 0; i < d_c; ++i) out[i] += e * kc[(size_t)p * d_c + i];
  }
  for (int i = 0; i < d_c; ++i) out[i] /= l;
  *lse = m + log(l);
}

int orc_decode(const orc_cfg* c, int B, int H, double scale, const uint16_t* q_lat,
               const uint16_t* q_rope, const uint8_t* pages, const int32_t* page_table,
               int max_pages, const int32_t* seq_lens, const uint16_t* sink,
               const uint16_t* local, int n_sel, const int32_t* sel_b, const int32_t* sel_h,
               int p_begin, int p_end, double* out, double* lse) {
  if (orc_check_cfg(c)) return -1;
  const int n_rows = n_sel > 0 ? n_sel : B * H;
  for (int b = 0; b < B; ++b) {
    /* rows of this sequence */
    int cnt = 0;
    for (int r = 0; r < n_rows; ++r)
      if ((n_sel > 0 ? sel_b[r] : r / H) == b) cnt++;
    if (cnt == 0) continue;
    int L = seq_lens[b];
    int lo = p_begin < 0 ? 0 : p_begin;
    int hi = (p_end < 0 || p_end > L) ? L : p_end;
    int n = hi > lo ? hi - lo : 0;
    /* gather and dequantize the sequence once */
    double* kc = (double*)malloc(sizeof(double) * ((size_t)n * c->d_c + 1));
    double* kr = (double*)malloc(sizeof(double) * ((size_t)n * c->d_r + 1));
    if (!kc || !kr) {
      free(kc);
      free(kr);
      return -2;
    }
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int p = 0; p < n; ++p)
      if (orc_token_values(c, b, lo + p, pages, page_table, max_pages, seq_lens, sink, local,
                           kc + (size_t)p * c->d_c, kr + (size_t)p * c->d_r))
        bad = 1;
    if (bad) {
      free(kc);
      free(kr);
      return -1;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
      int rb = n_sel > 0 ? sel_b[r] : r / H;
      if (rb != b) continue;
      int h = n_sel > 0 ? sel_h[r] : r % H;
      double ql[1024], qr[1024];
      for (int i = 0; i < c->d_c; ++i)
        ql[i] = orc_bf16_to_f32(q_lat[((size_t)b * H + h) * c->d_c + i]);
      for (int i = 0; i < c->d_r; ++i)
        qr[i] = orc_bf16_to_f32(q_rope[((size_t)b * H + h) * c->d_r + i]);
      double* score = (double*)malloc(sizeof(double) * ((size_t)n + 1));
      attend(n, c->d_c, c->d_r, scale, ql, qr, kc, kr, score, out + (size_t)r * c->d_c,
             lse + r);
      free(score);
    }
    free(kc);
    free(kr);
  }
  return 0;
}

/* Merge partial softmax results: lse = log sum_s exp(lse_s),
 * out = sum_s exp(lse_s - lse) * o_s; empty parts (lse_s = -inf) drop out. */
void orc_combine(int n, int d, const double* o_s, const double* lse_s, double* out,
                 double* lse) {
  double m = -INFINITY;
  for (int s = 0; s < n; ++s)
    if (lse_s[s] > m) m = lse_s[s];
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  if (m == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int s = 0; s < n; ++s) l += exp(lse_s[s] - m);
  *lse = m + log(l);
  for (int s = 0; s < n; ++s) {
    double w = exp(lse_s[s] - *lse);
    for (int i = 0; i < d; ++i) out[i] += w * o_s[(size_t)s * d + i];
  }
}

/* ---------------- paired BF16 cache (the baseline of Figure 5(b), Table 9) ----------------
 *
 * The unquantized cache that the low-bit kernel is measured against keeps
 * every token's [c | k_rope] row in BF16. Reading taken here (the pages name
 * the baseline but not its layout): the same paging as the packed cache, one
 * page = page_size rows of d_c + d_r bf16 values, row = slot = p mod
 * page_size, page = page_table[b][p div page_size]; no protected buffers. */

size_t orc_bf16_page_bytes(const orc_cfg* c) {
  return (size_t)c->page_size * (size_t)(c->d_c + c->d_r) * 2u;
}

int orc_bf16_write(const orc_cfg* c, int n, const uint16_t* c_kv, const uint16_t* k_rope,
                   const int32_t* seq_idx, const int32_t* pos, const int32_t* page_table,
                   int B, int max_pages, uint16_t* pages, int64_t num_pages) {
  if (orc_check_cfg(c)) return -1;
  const int D = c->d_c + c->d_r;
  for (int t = 0; t < n; ++t) {
    int b = seq_idx[t], p = pos[t];
    if (b < 0 || b >= B || p < 0 || p >= max_pages * c->page_size) return -1;
    int64_t page = page_table[(size_t)b * max_pages + p / c->page_size];
    if (page < 0 || page >= num_pages) return -1;
    uint16_t* row = pages + ((size_t)page * c->page_size + p % c->page_size) * D;
    for (int i = 0; i < c->d_c; ++i) row[i] = c_kv[(size_t)t * c->d_c + i];
    for (int i = 0; i < c->d_r; ++i) row[c->d_c + i] = k_rope[(size_t)t * c->d_r + i];
  }
  return 0;
}

/* Exact attention (fp64) of each selected (b, h) over the bf16 rows of tokens
 * [0, seq_lens[b]); same row selection and outputs as orc_decode. */
int orc_bf16_decode(const orc_cfg* c, int B, int H, double scale, const uint16_t* q_lat,
                    const uint16_t* q_rope, const uint16_t* pages, const int32_t* page_table,
                    int max_pages, const int32_t* seq_lens, int n_sel, const int32_t* sel_b,
                    const int32_t* sel_h, double* out, double* lse) {
  if (orc_check_cfg(c)) return -1;
  const int D = c->d_c + c->d_r;
  const int n_rows = n_sel > 0 ? n_sel : B * H;
  for (int b = 0; b < B; ++b) {
    int cnt = 0;
    for (int r = 0; r < n_rows; ++r)
      if ((n_sel > 0 ? sel_b[r] : r / H) == b) cnt++;
    if (cnt == 0) continue;
    const int n = seq_lens[b] > 0 ? seq_lens[b] : 0;
    if (n > max_pages * c->page_size) return -1;
    double* kc = (double*)malloc(sizeof(double) * ((size_t)n * c->d_c + 1));
    double* kr = (double*)malloc(sizeof(double) * ((size_t)n * c->d_r + 1));
    if (!kc || !kr) {
      free(kc);
      free(kr);
      return -2;
    }
    for (int p = 0; p < n; ++p) {
      int64_t page = page_table[(size_t)b * max_pages + p / c->page_size];
      const uint16_t* row = pages + ((size_t)page * c->page_size + p % c->page_size) * D;
      for (int i = 0; i < c->d_c; ++i) kc[(size_t)p * c->d_c + i] = orc_bf16_to_f32(row[i]);
      for (int i = 0; i < c->d_r; ++i)
        kr[(size_t)p * c->d_r + i] = orc_bf16_to_f32(row[c->d_c + i]);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
      int rb = n_sel > 0 ? sel_b[r] : r / H;
      if (rb != b) continue;
      int h = n_sel > 0 ? sel_h[r] : r % H;
      double ql[1024], qr[1024];
      for (int i = 0; i < c->d_c; ++i)
        ql[i] = orc_bf16_to_f32(q_lat[((size_t)b * H + h) * c->d_c + i]);
      for (int i = 0; i < c->d_r; ++i)
        qr[i] = orc_bf16_to_f32(q_rope[((size_t)b * H + h) * c->d_r + i]);
      double* score = (double*)malloc(sizeof(double) * ((size_t)n + 1));
      attend(n, c->d_c, c->d_r, scale, ql, qr, kc, kr, score, out + (size_t)r * c->d_c,
             lse + r);
      free(score);
    }
    free(kc);
    free(kr);
  }
  return 0;
}

/* ---------------- simulated quantize-dequantize (QDQ, Figure 3 caption) ----------------
 *
 * Each group of each token row goes through the writer's quantizer (readings
 * Q1-Q3) and comes back as x^ = q * s16 + z16. Reading taken here: that value
 * is rounded to fp32 (nearest even; it is exact in fp64) and then to bf16
 * (nearest even), the precision of the input rows. */
static uint16_t dequant_bf16(uint8_t q, uint16_t s16, uint16_t z16) {
  double v = (double)q * orc_f16_to_f64(s16) + orc_f16_to_f64(z16); /* exact */
  volatile float f = (float)v; /* nearest even */
  return orc_f64_to_bf16((double)f);
}

static void qdq_vector(const uint16_t* in, int d, int bits, int group, uint16_t* out) {
  float x[1024];
  uint8_t q[1024];
  for (int g = 0; g < d / group; ++g) {
    uint16_t s16, z16;
    for (int i = 0; i < group; ++i) x[i] = orc_bf16_to_f32(in[g * group + i]);
    orc_quantize_group(x, group, bits, &s16, &z16, q);
    for (int i = 0; i < group; ++i) out[g * group + i] = dequant_bf16(q[i], s16, z16);
  }
}

int orc_qdq(const orc_cfg* c, int n, const uint16_t* c_kv, const uint16_t* k_rope,
            uint16_t* out_c, uint16_t* out_r) {
  if (orc_check_cfg(c)) return -1;
  for (int t = 0; t < n; ++t) {
    qdq_vector(c_kv + (size_t)t * c->d_c, c->d_c, c->c_bits, group_of(c, c->d_c),
               out_c + (size_t)t * c->d_c);
    qdq_vector(k_rope + (size_t)t * c->d_r, c->d_r, c->r_bits, group_of(c, c->d_r),
               out_r + (size_t)t * c->d_r);
  }
  return 0;
}
