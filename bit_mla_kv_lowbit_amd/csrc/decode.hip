// Absorbed-MLA decode over the mixed BF16 / packed low-bit cache, for gfx950.
//
// QuantMLA (Figure 8 caption; abstract): attention unpacks and dequantizes the
// packed codes itself, takes protected sink / recent tokens from BF16 buffers,
// uses one reconstructed content tile for both the matching (QK) and the
// aggregation (PV) product, and normalizes all valid tokens with one softmax.
// The decode is the absorbed (MQA) form: all heads share the latent (GQLA card).
//
// Work decomposition: one workgroup = one (sequence, page range, 16-head
// block); 4 wavefronts; the page range is walked one 64-token page at a time,
// with the next page's codes loaded into registers while the current page is
// computed. Per page:
//   1. wave w takes tokens 16w..16w+15; lane (token t, sub-block j) holds the
//      8-channel sub-block j of every group of token t (the code order makes
//      each 128-bit load deliver one sub-block of 4 (INT4) or 8 (INT2) groups);
//   2. scores, exactly per group: the integer codes c (exact in fp16) are the
//      B operand of v_mfma_f32_16x16x32_f16, one MFMA per 32-channel group gives
//      D_g = q_g . c_g; then S = sum_g s_g D_g + sum_g z_g Q_g in fp32, with
//      Q_g = sum of q over group g (the z term is one more MFMA pair with Q_g
//      split into fp16 hi + lo). Rounding the reconstructed keys to fp16 first
//      would cost ~1e-3 in the scores of wide-range (outlier) groups;
//   3. the reconstructed content tile x = c * s + z (one packed fp16 FMA per
//      channel pair) goes to LDS token-major, the scores to a small LDS array;
//   4. every wave takes the page's 64 scores per head, updates the running max
//      and sum (log2 domain) and forms P in fp16;
//   5. wave w accumulates O^T for channels 128w..128w+127: the V^T operand is
//      read from the token-major tile with ds_read_b64_tr_b16, P^T from registers.
// The partial (O / l, log-sum-exp) of each page range is merged by
// combine_kernel (split-K over the sequence with an LSE combine).
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

constexpr float LN2 = 0.69314718055994530942f;
constexpr uint32_t MAGIC = 0x64006400u;  // fp16 pair (1024, 1024)
constexpr uint32_t ONE_ZERO = 0x00003C00u;  // (s, z) = (1.0, 0.0): a BF16 token

typedef __attribute__((address_space(3))) short4v lds_short4;

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// Raw data one lane loads for one page: its sub-block j of every code group of
// its token, and the token's (scale, zero) row.
template <int CB>
struct PageRegs {
  u32x4 c[CB == 4 ? 4 : 2];  // content code chunks
  u32x4 sz[4];               // content (s, z) words of groups 0..15
  u32x2 rsz;                 // RoPE (s, z) words of groups 16, 17
  u32x2 r;                   // RoPE code words (groups 16, 17)
};

template <int CB>
__device__ __forceinline__ void load_page(PageRegs<CB>& t, const uint8_t* page_base, int slot,
                                          int j) {
  using G = PageGeom<CB>;
  const uint8_t* crow = page_base + G::OFF_CC + slot * G::CC;
#pragma unroll
  for (int ld = 0; ld < (CB == 4 ? 4 : 2); ++ld)
    t.c[ld] = *reinterpret_cast<const u32x4*>(crow + 64 * ld + 16 * j);
  const uint8_t* srow = page_base + G::OFF_CS + slot * G::CS;
#pragma unroll
  for (int q = 0; q < 4; ++q) t.sz[q] = *reinterpret_cast<const u32x4*>(srow + 16 * q);
  t.rsz = *reinterpret_cast<const u32x2*>(page_base + G::OFF_RS + slot * G::RS);
  t.r = *reinterpret_cast<const u32x2*>(page_base + G::OFF_RC + slot * G::RC + 8 * j);
}

// Exact codes of channels 8j..8j+7 (pairs (0,1) (2,3) (4,5) (6,7)) of one group
// from its code word. Codes at bit offsets below 10 are turned into fp16
// 1024 + 2^o * c with one and-or, then back to c with one exact packed FMA.
__device__ __forceinline__ half8 codes4(uint32_t wd) {
  const half2v m1024 = as_h2(0xE400E400u);  // -1024
  const half2v r16 = as_h2(0x2C002C00u);    // 1/16
  const half2v m64 = as_h2(0xD400D400u);    // -64
  const uint32_t t = wd >> 8;
  const half2v p0 = as_h2((wd & 0x000F000Fu) | MAGIC) + m1024;
  const half2v p1 = __builtin_elementwise_fma(as_h2((wd & 0x00F000F0u) | MAGIC), r16, m64);
  const half2v p2 = as_h2((t & 0x000F000Fu) | MAGIC) + m1024;
  const half2v p3 = __builtin_elementwise_fma(as_h2((t & 0x00F000F0u) | MAGIC), r16, m64);
  return (half8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Same for 2-bit codes: code block e of the word (pairs at bits 8e + 2i, 24 + ... ).
__device__ __forceinline__ half8 codes2(uint32_t wd, int e) {
  const uint32_t t = e ? wd >> 8 : wd;
  const half2v m1024 = as_h2(0xE400E400u);
  const half2v r4 = as_h2(0x34003400u), m256 = as_h2(0xDC00DC00u);    // 1/4, -256
  const half2v r16 = as_h2(0x2C002C00u), m64 = as_h2(0xD400D400u);    // 1/16, -64
  const half2v r64 = as_h2(0x24002400u), m16 = as_h2(0xCC00CC00u);    // 1/64, -16
  const half2v p0 = as_h2((t & 0x00030003u) | MAGIC) + m1024;
  const half2v p1 = __builtin_elementwise_fma(as_h2((t & 0x000C000Cu) | MAGIC), r4, m256);
  const half2v p2 = __builtin_elementwise_fma(as_h2((t & 0x00300030u) | MAGIC), r16, m64);
  const half2v p3 = __builtin_elementwise_fma(as_h2((t & 0x00C000C0u) | MAGIC), r64, m16);
  return (half8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Code word of group g (0..17) for this lane's sub-block.
template <int CB>
__device__ __forceinline__ half8 group_codes(const PageRegs<CB>& t, int g) {
  if (g >= NG_C) return codes4(g == NG_C ? t.r.x : t.r.y);
  if (CB == 4) return codes4(t.c[g >> 2][g & 3]);
  return codes2(t.c[g >> 3][(g >> 1) & 3], g & 1);
}

template <int CB>
__device__ __forceinline__ uint32_t group_sz(const PageRegs<CB>& t, int g) {
  if (g >= NG_C) return g == NG_C ? t.rsz.x : t.rsz.y;
  return t.sz[g >> 2][g & 3];
}

// Reconstructed fp16 values x = c * s + z (one rounding per value).
__device__ __forceinline__ half8 reconstruct(half8 c, uint32_t sz) {
  const half2v szh = as_h2(sz);
  const half2v s2 = __builtin_shufflevector(szh, szh, 0, 0);
  const half2v z2 = __builtin_shufflevector(szh, szh, 1, 1);
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v x = __builtin_elementwise_fma((half2v){c[2 * i], c[2 * i + 1]}, s2, z2);
    r[2 * i] = x.x;
    r[2 * i + 1] = x.y;
  }
  return r;
}

// One page for one wave: scores of its 16 tokens (S[4 heads of this lane x
// token t16]) and the content tile rows. EDGE pages may hold BF16-protected
// tokens and tokens past the end; interior pages are all packed and valid.
__device__ __forceinline__ int tile_off(int row, int ch);

template <int CB, bool EDGE>
__device__ __forceinline__ float4v page_scores(PageRegs<CB>& t, const half8* qlds, int lane,
                                               const half8& qz1, const half8& qz2,
                                               _Float16* tile, int row, int j, int src,
                                               const uint16_t* brow) {
  // src: 0 = packed, 1 = BF16 row, 2 = nothing (past the end)
  if (EDGE) {
    if (src != 0) {
      const uint32_t v = src == 1 ? ONE_ZERO : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) t.sz[q] = (u32x4){v, v, v, v};
      t.rsz = (u32x2){v, v};
    }
  }
  // z term: lanes of even j carry z of groups 0..7, odd j of groups 8..15; the
  // matching Q_g (hi in j = 0, 1, lo in j = 2, 3) is in qz1. Groups 16, 17: qz2.
  half8 zb1, zb2;
  {
    const u32x4 a = (j & 1) ? t.sz[2] : t.sz[0];
    const u32x4 b = (j & 1) ? t.sz[3] : t.sz[1];
    const uint32_t z01 = __builtin_amdgcn_perm(a.y, a.x, 0x07060302u);
    const uint32_t z23 = __builtin_amdgcn_perm(a.w, a.z, 0x07060302u);
    const uint32_t z45 = __builtin_amdgcn_perm(b.y, b.x, 0x07060302u);
    const uint32_t z67 = __builtin_amdgcn_perm(b.w, b.z, 0x07060302u);
    const half2v h0 = as_h2(z01), h1 = as_h2(z23), h2 = as_h2(z45), h3 = as_h2(z67);
    zb1 = (half8){h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
    const half2v hr = as_h2(__builtin_amdgcn_perm(t.rsz.y, t.rsz.x, 0x07060302u));
    zb2 = (half8){hr.x, hr.y, 0, 0, 0, 0, 0, 0};
  }
  float4v S = {0.f, 0.f, 0.f, 0.f};
  S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz1, zb1, S, 0, 0, 0);
  S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz2, zb2, S, 0, 0, 0);
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 18; ++g) {
    half8 c = group_codes<CB>(t, g);
    if (EDGE) {
      if (src == 2) c = (half8){};
      const int ch = g < NG_C ? GROUP * g + 8 * j : D_C + GROUP * (g - NG_C) + 8 * j;
      if (src == 1) c = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(brow + ch));
    }
    const uint32_t sz = group_sz<CB>(t, g);
    const float4v D = __builtin_amdgcn_mfma_f32_16x16x32_f16(qlds[g * 64 + lane], c, zero4, 0, 0, 0);
    const float s = (float)as_h2(sz).x;
    S += s * D;
    if (g < NG_C)
      *reinterpret_cast<half8*>(tile + tile_off(row, GROUP * g + 8 * j)) = reconstruct(c, sz);
  }
  return S;
}

// LDS tile of reconstructed content values, 128 token rows x 512 fp16, with
// the 16-byte chunk index of each row XOR-swizzled so that the transposing
// reads of 16 rows and the row writes spread over the banks.
__device__ __forceinline__ int tile_off(int row, int ch) {
  const int chunk = (ch >> 3) ^ ((row & 3) | (((row >> 3) & 3) << 2));
  return row * D_C + chunk * 8 + (ch & 7);
}

template <int CB>
__global__ __launch_bounds__(512, 1) void decode_h16_kernel(DecodeArgs a) {
  using G = PageGeom<CB>;
  constexpr int TOK = 2 * PAGE;  // tokens per iteration: two pages
  __shared__ __attribute__((aligned(16))) _Float16 tile[TOK * D_C];
  __shared__ __attribute__((aligned(16))) float sx[16 * (TOK + 4)];
  __shared__ half8 qlds[18 * 64];  // Q A-operand registers of every group, per lane
  constexpr int SXS = TOK + 4;

  const int split = blockIdx.x, hb = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, j = lane >> 4, t16 = lane & 15;
  const int H = a.H;
  const int h = hb * 16 + t16;
  const int L = a.seq_lens[b];
  const int n_pages_seq = (L + PAGE - 1) / PAGE;
  const int pg0 = split * a.pages_per_split;
  const int pg1 = min(pg0 + a.pages_per_split, n_pages_seq);
  const int row_tok = 16 * w + t16;       // this lane's token row in the tile (0..127)
  const int half_pg = w >> 2;             // which of the two pages
  const int slot = 16 * (w & 3) + t16;    // slot in that page

  // Q as the A operand (lane = head t16; channels 32g + 8j .. +7 of group g),
  // kept in LDS, and the per-group sums Q_g split into fp16 hi + lo for the z term.
  half8 qz1, qz2;
  {
    const uint16_t* ql = a.q_lat + ((int64_t)b * H + h) * D_C;
    const uint16_t* qr = a.q_rope + ((int64_t)b * H + h) * D_R;
    // qz1 slot i: Q_{8 (j & 1) + i} (hi part for j < 2, lo part for j >= 2);
    // qz2 slots 0, 1: Q_16, Q_17 (hi for j = 0, lo for j = 1, zero otherwise)
    const bool lo_part = j >= 2;
    const int qz1_half = j & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qz1[i] = (_Float16)0.f;
      qz2[i] = (_Float16)0.f;
    }
#pragma unroll
    for (int g = 0; g < 18; ++g) {
      const uint16_t* src = g < NG_C ? ql + GROUP * g + 8 * j : qr + GROUP * (g - NG_C) + 8 * j;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src);
      if (w == 0) qlds[g * 64 + lane] = bf16x8_to_f16x8(raw);
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += bf16_to_f32(raw[e] & 0xffffu) + bf16_to_f32(raw[e] >> 16);
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const _Float16 hi = (_Float16)sum;
      const _Float16 lo = (_Float16)(sum - (float)hi);
      if (g < NG_C) {
        if ((g >> 3) == qz1_half) qz1[g & 7] = lo_part ? lo : hi;
      } else {
        if (j < 2) qz2[g - NG_C] = j == 1 ? lo : hi;
      }
    }
  }
  __syncthreads();

  float4v oacc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) oacc[mb] = (float4v){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;

  PageRegs<CB> cur;
  if (pg0 + half_pg < pg1)
    load_page<CB>(cur, a.pages + (int64_t)ptab[pg0 + half_pg] * G::BYTES, slot, j);

  for (int pg = pg0; pg < pg1; pg += 2) {
    PageRegs<CB> nxt;
    const int my_next = pg + 2 + half_pg;
    if (my_next < pg1) load_page<CB>(nxt, a.pages + (int64_t)ptab[my_next] * G::BYTES, slot, j);

    const int my_pg = pg + half_pg;
    const int p0 = my_pg * PAGE;
    const int p = p0 + slot;
    float4v S;
    const bool interior = my_pg < pg1 && p0 >= a.n_sink && p0 + PAGE <= L - a.n_local;
    if (interior) {
      S = page_scores<CB, false>(cur, qlds, lane, qz1, qz2, tile, row_tok, j, 0, nullptr);
    } else {
      int src = 2;
      const uint16_t* brow = a.sink;
      if (my_pg < pg1 && p < L) {
        if (p < a.n_sink) {
          src = 1;
          brow = a.sink + ((int64_t)b * a.n_sink + p) * D_ALL;
        } else if (p >= L - a.n_local) {
          src = 1;
          brow = a.local + ((int64_t)b * a.n_local + p % a.n_local) * D_ALL;
        } else {
          src = 0;
        }
      }
      S = page_scores<CB, true>(cur, qlds, lane, qz1, qz2, tile, row_tok, j, src, brow);
      if (src == 2) S = (float4v){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // scores to LDS: sx[head][token]
#pragma unroll
    for (int i = 0; i < 4; ++i) sx[(4 * j + i) * SXS + row_tok] = S[i];
    __syncthreads();

    // softmax update for head t16 over the 128 tokens (log2 domain); lane holds
    // tokens 32 kb + 8 j + i (kb = 0..3, i = 0..7) as the PV K slots
    float xv[32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const float* srcp = sx + t16 * SXS + 32 * kb + 8 * j;
      const float4v v0 = *reinterpret_cast<const float4v*>(srcp);
      const float4v v1 = *reinterpret_cast<const float4v*>(srcp + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[8 * kb + i] = v0[i];
        xv[8 * kb + 4 + i] = v1[i];
      }
    }
    float mx = xv[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, xv[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) oacc[mb] *= alpha;
    }
    m_run = m_new;
    half8 pB[4];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(xv[8 * kb + i], sl2, -m_use));
        psum += pv;
        pB[kb][i] = (_Float16)pv;
      }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run += psum;

    // O^T[64 channels of this wave x 16 heads] += V^T P^T over the 128 tokens
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int row = 32 * kb + 8 * j + (t16 >> 2);
        const int col = 64 * w + 16 * mb + 4 * (t16 & 3);
        const short4v lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + tile_off(row, col)));
        const short4v hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(tile + tile_off(row + 4, col)));
        const half4 l4 = __builtin_bit_cast(half4, lo), h4 = __builtin_bit_cast(half4, hi);
        const half8 av = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
        oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pB[kb], oacc[mb], 0, 0, 0);
      }
    }
    __syncthreads();
    cur = nxt;
  }

  // partial result of this page range: O / l and its log-sum-exp
  const int64_t orow = ((int64_t)b * a.n_split + split) * H + h;
  if (l_run > 0.f) {
    const float inv = 1.f / l_run;
    float* dst = a.ws_o + orow * D_C + 64 * w + 4 * j;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) *reinterpret_cast<float4v*>(dst + 16 * mb) = oacc[mb] * inv;
  }
  if (w == 0 && j == 0)
    a.ws_lse[orow] = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
}

// Merge the page-range partials of one (sequence, head, 128-channel quarter):
// lse = log sum exp(lse_s), out = sum_s exp(lse_s - lse) * o_s; empty ranges
// (lse_s = -inf) are skipped. 8 split lanes x 32 channel lanes per block.
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  __shared__ float4v part[8][32];
  const int row = blockIdx.x >> 2, cq = blockIdx.x & 3;
  const int b = row / a.H, h = row % a.H;
  const int sl = threadIdx.x >> 5, ct = threadIdx.x & 31;
  const int ns = a.n_split;
  const float* lses = a.ws_lse + (int64_t)b * ns * a.H + h;
  float m = -INFINITY;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, lses[(int64_t)s * a.H]);
  float lse = -INFINITY;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY) {
    float sum = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ls = lses[(int64_t)s * a.H];
      if (ls != -INFINITY) sum += __expf(ls - m);
    }
    lse = m + __logf(sum);
    const int c0 = 128 * cq + 4 * ct;
    for (int s = sl; s < ns; s += 8) {
      const float ls = lses[(int64_t)s * a.H];
      if (ls == -INFINITY) continue;
      const float4v o = *reinterpret_cast<const float4v*>(
          a.ws_o + (((int64_t)b * ns + s) * a.H + h) * D_C + c0);
      acc += __expf(ls - lse) * o;
    }
  }
  part[sl][ct] = acc;
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int k = 1; k < 8; ++k) acc += part[k][ct];
    uint16_t* op = a.out + ((int64_t)b * a.H + h) * D_C + 128 * cq + 4 * ct;
    u32x2 packed;
    packed.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    packed.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(op) = packed;
    if (ct == 0 && cq == 0) a.lse[(int64_t)b * a.H + h] = lse;
  }
}

SplitPlan plan_splits(int B, int H, int max_pages) {
  // about one 8-wave workgroup per CU (256 CUs); at most 64 pages per range so
  // long sequences spread over many CUs; an even page count per range (the
  // kernel walks two pages per iteration)
  const int n_hb = H / 16;
  const int64_t base = (int64_t)(B > 0 ? B : 1) * n_hb;
  int want = (int)((256 + base - 1) / base);
  if (want < 1) want = 1;
  if (want > max_pages) want = max_pages;
  int pps = (max_pages + want - 1) / want;
  if (pps > 64) pps = 64;
  pps += pps & 1;
  SplitPlan sp;
  sp.pages_per_split = pps;
  sp.n_split = (max_pages + pps - 1) / pps;
  return sp;
}

size_t decode_workspace_bytes(int B, int H, int max_pages) {
  const SplitPlan sp = plan_splits(B, H, max_pages);
  return (size_t)B * sp.n_split * H * (D_C + 1) * sizeof(float);
}

hipError_t launch_decode(DecodeArgs a, int c_bits, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const dim3 grid(a.n_split, a.H / 16, a.B);
  if (c_bits == 4)
    decode_h16_kernel<4><<<grid, dim3(512), 0, stream>>>(a);
  else
    decode_h16_kernel<2><<<grid, dim3(512), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<<<dim3(a.B * a.H * 4), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
