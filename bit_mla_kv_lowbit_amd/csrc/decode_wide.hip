// Absorbed-MLA decode for 128 query heads per query token (DeepSeek-V3-shaped
// batches and the serving step), for gfx950: every page is unpacked and
// dequantized once per 64 heads and shared by them.
//
// QuantMLA (Figure 8 caption; abstract): the kernel unpacks and dequantizes
// the packed codes itself, takes sink and recent tokens from their BF16 rows,
// uses one reconstructed content tile for matching (QK) and aggregation (PV),
// and normalizes all valid tokens with one softmax. Absorbed MLA is MQA over
// the shared latent (GQLA card), so one dequantized page serves every head.
//
// Work decomposition (length-aware, decided on the device from seq_lens): the
// pages of all (sequence, query token) pairs are laid end to end with a weight
// per page (2, or 3 for a page holding BF16 rows), and the line is cut into NC
// equal chunks. Workgroup (c, hh) takes the pages of chunk c for heads
// 64 hh .. 64 hh + 63 (the two workgroups of a chunk have ids c and c + NC, the
// same XCD, so the second read of a page hits that XCD's L2). A chunk may hold
// the tail of one sequence and the head of the next: each piece (segment) is
// folded into one (O / l, log-sum-exp) partial, or written as the final output
// when no other chunk touches that sequence; combine_wide_kernel merges the
// rest. A record per sequence names the chunks that touch it.
//
// A workgroup is 4 wavefronts (one per SIMD, one workgroup per CU) and walks
// its pages 32 tokens (half a page) per step:
//   producer  thread (token t, sub-block j, group half hf) loads its packed
//             codes and (scale, zero) words one step ahead, turns the codes
//             into exact fp16 integers (magic exponent) in a code tile, keeps
//             x = c * s + z in registers and writes it to the value tile after
//             the next barrier. A protected token's BF16 row goes to both
//             tiles as fp16 values with (scale, zero) = (1, 0);
//   scores    wave (head pair hp, group half gh): S = sum_g s_g (q_g . c_g) +
//             sum_g z_g Q_g for 32 heads over 9 of the 18 groups, one
//             v_mfma_f32_16x16x32_f16 per (16 heads, 16 tokens, group) on the
//             exact codes, the scale applied on the VALU; the two waves of a
//             pair exchange their partial sums through LDS, so both hold the
//             same full scores and take the same softmax decisions;
//   softmax   P = 2^(S scale log2e - M) against a reference max per head that
//             moves only when a score exceeds it by more than 2^8 (then O and
//             l are rescaled by the published factor); P to an LDS buffer;
//   PV        wave w: O^T for channels 128 w .. 128 w + 127 of all 64 heads
//             (128 accumulators per lane), V^T and P^T read transposed
//             (ds_read_b64_tr_b16).
// Three barriers per step (scores done, P ready, next tiles ready); the code
// and scale tiles are double-buffered, the value tile is single.
#include "mla_common.h"
#include "mla_kernels.h"
#include "decode_ops.h"

namespace mla {
namespace {

constexpr int NT = 512;         // threads per workgroup (8 waves, two per SIMD)
constexpr int WR = 64;          // query rows (heads) per workgroup
constexpr int RG = 128;         // rows per query token on this path
constexpr int ST = 32;          // tokens per step
constexpr int VT = D_C + 8;     // value tile row stride in halves (1040 bytes)
constexpr int PT = WR + 8;      // P buffer row stride in halves (144 bytes)
constexpr int NCH = 128;        // chunks of the page line (workgroups: 2 NCH)

constexpr int CT = D_ALL + 8;   // code tile row stride in halves (1168 bytes)
constexpr int SZT = 20;         // (scale, zero) words per token row (18 used)

// Double-buffered by step parity. In iteration k the score waves read the code
// and (scale, zero) tiles of step k and write P of step k, while the PV waves
// read the value tile and P of step k - 1 and fill the code, (scale, zero) and
// value tiles of step k + 1 (each PV wave only its own value columns).
struct WideLds {
  _Float16 code[2][ST * CT];     // fp16 codes (or BF16-row values) of 18 groups, token-major
  uint32_t sz[2][ST * SZT];      // (scale, zero) fp16 pairs per token and group
  _Float16 val[2][ST * VT];      // reconstructed content values, token-major
  _Float16 p[2][ST * PT];        // P: token rows x 64 heads
  float alpha[2][WR];            // rescale factor of each head's moved reference
  int flag[2][4];                // per head block: its reference moved in that step
  float lsum[WR];                // sum of P per head
  float mref[WR];                // final reference max per head
  int seg_first, seg_last, p_first;
  int scan[NT / 64];
};

// Weight of the pages of one (sequence, query token): 2 per page, 1 more for a
// page holding BF16 rows (the sink page and the window pages).
struct SeqW {
  int L, Lq, n_s, lo_start, n_pages, wp, sinkw, W;
  __device__ int wb(int k) const { return 2 * k + sinkw * min(k, 1) + max(0, k - wp); }
  // first page i in [0, n_pages] with wb(i) >= target
  __device__ int first_page(int target) const {
    int lo = 0, hi = n_pages;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (wb(mid) >= target) hi = mid;
      else lo = mid + 1;
    }
    return lo;
  }
};

__device__ __forceinline__ SeqW seq_weight(const DecodeArgs& a, int v, int L_raw) {
  SeqW s;
  const int qi = v % a.s_q;
  const int Lg = a.max_pages * PAGE;
  s.L = min(max(L_raw, 0), Lg);
  s.n_s = min(a.n_sink, s.L);
  s.lo_start = max(a.n_sink, s.L - a.n_local);
  s.Lq = max(0, s.L - (a.s_q - 1 - qi));
  s.n_pages = (s.Lq + PAGE - 1) / PAGE;
  s.wp = min(s.lo_start / PAGE, s.n_pages);
  s.sinkw = (s.n_s > 0 && s.wp > 0) ? 1 : 0;
  s.W = s.wb(s.n_pages);
  return s;
}

__device__ __forceinline__ SeqW seq_weight(const DecodeArgs& a, int v) {
  return seq_weight(a, v, a.seq_lens[v / a.s_q]);
}

// The same for a v every lane agrees on: the length is read with a scalar load
// and every field is kept in scalar registers.
__device__ __forceinline__ SeqW seq_weight_uniform(const DecodeArgs& a, int v) {
  v = __builtin_amdgcn_readfirstlane(v);
  const int L_raw = *(const_i32*)(a.seq_lens + v / a.s_q);
  SeqW s = seq_weight(a, v, L_raw);
  s.L = __builtin_amdgcn_readfirstlane(s.L);
  s.Lq = __builtin_amdgcn_readfirstlane(s.Lq);
  s.n_s = __builtin_amdgcn_readfirstlane(s.n_s);
  s.lo_start = __builtin_amdgcn_readfirstlane(s.lo_start);
  s.n_pages = __builtin_amdgcn_readfirstlane(s.n_pages);
  s.wp = __builtin_amdgcn_readfirstlane(s.wp);
  s.sinkw = __builtin_amdgcn_readfirstlane(s.sinkw);
  s.W = __builtin_amdgcn_readfirstlane(s.W);
  return s;
}

// Chunk that owns weight position u (0 <= u < W): chunk k covers
// [k W / nc, (k + 1) W / nc).
__device__ __forceinline__ int owner(int64_t u, int64_t W, int nc) {
  if (u >= W) return nc - 1;
  return (int)min((int64_t)nc - 1, ((u + 1) * nc - 1) / W);
}

// Packed data of one token that a converter lane (token, sub-block j) loads
// for its channel quarter cq: the content codes of groups 4 cq .. 4 cq + 3
// (C4: one 16-byte chunk; C2: two words), their (scale, zero) words, and for
// cq < 2 the code word and (scale, zero) word of RoPE group cq.
struct ConvRaw {
  u32x4 c, s;
  uint32_t r, rs;
};

// (A group of 2 or 4 blocks has one (scale, zero) word: it is repeated for
// each of its blocks, so the tiles always hold one word per block.)
template <int F>
__device__ __forceinline__ void conv_load(ConvRaw& t, __amdgpu_buffer_rsrc_t rs, int slot, int j,
                                          int cq) {
  using G = PageGeom<F>;
  if constexpr (G::CB == 4) {
    t.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, slot * G::CC + 16 * j + 64 * cq, G::OFF_CC, 0));
  } else {
    const u32x2 c2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
        rs, slot * G::CC + 16 * j + 64 * (cq >> 1) + 8 * (cq & 1), G::OFF_CC, 0));
    t.c = (u32x4){c2.x, c2.y, 0u, 0u};
  }
  if constexpr (G::GM == 1) {
    t.s = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, slot * G::CS + 16 * cq, G::OFF_CS, 0));
  } else if constexpr (G::GM == 2) {
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  rs, slot * G::CS + 8 * cq, G::OFF_CS, 0));
    t.s = (u32x4){w.x, w.x, w.y, w.y};
  } else {
    const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::CS + 4 * cq, G::OFF_CS, 0);
    t.s = (u32x4){w, w, w, w};
  }
  if (cq < NG_R) {
    // 4-bit: word cq of chunk j; 2-bit: both blocks share the chunk's word
    t.r = G::RB == 4 ? __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::RC + 8 * j + 4 * cq, G::OFF_RC, 0)
                     : __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::RC + 4 * j, G::OFF_RC, 0);
    t.rs = __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::RS + (G::GMR == 1 ? 4 * cq : 0),
                                                G::OFF_RS, 0);
  }
}

// One converter lane's share of a step: codes of its groups into the code
// tile, (scale, zero) words into their tile (lanes j = 0), and the
// reconstructed values of its content groups into the value tile. A token with
// a BF16 row (brow) takes its values with (scale, zero) = (1, 0); an invalid
// token zeros.
template <int F>
__device__ __forceinline__ void convert_tok(const ConvRaw& t, _Float16* crow, uint32_t* zrow,
                                            _Float16* vrow, int j, int cq, bool mixed, bool valid,
                                            const uint16_t* brow) {
  u32x4 sw = t.s;
  uint32_t rsw = t.rs;
  half8 c[4], r;
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = fmt_cb(F) == 4 ? codes4(t.c[e]) : codes2(t.c[e >> 1], e & 1);
  r = fmt_rb(F) == 4 ? codes4(t.r) : codes2(t.r, cq);
  if (mixed) {
    if (brow != nullptr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(brow + GROUP * (4 * cq + e) + 8 * j));
        sw[e] = 0x00003C00u;  // scale 1, zero 0
      }
      if (cq < NG_R) {
        r = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(brow + D_C + GROUP * cq + 8 * j));
        rsw = 0x00003C00u;
      }
    } else if (!valid) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = (half8){};
        sw[e] = 0u;
      }
      r = (half8){};
      rsw = 0u;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int g = 4 * cq + e;
    *reinterpret_cast<half8*>(crow + GROUP * g + 8 * j) = c[e];
    *reinterpret_cast<half8*>(vrow + GROUP * g + 8 * j) = reconstruct(c[e], sw[e]);
  }
  if (cq < NG_R) *reinterpret_cast<half8*>(crow + D_C + GROUP * cq + 8 * j) = r;
  if (j == 0) {
    *reinterpret_cast<u32x4*>(zrow + 4 * cq) = sw;
    if (cq < NG_R) zrow[NG_C + cq] = rsw;
  }
}

// Scores of 16 heads for the two token blocks of a step (lane: token t16 of
// each block, sub-block j), from the code and (scale, zero) tiles, exactly per
// group: integer codes (or BF16-row values with scale 1) are the MFMA B
// operand, each group's product is scaled on the VALU one group later, and the
// zero points enter through two MFMAs against the group sums of q (hi and lo
// fp16 parts). Both blocks go through the group loop together.
__device__ __forceinline__ void step_scores(const _Float16* code, const uint32_t* sz,
                                            const half8 (&qA)[18], const half8& qz1,
                                            const half8& qz2, int j, int t16, float4v (&S)[2]) {
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
  float sc[2][NG_C + NG_R];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const uint32_t* zrow = sz + (16 * tb + t16) * SZT;
    u32x4 w4[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) w4[k] = *reinterpret_cast<const u32x4*>(zrow + 4 * k);
    uint32_t wd[20];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      wd[4 * k] = w4[k].x;
      wd[4 * k + 1] = w4[k].y;
      wd[4 * k + 2] = w4[k].z;
      wd[4 * k + 3] = w4[k].w;
    }
#pragma unroll
    for (int g = 0; g < NG_C + NG_R; ++g) sc[tb][g] = (float)as_h2(wd[g]).x;
    // z operands (K slot 8 j + i): zb1 holds the z of content groups 0..7 in
    // lanes j < 2 and the RoPE groups' z in slots 0, 1 of lanes j >= 2; zb2 the
    // z of content groups 8..15
    const bool lowj = j < 2;
    const uint32_t rz = z_pair(wd[16], wd[17]);
    const u32x4 z1 = {lowj ? z_pair(wd[0], wd[1]) : rz, lowj ? z_pair(wd[2], wd[3]) : 0u,
                      lowj ? z_pair(wd[4], wd[5]) : 0u, lowj ? z_pair(wd[6], wd[7]) : 0u};
    const u32x4 z2 = {z_pair(wd[8], wd[9]), z_pair(wd[10], wd[11]), z_pair(wd[12], wd[13]),
                      z_pair(wd[14], wd[15])};
    S[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz1, __builtin_bit_cast(half8, z1), zero4, 0, 0, 0);
    S[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz2, __builtin_bit_cast(half8, z2), S[tb], 0, 0, 0);
  }
  const _Float16* c0 = code + t16 * CT + 8 * j;
  const _Float16* c1 = code + (16 + t16) * CT + 8 * j;
  // B operands read PF groups ahead of their MFMAs (LDS latency)
  constexpr int PF = 6;
  half8 Bw[PF][2];
#pragma unroll
  for (int g = 0; g < PF; ++g) {
    Bw[g][0] = *reinterpret_cast<const half8*>(c0 + GROUP * g);
    Bw[g][1] = *reinterpret_cast<const half8*>(c1 + GROUP * g);
  }
  float4v Dp0 = zero4, Dp1 = zero4;
#pragma unroll
  for (int g = 0; g < NG_C + NG_R; ++g) {
    const half8 B0 = Bw[g % PF][0];
    const half8 B1 = Bw[g % PF][1];
    if (g + PF < NG_C + NG_R) {
      const int gn = g + PF;
      const int ch = gn < NG_C ? GROUP * gn : D_C + GROUP * (gn - NG_C);
      Bw[g % PF][0] = *reinterpret_cast<const half8*>(c0 + ch);
      Bw[g % PF][1] = *reinterpret_cast<const half8*>(c1 + ch);
    }
    const float4v D0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[g], B0, zero4, 0, 0, 0);
    const float4v D1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[g], B1, zero4, 0, 0, 0);
    if (g > 0) {
      S[0] += sc[0][g - 1] * Dp0;
      S[1] += sc[1][g - 1] * Dp1;
    }
    Dp0 = D0;
    Dp1 = D1;
  }
  S[0] += sc[0][NG_C + NG_R - 1] * Dp0;
  S[1] += sc[1][NG_C + NG_R - 1] * Dp1;
}

// Row maximum over the 16 lanes of a row (DPP).
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)));
  return v;
}

// One segment (pages [i_begin, i_begin + n_steps / 2) of sequence v, rows
// 64 hh .. 64 hh + 63). Waves 0..3 score head block hb = w over every group;
// waves 4..7 own channel quarter cq = w - 4: they convert its codes (content
// groups 4 cq .. 4 cq + 3, RoPE group cq) and accumulate O^T for its channels
// 128 cq .. 128 cq + 127 of all 64 heads. Iteration k: scores of step k, PV of
// step k - 1 and conversion of step k + 1; one barrier per iteration.
template <int F>
__device__ __forceinline__ void segment(WideLds& sm, const DecodeArgs& a, const SeqW& s, int v,
                                        int b, int hh, int i_begin, int n_steps, bool direct,
                                        int slot, int w, int lane) {
  const int j = lane >> 4, t16 = lane & 15;
  const int* ptab = a.page_table + (int64_t)b * a.max_pages;
  auto step_p0 = [&](int st) { return PAGE * (i_begin + (st >> 1)) + ST * (st & 1); };
  if (w < 4) {
    // ================= score wave: 16 heads, all 18 groups =================
    const int hb = w;
    const float sl2 = a.scale_log2;
    half8 qA[NG_C + NG_R];
    half8 qz1, qz2;
    {
      const int64_t row = (int64_t)v * RG + WR * hh + 16 * hb + t16;
#pragma unroll
      for (int g = 0; g < NG_C + NG_R; ++g) {
        const uint16_t* src = g < NG_C ? a.q_lat + row * D_C + GROUP * g + 8 * j
                                       : a.q_rope + row * D_R + GROUP * (g - NG_C) + 8 * j;
        qA[g] = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(src));
      }
      // group sums Q_g of head t16 (one MFMA with a ones operand); the z
      // operands hold content groups 0..7 (lanes j < 2, else the RoPE groups)
      // and 8..15 in fp16 hi (j even) and lo (j odd) parts
      const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
      const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
      float qs[NG_C + NG_R];
#pragma unroll
      for (int g = 0; g < NG_C + NG_R; ++g)
        qs[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, qA[g], zero4, 0, 0, 0)[0];
      const bool lo_part = (j & 1) != 0, lowj = j < 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v1 = lowj ? qs[i] : (i < NG_R ? qs[NG_C + i] : 0.f);
        const float v2 = lowj ? qs[8 + i] : 0.f;
        const _Float16 h1 = (_Float16)v1, h2 = (_Float16)v2;
        qz1[i] = lo_part ? (_Float16)(v1 - (float)h1) : h1;
        qz2[i] = lo_part ? (_Float16)(v2 - (float)h2) : h2;
      }
    }
    float4v M = {M_NONE, M_NONE, M_NONE, M_NONE};  // reference max of heads 4 j + i
    float4v l = {0.f, 0.f, 0.f, 0.f};              // sum of P over the lane's tokens
    __syncthreads();  // step 0 converted
    for (int it = 0; it <= n_steps; ++it) {
      if (it < n_steps) {
        const int buf = it & 1;
        const int p0 = step_p0(it);
        float4v S[2];
        step_scores(sm.code[buf], sm.sz[buf], qA, qz1, qz2, j, t16, S);
        // ---- softmax over the step's 32 tokens, in the wave ----
        bool big = false;
        float4v u[2], t[2];  // scores in log2 units (invalid: -inf) and u - M
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const bool valid = p0 + 16 * tb + t16 < s.Lq;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u[tb][i] = valid ? S[tb][i] * sl2 : -INFINITY;
            t[tb][i] = u[tb][i] - M[i];
            big |= t[tb][i] > TAU;
          }
        }
        const bool move = __builtin_amdgcn_ballot_w64(big) != 0;
        if (move) {
          // the step's maximum per head becomes the reference
          float4v mn, al;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mn[i] = fmaxf(M[i], row_max(fmaxf(u[0][i], u[1][i])));
            al[i] = __builtin_amdgcn_exp2f(M[i] - mn[i]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) t[tb][i] = u[tb][i] - mn[i];
          }
          l *= al;
          M = mn;
          if (t16 == 0) *reinterpret_cast<float4v*>(sm.alpha[buf] + 16 * hb + 4 * j) = al;
        }
        if (lane == 0) sm.flag[buf][hb] = move ? 1 : 0;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          float4v pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(t[tb][i]);
          l += pv;
          u32x2 ph;
          ph.x = as_u32((half2v){(_Float16)pv[0], (_Float16)pv[1]});
          ph.y = as_u32((half2v){(_Float16)pv[2], (_Float16)pv[3]});
          *reinterpret_cast<u32x2*>(sm.p[buf] + (16 * tb + t16) * PT + 16 * hb + 4 * j) = ph;
        }
      }
      __syncthreads();
    }
    // sum of P and reference max per head for the PV waves
    float4v l4 = l;
#pragma unroll
    for (int i = 0; i < 4; ++i) l4[i] = row_sum(l4[i]);
    if (t16 == 0) {
      *reinterpret_cast<float4v*>(sm.lsum + 16 * hb + 4 * j) = l4;
      *reinterpret_cast<float4v*>(sm.mref + 16 * hb + 4 * j) = M;
    }
    __syncthreads();
  } else {
    // ======== converter + PV wave: channel quarter cq, all 64 heads ========
    const int cq = w - 4;
    auto step_rsrc = [&](int st) {
      const int pid = __builtin_amdgcn_readfirstlane(
          st < n_steps ? *(const_i32*)(ptab + i_begin + (st >> 1)) : 0);
      return page_rsrc<F>(a.pages, pid, st < n_steps);
    };
    auto load_step = [&](ConvRaw (&r)[2], int st) {
      const __amdgpu_buffer_rsrc_t rs = step_rsrc(st);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) conv_load<F>(r[tb], rs, ST * (st & 1) + 16 * tb + t16, j, cq);
    };
    auto convert_step = [&](const ConvRaw (&r)[2], int st) {
      const int buf = st & 1;
      const int p0 = step_p0(st);
      const bool mixed = p0 < s.n_s || p0 + ST > min(s.lo_start, s.Lq);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int row = 16 * tb + t16;
        const int p = p0 + row;
        const bool valid = p < s.Lq;
        const uint16_t* brow = nullptr;
        if (mixed && valid && (p < s.n_s || p >= s.lo_start))
          brow = p < s.n_s ? a.sink + ((int64_t)b * a.n_sink + p) * D_ALL
                           : a.local + ((int64_t)b * a.n_local + p % a.n_local) * D_ALL;
        convert_tok<F>(r[tb], sm.code[buf] + row * CT, sm.sz[buf] + row * SZT,
                        sm.val[buf] + row * VT, j, cq, mixed, valid, brow);
      }
    };
    // raw codes of steps of parity 0 and 1, loaded two iterations ahead
    ConvRaw raw0[2], raw1[2];
    load_step(raw0, 0);
    load_step(raw1, 1);
    convert_step(raw0, 0);
    load_step(raw0, 2);
    float4v O[8][4];  // [channel block][head block]: channel 128 cq + 16 cb + 4 j + i, head 16 k + t16
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int k = 0; k < 4; ++k) O[cb][k] = (float4v){0.f, 0.f, 0.f, 0.f};
    const int trow = 8 * j + 2 * (t16 >> 2);
    __syncthreads();  // step 0 converted
    for (int it = 0; it <= n_steps; ++it) {
      if (it >= 1) {
        const int buf = (it - 1) & 1;
        const int4 fl = *reinterpret_cast<const int4*>(sm.flag[buf]);
        if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
          const int fv[4] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (!fv[k]) continue;
            const float al = sm.alpha[buf][16 * k + t16];
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) O[cb][k] *= al;
          }
        }
        half8 pB[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pB[k] = tr_pair(sm.p[buf] + trow * PT + 16 * k + 4 * (t16 & 3),
                          sm.p[buf] + (trow + 1) * PT + 16 * k + 4 * (t16 & 3));
        const _Float16* vt = sm.val[buf];
        half8 av = tr_pair(vt + trow * VT + 128 * cq + 4 * (t16 & 3),
                           vt + (trow + 1) * VT + 128 * cq + 4 * (t16 & 3));
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const half8 cur = av;
          if (cb + 1 < 8) {
            const int col = 128 * cq + 16 * (cb + 1) + 4 * (t16 & 3);
            av = tr_pair(vt + trow * VT + col, vt + (trow + 1) * VT + col);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k)
            O[cb][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur, pB[k], O[cb][k], 0, 0, 0);
        }
      }
      // the next step into the other buffers (this wave's value columns of
      // buffer (k + 1) & 1 were last read by its own PV just above)
      if (it + 1 < n_steps) {
        if ((it + 1) & 1) {
          convert_step(raw1, it + 1);
          load_step(raw1, it + 3);
        } else {
          convert_step(raw0, it + 1);
          load_step(raw0, it + 3);
        }
      }
      __syncthreads();
    }
    __syncthreads();  // sums and maxima of the score waves
    // ---- normalize and write: out directly, or a partial for the combine ----
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int h = 16 * k + t16;  // row within the workgroup's 64
      const float lt = sm.lsum[h];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse_v = lt > 0.f ? (sm.mref[h] + __log2f(lt)) * LN2 : -INFINITY;
      const int64_t orow = (int64_t)v * RG + WR * hh + h;
      if (direct) {
        uint16_t* dst = a.out + orow * D_C + 128 * cq + 4 * j;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const float4v o = O[cb][k] * inv;
          u32x2 pk;
          pk.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
          pk.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
          *reinterpret_cast<u32x2*>(dst + 16 * cb) = pk;
        }
        if (cq == 0 && j == 0) a.lse[orow] = lse_v;
      } else {
        const int64_t prow = (int64_t)slot * RG + WR * hh + h;
        _Float16* dst = a.ws_o + prow * D_C + 128 * cq + 4 * j;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const float4v o = O[cb][k] * inv;
          u32x2 pk;
          pk.x = as_u32((half2v){(_Float16)o[0], (_Float16)o[1]});
          pk.y = as_u32((half2v){(_Float16)o[2], (_Float16)o[3]});
          *reinterpret_cast<u32x2*>(dst + 16 * cb) = pk;
        }
        if (cq == 0 && j == 0) a.ws_lse[prow] = lse_v;
      }
    }
  }
  __syncthreads();  // LDS is reused by the next segment
}

template <int F>
__global__ __launch_bounds__(NT, 1) void decode_wide_kernel(DecodeArgs a) {
  __shared__ WideLds sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int nc_all = gridDim.x >> 1;
  const int c = (int)blockIdx.x % nc_all, hh = (int)blockIdx.x / nc_all;
  const int V = a.B * a.s_q;

  // ---- the chunk of the page line this workgroup owns ----
  const int per = (V + NT - 1) / NT;
  const int v0 = min(V, tid * per), v1 = min(V, v0 + per);
  int my_w = 0;
  for (int v = v0; v < v1; ++v) my_w += seq_weight(a, v).W;
  // exclusive scan over the threads (wave scan, then across the waves)
  int incl = my_w;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sm.scan[w] = incl;
  if (tid == 0) {
    sm.seg_first = 0x7fffffff;
    sm.seg_last = -1;
  }
  __syncthreads();
  int wave_base = 0, W = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    wave_base += k < w ? sm.scan[k] : 0;
    W += sm.scan[k];
  }
  W = __builtin_amdgcn_readfirstlane(W);
  const int my_base = wave_base + incl - my_w;
  const int nce = min(nc_all, max(1, W / 3));  // chunks at least 3 weight units wide
  if (c >= nce) return;  // uniform: no pages for this workgroup
  const int64_t cw0 = (int64_t)c * W / nce, cw1 = (int64_t)(c + 1) * W / nce;
  {
    int P = my_base;
    for (int v = v0; v < v1; ++v) {
      const SeqW s = seq_weight(a, v);
      int o0 = 1, o1 = 0;
      if (s.W > 0) {
        o0 = owner(P, W, nce);
        o1 = owner(P + s.wb(s.n_pages - 1), W, nce);
        if (o0 <= c && c <= o1) {
          atomicMin(&sm.seg_first, v);
          atomicMax(&sm.seg_last, v);
        }
      }
      if (hh == 0 && owner(P, W, nce) == c)
        *reinterpret_cast<int2*>(a.ws_meta + 2 * v) = make_int2(o0, o1);
      P += s.W;
    }
  }
  __syncthreads();
  const int seg_first = __builtin_amdgcn_readfirstlane(sm.seg_first);
  const int seg_last = __builtin_amdgcn_readfirstlane(sm.seg_last);
  if (seg_first >= v0 && seg_first < v1) {
    int P = my_base;
    for (int v = v0; v < seg_first; ++v) P += seq_weight(a, v).W;
    sm.p_first = P;
  }
  __syncthreads();
  int P = __builtin_amdgcn_readfirstlane(sm.p_first);

  for (int v = seg_first; v <= seg_last; ++v) {
    const SeqW s = seq_weight_uniform(a, v);
    if (s.W == 0) continue;
    const int i_begin =
        __builtin_amdgcn_readfirstlane(s.first_page((int)max((int64_t)0, cw0 - P)));
    const int i_end =
        __builtin_amdgcn_readfirstlane(s.first_page((int)min((int64_t)s.W, cw1 - P)));
    const bool direct = __builtin_amdgcn_readfirstlane(
        owner(P, W, nce) == owner(P + s.wb(s.n_pages - 1), W, nce) ? 1 : 0) != 0;
    P += s.W;
    const int b = v / a.s_q;
    const int n_steps = __builtin_amdgcn_readfirstlane(
        min(2 * (i_end - i_begin), (s.Lq - PAGE * i_begin + ST - 1) / ST));
    segment<F>(sm, a, s, v, b, hh, i_begin, n_steps, direct, v + c, w, lane);
  }
}

// Merge the partials of sequences touched by more than one chunk: one wave per
// (sequence, row), 8 channels per lane. Sequences with no token get out = 0 and
// lse = -inf; those written directly by the decode are skipped.
__global__ __launch_bounds__(256) void combine_wide_kernel(DecodeArgs a) {
  const int64_t rowg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // v * 128 + r
  const int V = a.B * a.s_q;
  if (rowg >= (int64_t)V * RG) return;
  const int v = (int)(rowg / RG), r = (int)(rowg % RG);
  const int ch = 8 * (threadIdx.x & 63);
  const int2 m = *reinterpret_cast<const int2*>(a.ws_meta + 2 * v);
  uint16_t* dst = a.out + rowg * D_C + ch;
  if (m.x > m.y) {
    *reinterpret_cast<u32x4*>(dst) = (u32x4){0u, 0u, 0u, 0u};
    if ((threadIdx.x & 63) == 0) a.lse[rowg] = -INFINITY;
    return;
  }
  if (m.x == m.y) return;
  float mx = -INFINITY;
  for (int k = m.x; k <= m.y; ++k) mx = fmaxf(mx, a.ws_lse[(int64_t)(v + k) * RG + r]);
  float l = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = m.x; k <= m.y; ++k) {
    const int64_t prow = (int64_t)(v + k) * RG + r;
    const float ls = a.ws_lse[prow];
    if (ls == -INFINITY) continue;
    const float fw = __expf(ls - mx);
    const half8 o = *reinterpret_cast<const half8*>(a.ws_o + prow * D_C + ch);
    l += fw;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)o[e] * fw;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  u32x4 pk;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    pk[e] = f32_to_bf16_rne(acc[2 * e] * inv) | (f32_to_bf16_rne(acc[2 * e + 1] * inv) << 16);
  *reinterpret_cast<u32x4*>(dst) = pk;
  if ((threadIdx.x & 63) == 0) a.lse[rowg] = l > 0.f ? mx + __logf(l) : -INFINITY;
}

}  // namespace

size_t wide_workspace_bytes(int B, int s_q) {
  const size_t V = (size_t)B * s_q;
  const size_t meta = (V * 8 + 255) / 256 * 256;
  const size_t slots = (size_t)NCH + V;
  return meta + slots * RG * sizeof(float) + slots * RG * D_C * sizeof(_Float16);
}

hipError_t launch_decode_wide(DecodeArgs a, void* workspace, int fmt, hipStream_t stream) {
  const size_t V = (size_t)a.B * a.s_q;
  const size_t meta = (V * 8 + 255) / 256 * 256;
  const size_t slots = (size_t)NCH + V;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  a.ws_meta = reinterpret_cast<int32_t*>(base);
  a.ws_lse = reinterpret_cast<float*>(base + meta);
  a.ws_o = reinterpret_cast<_Float16*>(base + meta + slots * RG * sizeof(float));
  const dim3 grid(2 * NCH);
#define MLA_LAUNCH_WIDE(F) decode_wide_kernel<F><<<grid, dim3(NT), 0, stream>>>(a)
  MLA_FOR_PACKED_FMT(fmt, MLA_LAUNCH_WIDE)
#undef MLA_LAUNCH_WIDE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)V * RG;
  combine_wide_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
