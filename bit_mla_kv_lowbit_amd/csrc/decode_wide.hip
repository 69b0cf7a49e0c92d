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
// A workgroup is 8 wavefronts (two per SIMD, one workgroup per CU) that all do
// the same work on a step of 32 tokens (half a page):
//   convert  each wave takes 16 tokens x a quarter of the blocks: packed
//            codes (loaded two steps ahead) become exact fp16 integers
//            (magic exponent) in a code tile, the scales and zero points go
//            to their tiles, x = c * s + z to the value tile; a protected
//            token's BF16 row enters as fp16 values with (scale, zero) = (1, 0);
//   scores   wave (head block hb, K half kh): S = sum_g s_g (c_g . q_g) +
//            sum_g z_g Q_g for 16 heads over 9 of the 18 blocks, one
//            v_mfma_f32_16x16x32_f16 per (16 tokens, block) on the exact
//            codes, the scale applied on the VALU; the two waves of a head
//            block add their partial sums through LDS;
//   softmax  P = 2^(S scale log2e - M) against a reference max per head that
//            moves only when a score exceeds it by more than 2^8 (then O and
//            l are rescaled); both waves of a head block compute the same P,
//            which stays in registers;
//   PV       wave (hb, kh): O^T of its 16 heads for content channels
//            256 kh .. 256 kh + 255 (64 accumulators per lane), V^T read
//            transposed (ds_read_b64_tr_b16), P the B operand.
// Two barriers per step (partial scores ready; next step converted).
//
// The same kernel decodes the paired BF16 cache the pages normalize their
// latency to (Figure 5(b), Table 9) at 128 heads: its pages' rows enter the
// value buffer as fp16 (exact), and the scores are one plain MFMA chain over
// the values, with no scales, zero points or code tile; chunking, softmax, PV
// and combine are the packed cache's.
#include "mla_common.h"
#include "mla_kernels.h"
#include "decode_ops.h"

namespace mla {
namespace {

constexpr int NT = 512;          // threads per workgroup (8 waves, two per SIMD)
constexpr int WR = 64;           // query rows (heads) per workgroup
constexpr int RG = 128;          // rows per query token on this path
constexpr int ST = 32;           // tokens per step
constexpr int NCH = 128;         // chunks of the page line (workgroups: 2 NCH)
constexpr int NB = NG_C + NG_R;  // 18 blocks of 32 channels per token ([c | k_rope])
constexpr int KH = 9;            // blocks per K half: content 8 kh .. 8 kh + 7 and RoPE block kh
// Row strides in halves, chosen by measuring LDS bank conflicts and the v3
// step time over a range of paddings: code tile 312 dwords, value tile 264
// dwords (8 mod 64: the 8 consecutive rows of 8 dwords that a transposing read
// serves per cycle cover the 64 banks once).
constexpr int CT = D_ALL + 48;
constexpr int VT = D_C + 16;
// z tile row: 8 words per block quarter q (the (z, z) words of content blocks
// 4q .. 4q + 3, then RoPE block q for q < 2), padded to 36 words (36 mod 64:
// 16 consecutive rows hit distinct banks); scale tile rows are ordered the
// same way (5 per quarter).
constexpr int ZW = 36;
constexpr int NSR = 20;          // scale tile rows

// In iteration k the scores of step k read the code, scale and z tiles before
// the first barrier; after it every wave runs the PV product of step k on
// value buffer k & 1 and then converts step k + 1 into the code, scale and z
// tiles and value buffer (k + 1) & 1, which the second barrier publishes.
struct WideLds {
  _Float16 code[ST * CT];          // exact codes (or BF16-row values) of the 18 blocks, token-major
  _Float16 val[2][ST * VT];        // reconstructed content values, token-major
  _Float16 scl[NSR][ST];           // fp16 scale per block (row order above) and token (order below)
  uint32_t zop[ST * ZW];           // per token: (z, z) words, layout above
  float4v xs[NT / 64][2][64];      // each wave's partial scores [token block][lane]
  int seg_first, seg_last, p_first;
  int scan[NT / 64];
};

// Scale tile row of content block g (0..15) and of RoPE block NG_C + q.
__device__ __forceinline__ int scale_row(int g) { return g < NG_C ? 5 * (g >> 2) + (g & 3) : 5 * (g - NG_C) + 4; }

// Position in a scale row of token 16 tb + r (r < 16): the 8 tokens whose
// scores a lane holds (rows 4 (r / 4) .. + 3 of both token blocks) are adjacent.
__device__ __forceinline__ int scale_pos(int row) {
  return 8 * ((row & 15) >> 2) + 4 * (row >> 4) + (row & 3);
}

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
template <int F>
struct ConvRaw {
  u32x4 c, s;
  uint32_t r, rs;
};
// BF16 pages (the paired baseline): the lane's 8 channels of content blocks
// 4 cq .. 4 cq + 3 and of RoPE block cq & 1, as stored
template <>
struct ConvRaw<16> {
  u32x4 c[4];
  u32x4 r;
};

// (A group of 2 or 4 blocks has one (scale, zero) word: it is repeated for
// each of its blocks, so the tiles always hold one word per block.)
template <int F>
__device__ __forceinline__ void conv_load(ConvRaw<F>& t, __amdgpu_buffer_rsrc_t rs, int slot, int j,
                                          int cq) {
  using G = PageGeom<F>;
  if constexpr (F == 16) {
    // token rows of 576 bf16: block g, sub-block j at bytes 64 g + 16 j
#pragma unroll
    for (int e = 0; e < 4; ++e)
      t.c[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, slot * G::ROW + 64 * (4 * cq + e) + 16 * j, 0, 0));
    t.r = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, slot * G::ROW + 2 * D_C + 64 * (cq & 1) + 16 * j, 0, 0));
    return;
  } else {
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
  // RoPE block cq (used for cq < 2; the other quarters load block cq - 2 too,
  // so the loads are unconditional and the prefetch registers need no merge)
  const int rq = cq & 1;
  // 4-bit: word rq of chunk j; 2-bit: both blocks share the chunk's word
  t.r = G::RB == 4 ? __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::RC + 8 * j + 4 * rq, G::OFF_RC, 0)
                   : __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::RC + 4 * j, G::OFF_RC, 0);
  t.rs = __builtin_amdgcn_raw_buffer_load_b32(rs, slot * G::RS + (G::GMR == 1 ? 4 * rq : 0),
                                              G::OFF_RS, 0);
  }
}

// One converter lane's share of a step (token row `row` of the step, sub-block
// j, block quarter cq): exact fp16 codes of blocks 4 cq .. 4 cq + 3 (and RoPE
// block cq when cq < 2) into the code tile; for j = 0 the blocks' fp16 scales
// and (z, z) words into the scale and z tiles; the reconstructed values
// x = c * s + z of its 4 content blocks into value buffer buf. A token with a
// BF16 row (brow) takes its values with (scale, zero) = (1, 0); an invalid
// token zeros.
template <int F>
__device__ __forceinline__ void convert_tok(const ConvRaw<F>& t, WideLds& sm, int buf, int row, int j,
                                            int cq, bool mixed, bool valid, const uint16_t* brow) {
  u32x4 sw;
  uint32_t rsw;
  half8 c[4], r;
  if constexpr (F == 16) {
    // BF16 rows enter as fp16 values (exact) with (scale, zero) = (1, 0)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = bf16x8_to_f16x8(t.c[e]);
      sw[e] = 0x00003C00u;
    }
    r = bf16x8_to_f16x8(t.r);
    rsw = 0x00003C00u;
  } else {
    sw = t.s;
    rsw = t.rs;
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = fmt_cb(F) == 4 ? codes4(t.c[e]) : codes2(t.c[e >> 1], e & 1);
    r = fmt_rb(F) == 4 ? codes4(t.r) : codes2(t.r, cq & 1);
  }
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
  _Float16* crow = sm.code + row * CT;
  _Float16* vrow = sm.val[buf] + row * VT;
  if constexpr (F == 16) {
    // the values are what both products read: content into the value buffer
    // only, RoPE into the code tile; no scales or zero points
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<half8*>(vrow + GROUP * (4 * cq + e) + 8 * j) = c[e];
    if (cq < NG_R) *reinterpret_cast<half8*>(crow + D_C + GROUP * cq + 8 * j) = r;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *reinterpret_cast<half8*>(crow + GROUP * (4 * cq + e) + 8 * j) = c[e];
    *reinterpret_cast<half8*>(vrow + GROUP * (4 * cq + e) + 8 * j) = reconstruct(c[e], sw[e]);
  }
  if (cq < NG_R) *reinterpret_cast<half8*>(crow + D_C + GROUP * cq + 8 * j) = r;
  if (j == 0) {
    _Float16* sc = &sm.scl[5 * cq][scale_pos(row)];
    uint32_t* zr = sm.zop + row * ZW + 8 * cq;
    u32x4 zz;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[ST * e] = as_h2(sw[e]).x;
      zz[e] = (sw[e] & 0xffff0000u) | (sw[e] >> 16);  // (z, z)
    }
    *reinterpret_cast<u32x4*>(zr) = zz;
    if (cq < NG_R) {
      sc[ST * 4] = as_h2(rsw).x;
      zr[4] = (rsw & 0xffff0000u) | (rsw >> 16);
    }
  }
}

// Block k (0..8) of K half kh: content block 8 kh + k, then RoPE block 16 + kh.
__device__ __forceinline__ int half_block(int kh, int k) { return k < 8 ? 8 * kh + k : NG_C + kh; }

// Partial scores of 16 heads (lane: head t16, rows 4 j .. 4 j + 3 of each
// token block) over the wave's K half (its 9 blocks), exactly per block:
// integer codes (or BF16-row values with scale 1) are the MFMA A operand, q the
// B operand, and each block's product is scaled on the VALU; the zero points
// enter through one MFMA per token block whose A operand holds (z, z) per block
// against the (hi, lo) fp16 parts of the group sums of q.
__device__ __forceinline__ void step_scores(const WideLds& sm, int kh,
                                            const half8 (&qA)[KH], const half8& qz, int j,
                                            int t16, float4v (&S)[2]) {
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
  const _Float16* c0 = sm.code + t16 * CT + 8 * j;
  const _Float16* c1 = c0 + 16 * CT;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    // z operand: quarters 2 kh and 2 kh + 1 (j = 0, 1), the RoPE block's
    // word (j = 2; in quarter kh), zeros (j = 3)
    const uint32_t* zr = sm.zop + (16 * tb + t16) * ZW;
    u32x4 zw = *reinterpret_cast<const u32x4*>(zr + (j < 2 ? 16 * kh + 8 * j : 8 * kh + 4));
    if (j >= 2) zw = (u32x4){j == 2 ? zw[0] : 0u, 0u, 0u, 0u};
    S[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, zw), qz, zero4, 0, 0, 0);
  }
  // A operands and scales read PF blocks ahead of their MFMAs (LDS latency)
  constexpr int PF = 2;
  half8 Aw[PF][2], Sw[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    Aw[k][0] = *reinterpret_cast<const half8*>(c0 + GROUP * half_block(kh, k));
    Aw[k][1] = *reinterpret_cast<const half8*>(c1 + GROUP * half_block(kh, k));
    Sw[k] = *reinterpret_cast<const half8*>(sm.scl[scale_row(half_block(kh, k))] + 8 * j);
  }
#pragma unroll
  for (int k = 0; k < KH; ++k) {
    const half8 A0 = Aw[k % PF][0], A1 = Aw[k % PF][1], sc = Sw[k % PF];
    if (k + PF < KH) {
      Aw[k % PF][0] = *reinterpret_cast<const half8*>(c0 + GROUP * half_block(kh, k + PF));
      Aw[k % PF][1] = *reinterpret_cast<const half8*>(c1 + GROUP * half_block(kh, k + PF));
      Sw[k % PF] = *reinterpret_cast<const half8*>(sm.scl[scale_row(half_block(kh, k + PF))] + 8 * j);
    }
    const float4v D0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qA[k], zero4, 0, 0, 0);
    const float4v D1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qA[k], zero4, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[0][i] += (float)sc[i] * D0[i];
      S[1][i] += (float)sc[4 + i] * D1[i];
    }
  }
}

// Partial scores of the BF16 baseline, in the same lane layout: the values
// (content from value buffer vt, RoPE from the code tile) are the A operand of
// one MFMA chain over the wave's 9 blocks; there is no scale or zero point.
__device__ __forceinline__ void step_scores_bf16(const WideLds& sm, const _Float16* vt, int kh,
                                                 const half8 (&qA)[KH], int j, int t16,
                                                 float4v (&S)[2]) {
  S[0] = S[1] = (float4v){0.f, 0.f, 0.f, 0.f};
  const _Float16* v0 = vt + t16 * VT + 8 * j;
  const _Float16* r0 = sm.code + t16 * CT + D_C + GROUP * kh + 8 * j;
#pragma unroll
  for (int k = 0; k < KH; ++k) {
    const _Float16* p = k < 8 ? v0 + GROUP * (8 * kh + k) : r0;
    const int stride = k < 8 ? 16 * VT : 16 * CT;
    const half8 A0 = *reinterpret_cast<const half8*>(p);
    const half8 A1 = *reinterpret_cast<const half8*>(p + stride);
    S[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qA[k], S[0], 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qA[k], S[1], 0, 0, 0);
  }
}

// One segment: pages [i_begin, i_begin + n_steps / 2) of (sequence, query
// token) v, heads 64 hh .. 64 hh + 63. Wave w scores head block hb = w & 3
// over K half kh = w >> 2 and accumulates O^T of those 16 heads for content
// channels 256 kh .. 256 kh + 255; it also converts token block w >> 2, block
// quarter w & 3 of every step. The two waves of a head block add their
// partial scores through LDS (the same sum in both, so both take the same
// softmax decisions and hold the same P, which stays in registers as the B
// operand of the PV product). Iteration k: scores of step k, barrier, softmax
// and PV of step k, conversion of step k + 1, barrier.
template <int F>
__device__ __forceinline__ void segment(WideLds& sm, const DecodeArgs& a, const SeqW& s, int v,
                                        int b, int hh, int i_begin, int n_steps, bool direct,
                                        int slot, int w, int lane) {
  const int j = lane >> 4, t16 = lane & 15;
  const int hb = w & 3, kh = w >> 2;
  const int crow = 16 * (w >> 2) + t16, cq = w & 3;  // converter: token row, block quarter
  auto step_p0 = [&](int st) { return PAGE * (i_begin + (st >> 1)) + ST * (st & 1); };
  // Page ids come through vector loads (in order with the code loads, so a
  // prefetched id is waited for precisely; a scalar load would be waited for
  // with every LDS access after it), two iterations ahead of their use.
  const __amdgpu_buffer_rsrc_t pt_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.page_table + (int64_t)b * a.max_pages), (short)0, a.max_pages * 4, 0x00020000);
  auto pid_load = [&](int st) {  // page id of step st (0 past the page table: range-checked offset)
    return __builtin_amdgcn_raw_buffer_load_b32(pt_rs, 4 * (i_begin + (st >> 1)), 0, 0);
  };
  auto load_step = [&](ConvRaw<F>& r, int st, uint32_t pid) {
    const __amdgpu_buffer_rsrc_t rs =
        page_rsrc<F>(a.pages, __builtin_amdgcn_readfirstlane(pid), st < n_steps);
    conv_load<F>(r, rs, ST * (st & 1) + crow, j, cq);
  };
  auto convert_step = [&](const ConvRaw<F>& r, int st) {
    const int p0 = step_p0(st);
    const bool mixed = p0 < s.n_s || p0 + ST > min(s.lo_start, s.Lq);
    const int p = p0 + crow;
    const bool valid = p < s.Lq;
    const uint16_t* brow = nullptr;
    if constexpr (F != 16) {  // the BF16 baseline has no protected buffers
      if (mixed && valid && (p < s.n_s || p >= s.lo_start))
        brow = p < s.n_s ? a.sink + ((int64_t)b * a.n_sink + p) * D_ALL
                         : a.local + ((int64_t)b * a.n_local + p % a.n_local) * D_ALL;
    }
    convert_tok<F>(r, sm, st & 1, crow, j, cq, mixed, valid, brow);
  };

  // ---- Q operands of the wave's 9 blocks and its z operand ----
  const float sl2 = a.scale_log2;
  const int64_t qrow = (int64_t)v * RG + WR * hh + 16 * hb + t16;
  half8 qA[KH];
  half8 qz;
  {
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const int g = half_block(kh, k);
      const uint16_t* src = g < NG_C ? a.q_lat + qrow * D_C + GROUP * g + 8 * j
                                     : a.q_rope + qrow * D_R + GROUP * (g - NG_C) + 8 * j;
      qA[k] = bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(src));
    }
    // group sums of head t16 (one MFMA with a ones operand each); the z
    // operand word 4 j + e of the lane holds (hi, lo) of the sum of half block
    // 4 j + e (j < 2: content blocks; word 8: the RoPE block)
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
    float qs[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k)
      qs[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, qA[k], zero4, 0, 0, 0)[0];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = j == 0 ? qs[e] : j == 1 ? qs[4 + e] : (j == 2 && e == 0) ? qs[8] : 0.f;
      const _Float16 hi = (_Float16)q;
      qz[2 * e] = hi;
      qz[2 * e + 1] = (_Float16)(q - (float)hi);
    }
  }

  // ---- raw data of steps of parity 0 and 1, loaded two iterations ahead ----
  ConvRaw<F> raw0, raw1;
  load_step(raw0, 0, pid_load(0));
  load_step(raw1, 1, pid_load(1));
  convert_step(raw0, 0);
  load_step(raw0, 2, pid_load(2));
  uint32_t pid1 = pid_load(3), pid0 = pid_load(4);  // next ids for raw1 / raw0
  float4v O[16];  // channel 256 kh + 16 cb + 4 j + i of head t16
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) O[cb] = (float4v){0.f, 0.f, 0.f, 0.f};
  float M = M_NONE;  // reference max of head t16 (log2 units)
  float l = 0.f;     // sum of P over the lane's tokens
  const int tr_lo = (4 * j + (t16 >> 2)) * VT + 4 * (t16 & 3) + 256 * kh;
  const int tr_hi = tr_lo + 16 * VT;
  __syncthreads();  // step 0 converted

  // One iteration; rnext holds the raw data of step it + 1 and is reloaded
  // with step it + 3, whose page id pnext was loaded two iterations ago (the
  // loads are unconditional: past the last step the page descriptor has an
  // empty range). Called with raw1 and raw0 in turn, so each prefetch lands in
  // fixed registers.
  auto iteration = [&](int it, ConvRaw<F>& rnext, uint32_t& pnext) {
    const int buf = it & 1;
    const int p0 = step_p0(it);
    float4v S[2];
    if constexpr (F == 16) step_scores_bf16(sm, sm.val[buf], kh, qA, j, t16, S);
    else step_scores(sm, kh, qA, qz, j, t16, S);
    sm.xs[w][0][lane] = S[0];
    sm.xs[w][1][lane] = S[1];
    __syncthreads();  // partial scores of both K halves
    S[0] += sm.xs[w ^ 4][0][lane];
    S[1] += sm.xs[w ^ 4][1][lane];
    // ---- softmax over the step's 32 tokens (the same in both waves of the pair) ----
    bool big = false;
    float u[2][4], t[2][4];  // scores in log2 units (invalid: -inf) and u - M
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = p0 + 16 * tb + 4 * j + i < s.Lq;
        u[tb][i] = valid ? S[tb][i] * sl2 : -INFINITY;
        t[tb][i] = u[tb][i] - M;
        big |= t[tb][i] > TAU;
      }
    }
    if (__builtin_amdgcn_ballot_w64(big) != 0) {
      // the step's maximum per head becomes the reference (lanes t16 + 16 j
      // hold the same head)
      float m8 = u[0][0];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) m8 = fmaxf(m8, u[tb][i]);
      m8 = fmaxf(m8, __shfl_xor(m8, 16, 64));
      m8 = fmaxf(m8, __shfl_xor(m8, 32, 64));
      const float mn = fmaxf(M, m8);
      const float al = __builtin_amdgcn_exp2f(M - mn);
      l *= al;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) O[cb] *= al;
      M = mn;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) t[tb][i] = u[tb][i] - M;
    }
    half8 pB;  // K slot 4 tb + i: token 16 tb + 4 j + i
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(t[tb][i]);
        l += pv;
        pB[4 * tb + i] = (_Float16)pv;
      }
    // ---- PV: O^T += V^T P over the step's 32 tokens ----
    const _Float16* vt = sm.val[buf];
    half8 av = tr_pair(vt + tr_lo, vt + tr_hi);
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
      const half8 cur = av;
      if (cb + 1 < 16) av = tr_pair(vt + tr_lo + 16 * (cb + 1), vt + tr_hi + 16 * (cb + 1));
      O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur, pB, O[cb], 0, 0, 0);
    }
    // the next step into the code, scale and z tiles (every wave's scores of
    // this step are done) and the other value buffer (last read by the PV
    // product of step it - 1)
    if (it + 1 < n_steps) convert_step(rnext, it + 1);
    load_step(rnext, it + 3, pnext);
    pnext = pid_load(it + 5);
    __syncthreads();  // step it + 1 converted; every wave is done with the partials
  };
  for (int it = 0; it < n_steps; it += 2) {
    iteration(it, raw1, pid1);
    if (it + 1 < n_steps) iteration(it + 1, raw0, pid0);
  }

  // ---- normalize and write: out directly, or a partial for the combine ----
  float lt = l + __shfl_xor(l, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (M + __log2f(lt)) * LN2 : -INFINITY;
  const int h = 16 * hb + t16;  // row within the workgroup's 64
  const int64_t orow = (int64_t)v * RG + WR * hh + h;
  if (direct) {
    uint16_t* dst = a.out + orow * D_C + 256 * kh + 4 * j;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
      const float4v o = O[cb] * inv;
      u32x2 pk;
      pk.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
      pk.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
      *reinterpret_cast<u32x2*>(dst + 16 * cb) = pk;
    }
    if (kh == 0 && j == 0) a.lse[orow] = lse_v;
  } else {
    const int64_t prow = (int64_t)slot * RG + WR * hh + h;
    _Float16* dst = a.ws_o + prow * D_C + 256 * kh + 4 * j;
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
      const float4v o = O[cb] * inv;
      u32x2 pk;
      pk.x = as_u32((half2v){(_Float16)o[0], (_Float16)o[1]});
      pk.y = as_u32((half2v){(_Float16)o[2], (_Float16)o[3]});
      *reinterpret_cast<u32x2*>(dst + 16 * cb) = pk;
    }
    if (kh == 0 && j == 0) a.ws_lse[prow] = lse_v;
  }
  __syncthreads();  // LDS is reused by the next segment
}

template <int F>
__global__ __launch_bounds__(NT, 1) void decode_wide_kernel(DecodeArgs a) {
  __shared__ WideLds sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // the z tile's padding words stay zero
  for (int i = tid; i < ST * ZW; i += NT) sm.zop[i] = 0u;
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
  if (fmt == 16) {
    decode_wide_kernel<16><<<grid, dim3(NT), 0, stream>>>(a);
  } else {
#define MLA_LAUNCH_WIDE(F) decode_wide_kernel<F><<<grid, dim3(NT), 0, stream>>>(a)
    MLA_FOR_PACKED_FMT(fmt, MLA_LAUNCH_WIDE)
#undef MLA_LAUNCH_WIDE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)V * RG;
  combine_wide_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
