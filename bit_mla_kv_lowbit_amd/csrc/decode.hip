// Absorbed-MLA decode over the mixed BF16 / packed low-bit cache, for gfx950.
//
// QuantMLA (Figure 8 caption; abstract): attention unpacks and dequantizes the
// packed codes itself, takes protected sink / recent tokens from BF16 buffers,
// uses one reconstructed content tile for both the matching (QK) and the
// aggregation (PV) product, and normalizes all valid tokens with one softmax.
// The decode is the absorbed (MQA) form: all heads share the latent (GQLA card).
//
// Work decomposition: one workgroup of 8 wavefronts (two per SIMD) = one
// (sequence, page range, 16-head block); the range is walked one 64-token page
// per iteration, the next page's codes being loaded into registers while the
// current one is used. Wave w takes the 16 tokens 16 (w & 3) .. +15 of the page
// and half of the code groups (set w >> 2: content groups 8s .. 8s + 7 and RoPE
// group s); lane (token t, sub-block j) holds the 8-channel sub-block j of each
// of those groups (the code order makes one 128-bit load deliver one sub-block
// of 4 (INT4) or 8 (INT2) groups). Per page:
//   1. partial scores, exactly per group: the integer codes c (exact in fp16)
//      are the B operand of v_mfma_f32_16x16x32_f16, one MFMA per 32-channel
//      group gives D_g = q_g . c_g; then S = sum_g s_g D_g + sum_g z_g Q_g in
//      fp32, with Q_g = sum of q over group g (the z term is one more MFMA with
//      Q_g split into fp16 hi + lo). Rounding the reconstructed keys to fp16
//      first would cost ~1e-3 in the scores of wide-range (outlier) groups;
//   2. the reconstructed content values x = c * s + z (one packed fp16 FMA per
//      channel pair) go to an LDS tile, token-major; the two partial scores of
//      each token to a small LDS array;
//   3. softmax once per head (wave w owns heads 2w, 2w + 1): running max and
//      sum in the log2 domain, P in fp16 and each head's rescale factor to LDS;
//   4. wave w accumulates O^T for channels 64w .. 64w + 63: the V^T operand is
//      read from the token-major tile with ds_read_b64_tr_b16, P^T from LDS.
// One extra workgroup per (sequence, head block) attends over the BF16-protected
// tokens the same way (the page workgroups mask them out). The partials (O / l,
// log-sum-exp) of all workgroups of a sequence are merged by combine_kernel
// (split-K over the sequence with an LSE combine: one global softmax).
#include "mla_common.h"
#include "mla_kernels.h"

#include <type_traits>

namespace mla {

constexpr float LN2 = 0.69314718055994530942f;
constexpr uint32_t MAGIC = 0x64006400u;  // fp16 pair (1024, 1024)
constexpr uint32_t ONE_ZERO = 0x00003C00u;  // (s, z) = (1.0, 0.0): a BF16 token

typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int SXS = PAGE + 4;  // floats per partial-score row
constexpr int PS = PAGE + 8;   // halves per P row

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// (a & m) | o in one VALU op (the compiler otherwise emits an and plus an or)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// Raw data one lane loads for one page: sub-block j of its token in each of the
// wave's 9 code groups, and those groups' (scale, zero) words.
template <int CB>
struct PageRegs {
  u32x4 c[CB == 4 ? 2 : 1];  // content code chunks (8 groups)
  u32x4 sz[2];               // content (s, z) words of the 8 groups
  uint32_t r;                // RoPE code word (group 16 + set)
  uint32_t rsz;              // RoPE (s, z) word
};

// Byte offsets, inside a page, of what one lane (slot, sub-block j, set gs) loads.
template <int CB>
struct LaneOffsets {
  uint32_t c, s, r, rs;
  __device__ LaneOffsets(int slot, int j, int gs) {
    using G = PageGeom<CB>;
    c = G::OFF_CC + slot * G::CC + (CB == 4 ? 128 : 64) * gs + 16 * j;
    s = G::OFF_CS + slot * G::CS + 32 * gs;
    r = G::OFF_RC + slot * G::RC + 8 * j + 4 * gs;
    rs = G::OFF_RS + slot * G::RS + 4 * gs;
  }
};

// Buffer descriptor of one physical page (raw byte addressing, range = page).
template <int CB>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* pages, int pid,
                                                            bool any = true) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(pages + (int64_t)pid * PageGeom<CB>::BYTES), (short)0,
      any ? PageGeom<CB>::BYTES : 0, 0x00020000);
}

template <int CB>
__device__ __forceinline__ void load_page(PageRegs<CB>& t, __amdgpu_buffer_rsrc_t rs,
                                          const LaneOffsets<CB>& o) {
#pragma unroll
  for (int m = 0; m < (CB == 4 ? 2 : 1); ++m)
    t.c[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.c + 64 * m, 0, 0));
#pragma unroll
  for (int m = 0; m < 2; ++m)
    t.sz[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.s + 16 * m, 0, 0));
  t.r = __builtin_amdgcn_raw_buffer_load_b32(rs, o.r, 0, 0);
  t.rsz = __builtin_amdgcn_raw_buffer_load_b32(rs, o.rs, 0, 0);
}

// Exact codes of channels 8j..8j+7 (pairs (0,1) (2,3) (4,5) (6,7)) of one group
// from its code word. Codes at bit offsets below 10 are turned into fp16
// 1024 + 2^o * c with one and-or, then back to c with one exact packed FMA.
__device__ __forceinline__ half8 codes4(uint32_t wd) {
  const half2v m1024 = as_h2(0xE400E400u);  // -1024
  const half2v r16 = as_h2(0x2C002C00u);    // 1/16
  const half2v m64 = as_h2(0xD400D400u);    // -64
  const uint32_t t = wd >> 8;
  const half2v p0 = as_h2(and_or(wd, 0x000F000Fu, MAGIC)) + m1024;
  const half2v p1 = __builtin_elementwise_fma(as_h2(and_or(wd, 0x00F000F0u, MAGIC)), r16, m64);
  const half2v p2 = as_h2(and_or(t, 0x000F000Fu, MAGIC)) + m1024;
  const half2v p3 = __builtin_elementwise_fma(as_h2(and_or(t, 0x00F000F0u, MAGIC)), r16, m64);
  return (half8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Same for 2-bit codes: code block e of the word (pairs at bits 8e + 2i, 24 + ... ).
__device__ __forceinline__ half8 codes2(uint32_t wd, int e) {
  const uint32_t t = e ? wd >> 8 : wd;
  const half2v m1024 = as_h2(0xE400E400u);
  const half2v r4 = as_h2(0x34003400u), m256 = as_h2(0xDC00DC00u);    // 1/4, -256
  const half2v r16 = as_h2(0x2C002C00u), m64 = as_h2(0xD400D400u);    // 1/16, -64
  const half2v r64 = as_h2(0x24002400u), m16 = as_h2(0xCC00CC00u);    // 1/64, -16
  const half2v p0 = as_h2(and_or(t, 0x00030003u, MAGIC)) + m1024;
  const half2v p1 = __builtin_elementwise_fma(as_h2(and_or(t, 0x000C000Cu, MAGIC)), r4, m256);
  const half2v p2 = __builtin_elementwise_fma(as_h2(and_or(t, 0x00300030u, MAGIC)), r16, m64);
  const half2v p3 = __builtin_elementwise_fma(as_h2(and_or(t, 0x00C000C0u, MAGIC)), r64, m16);
  return (half8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Codes of local group lg (0..7: content group 8 set + lg; 8: RoPE group).
template <int CB>
__device__ __forceinline__ half8 group_codes(const PageRegs<CB>& t, int lg) {
  if (lg == 8) return codes4(t.r);
  if (CB == 4) return codes4(t.c[lg >> 2][lg & 3]);
  return codes2(t.c[0][lg >> 1], lg & 1);
}

template <int CB>
__device__ __forceinline__ uint32_t group_sz(const PageRegs<CB>& t, int lg) {
  return lg == 8 ? t.rsz : t.sz[lg >> 2][lg & 3];
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

// LDS tile of reconstructed content values, 64 token rows x 512 fp16. The
// 16-byte chunk index of each row is XOR-ed with f(row) so that (64 banks of
// 4 bytes): a transposing read (8 rows 8j + x or 8j + 4 + x, x < 4, per 32
// lanes, 32 bytes each) hits 8 distinct 32-byte bank segments (f bits 1..3 =
// row bits 0, 1, 3; f bit 0 = row bit 2 is constant within one read), and a
// row write (16 consecutive rows, one chunk each) hits 16 distinct chunks.
__device__ __forceinline__ int tile_off(int row, int ch) {
  const int f = ((row >> 2) & 1) | ((row & 3) << 1) | (((row >> 3) & 1) << 3);
  return row * D_C + (((ch >> 3) ^ f) << 3) + (ch & 7);
}

// Channel (in the [content | rope] row) of sub-block j of local group lg of set gs.
__device__ __forceinline__ int group_channel(int lg, int gs, int j) {
  return lg < 8 ? GROUP * (8 * gs + lg) + 8 * j : D_C + GROUP * gs + 8 * j;
}

// Softmax and PV state of one wave.
struct AttnState {
  float4v oacc[4];     // O^T of channels 64w + 16mb + 4j + i, head t16
  float m_run, l_run;  // running max (log2 domain) and sum of head hh (waves 0, 1)
};

// O^T[64 channels of wave w x 16 heads] += V^T P^T over one page's 64 tokens,
// after rescaling by the page's factor; V^T is read transposed from the tile.
// The eight MFMAs are issued one per code group from inside the next page's
// score loop (pv_step), so their LDS reads and MFMA latency hide under the
// score arithmetic.
struct PvCtx {
  const _Float16* tile;
  half8 pB[2];
};

__device__ __forceinline__ void pv_begin(PvCtx& c, AttnState& st, const _Float16* tile,
                                         const _Float16* plds, const float* alds, int j,
                                         int t16) {
  const float alpha = alds[t16];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) st.oacc[mb] *= alpha;
  c.tile = tile;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    c.pB[kb] = *reinterpret_cast<const half8*>(plds + t16 * PS + 32 * kb + 8 * j);
}

__device__ __forceinline__ void pv_step(AttnState& st, const PvCtx& c, int i, int w, int j,
                                        int t16) {
  const int mb = i >> 1, kb = i & 1;
  const int trow = 32 * kb + 8 * j + (t16 >> 2);
  const int col = 64 * w + 16 * mb + 4 * (t16 & 3);
  const short4v lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(c.tile + tile_off(trow, col)));
  const short4v hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(c.tile + tile_off(trow + 4, col)));
  const half4 l4 = __builtin_bit_cast(half4, lo), h4 = __builtin_bit_cast(half4, hi);
  const half8 av = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
  st.oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, c.pB[kb], st.oacc[mb], 0, 0, 0);
}

// Partial scores of one wave (S[i]: head 4j + i, its token) over its 9 groups,
// plus the content tile rows of those groups. MASKED: a token with keep false
// (protected, past the end or past the range) gets zero (scale, zero) words, so
// its codes contribute 0, and a -inf score.
template <int CB, bool MASKED, bool PV>
__device__ __forceinline__ float4v packed_scores(PageRegs<CB>& t, const half8 (&qA)[9],
                                                 const half8& qz, _Float16* tile, int row,
                                                 int gs, int j, bool keep, AttnState& st,
                                                 const PvCtx& pv, int w, int t16) {
  if (MASKED) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) t.sz[m][e] = keep ? t.sz[m][e] : 0u;
    t.rsz = keep ? t.rsz : 0u;
  }
  // z term: lanes j = 0, 1 carry the z of the 8 content groups (matching the hi
  // and lo parts of Q_g in qz), lanes j = 2, 3 the RoPE group's z in slot 0
  half8 zb;
  {
    const half2v h0 = as_h2(__builtin_amdgcn_perm(t.sz[0].y, t.sz[0].x, 0x07060302u));
    const half2v h1 = as_h2(__builtin_amdgcn_perm(t.sz[0].w, t.sz[0].z, 0x07060302u));
    const half2v h2 = as_h2(__builtin_amdgcn_perm(t.sz[1].y, t.sz[1].x, 0x07060302u));
    const half2v h3 = as_h2(__builtin_amdgcn_perm(t.sz[1].w, t.sz[1].z, 0x07060302u));
    const _Float16 zr = as_h2(t.rsz).y;
    const bool content = j < 2;
    zb = (half8){content ? h0.x : zr, content ? h0.y : (_Float16)0.f,
                 content ? h1.x : (_Float16)0.f, content ? h1.y : (_Float16)0.f,
                 content ? h2.x : (_Float16)0.f, content ? h2.y : (_Float16)0.f,
                 content ? h3.x : (_Float16)0.f, content ? h3.y : (_Float16)0.f};
  }
  float4v S = {0.f, 0.f, 0.f, 0.f};
  S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz, zb, S, 0, 0, 0);
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int lg = 0; lg < 9; ++lg) {
    if (PV && lg < 8) pv_step(st, pv, lg, w, j, t16);
    const half8 c = group_codes<CB>(t, lg);
    const uint32_t sz = group_sz<CB>(t, lg);
    const float4v D = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[lg], c, zero4, 0, 0, 0);
    S += (float)as_h2(sz).x * D;
    if (lg < 8)
      *reinterpret_cast<half8*>(tile + tile_off(row, group_channel(lg, gs, j))) = reconstruct(c, sz);
  }
  if (MASKED && !keep) S = (float4v){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  return S;
}

// Partial scores and tile rows of a BF16 token (exact in fp16): one MFMA chain
// over the wave's 9 groups; the 9 row pieces are loaded before use. Invalid
// tokens read a valid row (in bounds) and are then zeroed / set to -inf.
template <bool PV>
__device__ __forceinline__ float4v bf16_scores(const uint16_t* rowp, bool valid,
                                               const half8 (&qA)[9], _Float16* tile, int row,
                                               int gs, int j, AttnState& st, const PvCtx& pv,
                                               int w, int t16) {
  u32x4 raw[9];
#pragma unroll
  for (int lg = 0; lg < 9; ++lg)
    raw[lg] = *reinterpret_cast<const u32x4*>(rowp + group_channel(lg, gs, j));
  float4v S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int lg = 0; lg < 9; ++lg) {
    if (PV && lg < 8) pv_step(st, pv, lg, w, j, t16);
    half8 kv = bf16x8_to_f16x8(raw[lg]);
    kv = valid ? kv : (half8){};
    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[lg], kv, S, 0, 0, 0);
    if (lg < 8) *reinterpret_cast<half8*>(tile + tile_off(row, group_channel(lg, gs, j))) = kv;
  }
  if (!valid) S = (float4v){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  return S;
}



// Reductions over the 8 lanes of an aligned octet with DPP lane moves (no LDS
// round trip): swap neighbours, swap pairs, then mirror within the half-row.
__device__ __forceinline__ float octet_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)));
  return v;
}
__device__ __forceinline__ float octet_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

// Softmax of one page, once per head, by waves 0 and 1 (lane: head
// hh = 8w + lane / 8, tokens 8 tl .. 8 tl + 7 with tl = lane % 8), from the two
// partial scores in LDS; writes P (fp16) and each head's rescale factor.
__device__ __forceinline__ void softmax_page(AttnState& st, const float* sxp, _Float16* plds,
                                             float* alds, int hh, int tl, float sl2) {
  float sv[8];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const float4v a0 = *reinterpret_cast<const float4v*>(sxp + hh * SXS + 8 * tl + 4 * h2);
    const float4v a1 = *reinterpret_cast<const float4v*>(sxp + (16 + hh) * SXS + 8 * tl + 4 * h2);
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[4 * h2 + i] = a0[i] + a1[i];
  }
  float mx = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
  mx = octet_max(mx);
  const float m_new = fmaxf(st.m_run, mx * sl2);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_use);
  half8 ph;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float pv = __builtin_amdgcn_exp2f(fmaf(sv[i], sl2, -m_use));
    psum += pv;
    ph[i] = (_Float16)pv;
  }
  psum = octet_sum(psum);
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
  *reinterpret_cast<half8*>(plds + hh * PS + 8 * tl) = ph;
  if (tl == 0) alds[hh] = alpha;
}

// Work items of a sequence: its packed pages (the pages that hold packed
// tokens, protected tokens in them masked out), then its BF16-protected tokens
// (sink, then recent window) in chunks of 64. Workgroup `split` takes items
// [split * ipp, (split + 1) * ipp) with ipp = ceil(items / n_split), and writes
// one partial (O / l, lse) that combine_kernel merges.
template <int CB>
__global__ __launch_bounds__(512, 1) void decode_h16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 tile[2 * PAGE * D_C];
  __shared__ __attribute__((aligned(16))) float sxp[32 * SXS];
  __shared__ __attribute__((aligned(16))) _Float16 plds[2 * 16 * PS];
  __shared__ float alds[16];
  __shared__ int pids[MAX_ITEMS];  // physical pages of this workgroup's packed items

  // Workgroup -> (page range u = (b, split), head block hb). Consecutive
  // workgroups go to the 8 XCDs in turn, and each XCD has its own L2: the head
  // blocks of one page range get ids that are equal mod 8, so the page range is
  // read from HBM once and served from that XCD's L2 to the other head blocks.
  const int n_hb = a.H / 16;
  const int gsz = 8 * n_hb;
  const int u = (int)(blockIdx.x / gsz) * 8 + (int)(blockIdx.x % 8);
  if (u >= a.B * a.n_split) return;  // padding of the last group of 8 ranges
  const int hb = (int)(blockIdx.x % gsz) / 8;
  const int b = u / a.n_split, split = u % a.n_split;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int lane = tid & 63, j = lane >> 4, t16 = lane & 15;
  const int gs = w >> 2;                  // code-group set of this wave
  const int row = 16 * (w & 3) + t16;     // token row of this lane in the page / tile
  const int hh = 8 * (w & 1) + (lane >> 3);  // softmax (waves 0, 1): head of this lane
  const int tl = lane & 7;                   // softmax: tokens 8 tl .. 8 tl + 7
  const int H = a.H;
  const int h = hb * 16 + t16;
  // lengths are clamped to what the page table can hold
  const int L = min(max(a.seq_lens[b], 0), a.max_pages * PAGE);
  const float sl2 = a.scale_log2;

  // items of this sequence and of this workgroup
  const int lo_p = a.n_sink, hi_p = L - a.n_local;       // packed: lo_p <= p < hi_p
  const int n_pp = hi_p > lo_p ? (hi_p + PAGE - 1) / PAGE : 0;
  const int n_s = min(a.n_sink, L);
  const int lo_start = max(a.n_sink, L - a.n_local);
  const int n_prot = n_s + max(0, L - lo_start);
  const int n_items = n_pp + (n_prot + PAGE - 1) / PAGE;
  const int ipp = (n_items + a.n_split - 1) / a.n_split;
  const int it0 = min(split * ipp, n_items), it1 = min(it0 + ipp, n_items);
  const int n_it = it1 - it0;
  const int n_pk = max(0, min(it1, n_pp) - it0);  // packed items of this workgroup

  // Q as the A operand for the wave's 9 groups (lane = head t16; channels
  // 8j .. 8j + 7 of each group), and qz: the z-term A operand holding the group
  // sums Q_g split into fp16 hi (lanes j = 0, 2) and lo (j = 1, 3) parts, content
  // groups in lanes j < 2, the RoPE group in slot 0 of lanes j >= 2.
  half8 qA[9];
  half8 qz;
  {
    const uint16_t* qrow_l = a.q_lat + ((int64_t)b * H + h) * D_C;
    const uint16_t* qrow_r = a.q_rope + ((int64_t)b * H + h) * D_R;
    u32x4 raw[9];
#pragma unroll
    for (int lg = 0; lg < 9; ++lg) {
      const int ch = group_channel(lg, gs, j);
      raw[lg] = *reinterpret_cast<const u32x4*>(ch < D_C ? qrow_l + ch : qrow_r + (ch - D_C));
    }
    float qs[9];
#pragma unroll
    for (int lg = 0; lg < 9; ++lg) {
      qA[lg] = bf16x8_to_f16x8(raw[lg]);
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sum += bf16_to_f32(raw[lg][e] & 0xffffu) + bf16_to_f32(raw[lg][e] >> 16);
      qs[lg] = sum;
    }
#pragma unroll
    for (int lg = 0; lg < 9; ++lg) {
      qs[lg] += __shfl_xor(qs[lg], 16);
      qs[lg] += __shfl_xor(qs[lg], 32);
    }
    const bool lo_part = (j & 1) != 0, content = j < 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = content ? qs[i] : (i == 0 ? qs[8] : 0.f);
      const _Float16 hi = (_Float16)v;
      qz[i] = lo_part ? (_Float16)(v - (float)hi) : hi;
    }
  }

  AttnState st;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) st.oacc[mb] = (float4v){0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  if (tid < n_pk) pids[tid] = a.page_table[(int64_t)b * a.max_pages + it0 + tid];
  __syncthreads();

  // Packed items: the page after the one being scored is in flight. Loads
  // past the packed items repeat the last packed page; with no packed item the
  // descriptor has an empty range (loads return 0, touch nothing). The loads
  // stay unconditional so the wait counts are static and a wait for one page
  // never waits for the prefetch issued after it.
  const LaneOffsets<CB> lo(row, j, gs);
  auto page_at = [&](int k) {
    const int pid = __builtin_amdgcn_readfirstlane(pids[max(0, min(k, n_pk - 1))]);
    return page_rsrc<CB>(a.pages, n_pk > 0 ? pid : 0, n_pk > 0);
  };
  auto score_item = [&](PageRegs<CB>& cur, int k, _Float16* tbuf, const PvCtx& pv,
                        auto pv_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    const int item = it0 + k;
    if (item < n_pp) {
      const int p0 = item * PAGE;
      if (p0 >= lo_p && p0 + PAGE <= hi_p)
        return packed_scores<CB, false, PV>(cur, qA, qz, tbuf, row, gs, j, true, st, pv, w, t16);
      const int p = p0 + row;
      return packed_scores<CB, true, PV>(cur, qA, qz, tbuf, row, gs, j, p >= lo_p && p < hi_p, st,
                                         pv, w, t16);
    }
    // BF16-protected tokens: q < n_s are the sink tokens, the rest the recent
    // window lo_start .. L - 1 (ring slots p mod n_local)
    const int q = (item - n_pp) * PAGE + row;
    const bool valid = q < n_prot;
    const int qc = min(q, n_prot - 1);
    const uint16_t* rowp =
        qc < n_s ? a.sink + ((int64_t)b * a.n_sink + qc) * D_ALL
                 : a.local + ((int64_t)b * a.n_local + (lo_start + qc - n_s) % a.n_local) * D_ALL;
    return bf16_scores<PV>(rowp, valid, qA, tbuf, row, gs, j, st, pv, w, t16);
  };

  // Pipeline: the PV product of item k runs inside the score loop of item
  // k + 1 (double-buffered tile and P), so the MFMA / LDS work of one overlaps
  // the VALU work of the other; two barriers per item. Two register sets: the
  // set that held item k is reloaded with item k + 2 at the start of the
  // phase that scores item k + 1 (the loop is unrolled by two so each set
  // keeps its registers).
  constexpr int TILE = PAGE * D_C, PL = 16 * PS;
  PageRegs<CB> ra, rb;
  auto put_scores = [&](const float4v& S) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sxp[(gs * 16 + 4 * j + i) * SXS + row] = S[i];
  };
  auto phase = [&](int k, PageRegs<CB>& cur, PageRegs<CB>& ahead) {
    const int cb = k & 1, nb = cb ^ 1;
    load_page<CB>(ahead, page_at(k + 2), lo);
    PvCtx pv;
    pv_begin(pv, st, tile + cb * TILE, plds + cb * PL, alds, j, t16);
    const bool more = k + 1 < n_it;
    if (more) {
      put_scores(score_item(cur, k + 1, tile + nb * TILE, pv, std::true_type()));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) pv_step(st, pv, i, w, j, t16);
    }
    __syncthreads();
    if (more && w < 2) softmax_page(st, sxp, plds + nb * PL, alds, hh, tl, sl2);
    __syncthreads();
    return more;
  };
  if (n_it > 0) {
    load_page<CB>(ra, page_at(0), lo);
    load_page<CB>(rb, page_at(1), lo);
    put_scores(score_item(ra, 0, tile, PvCtx{}, std::false_type()));
    __syncthreads();
    if (w < 2) softmax_page(st, sxp, plds, alds, hh, tl, sl2);
    __syncthreads();
    for (int k = 0;; k += 2) {
      if (!phase(k, rb, ra)) break;
      if (!phase(k + 1, ra, rb)) break;
    }
  }

  // O / l and the log-sum-exp (l and m live in the lanes that own each head's
  // softmax): the output itself when a sequence has a single page range, else
  // the range's partial
  if (w < 2 && tl == 0) alds[hh] = st.l_run > 0.f ? 1.f / st.l_run : 0.f;
  __syncthreads();
  const float inv = alds[t16];
  if (a.n_split == 1) {
    uint16_t* dst = a.out + ((int64_t)b * H + h) * D_C + 64 * w + 4 * j;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const float4v o = st.oacc[mb] * inv;
      u32x2 packed;
      packed.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
      packed.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
      *reinterpret_cast<u32x2*>(dst + 16 * mb) = packed;
    }
    if (w < 2 && tl == 0)
      a.lse[(int64_t)b * H + hb * 16 + hh] =
          st.l_run > 0.f ? (st.m_run + __log2f(st.l_run)) * LN2 : -INFINITY;
    return;
  }
  const int64_t orow = ((int64_t)b * a.n_split + split) * H + h;
  if (inv > 0.f) {
    float* dst = a.ws_o + orow * D_C + 64 * w + 4 * j;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) *reinterpret_cast<float4v*>(dst + 16 * mb) = st.oacc[mb] * inv;
  }
  if (w < 2 && tl == 0) {
    const int64_t lrow = ((int64_t)b * a.n_split + split) * H + hb * 16 + hh;
    a.ws_lse[lrow] = st.l_run > 0.f ? (st.m_run + __log2f(st.l_run)) * LN2 : -INFINITY;
  }
}

// Merge the page-range partials of one (sequence, head, 128-channel quarter):
// lse = log sum exp(lse_s), out = sum_s exp(lse_s - lse) * o_s. Eight split
// lanes each fold their share of the ranges with a running max (empty ranges,
// lse_s = -inf, are skipped), then the eight running states are merged.
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  __shared__ float4v part[8][32];
  __shared__ float pm[8], pl[8];
  const int row = blockIdx.x >> 2, cq = blockIdx.x & 3;
  const int b = row / a.H, h = row % a.H;
  const int tid = threadIdx.x, sl = tid >> 5, ct = tid & 31;
  const int ns = a.n_split;
  const int c0 = 128 * cq + 4 * ct;
  const float* lses = a.ws_lse + (int64_t)b * ns * a.H + h;
  const float* base = a.ws_o + ((int64_t)b * ns * a.H + h) * D_C + c0;
  const int64_t stride = (int64_t)a.H * D_C;

  float m = -INFINITY, l = 0.f;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = sl; s < ns; s += 8) {
    const float ls = lses[(int64_t)s * a.H];
    if (ls == -INFINITY) continue;
    const float4v o = *reinterpret_cast<const float4v*>(base + s * stride);
    const float m_new = fmaxf(m, ls);
    const float fo = __expf(m - m_new), fs = __expf(ls - m_new);
    acc = acc * fo + o * fs;
    l = l * fo + fs;
    m = m_new;
  }
  part[sl][ct] = acc;
  if (ct == 0) {
    pm[sl] = m;
    pl[sl] = l;
  }
  __syncthreads();
  if (sl == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, pm[k]);
    float4v tot = {0.f, 0.f, 0.f, 0.f};
    float lt = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (pm[k] == -INFINITY) continue;
      const float f = __expf(pm[k] - M);
      tot += part[k][ct] * f;
      lt += pl[k] * f;
    }
    tot *= lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = a.out + ((int64_t)b * a.H + h) * D_C + c0;
    u32x2 packed;
    packed.x = f32_to_bf16_rne(tot[0]) | (f32_to_bf16_rne(tot[1]) << 16);
    packed.y = f32_to_bf16_rne(tot[2]) | (f32_to_bf16_rne(tot[3]) << 16);
    *reinterpret_cast<u32x2*>(op) = packed;
    if (ct == 0 && cq == 0) a.lse[(int64_t)b * a.H + h] = lt > 0.f ? M + __logf(lt) : -INFINITY;
  }
}

SplitPlan plan_splits(int B, int H, int max_pages) {
  // one 8-wave workgroup per CU (256 CUs) when the batch is small; enough
  // workgroups that none takes more than MAX_ITEMS items (a sequence has at
  // most max_pages packed pages plus 5 chunks of protected tokens, since
  // n_sink + n_local <= 320)
  const int n_hb = H / 16;
  const int64_t base = (int64_t)(B > 0 ? B : 1) * n_hb;
  int n = (int)(256 / base);
  const int items = max_pages + 5;
  const int need = (items + MAX_ITEMS - 1) / MAX_ITEMS;
  if (n < need) n = need;
  if (n > items) n = items;
  if (n < 1) n = 1;
  SplitPlan sp;
  sp.n_split = n;
  sp.pages_per_split = (items + n - 1) / n;  // upper bound, informational
  return sp;
}

size_t decode_workspace_bytes(int B, int H, int max_pages) {
  const SplitPlan sp = plan_splits(B, H, max_pages);
  return (size_t)B * sp.n_split * H * (D_C + 1) * sizeof(float);
}

hipError_t launch_decode(DecodeArgs a, int c_bits, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int n_u = a.B * a.n_split;
  const dim3 grid((n_u + 7) / 8 * 8 * (a.H / 16));
  if (c_bits == 4)
    decode_h16_kernel<4><<<grid, dim3(512), 0, stream>>>(a);
  else
    decode_h16_kernel<2><<<grid, dim3(512), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;  // one range: output written directly
  combine_kernel<<<dim3(a.B * a.H * 4), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
