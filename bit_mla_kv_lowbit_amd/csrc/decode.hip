// Absorbed-MLA decode over the mixed BF16 / packed low-bit cache, for gfx950.
//
// QuantMLA (Figure 8 caption; abstract): attention unpacks and dequantizes the
// packed codes itself, takes protected sink / recent tokens from BF16 buffers,
// uses one reconstructed content tile for both the matching (QK) and the
// aggregation (PV) product, and normalizes all valid tokens with one softmax.
// The decode is the absorbed (MQA) form: all heads share the latent (GQLA card).
//
// Work decomposition: one workgroup of 4 wavefronts (one per SIMD) = one
// (sequence, page range, 16-head block); the range is walked one 64-token page
// per iteration, the next page's codes being loaded into registers while the
// current one is used. Wave w owns the 16 tokens 16w .. 16w + 15 of every page
// for the scores and the softmax, and the 128 output channels 128w .. 128w + 127
// for the PV product. Lane (token t, sub-block j) holds the 8-channel sub-block
// j of each of its token's 18 code groups (16 content, 2 RoPE; the code order
// makes one 128-bit load deliver one sub-block of 4 (INT4) or 8 (INT2) groups)
// and all (scale, zero) words of its token. Per page:
//   1. scores, exactly per group: the integer codes c (exact in fp16) are the
//      B operand of v_mfma_f32_16x16x32_f16, one MFMA per 32-channel group
//      gives D_g = q_g . c_g; then S = sum_g s_g D_g + sum_g z_g Q_g in fp32,
//      with Q_g = sum of q over group g (the z term is two more MFMAs with Q_g
//      split into fp16 hi + lo). Rounding the reconstructed keys to fp16 first
//      would cost ~1e-3 in the scores of wide-range (outlier) groups;
//   2. the reconstructed content values x = c * s + z (one packed fp16 FMA per
//      channel pair) go to an LDS tile, token-major;
//   3. softmax in the wave, with a reference max per head that all waves
//      share: P = 2^(S log2e scale - M). M only moves when a score exceeds it
//      by more than 2^8 (then the wave uses its own page max, publishes it, and
//      every wave rescales by the same factors after the barrier), so P stays
//      below 256 in fp16 and in the common case nothing is rescaled;
//   4. after the page's barrier, wave w accumulates O^T for its channels:
//      V^T and P^T are read transposed from LDS with ds_read_b64_tr_b16; a
//      second barrier frees the tile for the next page.
// Two workgroups share each CU, so one's PV product and barriers overlap the
// other's score loop. The partials (O / l, log-sum-exp) of the workgroups of a sequence are merged by
// combine_kernel (split-K over the sequence with an LSE combine: one global
// softmax); a sequence with a single page range writes its output directly.
//
// The same kernel serves two related calls. With s_q query tokens per
// sequence (multi-token prediction, GQLA card) the rows of query token i form
// their own head blocks and attend to the first L - (s_q - 1 - i) tokens. With
// F = 16 it decodes the paired BF16 cache the pages normalize their latency
// to (Figure 5(b), Table 9): BF16 rows instead of codes, bf16 MFMA for the
// scores, the same tile, softmax, PV and combine.
#include "mla_common.h"
#include "mla_kernels.h"
#include "decode_ops.h"

#include <type_traits>

namespace mla {

constexpr int WAVES = 4;  // wavefronts per workgroup

// Scores of the BF16 baseline use bf16 MFMA on Q and the rows as stored
// (bf16 values travel in half8 bit containers). Its PV product stays in fp16
// like the packed cache's: P in bf16 (8 significant bits) would move outputs
// by up to 2^-9 of the value spread, too much for outlier channels.
__device__ __forceinline__ float4v mma_bf16(const half8& a, const half8& b, const float4v& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight bf16 (bit patterns) -> fp16. Truncation is exact here: bf16 values in
// the fp16 normal range fit in 11 significant bits (below it, fp16 subnormals
// lose at most 2^-24).
__device__ __forceinline__ half8 bf16x8_to_f16x8_rtz(u32x4 w) {
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = __builtin_bit_cast(
        half2v, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[i] << 16),
                                           __uint_as_float(w[i] & 0xffff0000u)));
    r[2 * i] = h.x;
    r[2 * i + 1] = h.y;
  }
  return r;
}

// LDS tile of reconstructed content values, 64 token rows x 512 fp16, rows
// padded to TS halves (1040 bytes = 16 mod 256: 64 banks of 4 bytes). A row
// write (16 lanes: 16 consecutive rows, 16 bytes each) hits 16 distinct 16-byte
// bank slots. The PV operands map K slot jj (0..3) of lane group j to token
// 8j + 2jj and slot 4 + jj to token 8j + 2jj + 1 (plus 32 per K-block), so a
// transposing read (32 lanes: 8 rows 2 apart, 32 bytes each) hits 8 distinct
// 32-byte bank segments. All per-lane addresses are a base plus constants.
constexpr int TS = D_C + 8;
// P buffer of one page, 64 token rows x 16 heads (fp16), rows padded to PS
// halves (48 bytes): conflict-free row writes (8 bytes per lane) and the same
// transposing reads as the tile.
constexpr int PS = 24;
constexpr int TILE = PAGE * TS;

// Softmax and PV state of one lane: O^T of channels 128w + 16mb + 4j + i and
// head t16; the reference max of head t16 (PV side) and of heads 4j + i
// (score side: the same values, kept in both lane layouts) and the partial
// sums of exp over the lane's tokens for heads 4j + i.
struct AttnState {
  float4v oacc[8];
  float m_pv;
  float4v m_sc;
  float4v l_sc;
  float4v psum;  // this page's P of the lane's token, heads 4j + i (until folded into l_sc)
};

// PV operands of one page: the tile it reads, P^T (B operand, K-blocks 0, 1)
// and the V^T operand of the next PV step (read one step ahead).
struct PvCtx {
  const _Float16* tile;
  half8 pB[2];
  half8 av;
};

// V^T operand of PV step i = 2 mb + kb: channels of block mb of wave w, the 32
// tokens of K-block kb.
__device__ __forceinline__ half8 pv_load(const PvCtx& c, int i, int w, int j, int t16) {
  const int mb = i >> 1, kb = i & 1;
  const int trow = 32 * kb + 8 * j + 2 * (t16 >> 2);
  const int col = 128 * w + 16 * mb + 4 * (t16 & 3);
  return tr_pair(c.tile + trow * TS + col, c.tile + (trow + 1) * TS + col);
}

// O^T[16 channels, block mb of wave w x 16 heads] += V^T P^T over the 32 tokens
// of K-block kb (step i = 2 mb + kb), after issuing the reads of step i + 1.
__device__ __forceinline__ void pv_step(AttnState& st, PvCtx& c, int i, int w, int j, int t16) {
  const half8 cur = c.av;
  if (i + 1 < 16) c.av = pv_load(c, i + 1, w, j, t16);
  const int mb = i >> 1, kb = i & 1;
  st.oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur, c.pB[kb], st.oacc[mb], 0, 0, 0);
}

// LDS exchange of one page between the score side and the PV side.
struct PageLds {
  _Float16* pbuf;  // [64 rows][PS]: 16 heads
  float* mref;     // [4 waves][16 heads]: a wave's page reference max (when flagged)
  int* flag;       // [4 waves]: the wave used its own page max
};

// Softmax of the wave's 16 tokens of a page, from the scores S (heads 4j + i,
// the lane's token): P to the page's LDS buffer, the flag (and reference max)
// of the wave, P of the lane's token kept in st.psum.
__device__ __forceinline__ void softmax_tokens(AttnState& st, const float4v& S, const PageLds& pl,
                                               float sl2, int w, int lane, int row, int j,
                                               int t16) {
  float4v t;
  bool big = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[i] = fmaf(S[i], sl2, -st.m_sc[i]);
    big |= t[i] > TAU;
  }
  const bool any_big = __builtin_amdgcn_ballot_w64(big) != 0;
  if (any_big) {
    // the wave's own page max per head (over its 16 tokens: the 16 lanes of a
    // row), at least the shared reference
    float4v mx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = S[i] * sl2;
      v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true)));
      v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true)));
      v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true)));
      v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true)));
      mx[i] = fmaxf(st.m_sc[i], v);
      t[i] = fmaf(S[i], sl2, -mx[i]);
    }
    if (t16 == 0) *reinterpret_cast<float4v*>(pl.mref + 16 * w + 4 * j) = mx;
  }
  if (lane == 0) pl.flag[w] = any_big ? 1 : 0;
  float4v p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(t[i]);
  st.psum = p;
  u32x2 ph;
  ph.x = as_u32((half2v){(_Float16)p[0], (_Float16)p[1]});
  ph.y = as_u32((half2v){(_Float16)p[2], (_Float16)p[3]});
  *reinterpret_cast<u32x2*>(pl.pbuf + row * PS + 4 * j) = ph;
}

// PV side of a page after its barrier: P^T operands, and the shared reference
// max moved where a wave flagged it (O, the P operands and the partial sums
// rescaled by the same factors in every wave, so all waves keep equal maxima).
__device__ __forceinline__ void pv_begin(PvCtx& c, AttnState& st, const _Float16* tile,
                                         const PageLds& pl, int w, int j, int t16) {
  c.tile = tile;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int trow = 32 * kb + 8 * j + 2 * (t16 >> 2);
    c.pB[kb] = tr_pair(pl.pbuf + trow * PS + 4 * (t16 & 3), pl.pbuf + (trow + 1) * PS + 4 * (t16 & 3));
  }
  c.av = pv_load(c, 0, w, j, t16);
  const int4 fl = *reinterpret_cast<const int4*>(pl.flag);
  const int any = __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w);
  if (!any) {
    st.l_sc += st.psum;
    return;
  }
  const int f[4] = {fl.x, fl.y, fl.z, fl.w};
  // PV side: head t16
  float mp = st.m_pv;
#pragma unroll
  for (int v = 0; v < WAVES; ++v)
    if (f[v]) mp = fmaxf(mp, pl.mref[16 * v + t16]);
  const float alpha = __builtin_amdgcn_exp2f(st.m_pv - mp);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.oacc[mb] *= alpha;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int src = 2 * kb + (j >> 1);  // wave that produced these 8 tokens
    const float ref = f[src] ? pl.mref[16 * src + t16] : st.m_pv;
    const float fs = __builtin_amdgcn_exp2f(ref - mp);
#pragma unroll
    for (int e = 0; e < 8; ++e) c.pB[kb][e] = (_Float16)((float)c.pB[kb][e] * fs);
  }
  st.m_pv = mp;
  // score side: heads 4j + i, and this wave's partial sums of the page
  float4v ms = st.m_sc;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    if (!f[v]) continue;
    const float4v mr = *reinterpret_cast<const float4v*>(pl.mref + 16 * v + 4 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) ms[i] = fmaxf(ms[i], mr[i]);
  }
  const float4v own = f[w] ? *reinterpret_cast<const float4v*>(pl.mref + 16 * w + 4 * j) : st.m_sc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.l_sc[i] = st.l_sc[i] * __builtin_amdgcn_exp2f(st.m_sc[i] - ms[i]) +
                 st.psum[i] * __builtin_amdgcn_exp2f(own[i] - ms[i]);
  st.m_sc = ms;
}

// Scores of the lane's token (S[i]: head 4j + i) over its 18 groups, plus the
// content tile row of the token.
template <int F>
__device__ __forceinline__ float4v packed_scores(const PageRegs<F>& t, const half8 (&qA)[18],
                                                 const half8& qz1, const half8& qz2,
                                                 _Float16* tile, int row, int j) {
  // z operands (K slot 8j + i): zb1 holds the z of content groups 0..7 in lanes
  // j < 2 and the RoPE groups' z in slots 0, 1 of lanes j >= 2; zb2 the z of
  // content groups 8..15. qz1 / qz2 hold the matching fp16 hi (j even) and lo
  // (j odd) parts of the group sums Q_g.
  const bool lowj = j < 2;
  const uint32_t rz = z_pair(t.rsz.x, t.rsz.y);
  const u32x4 z1 = {lowj ? z_pair(t.sz[0].x, t.sz[0].y) : rz,
                    lowj ? z_pair(t.sz[0].z, t.sz[0].w) : 0u,
                    lowj ? z_pair(t.sz[1].x, t.sz[1].y) : 0u,
                    lowj ? z_pair(t.sz[1].z, t.sz[1].w) : 0u};
  const u32x4 z2 = {z_pair(t.sz[2].x, t.sz[2].y), z_pair(t.sz[2].z, t.sz[2].w),
                    z_pair(t.sz[3].x, t.sz[3].y), z_pair(t.sz[3].z, t.sz[3].w)};
  const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
  float4v S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz1, __builtin_bit_cast(half8, z1), zero4, 0, 0, 0);
  S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qz2, __builtin_bit_cast(half8, z2), S, 0, 0, 0);
  // each group's product is scaled one group later, when its MFMA has finished
  float4v Dp = zero4;
  float sp = 0.f;
#pragma unroll
  for (int g = 0; g < NG_C + NG_R; ++g) {
    const half8 c = g < NG_C ? content_codes<F>(t, g) : rope_codes<F>(t, g - NG_C);
    const uint32_t sz = g < NG_C ? content_sz<F>(t, g) : t.rsz[g - NG_C];
    const float4v D = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[g], c, zero4, 0, 0, 0);
    if (g > 0) S += sp * Dp;
    if (g < NG_C)
      *reinterpret_cast<half8*>(tile + row * TS + GROUP * g + 8 * j) = reconstruct(c, sz);
    Dp = D;
    sp = (float)as_h2(sz).x;
  }
  S += sp * Dp;
  return S;
}

// Scores and tile row of a token taken from the BF16 buffers (exact in fp16),
// for the lanes with use set: one MFMA chain over the 18 groups. The other
// lanes read a valid row (in bounds), contribute 0 and leave the tile alone.
__device__ __forceinline__ float4v bf16_scores(const uint16_t* rowp, bool use,
                                               const half8 (&qA)[18], _Float16* tile, int row,
                                               int j) {
  float4v S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 raw[9];
#pragma unroll
    for (int i = 0; i < 9; ++i)
      raw[i] = *reinterpret_cast<const u32x4*>(rowp + group_channel(9 * h + i, j));
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int g = 9 * h + i;
      half8 kv = bf16x8_to_f16x8(raw[i]);
      kv = use ? kv : (half8){};
      S = __builtin_amdgcn_mfma_f32_16x16x32_f16(qA[g], kv, S, 0, 0, 0);
      if (g < NG_C && use) *reinterpret_cast<half8*>(tile + row * TS + GROUP * g + 8 * j) = kv;
    }
  }
  return S;
}

// Q operands of groups Q_REG .. 17 of the BF16 baseline stay in LDS (one copy
// per workgroup, read once per page): its next page's raw rows take 72 VGPRs,
// and with all 18 Q operands in registers as well the kernel would spill.
constexpr int Q_REG = 10;
constexpr int Q_LDS = NG_C + NG_R - Q_REG;

// Scores and tile row of a token of a BF16 page (bf16 MFMA on the stored
// values, fp16 tile); a row with keep false contributes 0 and leaves a zero
// tile row. q_lds: the lane's Q operands of groups Q_REG.. (stride 64 lanes).
__device__ __forceinline__ float4v bf16_page_scores(const PageRegs<16>& t, bool keep,
                                                    const half8 (&qA)[18], const half8* q_lds,
                                                    _Float16* tile, int row, int j) {
  float4v S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < NG_C + NG_R; ++g) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 kv = keep ? t.k[g] : z;
    const half8 q = g < Q_REG ? qA[g] : q_lds[64 * (g - Q_REG)];
    S = mma_bf16(q, __builtin_bit_cast(half8, kv), S);
    if (g < NG_C)
      *reinterpret_cast<half8*>(tile + row * TS + GROUP * g + 8 * j) = bf16x8_to_f16x8_rtz(kv);
  }
  return S;
}

// Page range [it0, it0 + n_it) of workgroup `split` (of n_split) over the
// first L tokens of a sequence whose protected tokens are p < n_s and
// p >= lo_start. Pages with protected tokens cost more than a packed page
// (their BF16 rows are read when they are scored), so the boundaries balance
// the weight c(i) of pages 0 .. i - 1, in half-page units: 2 per page, 1 more
// for the sink page and 3 more for each page from the one holding the
// window's first token (1.5 and 2.5 packed pages; measured against 2 and 2 on
// the V2-Lite- and C2R4-shaped batches, about 1 % faster).
// Split s starts at the smallest i with c(i) >= s * W / n_split.
struct PageRange {
  int it0, n_it;
};
__device__ __forceinline__ PageRange page_range(int L, int n_s, int lo_start, int split,
                                                int n_split) {
  const int n_items = (L + PAGE - 1) / PAGE;
  const int wp = min(lo_start / PAGE, n_items);
  const int sink_w = n_s > 0 ? 1 : 0;
  auto weight_before = [&](int i) { return 2 * i + sink_w * min(i, 1) + 3 * max(0, i - wp); };
  const int64_t W = weight_before(n_items);
  auto first_item = [&](int s) {
    int lo_i = 0, hi_i = n_items;
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i) >> 1;
      if ((int64_t)weight_before(mid) * n_split >= (int64_t)s * W) hi_i = mid;
      else lo_i = mid + 1;
    }
    return lo_i;
  };
  const int i0 = first_item(split);
  const int i1 = first_item(split + 1);  // i1 - i0 <= MAX_ITEMS by the split plan
  return {i0, i1 - i0};
}

// Work items of a sequence: its pages (protected tokens taken from the BF16
// buffers in their own slots). Workgroup `split` takes a contiguous range of
// the pages (an even share of their cost), and writes one partial (O / l,
// lse) that combine_kernel merges.
template <int F>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 tile[TILE];
  __shared__ __attribute__((aligned(16))) _Float16 pbuf[PAGE * PS];
  __shared__ __attribute__((aligned(16))) float mref[WAVES * 16];
  __shared__ __attribute__((aligned(16))) int flag[WAVES];
  __shared__ __attribute__((aligned(16))) float lsum[WAVES * 16];
  // physical pages of the first 256 items (a longer range, where the split
  // plan makes one, reads the rest from the page table with scalar loads)
  __shared__ int pids[256];
  __shared__ __attribute__((aligned(16))) half8 q_lds[F == 16 ? Q_LDS * 64 : 1];

  // All scalar arguments are read up front (one round trip, not one per first
  // use: the length, the page table and the first page already form a chain
  // of dependent reads, done with scalar loads so that they do not queue
  // behind the vector reads of Q).
  const int H = a.H, n_split = a.n_split, max_pages = a.max_pages;
  const int n_sink = a.n_sink, n_local = a.n_local;
  const uint16_t* const q_lat = a.q_lat;
  const uint16_t* const q_rope = a.q_rope;
  const int32_t* const seq_lens = a.seq_lens;
  const int32_t* const page_table = a.page_table;
  asm volatile("" ::"s"(H), "s"(n_split), "s"(max_pages), "s"(n_sink), "s"(n_local), "s"(q_lat),
               "s"(q_rope), "s"(seq_lens), "s"(page_table), "s"(a.B));

  // Workgroup -> (page range u = (b, split), head block hb). Consecutive
  // workgroups go to the 8 XCDs in turn, and each XCD has its own L2: the head
  // blocks of one page range get ids that are equal mod 8, so the page range is
  // read from HBM once and served from that XCD's L2 to the other head blocks.
  const int n_hb = H / 16;
  const int gsz = 8 * n_hb;
  const int u = (int)(blockIdx.x / gsz) * 8 + (int)(blockIdx.x % 8);
  if (u >= a.B * n_split) return;  // padding of the last group of 8 ranges
  const int hb = (int)(blockIdx.x % gsz) / 8;
  const int b = __builtin_amdgcn_readfirstlane(u / n_split);
  const int split = __builtin_amdgcn_readfirstlane(u % n_split);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int lane = tid & 63, j = lane >> 4, t16 = lane & 15;
  const int row = 16 * w + t16;  // token row of this lane in the page / tile
  const int h = hb * 16 + t16;

  // This workgroup's page range. The length arrives one round trip after the
  // arguments, and the page table one more after it; so the range is first
  // computed for a sequence that fills its page-table row (the common case of
  // a batch of equal lengths) and its page ids are read at once, while the
  // length and Q are in flight. A range that turns out different is read
  // again.
  const int L_raw = *(volatile const_i32*)(seq_lens + b);  // volatile: issued first

  // Q of the 16 heads is read once per workgroup (16 B per thread and chunk),
  // converted to fp16 and staged in the tile (rows of QS halves) before the
  // waves take their operands from it.
  constexpr int QS = D_ALL + 8;
  constexpr int NCH = 16 * (D_ALL / 8);  // 8-channel chunks
  u32x4 qv[(NCH + 255) / 256];
  {
    const uint16_t* ql = q_lat + ((int64_t)b * H + hb * 16) * D_C;
    const uint16_t* qr = q_rope + ((int64_t)b * H + hb * 16) * D_R;
#pragma unroll
    for (int i = 0; i < (NCH + 255) / 256; ++i) {
      const int c = min(tid + 256 * i, NCH - 1), hh = c / (D_ALL / 8), k = c % (D_ALL / 8);
      qv[i] = *reinterpret_cast<const u32x4*>(k < D_C / 8 ? ql + hh * D_C + 8 * k
                                                        : qr + hh * D_R + 8 * (k - D_C / 8));
    }
  }
  const int Lg = max_pages * PAGE;
  const int* ptab_b = page_table + (int64_t)b * max_pages;
  const PageRange rg = page_range(Lg, min(n_sink, Lg), max(n_sink, Lg - n_local), split, n_split);
  const int pid0_g = rg.n_it > 0 ? *(const_i32*)(ptab_b + rg.it0) : 0;
  const int pidm_g = tid < rg.n_it ? ptab_b[rg.it0 + tid] : 0;

  // lengths are clamped to what the page table can hold
  const int L = min(max(L_raw, 0), Lg);
  const float sl2 = a.scale_log2;
  // Token p of a page is taken from the packed codes, or from the BF16 buffers
  // if it is protected (p < n_s: sink; p >= lo_start: the recent window, ring
  // slot p mod n_local), or is masked if p >= Lq. With s_q query tokens per
  // sequence (the last s_q tokens of the cache), the heads of query token qi
  // attend causally to p < Lq = L - (s_q - 1 - qi); the protected set is the
  // cache's (its length L).
  const int n_s = min(n_sink, L);
  const int lo_start = max(n_sink, L - n_local);  // first token of the recent window
  const int qi = (hb * 16) / a.h_per_q;
  const int Lq = max(0, L - (a.s_q - 1 - qi));
  const PageRange rr = Lq == Lg ? rg : page_range(Lq, n_s, lo_start, split, n_split);
  const int it0 = rr.it0;
  const int n_it = rr.n_it;
  const int n_pk = n_it;  // every item is a page of the page table
  const int mix_from = min(lo_start, Lq);  // pages reaching past it have BF16 or masked rows
  int pid0 = pid0_g, pid_mine = pidm_g;
  if (rr.it0 != rg.it0 || rr.n_it != rg.n_it) {
    pid0 = n_pk > 0 ? *(const_i32*)(ptab_b + it0) : 0;
    pid_mine = tid < n_pk ? ptab_b[it0 + tid] : 0;
  }

  // The first page stays in flight while Q is converted. Loads past the last
  // item repeat it; with no item the descriptor has an empty range (loads
  // return 0, touch nothing), so the loads stay unconditional and the wait
  // counts static.
  const LaneOffsets<F> lo(row, j);
  PageRegs<F> regs;
  load_page<F>(regs, page_rsrc<F>(a.pages, pid0, n_pk > 0), lo);
#pragma unroll
  for (int i = 0; i < (NCH + 255) / 256; ++i) {
    const int c = tid + 256 * i, hh = c / (D_ALL / 8), k = c % (D_ALL / 8);
    if (c < NCH)
      *reinterpret_cast<half8*>(tile + hh * QS + 8 * k) =
          F == 16 ? __builtin_bit_cast(half8, qv[i]) : bf16x8_to_f16x8(qv[i]);
  }
  __syncthreads();  // Q staged

  // Q as fp16 A operands, and the z-term A operands (see packed_scores).
  half8 qA[NG_C + NG_R];
  half8 qz1, qz2;
  {
    // group sums Q_g of head t16: one MFMA with a ones A operand (Q as the B
    // operand has the same lane layout as the A operand)
    float qs[NG_C + NG_R];
#pragma unroll
    for (int g = 0; g < NG_C + NG_R; ++g)
      qA[g] = *reinterpret_cast<const half8*>(tile + t16 * QS + group_channel(g, j));
    if constexpr (F == 16) {
      if (w == 0) {
#pragma unroll
        for (int g = Q_REG; g < NG_C + NG_R; ++g) q_lds[64 * (g - Q_REG) + lane] = qA[g];
      }
    } else {
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
    const float4v zero4 = {0.f, 0.f, 0.f, 0.f};
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
  }

  AttnState st;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.oacc[mb] = (float4v){0.f, 0.f, 0.f, 0.f};
  st.m_pv = M_NONE;
  st.m_sc = (float4v){M_NONE, M_NONE, M_NONE, M_NONE};
  st.l_sc = (float4v){0.f, 0.f, 0.f, 0.f};
  st.psum = (float4v){0.f, 0.f, 0.f, 0.f};

  if (tid < n_pk) pids[tid] = pid_mine;
  __syncthreads();  // page ids in LDS; Q read out of the tile before it is overwritten

  auto score_item = [&](const PageRegs<F>& cur, int k) {
    const int p0 = (it0 + k) * PAGE;
    const bool mixed = p0 < n_s || p0 + PAGE > mix_from;  // not every token packed
    const int p = p0 + row;
    const bool valid = p < Lq;
    const bool prot = valid && (p < n_s || p >= lo_start);
    if constexpr (F == 16) {
      // BF16 baseline: no protected buffers; a partial last page masks its tail
      float4v S = bf16_page_scores(cur, !mixed || valid, qA, q_lds + lane, tile, row, j);
      if (!valid) S = (float4v){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      return S;
    } else {
      PageRegs<F> t = cur;
      if (mixed) mask_token<F>(t, valid && !prot);
      float4v S = packed_scores<F>(t, qA, qz1, qz2, tile, row, j);
      if (mixed) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);  // pages with BF16 rows are the slow ones
        const uint64_t pm = __builtin_amdgcn_ballot_w64(prot);
        if (pm != 0) {
          // lanes without a protected token read the first protected lane's row
          const int src = (int)__builtin_ctzll(pm);
          const int pp = prot ? p : __builtin_amdgcn_readlane(p, src);
          const uint16_t* rowp = pp < n_s ? a.sink + ((int64_t)b * n_sink + pp) * D_ALL
                                          : a.local + ((int64_t)b * n_local + pp % n_local) * D_ALL;
          S += bf16_scores(rowp, prot, qA, tile, row, j);
        }
        if (!valid) S = (float4v){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
      return S;
    }
  };

  // Per item: scores, tile rows and softmax of the item, then (after a
  // barrier) its PV product, then a barrier before the next item overwrites
  // the tile. The next page's codes are loaded into the same registers as soon
  // as the scores have used them, so they arrive during the PV product; two
  // workgroups share each CU, so one's PV / barriers overlap the other's
  // scores.
  const PageLds pl{pbuf, mref, flag};
  if (n_it > 0) {
    for (int k = 0;; ++k) {
      const int kn = max(0, min(k + 1, n_pk - 1));
      const int pid_next = kn < 256 ? pids[kn] : *(const_i32*)(ptab_b + it0 + kn);  // read ahead
      const float4v S = score_item(regs, k);
      // From the softmax to the end of the PV product the wave's instructions
      // take precedence over those of the other workgroup's wave on the SIMD
      // (its score loop), so the short, latency-bound stretches around the
      // barrier do not wait behind a long run of VALU work.
      __builtin_amdgcn_s_setprio(2);
      softmax_tokens(st, S, pl, sl2, w, lane, row, j, t16);
      load_page<F>(regs, page_rsrc<F>(a.pages, n_pk > 0 ? __builtin_amdgcn_readfirstlane(pid_next) : 0,
                                        n_pk > 0), lo);
      __syncthreads();
      PvCtx pv;
      pv_begin(pv, st, tile, pl, w, j, t16);
#pragma unroll
      for (int i = 0; i < 16; ++i) pv_step(st, pv, i, w, j, t16);
      __builtin_amdgcn_s_setprio(0);
      if (k + 1 >= n_it) break;
      __syncthreads();
    }
  }

  // l of each head: the lanes' partial sums (heads 4j + i) over the wave's 16
  // tokens, then over the four waves; all waves hold the same reference max.
  {
    float4v l4 = st.l_sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) l4[i] = row_sum(l4[i]);
    if (t16 == 0) *reinterpret_cast<float4v*>(lsum + 16 * w + 4 * j) = l4;
  }
  __syncthreads();
  const float l = lsum[t16] + lsum[16 + t16] + lsum[32 + t16] + lsum[48 + t16];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_v = l > 0.f ? (st.m_pv + __log2f(l)) * LN2 : -INFINITY;
  if (n_split == 1) {
    uint16_t* dst = a.out + ((int64_t)b * H + h) * D_C + 128 * w + 4 * j;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float4v o = st.oacc[mb] * inv;
      u32x2 packed;
      packed.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
      packed.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
      *reinterpret_cast<u32x2*>(dst + 16 * mb) = packed;
    }
    if (w == 0 && j == 0) a.lse[(int64_t)b * H + h] = lse_v;
    return;
  }
  const int64_t orow = ((int64_t)b * n_split + split) * H + h;
  if (inv > 0.f) {
    _Float16* dst = a.ws_o + orow * D_C + 128 * w + 4 * j;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float4v o = st.oacc[mb] * inv;
      u32x2 packed;
      packed.x = as_u32((half2v){(_Float16)o[0], (_Float16)o[1]});
      packed.y = as_u32((half2v){(_Float16)o[2], (_Float16)o[3]});
      *reinterpret_cast<u32x2*>(dst + 16 * mb) = packed;
    }
  }
  if (w == 0 && j == 0) a.ws_lse[orow] = lse_v;
}

// Merge the page-range partials of one (sequence, head): lse = log sum
// exp(lse_s), out = sum_s exp(lse_s - lse) * o_s. A workgroup takes SL split
// lanes x CL channel lanes of 8 channels (64 / CL workgroups per row). Each
// split lane issues the loads of U of its ranges together and folds them with
// a running max (empty ranges, lse = -inf, hold no output); the SL states are
// then merged in LDS.
template <int SL, int CL, int U>
__global__ __launch_bounds__(SL * CL) void combine_kernel(DecodeArgs a) {
  __shared__ float part[SL][8][CL];
  __shared__ float pm[SL], pl[SL];
  constexpr int PER_ROW = 64 / CL;
  const int row = blockIdx.x / PER_ROW, cq = blockIdx.x % PER_ROW;
  const int b = row / a.H, h = row % a.H;
  const int tid = threadIdx.x, sl = tid / CL, cl = tid % CL;
  const int ch = 8 * (cq * CL + cl);
  const int ns = a.n_split;
  const float* lses = a.ws_lse + (int64_t)b * ns * a.H + h;
  const _Float16* base = a.ws_o + ((int64_t)b * ns * a.H + h) * D_C + ch;
  const int64_t stride = (int64_t)a.H * D_C;

  float m = -INFINITY, l = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = sl; s0 < ns; s0 += U * SL) {
    float ls[U];
    half8 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + SL * u, ns - 1);
      ls[u] = s0 + SL * u < ns ? lses[(int64_t)s * a.H] : -INFINITY;
      o[u] = *reinterpret_cast<const half8*>(base + (int64_t)s * stride);
    }
    float mc = ls[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mc = fmaxf(mc, ls[u]);
    if (mc == -INFINITY) continue;
    const float m_new = fmaxf(m, mc);
    const float r = __expf(m - m_new);  // 0 while m = -inf
    l *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = ls[u] != -INFINITY;
      const float f = ok ? __expf(ls[u] - m_new) : 0.f;
      l += f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ok ? (float)o[u][e] * f : 0.f;
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[sl][e][cl] = acc[e];
  if (cl == 0) {
    pm[sl] = m;
    pl[sl] = l;
  }
  __syncthreads();
  if (sl != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < SL; ++k) M = fmaxf(M, pm[k]);
  l = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    if (pm[k] == -INFINITY) continue;
    const float f = __expf(pm[k] - M);
    l += pl[k] * f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += part[k][e][cl] * f;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  u32x4 packed;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    packed[e] = f32_to_bf16_rne(acc[2 * e] * inv) | (f32_to_bf16_rne(acc[2 * e + 1] * inv) << 16);
  *reinterpret_cast<u32x4*>(a.out + ((int64_t)b * a.H + h) * D_C + ch) = packed;
  if (cl == 0 && cq == 0) a.lse[(int64_t)b * a.H + h] = l > 0.f ? M + __logf(l) : -INFINITY;
}

SplitPlan plan_splits(int B, int H, int max_pages) {
  // two 4-wave workgroups per CU (256 CUs) when the batch is small; enough
  // workgroups that none takes more than a cap of pages: the page weight is
  // at most 2 max_pages + 16 (the sink page +1, at most 5 pages of a
  // 256-token window +3 each) and every page weighs at least 2, so a share
  // spans fewer than (max_pages + 8) / n + 1 pages. The cap is 256 pages;
  // where it needs more splits than one round of 512 workgroups holds, a
  // single round with up to MAX_ITEMS pages per workgroup is used if that
  // suffices, else the split count is rounded up to whole rounds (no round
  // that leaves most CUs idle).
  const int n_hb = H / 16;
  const int64_t base = (int64_t)(B > 0 ? B : 1) * n_hb;
  const int n_round = (int)(512 / base);  // splits that make one full round
  int n = n_round;
  const int need256 = (max_pages + 8 + (256 - 4) - 1) / (256 - 4);
  const int need_max = (max_pages + 8 + (MAX_ITEMS - 4) - 1) / (MAX_ITEMS - 4);
  if (need256 > n) {
    if (n >= 1 && need_max <= n) {
      // one round, longer ranges
    } else if (n >= 1) {
      n = (need256 + n - 1) / n * n;
    } else {
      n = need256;
    }
  }
  if (n > max_pages) n = max_pages;
  if (n < 1) n = 1;
  SplitPlan sp;
  sp.n_split = n;
  sp.pages_per_split = (max_pages + n - 1) / n;  // informational
  return sp;
}

size_t decode_workspace_bytes(int B, int H, int max_pages) {
  const SplitPlan sp = plan_splits(B, H, max_pages);
  const size_t narrow = (size_t)B * sp.n_split * H * (sizeof(float) + D_C * sizeof(_Float16));
  // rows that may be s_q query tokens of 128 heads each (the 128-head path)
  const size_t wide = H % 128 == 0 ? wide_workspace_bytes(B, H / 128) : 0;
  return narrow > wide ? narrow : wide;
}

hipError_t launch_decode(DecodeArgs a, int fmt, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  // 128 heads per query token: one dequantization (or, for BF16 pages, one
  // conversion to fp16) per page and 64 heads, work split by page weight
  // (decode_wide.hip)
  if (a.h_per_q == 128) return launch_decode_wide(a, a.ws_lse, fmt, stream);
  const int n_u = a.B * a.n_split;
  const dim3 grid((n_u + 7) / 8 * 8 * (a.H / 16));
  if (fmt == 16) {
    decode_kernel<16><<<grid, dim3(256), 0, stream>>>(a);
  } else {
#define MLA_LAUNCH_NARROW(F) decode_kernel<F><<<grid, dim3(256), 0, stream>>>(a)
    MLA_FOR_PACKED_FMT(fmt, MLA_LAUNCH_NARROW)
#undef MLA_LAUNCH_NARROW
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;  // one range: output written directly
  // SL split lanes with U ranges each per round of loads (U covers a lane's
  // share up to 8); a row splits into four channel blocks when rows are few
  const int rows = a.B * a.H, ns = a.n_split;
  const dim3 g1(rows), g4(rows * 4);
  if (ns >= 8) {
    const int per = (ns + 7) / 8;
    if (rows < 1024) {
      if (per > 4) combine_kernel<8, 16, 8><<<g4, dim3(128), 0, stream>>>(a);
      else if (per > 2) combine_kernel<8, 16, 4><<<g4, dim3(128), 0, stream>>>(a);
      else if (per > 1) combine_kernel<8, 16, 2><<<g4, dim3(128), 0, stream>>>(a);
      else combine_kernel<8, 16, 1><<<g4, dim3(128), 0, stream>>>(a);
    } else {
      if (per > 4) combine_kernel<8, 64, 8><<<g1, dim3(512), 0, stream>>>(a);
      else if (per > 2) combine_kernel<8, 64, 4><<<g1, dim3(512), 0, stream>>>(a);
      else if (per > 1) combine_kernel<8, 64, 2><<<g1, dim3(512), 0, stream>>>(a);
      else combine_kernel<8, 64, 1><<<g1, dim3(512), 0, stream>>>(a);
    }
  } else if (ns >= 4) {
    combine_kernel<4, 64, 2><<<g1, dim3(256), 0, stream>>>(a);
  } else {
    combine_kernel<2, 64, 2><<<g1, dim3(128), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
