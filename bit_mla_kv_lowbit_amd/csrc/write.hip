// Fused cache writer for gfx950 (QuantMLA, Figure 8 caption: a packed copy of
// every incoming token plus BF16 copies of protected sink and recent tokens).
//
// One lane takes 8 channels of a token: a wavefront reads one token's 1 KB
// content row and writes its packed code row with one instruction each, and
// the 4 lanes of a 32-channel group exchange their extremes to find the
// group's scale and zero. The codes and the fp16 (scale, zero) pairs are
// bit-identical to a plain CPU evaluation with fp32 subtraction and correctly
// rounded division (nearest even): a reciprocal estimate decides each code
// whose quotient is not within 1e-5 of a half-integer, the others take the
// correctly rounded division.
//
// Also here: the writer of the paired BF16 cache (rows copied into page
// slots) and the simulated quantize-dequantize (Figure 3 caption), which
// shares the quantizer.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

// Merge the extremes of this lane with those of quad partner j ^ M (DPP quad
// permutation), the lower lane's channels counting as earlier.
template <int M>
__device__ __forceinline__ void quad_merge(float& lo, float& hi, int j) {
  constexpr int CTRL = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const float plo = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, lo), CTRL, 0xF, 0xF, false));
  const float phi = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hi), CTRL, 0xF, 0xF, false));
  const bool upper = (j & M) != 0;  // this lane holds the later channels
  const float lo_a = upper ? plo : lo, lo_b = upper ? lo : plo;
  const float hi_a = upper ? phi : hi, hi_b = upper ? hi : phi;
  lo = lo_b < lo_a ? lo_b : lo_a;
  hi = hi_b > hi_a ? hi_b : hi_a;
}

// Merge with the mirrored lane of the half row (CTRL 0x141: lane i <-> 7 - i
// within 8) or of the row (0x140: i <-> 15 - i within 16); the lanes with bit
// M of j set hold the later channels. After the quad merges every lane of a
// quad holds the quad's extremes, so one mirror step joins two quads, the
// next two 8-lane halves.
template <int CTRL, int M>
__device__ __forceinline__ void mirror_merge(float& lo, float& hi, int j) {
  const float plo = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, lo), CTRL, 0xF, 0xF, false));
  const float phi = __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, hi), CTRL, 0xF, 0xF, false));
  const bool upper = (j & M) != 0;
  const float lo_a = upper ? plo : lo, lo_b = upper ? lo : plo;
  const float hi_a = upper ? phi : hi, hi_b = upper ? hi : phi;
  lo = lo_b < lo_a ? lo_b : lo_a;
  hi = hi_b > hi_a ? hi_b : hi_a;
}

// Minimum and maximum of a group held by 4 GM consecutive lanes, aligned to
// 4 GM lanes (lane j of the group holds channels 8j..8j+7, its own extremes
// in lo / hi): on equal values (+0 / -0) the earlier channel wins, as in a
// scan over the group in channel order.
template <int GM>
__device__ __forceinline__ void group_extremes(float& lo, float& hi, int j) {
  quad_merge<1>(lo, hi, j);
  quad_merge<2>(lo, hi, j);
  if constexpr (GM >= 2) mirror_merge<0x141, 4>(lo, hi, j);
  if constexpr (GM >= 4) mirror_merge<0x140, 8>(lo, hi, j);
}

// The same extremes without the order of equal values (min / max over the
// group's 4 GM lanes, partners by DPP as in group_extremes). The hardware
// min / max are written out: the library forms would first quiet signaling
// NaNs, which the inputs (finite by the writer's contract) never hold.
__device__ __forceinline__ float vmin3(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmin2(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int GM>
__device__ __forceinline__ void group_minmax(float& lo, float& hi) {
  lo = vmin2(lo, dpp_f<0xB1>(lo));
  hi = vmax2(hi, dpp_f<0xB1>(hi));
  lo = vmin2(lo, dpp_f<0x4E>(lo));
  hi = vmax2(hi, dpp_f<0x4E>(hi));
  if constexpr (GM >= 2) {
    lo = vmin2(lo, dpp_f<0x141>(lo));
    hi = vmax2(hi, dpp_f<0x141>(hi));
  }
  if constexpr (GM >= 4) {
    lo = vmin2(lo, dpp_f<0x140>(lo));
    hi = vmax2(hi, dpp_f<0x140>(hi));
  }
}

// Asymmetric min-max quantization of one group of 32 GM channels held by
// 4 GM lanes (lane j of the group: channels 8j .. 8j + 7 in raw, bf16): fp16
// scale s = (hi - lo) / (2^bits - 1) and zero z = lo (both rounded to nearest
// even); the lane's codes q = clamp(rint((x - z) / s), 0, 2^bits - 1), all 0
// when s = 0. Every fp32 step matches one IEEE operation rounded to nearest
// even.
template <int GM>
__device__ __forceinline__ void quantize8(const u32x4& raw, int bits, int j, _Float16& s16,
                                          _Float16& z16, uint32_t (&q)[8]) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_to_f32(raw[e] & 0xffffu);
    x[2 * e + 1] = bf16_to_f32(raw[e] >> 16);
  }
  // The group's extremes: min / max over the lanes' values (v_min3 / v_max3,
  // then min / max with the DPP partners). Equal values only differ in bits
  // when they are zeros of opposite sign, so where an extreme is a zero the
  // wavefront takes the ordered scan instead, in which the first of equal
  // values wins.
  float lo = vmin2(vmin3(vmin3(x[0], x[1], x[2]), x[3], x[4]), vmin3(x[5], x[6], x[7]));
  float hi = vmax2(vmax3(vmax3(x[0], x[1], x[2]), x[3], x[4]), vmax3(x[5], x[6], x[7]));
  group_minmax<GM>(lo, hi);
  if (__builtin_amdgcn_ballot_w64(lo == 0.0f || hi == 0.0f) != 0) {
    lo = x[0];
    hi = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {  // strict compares: the first of equal values wins
      lo = x[i] < lo ? x[i] : lo;
      hi = x[i] > hi ? x[i] : hi;
    }
    group_extremes<GM>(lo, hi, j);
  }
  const float qmax = (float)((1 << bits) - 1);
  s16 = (_Float16)__fdiv_rn(__fsub_rn(hi, lo), qmax);  // nearest even
  z16 = (_Float16)lo;
  const float s = (float)s16, z = (float)z16;
  // rint(fl((x - z) / s)) without a correctly rounded division per value:
  // with rs = rcp(s) (1 ulp), t = d * rs lies within 4e-6 of fl(d / s) while
  // |d / s| <= 17, so both round to the same integer unless t is within 1e-5
  // of a half-integer; those values take the exact division. Beyond [-1, 17]
  // both clamp to the same code.
  // The exact divisions sit behind a wavefront-uniform branch (rarely taken;
  // as a per-lane select they would all be executed).
  // (t is within 1e-5 of a half-integer exactly when |t - rint(t)| > 0.5 - 1e-5;
  // the subtraction is exact for |t| <= 17.)
  // (s = 0: rs = 0 makes every quotient 0, hence every code 0)
  const float rs = s != 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
  float d[8], r[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = __fsub_rn(x[i], z);
    const float t = d[i] * rs;
    r[i] = rintf(t);
    near |= __builtin_fabsf(t - r[i]) > 0.5f - 1e-5f;
  }
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = d[i] * rs;
        if (__builtin_fabsf(t - r[i]) > 0.5f - 1e-5f) r[i] = rintf(__fdiv_rn(d[i], s));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = (uint32_t)__builtin_amdgcn_fmed3f(r[i], 0.0f, qmax);
}

// Quantize and store the 8 channels (sub-block j of 32-channel block gi) one
// lane holds of a token's content (rope false) or RoPE part, given the lanes
// of its group (4 per block, aligned); also its share of the BF16 copy when
// the token is protected.
template <int F>
__device__ __forceinline__ void quantize_store(const WriteArgs& a, const u32x4& raw, bool rope,
                                               int gi, int j, uint8_t* base, int slot,
                                               uint16_t* keep) {
  using G = PageGeom<F>;
  const int bits = rope ? G::RB : G::CB;
  _Float16 s16, z16;
  uint32_t q[8];
  // lane index inside the group: content groups span GM blocks, RoPE groups GMR
  int gsz;  // blocks per group
  if (rope) {
    gsz = G::GMR;
    quantize8<G::GMR>(raw, bits, 4 * (gi % G::GMR) + j, s16, z16, q);
  } else {
    gsz = G::GM;
    quantize8<G::GM>(raw, bits, 4 * (gi % G::GM) + j, s16, z16, q);
  }

  // pack (code order of the page layout, on 32-channel blocks): sub-block j of
  // a block goes to chunk j of the block's chunk row; channel 8j + 2i + k sits
  // at bit 16k + bits * (4e + i) of its 32-bit word, e = code block of the block.
  if (bits == 4) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v |= (q[2 * i] << (4 * i)) | (q[2 * i + 1] << (16 + 4 * i));
    if (rope)  // 2 blocks per 8-byte chunk: chunk j at 8j, word gi
      *reinterpret_cast<uint32_t*>(base + G::OFF_RC + slot * G::RC + 8 * j + 4 * gi) = v;
    else  // 4 blocks per 16-byte chunk: chunk (ld, j) at 16 (4 ld + j), word gi % 4
      *reinterpret_cast<uint32_t*>(base + G::OFF_CC + slot * G::CC + 16 * (4 * (gi >> 2) + j) +
                                   4 * (gi & 3)) = v;
  } else {
    // two blocks per word (code block e = gi mod 2): the block owns byte e
    // (even channels) and byte 2 + e (odd channels) of the word; content: 8
    // blocks per 16-byte chunk, RoPE: its 2 blocks in one word, chunk j at 4j
    uint32_t vlo = 0, vhi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vlo |= q[2 * i] << (2 * i);
      vhi |= q[2 * i + 1] << (2 * i);
    }
    uint8_t* wp = rope ? base + G::OFF_RC + slot * G::RC + 4 * j
                       : base + G::OFF_CC + slot * G::CC + 16 * (4 * (gi >> 3) + j) +
                             4 * ((gi >> 1) & 3);
    const int e = gi & 1;
    wp[e] = (uint8_t)vlo;
    wp[2 + e] = (uint8_t)vhi;
  }
  if (j == 0 && gi % gsz == 0) {  // the group's first lane stores its (scale, zero)
    const uint32_t sz = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
    uint8_t* szdst = rope ? base + G::OFF_RS + slot * G::RS + (gi / gsz) * 4
                          : base + G::OFF_CS + slot * G::CS + (gi / gsz) * 4;
    *reinterpret_cast<uint32_t*>(szdst) = sz;
  }
  if (keep) *reinterpret_cast<u32x4*>(keep + (rope ? D_C : 0) + gi * GROUP + 8 * j) = raw;
}

// Where token t goes: its page base and slot and its BF16 row (null unless
// protected); false for a token outside the page table (or of no sequence),
// which is dropped, never written out of bounds.
template <int F>
__device__ __forceinline__ bool token_dest(const WriteArgs& a, int t, uint8_t*& base, int& slot,
                                           uint16_t*& keep) {
  const int b = a.seq_idx ? a.seq_idx[t] : t;
  const int p = a.pos[t];
  if (b < 0 || b >= a.B || p < 0 || p >= a.max_pages * PAGE) return false;
  const int L = a.seq_lens[b];
  const int64_t page = a.page_table[(int64_t)b * a.max_pages + p / PAGE];
  base = a.pages + page * (int64_t)PageGeom<F>::BYTES;
  slot = p % PAGE;
  keep = nullptr;
  if (p < a.n_sink)
    keep = a.sink + ((int64_t)b * a.n_sink + p) * D_ALL;
  else if (a.n_local > 0 && p >= L - a.n_local)
    keep = a.local + ((int64_t)b * a.n_local + p % a.n_local) * D_ALL;
  return true;
}

// One wavefront writes TW tokens. Lane l holds channels 8l..8l+7 (group l / 4,
// sub-block l % 4) of a token's content, so each content pass reads the
// token's 1 KB row and writes its packed code row with one instruction each;
// a last pass takes the RoPE parts of all TW tokens (8 lanes each). The 4
// lanes of a group exchange their extremes to find its scale and zero. All
// loads of the wavefront (the tokens' indices with scalar loads, then every
// input row) are issued before the first token is quantized, so the chain of
// dependent reads is paid once per TW tokens.
template <int F>
__global__ __launch_bounds__(256) void write_kernel(WriteArgs a) {
  constexpr int TW = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) +
                                                        (threadIdx.x >> 6)));
  const int t0 = wave * TW;
  if (t0 >= a.n_tokens) return;
  const int nt = min(TW, a.n_tokens - t0);
  u32x4 raw[TW + 1];
  const int tr = t0 + (lane >> 3);  // token of this lane's RoPE part
  const int chr = 8 * (lane & 7);
#pragma unroll
  for (int k = 0; k < TW; ++k)
    raw[k] = *reinterpret_cast<const u32x4*>(a.c_kv + (int64_t)(t0 + min(k, nt - 1)) * D_C +
                                             8 * lane);
  raw[TW] = *reinterpret_cast<const u32x4*>(a.k_rope + (int64_t)min(tr, a.n_tokens - 1) * D_R +
                                            chr);
  uint8_t* base[TW];
  int slot[TW];
  uint16_t* keep[TW];
  bool ok[TW];
#pragma unroll
  for (int k = 0; k < TW; ++k)
    ok[k] = k < nt && token_dest<F>(a, t0 + k, base[k], slot[k], keep[k]);
#pragma unroll
  for (int k = 0; k < TW; ++k)
    if (ok[k]) quantize_store<F>(a, raw[k], false, lane >> 2, lane & 3, base[k], slot[k], keep[k]);
  // RoPE parts: the lanes of token k (8k .. 8k + 7) take its destination
  uint8_t* rb = nullptr;
  int rslot = 0;
  uint16_t* rkeep = nullptr;
  bool rok = false;
#pragma unroll
  for (int k = 0; k < TW; ++k) {
    if ((lane >> 3) == k) {
      rok = ok[k];
      rb = base[k];
      rslot = slot[k];
      rkeep = keep[k];
    }
  }
  if (rok) quantize_store<F>(a, raw[TW], true, (lane & 7) >> 2, lane & 3, rb, rslot, rkeep);
}

// Paired BF16 cache (the unquantized baseline of the Figure 5(b) and Table 9
// latency comparison): the token's [c | k_rope] row is copied into its page
// slot. One thread per 16-byte chunk (72 per token), so a wavefront stores
// whole rows with coalesced 128-bit writes.
__global__ __launch_bounds__(256) void write_bf16_kernel(WriteArgs a) {
  constexpr int CH = D_ALL / 8;  // 16-byte chunks per row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.n_tokens * CH) return;
  const int t = (int)(gid / CH), k = (int)(gid % CH);
  const int b = a.seq_idx ? a.seq_idx[t] : t;
  const int p = a.pos[t];
  if (b < 0 || b >= a.B || p < 0 || p >= a.max_pages * PAGE) return;
  const int64_t page = a.page_table[(int64_t)b * a.max_pages + p / PAGE];
  const u32x4 v = k < D_C / 8
                      ? reinterpret_cast<const u32x4*>(a.c_kv + (int64_t)t * D_C)[k]
                      : reinterpret_cast<const u32x4*>(a.k_rope + (int64_t)t * D_R)[k - D_C / 8];
  u32x4* row = reinterpret_cast<u32x4*>(a.pages + page * (int64_t)PageGeom<16>::BYTES +
                                        (int64_t)(p % PAGE) * PageGeom<16>::ROW);
  row[k] = v;
}

hipError_t launch_write(const WriteArgs& a, int fmt, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  if (fmt == 16) {
    const int64_t total = (int64_t)a.n_tokens * (D_ALL / 8);
    write_bf16_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
  }
  const int64_t waves = ((int64_t)a.n_tokens + 7) / 8;  // 8 tokens per wavefront
  const int threads = 256;
  const int64_t blocks = (waves * 64 + threads - 1) / threads;
#define MLA_LAUNCH_WRITE(F) write_kernel<F><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(a)
  MLA_FOR_PACKED_FMT(fmt, MLA_LAUNCH_WRITE)
#undef MLA_LAUNCH_WRITE
  return hipGetLastError();
}

// x^ = q * s + z of 8 codes as one fused multiply-add each, rounded to fp32
// and then to bf16 (nearest even), packed as 8 bf16.
__device__ __forceinline__ u32x4 dequant8(const uint32_t (&q)[8], _Float16 s16, _Float16 z16) {
  const float s = (float)s16, z = (float)z16;
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = __builtin_fmaf((float)q[2 * e], s, z);
    const float hi = __builtin_fmaf((float)q[2 * e + 1], s, z);
    v[e] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
  }
  return v;
}

// Simulated quantize-dequantize (Figure 3 caption): the writer's wavefront
// layout (8 tokens per wavefront: one content pass per token, lane l holding
// channels 8l..8l+7, then one pass over the 8 tokens' RoPE parts, 8 lanes
// each), so every group's lanes are consecutive and aligned; its quantizer,
// then dequant8. 16 B in and out per lane and pass.
template <int F>
__global__ __launch_bounds__(256) void qdq_kernel(QdqArgs a) {
  using G = PageGeom<F>;
  constexpr int TW = 8;
  const int lane = threadIdx.x & 63;
  const int64_t t0 = (int64_t)__builtin_amdgcn_readfirstlane(
                         (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6))) * TW;
  if (t0 >= a.n_tokens) return;
  const int nt = (int)min((int64_t)TW, a.n_tokens - t0);
  for (int k = 0; k < nt; ++k) {
    const int64_t off = (t0 + k) * D_C + 8 * lane;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(a.c_kv + off);
    _Float16 s16, z16;
    uint32_t q[8];
    quantize8<G::GM>(raw, G::CB, lane & (4 * G::GM - 1), s16, z16, q);
    *reinterpret_cast<u32x4*>(a.out_c + off) = dequant8(q, s16, z16);
  }
  // RoPE parts: token t0 + (lane >> 3), channels 8 (lane & 7); lanes of a token
  // past the end read the last token (every lane takes part in the exchange)
  const int64_t tr = t0 + (lane >> 3);
  const int64_t off = min(tr, (int64_t)a.n_tokens - 1) * D_R + 8 * (lane & 7);
  const u32x4 raw = *reinterpret_cast<const u32x4*>(a.k_rope + off);
  _Float16 s16, z16;
  uint32_t q[8];
  quantize8<G::GMR>(raw, G::RB, lane & (4 * G::GMR - 1), s16, z16, q);
  if (tr < a.n_tokens) *reinterpret_cast<u32x4*>(a.out_r + off) = dequant8(q, s16, z16);
}

hipError_t launch_qdq(const QdqArgs& a, int fmt, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  const int64_t waves = (a.n_tokens + 7) / 8;
  const dim3 grid((unsigned)((waves + 3) / 4));
#define MLA_LAUNCH_QDQ(F) qdq_kernel<F><<<grid, dim3(256), 0, stream>>>(a)
  MLA_FOR_PACKED_FMT(fmt, MLA_LAUNCH_QDQ)
#undef MLA_LAUNCH_QDQ
  return hipGetLastError();
}

}  // namespace mla
