// Device helpers shared by the decode kernels (gfx950): constants, fp16
// views, the magic-exponent code conversion, reconstruction, transposing LDS
// reads and lane reductions.
#pragma once
#include "mla_common.h"

namespace mla {

constexpr float LN2 = 0.69314718055994530942f;
constexpr uint32_t MAGIC = 0x64006400u;  // fp16 pair (1024, 1024)
constexpr float TAU = 8.f;               // lazy-rescale threshold (log2 units)
constexpr float M_NONE = -1e30f;         // reference max before any valid token

typedef __attribute__((address_space(3))) short4v lds_short4;
// read-only data read through the constant address space (scalar loads)
typedef __attribute__((address_space(4))) const int32_t const_i32;

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// (a & m) | o in one VALU op (the compiler otherwise emits an and plus an or)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

template <int F>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* pages, int pid,
                                                            bool any = true) {
  return __builtin_amdgcn_make_buffer_rsrc(
      (void*)(pages + (int64_t)pid * PageGeom<F>::BYTES), (short)0,
      any ? PageGeom<F>::BYTES : 0, 0x00020000);
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

// z halves of two (s, z) words, packed
__device__ __forceinline__ uint32_t z_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Two transposing 8-byte reads (rows r and r + 1 of each lane's pattern) of one
// 16-column block, as an 8-element operand.
__device__ __forceinline__ half8 tr_pair(const _Float16* lo_p, const _Float16* hi_p) {
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)lo_p);
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)hi_p);
  const half4 l4 = __builtin_bit_cast(half4, lo), h4 = __builtin_bit_cast(half4, hi);
  return (half8){l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
}

// Sum over the 16 lanes of a row (DPP butterfly: neighbours, pairs, half-row
// mirror, row mirror).
__device__ __forceinline__ float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
  return v;
}

// Raw data one lane loads for one page: sub-block j of its token in each of the
// 16 content blocks and the 2 RoPE blocks, and all (scale, zero) words of its
// token, one per 32-channel block (a group of 2 or 4 blocks repeats its word).
template <int F>
struct PageRegs {
  u32x4 c[fmt_cb(F) == 4 ? 4 : 2];  // content code chunks
  u32x4 sz[4];                      // content (s, z) words of blocks 0..15
  u32x2 r;                          // RoPE code words (4-bit: blocks 0, 1; 2-bit: .x)
  u32x2 rsz;                        // RoPE (s, z) words of blocks 0, 1
};

// BF16 baseline page: sub-block j of each of the token's 18 groups, raw bf16.
template <>
struct PageRegs<16> {
  u32x4 k[NG_C + NG_R];
};

// Byte offsets, inside a page, of what one lane (slot, sub-block j) loads,
// relative to the start of each region (the region starts go in the scalar
// offset of the buffer loads). The content code chunk m (16 bytes at + 64 m)
// holds sub-block j of blocks 4m .. 4m + 3 (INT4) or 8m .. 8m + 7 (INT2); the
// RoPE chunk j holds sub-block j of both RoPE blocks (8 bytes at 4 bits, 4 at 2).
template <int F>
struct LaneOffsets {
  uint32_t c, s, r, rs;
  __device__ LaneOffsets(int slot, int j) {
    using G = PageGeom<F>;
    c = slot * G::CC + 16 * j;
    s = slot * G::CS;
    r = slot * G::RC + (G::RB == 4 ? 8 : 4) * j;
    rs = slot * G::RS;
  }
};

// Buffer descriptor of one physical page (raw byte addressing, range = page;
// an empty range makes every load return 0 and touch nothing).
// BF16 page: sub-block j of group g of the row sits at + 64 g (RoPE groups
// follow the 16 content groups in the row).
template <>
struct LaneOffsets<16> {
  uint32_t c;
  __device__ LaneOffsets(int slot, int j) : c(slot * PageGeom<16>::ROW + 16 * j) {}
};

template <int F>
__device__ __forceinline__ void load_page(PageRegs<F>& t, __amdgpu_buffer_rsrc_t rs,
                                          const LaneOffsets<F>& o) {
  if constexpr (F == 16) {
#pragma unroll
    for (int g = 0; g < NG_C + NG_R; ++g)
      t.k[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.c, 64 * g, 0));
  } else {
    using G = PageGeom<F>;
#pragma unroll
    for (int m = 0; m < (G::CB == 4 ? 4 : 2); ++m)
      t.c[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.c, G::OFF_CC + 64 * m, 0));
    if constexpr (G::GM == 1) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        t.sz[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.s, G::OFF_CS + 16 * m, 0));
    } else if constexpr (G::GM == 2) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.s, G::OFF_CS + 16 * m, 0));
        t.sz[2 * m] = (u32x4){w.x, w.x, w.y, w.y};
        t.sz[2 * m + 1] = (u32x4){w.z, w.z, w.w, w.w};
      }
    } else {
      const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.s, G::OFF_CS, 0));
#pragma unroll
      for (int m = 0; m < 4; ++m) t.sz[m] = (u32x4){w[m], w[m], w[m], w[m]};
    }
    if constexpr (G::RB == 4) {
      t.r = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.r, G::OFF_RC, 0));
    } else {
      t.r = (u32x2){__builtin_amdgcn_raw_buffer_load_b32(rs, o.r, G::OFF_RC, 0), 0u};
    }
    if constexpr (G::GMR == 1) {
      t.rsz = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.rs, G::OFF_RS, 0));
    } else {
      const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rs, o.rs, G::OFF_RS, 0);
      t.rsz = (u32x2){w, w};
    }
  }
}

// Codes and (s, z) word of content block g (0..15).
template <int F>
__device__ __forceinline__ half8 content_codes(const PageRegs<F>& t, int g) {
  if (fmt_cb(F) == 4) return codes4(t.c[g >> 2][g & 3]);
  return codes2(t.c[g >> 3][(g & 7) >> 1], g & 1);
}
template <int F>
__device__ __forceinline__ uint32_t content_sz(const PageRegs<F>& t, int g) {
  return t.sz[g >> 2][g & 3];
}
// Codes of RoPE block gr (0, 1).
template <int F>
__device__ __forceinline__ half8 rope_codes(const PageRegs<F>& t, int gr) {
  if (fmt_rb(F) == 4) return codes4(t.r[gr]);
  return codes2(t.r.x, gr);
}

// Masked page: a token with keep false gets zero (scale, zero) words, so its
// codes contribute 0 to the scores and the tile (its score is set to -inf).
template <int F>
__device__ __forceinline__ void mask_token(PageRegs<F>& t, bool keep) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) t.sz[m][e] = keep ? t.sz[m][e] : 0u;
  t.rsz.x = keep ? t.rsz.x : 0u;
  t.rsz.y = keep ? t.rsz.y : 0u;
}

// Channel of sub-block j of group g (0..15 content, 16, 17 RoPE) in a
// [content | rope] row.
__device__ __forceinline__ int group_channel(int g, int j) {
  return g < NG_C ? GROUP * g + 8 * j : D_C + GROUP * (g - NG_C) + 8 * j;
}

}  // namespace mla
