// Shared device-side definitions for the gfx950 kernels: vector types, the
// fixed cache geometry and small conversion helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D_C = 512;     // content latent channels
constexpr int D_R = 64;      // RoPE key channels
constexpr int D_ALL = 576;   // row width of the bf16 sink/local buffers
constexpr int GROUP = 32;    // channels per (scale, zero) pair
constexpr int PAGE = 64;     // token slots per page
constexpr int NG_C = D_C / GROUP;  // 16 content groups
constexpr int NG_R = D_R / GROUP;  // 2 RoPE groups

// Byte geometry of one page for a content code width of CB bits (RoPE: 4 bits).
template <int CB>
struct PageGeom {
  static constexpr int CC = D_C * CB / 8;   // content code bytes per token
  static constexpr int RC = D_R * 4 / 8;    // RoPE code bytes per token (32)
  static constexpr int CS = NG_C * 4;       // content (s, z) bytes per token (64)
  static constexpr int RS = NG_R * 4;       // RoPE (s, z) bytes per token (8)
  static constexpr int OFF_CC = 0;
  static constexpr int OFF_RC = PAGE * CC;
  static constexpr int OFF_CS = PAGE * (CC + RC);
  static constexpr int OFF_RS = PAGE * (CC + RC + CS);
  static constexpr int BYTES = PAGE * (CC + RC + CS + RS);
};
// BF16 baseline page (CB = 16): 64 rows of [c (512) | k_rope (64)] bf16.
template <>
struct PageGeom<16> {
  static constexpr int ROW = D_ALL * 2;  // bytes per token row (1152)
  static constexpr int BYTES = PAGE * ROW;
};
static_assert(PageGeom<16>::BYTES == 73728, "BF16 page");
static_assert(PageGeom<4>::BYTES == 23040, "C4R4 page");
static_assert(PageGeom<2>::BYTES == 14848, "C2R4 page");
static_assert(PageGeom<4>::OFF_RC == 16384 && PageGeom<4>::OFF_CS == 18432 &&
              PageGeom<4>::OFF_RS == 22528, "C4R4 regions");

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two bf16 (packed in one dword, low half first) -> two fp16. Exact for
// bf16 values inside the fp16 normal range (8 significant bits fit in 11).
__device__ __forceinline__ half2v bf16x2_to_f16x2(uint32_t w) {
  float lo = __uint_as_float(w << 16);
  float hi = __uint_as_float(w & 0xffff0000u);
  half2v r;
  r.x = (_Float16)lo;
  r.y = (_Float16)hi;
  return r;
}

__device__ __forceinline__ half8 bf16x8_to_f16x8(u32x4 w) {
  half2v a = bf16x2_to_f16x2(w.x), b = bf16x2_to_f16x2(w.y), c = bf16x2_to_f16x2(w.z),
         d = bf16x2_to_f16x2(w.w);
  half8 r;
  r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
  r[4] = c.x; r[5] = c.y; r[6] = d.x; r[7] = d.y;
  return r;
}

}  // namespace mla
