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

// Cache format code F (a template parameter of the kernels): content code
// bits F & 31 (4 or 2; 16 is the paired BF16 cache), 2-bit RoPE codes when
// F & 32 is set (else 4-bit), quantization groups of 32 << (F >> 6) channels
// (32, 64 or 128). The workload formats keep small codes: C4R4 = 4 and
// C2R4 = 2 (groups of 32), the BF16 cache 16. The code order is the same for
// every group size (32-channel blocks of 8-channel sub-blocks); a group of 64
// or 128 channels has one (scale, zero) pair for its 2 or 4 blocks, and the
// 64-channel RoPE key is one group when the group is 128.
constexpr int fmt_code(int c_bits, int r_bits, int group) {
  return c_bits | (r_bits == 2 ? 32 : 0) | (group == 128 ? 128 : group == 64 ? 64 : 0);
}
constexpr int fmt_cb(int F) { return F & 31; }
constexpr int fmt_rb(int F) { return (F & 32) ? 2 : 4; }
constexpr int fmt_gm(int F) { return 1 << (F >> 6); }  // 32-channel blocks per content group
constexpr int fmt_gmr(int F) { return fmt_gm(F) < 2 ? fmt_gm(F) : 2; }  // per RoPE group

// Byte geometry of one page of format F.
template <int F>
struct PageGeom {
  static constexpr int CB = fmt_cb(F), RB = fmt_rb(F), GM = fmt_gm(F), GMR = fmt_gmr(F);
  static constexpr int CC = D_C * CB / 8;     // content code bytes per token
  static constexpr int RC = D_R * RB / 8;     // RoPE code bytes per token
  static constexpr int CS = NG_C / GM * 4;    // content (s, z) bytes per token
  static constexpr int RS = NG_R / GMR * 4;   // RoPE (s, z) bytes per token
  static constexpr int OFF_CC = 0;
  static constexpr int OFF_RC = PAGE * CC;
  static constexpr int OFF_CS = PAGE * (CC + RC);
  static constexpr int OFF_RS = PAGE * (CC + RC + CS);
  static constexpr int BYTES = PAGE * (CC + RC + CS + RS);
};
// BF16 baseline page (F = 16): 64 rows of [c (512) | k_rope (64)] bf16.
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
static_assert(PageGeom<fmt_code(4, 4, 64)>::BYTES == 64 * 324 &&
              PageGeom<fmt_code(4, 4, 128)>::BYTES == 64 * 308 &&
              PageGeom<fmt_code(4, 2, 32)>::BYTES == 64 * 344 &&
              PageGeom<fmt_code(2, 2, 32)>::BYTES == 64 * 216 &&
              PageGeom<fmt_code(2, 2, 128)>::BYTES == 64 * 164, "variant pages");

// Calls BODY(F) with F the compile-time code of a packed format (runtime
// value fmt, one of the twelve codes above); unknown codes do nothing.
#define MLA_FOR_PACKED_FMT(fmt, BODY) \
  switch (fmt) {                      \
    case 4: BODY(4); break;           \
    case 2: BODY(2); break;           \
    case 36: BODY(36); break;         \
    case 34: BODY(34); break;         \
    case 68: BODY(68); break;         \
    case 66: BODY(66); break;         \
    case 100: BODY(100); break;       \
    case 98: BODY(98); break;         \
    case 132: BODY(132); break;       \
    case 130: BODY(130); break;       \
    case 164: BODY(164); break;       \
    case 162: BODY(162); break;       \
    default: break;                   \
  }

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
