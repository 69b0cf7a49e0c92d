// Fused cache writer for gfx950 (QuantMLA, Figure 8 caption: a packed copy of
// every incoming token plus BF16 copies of protected sink and recent tokens).
//
// One thread quantizes one 32-channel group of one token (16 content groups +
// 2 RoPE groups per token), so a token's 18 groups are handled by 18
// neighbouring lanes and its 1152 input bytes are read in 64-byte pieces.
// Every fp32 step is a single IEEE operation rounded to nearest even
// (__fsub_rn / __fdiv_rn, no contraction), so the codes and the fp16
// (scale, zero) pairs are bit-identical to a plain CPU evaluation.
#include "mla_common.h"
#include "mla_kernels.h"

namespace mla {

// Load the 32 bf16 values of one group (64 bytes) and widen them to fp32.
__device__ __forceinline__ void load_group(const uint16_t* src, u32x4 (&raw)[4],
                                           float (&x)[GROUP]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) raw[k] = reinterpret_cast<const u32x4*>(src)[k];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * k + 2 * e] = bf16_to_f32(raw[k][e] & 0xffffu);
      x[8 * k + 2 * e + 1] = bf16_to_f32(raw[k][e] >> 16);
    }
  }
}

// Asymmetric min-max quantization of one group to `bits`-bit codes: fp16
// scale s = (hi - lo) / (2^bits - 1) and zero z = lo (both rounded to nearest
// even), q = clamp(rint((x - z) / s), 0, 2^bits - 1), all codes 0 when s = 0.
__device__ __forceinline__ void quantize_group(const float (&x)[GROUP], int bits, _Float16& s16,
                                               _Float16& z16, uint32_t (&q)[GROUP]) {
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int i = 1; i < GROUP; ++i) {  // strict compares: the first of equal values wins
    lo = x[i] < lo ? x[i] : lo;
    hi = x[i] > hi ? x[i] : hi;
  }
  const float qmax = (float)((1 << bits) - 1);
  const float s32 = __fdiv_rn(__fsub_rn(hi, lo), qmax);
  s16 = (_Float16)s32;  // round to nearest even
  z16 = (_Float16)lo;
  const float s = (float)s16, z = (float)z16;
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    float r = 0.0f;
    if (s != 0.0f) {
      r = rintf(__fdiv_rn(__fsub_rn(x[i], z), s));
      r = fminf(fmaxf(r, 0.0f), qmax);
    }
    q[i] = (uint32_t)r;
  }
}

template <int CB>
__global__ __launch_bounds__(256) void write_kernel(WriteArgs a) {
  using G = PageGeom<CB>;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.n_tokens * (NG_C + NG_R);
  if (gid >= total) return;
  const int t = (int)(gid / (NG_C + NG_R));
  const int g = (int)(gid % (NG_C + NG_R));
  const int b = a.seq_idx ? a.seq_idx[t] : t;
  const int p = a.pos[t];
  // tokens outside the page table (or of no sequence) are dropped, never
  // written out of bounds
  if (b < 0 || b >= a.B || p < 0 || p >= a.max_pages * PAGE) return;
  const int L = a.seq_lens[b];
  const int64_t page = a.page_table[(int64_t)b * a.max_pages + p / PAGE];
  const int slot = p % PAGE;
  uint8_t* base = a.pages + page * (int64_t)G::BYTES;

  const bool rope = g >= NG_C;
  const int gi = rope ? g - NG_C : g;
  const int bits = rope ? 4 : CB;
  const uint16_t* src = rope ? a.k_rope + (int64_t)t * D_R + gi * GROUP
                             : a.c_kv + (int64_t)t * D_C + gi * GROUP;

  // 32 bf16 values as 16 dwords (64 B)
  u32x4 raw[4];
  float x[GROUP];
  load_group(src, raw, x);
  _Float16 s16, z16;
  uint32_t q[GROUP];
  quantize_group(x, bits, s16, z16, q);

  // pack (code order of the page layout): sub-block j (channels 8j..8j+7 of the
  // group) goes to chunk j of the group's chunk row; channel 8j + 2i + k sits at
  // bit 16k + bits * (4e + i) of its 32-bit word, e = code block of the group.
  const uint32_t sz = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
  if (rope) {
    // 2 groups per chunk: chunk j = 8 bytes at 8j, word gi
    uint8_t* row = base + G::OFF_RC + slot * G::RC;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v |= (q[8 * j + 2 * i] << (4 * i)) | (q[8 * j + 2 * i + 1] << (16 + 4 * i));
      *reinterpret_cast<uint32_t*>(row + 8 * j + 4 * gi) = v;
    }
  } else if (bits == 4) {
    // 4 groups per 16-byte chunk: chunk (ld, j) at 16 (4 ld + j), word gi % 4
    uint8_t* row = base + G::OFF_CC + slot * G::CC;
    const int ld = gi >> 2, w = gi & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v |= (q[8 * j + 2 * i] << (4 * i)) | (q[8 * j + 2 * i + 1] << (16 + 4 * i));
      *reinterpret_cast<uint32_t*>(row + 16 * (4 * ld + j) + 4 * w) = v;
    }
  } else {
    // 8 groups per 16-byte chunk, two per word (code block e): the group owns
    // byte e (even channels) and byte 2 + e (odd channels) of the word
    uint8_t* row = base + G::OFF_CC + slot * G::CC;
    const int ld = gi >> 3, w = (gi >> 1) & 3, e = gi & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= q[8 * j + 2 * i] << (2 * i);
        hi |= q[8 * j + 2 * i + 1] << (2 * i);
      }
      uint8_t* wp = row + 16 * (4 * ld + j) + 4 * w;
      wp[e] = (uint8_t)lo;
      wp[2 + e] = (uint8_t)hi;
    }
  }
  uint8_t* szdst = rope ? base + G::OFF_RS + slot * G::RS + gi * 4
                        : base + G::OFF_CS + slot * G::CS + gi * 4;
  *reinterpret_cast<uint32_t*>(szdst) = sz;

  // BF16 retention of protected tokens
  uint16_t* keep = nullptr;
  if (p < a.n_sink)
    keep = a.sink + ((int64_t)b * a.n_sink + p) * D_ALL;
  else if (p >= L - a.n_local)
    keep = a.local + ((int64_t)b * a.n_local + p % a.n_local) * D_ALL;
  if (keep) {
    u32x4* kd = reinterpret_cast<u32x4*>(keep + (rope ? D_C + gi * GROUP : gi * GROUP));
#pragma unroll
    for (int k = 0; k < 4; ++k) kd[k] = raw[k];
  }
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

hipError_t launch_write(const WriteArgs& a, int c_bits, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  if (c_bits == 16) {
    const int64_t total = (int64_t)a.n_tokens * (D_ALL / 8);
    write_bf16_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
  }
  const int64_t total = (int64_t)a.n_tokens * (NG_C + NG_R);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (c_bits == 4)
    write_kernel<4><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(a);
  else
    write_kernel<2><<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(a);
  return hipGetLastError();
}

// Simulated quantize-dequantize (Figure 3 caption): one thread per (token,
// group) quantizes its group as the writer does and stores x^ = q * s + z,
// one fused multiply-add rounded to fp32, then rounded to bf16 (nearest even).
template <int CB>
__global__ __launch_bounds__(256) void qdq_kernel(QdqArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.n_tokens * (NG_C + NG_R)) return;
  const int t = (int)(gid / (NG_C + NG_R));
  const int g = (int)(gid % (NG_C + NG_R));
  const bool rope = g >= NG_C;
  const int gi = rope ? g - NG_C : g;
  const int64_t off = rope ? (int64_t)t * D_R + gi * GROUP : (int64_t)t * D_C + gi * GROUP;
  u32x4 raw[4];
  float x[GROUP];
  load_group((rope ? a.k_rope : a.c_kv) + off, raw, x);
  _Float16 s16, z16;
  uint32_t q[GROUP];
  quantize_group(x, rope ? 4 : CB, s16, z16, q);
  const float s = (float)s16, z = (float)z16;
  u32x4* dst = reinterpret_cast<u32x4*>((rope ? a.out_r : a.out_c) + off);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __builtin_fmaf((float)q[8 * k + 2 * e], s, z);
      const float hi = __builtin_fmaf((float)q[8 * k + 2 * e + 1], s, z);
      v[e] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
    }
    dst[k] = v;
  }
}

hipError_t launch_qdq(const QdqArgs& a, int c_bits, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  const int64_t total = (int64_t)a.n_tokens * (NG_C + NG_R);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (c_bits == 4)
    qdq_kernel<4><<<grid, dim3(256), 0, stream>>>(a);
  else
    qdq_kernel<2><<<grid, dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mla
