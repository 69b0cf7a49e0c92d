// Kernel argument blocks and launchers shared by the C-ABI entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct WriteArgs {
  int n_tokens;
  const uint16_t* c_kv;     // bf16 [n, 512]
  const uint16_t* k_rope;   // bf16 [n, 64]
  const int32_t* seq_idx;   // [n] or null (token t belongs to sequence t)
  const int32_t* pos;       // [n]
  const int32_t* seq_lens;  // [B], after the write
  const int32_t* page_table;
  int B, max_pages;
  uint8_t* pages;
  uint16_t* sink;
  uint16_t* local;
  int n_sink, n_local;
};

struct QdqArgs {
  int n_tokens;
  const uint16_t* c_kv;    // bf16 [n, 512]
  const uint16_t* k_rope;  // bf16 [n, 64]
  uint16_t* out_c;         // bf16 [n, 512]
  uint16_t* out_r;         // bf16 [n, 64]
};

struct DecodeArgs {
  const uint16_t* q_lat;   // bf16 [B, H, 512]
  const uint16_t* q_rope;  // bf16 [B, H, 64]
  const uint8_t* pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* seq_lens;
  const uint16_t* sink;
  const uint16_t* local;
  _Float16* ws_o;  // [B, n_split, H, 512] fp16 partial outputs (normalized)
  float* ws_lse;   // [B, n_split, H] fp32 partial log-sum-exp (natural log)
  int32_t* ws_meta;  // 128-head path: per (sequence, query token) the chunks touching it
  uint16_t* out;  // bf16 [B, H, 512]
  float* lse;     // fp32 [B, H]
  int B, H, n_split, pages_per_split, n_sink, n_local;
  // query tokens per sequence and heads per query token (H = s_q * h_per_q
  // rows per sequence; rows of query token i attend to p < len - (s_q - 1 - i))
  int s_q, h_per_q;
  float scale_log2;  // softmax_scale * log2(e)
};

// Upper bound on partials per sequence that the combine kernel merges.
constexpr int MAX_SPLITS = 2048;
// Upper bound on work items (pages or protected-token chunks) per workgroup.
constexpr int MAX_ITEMS = 512;

struct SplitPlan {
  int n_split;
  int pages_per_split;
};

SplitPlan plan_splits(int B, int H, int max_pages);
size_t decode_workspace_bytes(int B, int H, int max_pages);

// fmt: a format code of mla_common.h (fmt_code), or 16 for the BF16 pages
hipError_t launch_write(const WriteArgs& a, int fmt, hipStream_t stream);
hipError_t launch_decode(DecodeArgs a, int fmt, hipStream_t stream);
hipError_t launch_qdq(const QdqArgs& a, int fmt, hipStream_t stream);

// 128 heads per query token (packed caches): each page is dequantized once per
// 64 heads; work split by page weight on the device (decode_wide.hip).
size_t wide_workspace_bytes(int B, int s_q);
hipError_t launch_decode_wide(DecodeArgs a, void* workspace, int fmt, hipStream_t stream);

}  // namespace mla
