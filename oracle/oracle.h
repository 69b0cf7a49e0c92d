/*
 * CPU oracle for low-bit MLA KV caching and decode.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain-loop statement of
 * what the GPU path must compute. Only tests/, __graft_entry__.smoke() and
 * bench.py's cpu_baseline leg may load it. The product library never links,
 * loads or calls anything here, and nothing here is shared with the HIP code.
 *
 * The method is QuantMLA ("QuantMLA: Function-Aligned Dual-Path Quantization
 * for Low-Bit MLA KV Caching"):
 *   - packed INT4 content latent + INT4 RoPE key (C4R4), or INT2 content with
 *     an INT4 RoPE key (C2R4): abstract;
 *   - a fused writer packs every incoming token and keeps pre-quantization
 *     BF16 copies of the protected sink and recent tokens: Figure 8 caption,
 *     Figure 3 caption;
 *   - protection policy sink4/local128: Figure 5 caption, Table 9 caption;
 *   - attention reads BF16 for protected tokens and dequantized codes
 *     otherwise, under one global softmax: Figure 8 caption;
 *   - the decode is the absorbed (MQA) form of MLA in which every head attends
 *     over the shared latent: GQLA card on the same cards page.
 * The pages give no quantizer formula, bit order or page layout; the readings
 * taken here are listed in the comments of oracle.c.
 *
 * All buffers are host memory owned by the caller. bf16 and fp16 values are
 * passed as their raw uint16_t bit patterns.
 */
#ifndef MLA_ORACLE_H
#define MLA_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t d_c;       /* content latent width (512 in the workloads) */
  int32_t d_r;       /* decoupled RoPE key width (64) */
  int32_t c_bits;    /* content code width: 4 or 2 */
  int32_t r_bits;    /* RoPE code width: 4 or 2 */
  int32_t group;     /* channels per quantization group: 32, 64 or 128 */
  int32_t page_size; /* token slots per page (64) */
  int32_t n_sink;    /* leading protected tokens (4) */
  int32_t n_local;   /* trailing protected tokens (128) */
} orc_cfg;

/* 0 on success, negative on a rejected argument. */
int orc_check_cfg(const orc_cfg* cfg);

/* IEEE-754 binary32 -> binary16 with round-to-nearest-even (bit pattern). */
uint16_t orc_f32_to_f16(float x);
double orc_f16_to_f64(uint16_t h);
float orc_bf16_to_f32(uint16_t b);
/* binary64 -> bfloat16 with round-to-nearest-even (bit pattern). */
uint16_t orc_f64_to_bf16(double x);

/* Quantize one group of n fp32 values to `bits`-bit codes (one code per byte
 * in `codes`), returning the fp16 scale and zero bit patterns. */
void orc_quantize_group(const float* x, int n, int bits, uint16_t* s16, uint16_t* z16,
                        uint8_t* codes);

/* Byte offsets of the four regions inside one page and the page size. */
size_t orc_page_bytes(const orc_cfg* cfg);
void orc_page_regions(const orc_cfg* cfg, size_t off[4]);

/* Fused writer. Every token t gets a packed copy in page
 * page_table[seq_idx[t]][pos[t] / page_size], slot pos[t] % page_size, and a
 * BF16 copy in sink/local when it is protected under seq_lens (the lengths
 * after this write). Returns 0, or -1 if an index is out of range. */
int orc_write(const orc_cfg* cfg, int n_tokens, const uint16_t* c_kv, const uint16_t* k_rope,
              const int32_t* seq_idx, const int32_t* pos, const int32_t* seq_lens,
              const int32_t* page_table, int B, int max_pages, uint8_t* pages, int64_t num_pages,
              uint16_t* sink, uint16_t* local);

/* Source of token p in a sequence of length L: 0 = sink buffer, 1 = local
 * ring, 2 = packed page. */
int orc_token_source(const orc_cfg* cfg, int p, int L);

/* Values of token p of sequence b as seen by attention, in fp64:
 * kc[d_c] (content) and kr[d_r] (RoPE key). Returns 0 or -1. */
int orc_token_values(const orc_cfg* cfg, int b, int p, const uint8_t* pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const uint16_t* sink, const uint16_t* local, double* kc, double* kr);

/* Absorbed-MLA decode over tokens [p_begin, p_end) of each selected (b, h)
 * (clipped to [0, seq_lens[b])). p_end < 0 means "to the end". n_sel = 0
 * selects every (b, h) in row-major order; otherwise sel_b/sel_h list the
 * pairs. out is fp64 [n_rows][d_c], lse fp64 [n_rows] (natural log of the
 * sum of exp(scale * score)). An empty range gives out = 0, lse = -inf. */
int orc_decode(const orc_cfg* cfg, int B, int H, double scale, const uint16_t* q_lat,
               const uint16_t* q_rope, const uint8_t* pages, const int32_t* page_table,
               int max_pages, const int32_t* seq_lens, const uint16_t* sink,
               const uint16_t* local, int n_sel, const int32_t* sel_b, const int32_t* sel_h,
               int p_begin, int p_end, double* out, double* lse);

/* Merge n partial results (o_s[n][d], lse_s[n]) of one row into (out, lse). */
void orc_combine(int n, int d, const double* o_s, const double* lse_s, double* out, double* lse);

/* Paired BF16 cache, the unquantized baseline the low-bit kernel is measured
 * against (Figure 5(b) caption, Table 9 caption). Page = page_size rows of
 * [c (d_c) | k_rope (d_r)] bf16; row = slot of the token. */
size_t orc_bf16_page_bytes(const orc_cfg* cfg);
/* Copy each token's row into its page slot. Returns 0, or -1 on an index out
 * of range. */
int orc_bf16_write(const orc_cfg* cfg, int n_tokens, const uint16_t* c_kv,
                   const uint16_t* k_rope, const int32_t* seq_idx, const int32_t* pos,
                   const int32_t* page_table, int B, int max_pages, uint16_t* pages,
                   int64_t num_pages);
/* Exact (fp64) attention over tokens [0, seq_lens[b]) of the BF16 cache; row
 * selection and outputs as in orc_decode. */
int orc_bf16_decode(const orc_cfg* cfg, int B, int H, double scale, const uint16_t* q_lat,
                    const uint16_t* q_rope, const uint16_t* pages, const int32_t* page_table,
                    int max_pages, const int32_t* seq_lens, int n_sel, const int32_t* sel_b,
                    const int32_t* sel_h, double* out, double* lse);

/* Simulated quantize-dequantize (QDQ, Figure 3 caption): every group of every
 * token row through the writer's quantizer and back, x^ = q * s16 + z16,
 * rounded to fp32 and then to bf16 (both nearest even). out_c [n][d_c] and
 * out_r [n][d_r] are bf16 bit patterns. Returns 0 or -1. */
int orc_qdq(const orc_cfg* cfg, int n_tokens, const uint16_t* c_kv, const uint16_t* k_rope,
            uint16_t* out_c, uint16_t* out_r);

/* Threads the oracle's parallel loops use, and a way to change it (n > 0). */
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
