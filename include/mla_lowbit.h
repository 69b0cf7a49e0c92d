/*
 * mla_lowbit: packed low-bit MLA KV cache writer and absorbed-MLA decode for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is QuantMLA ("QuantMLA: Function-Aligned Dual-Path Quantization
 * for Low-Bit MLA KV Caching", newx.sg summary page and thelatestinai.com
 * cards page):
 *   - the cache keeps the content latent c_kv and the decoupled RoPE key
 *     k_rope as low-bit codes: INT4 + INT4 ("C4R4") or INT2 content with an
 *     INT4 RoPE key ("C2R4") (abstract);
 *   - a fused writer packs every incoming token; sink and recent tokens also
 *     keep their original unquantized BF16 rows, in buffers of their own
 *     (Figure 8 caption; Figure 3 caption);
 *   - the protection policy is sink4/local128 (Figure 5 and Table 9 captions);
 *   - attention unpacks and dequantizes inside the kernel, reads BF16 values
 *     for protected tokens, shares one reconstructed content tile between the
 *     matching (QK) and aggregation (PV) products, and normalizes all valid
 *     tokens with one softmax (Figure 8 caption; abstract);
 *   - decode is the absorbed (MQA) form of MLA: every query head attends over
 *     the one shared latent (GQLA card on the same cards page).
 * The pages fix no quantizer formula, code order, page layout or partitioning;
 * the choices made here are stated below.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers, owned and allocated by the
 *     caller, 16-byte aligned. The library never allocates, frees,
 *     synchronizes or keeps state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work on it and return; results are ready when the stream reaches them.
 *   - bf16 / fp16 arrays hold the raw 16-bit patterns.
 *   - Return value: MLA_LOWBIT_OK (0) or a negative error code. Arguments are
 *     validated on the host before anything is launched; on an error nothing
 *     is enqueued. Contents of device buffers are not validated: an
 *     out-of-range page-table entry, position or length is undefined behaviour.
 *   - Calls are reentrant and thread-safe.
 *
 * Quantizer (per token, per group of cfg->group contiguous channels, 32 in
 * the C4R4 / C2R4 workloads, 64 or 128 as variants; a group never spans the
 * content / RoPE boundary, and at group 128 the 64-channel RoPE key is one
 * group; bit-exact):
 *   lo = min, hi = max of the group (bf16 values widened to fp32);
 *   s = fp16_rne(fp32(hi - lo) / fp32(2^b - 1)), z = fp16_rne(lo);
 *   q = 0 if s == 0, else clamp(rint_even((x - z) / s), 0, 2^b - 1) in fp32;
 *   the decode reconstructs x = q * s + z.
 *
 * Page layout (page_size = 64 token slots; slot = pos % 64 in page
 * page_table[b][pos / 64]); four token-major regions, C4R4 / C2R4:
 *   content codes  [64][256 | 128] B   at 0
 *   RoPE codes     [64][32] B          at 16384 | 8192
 *   content (s,z)  [64][16][2] fp16    at 18432 | 10240
 *   RoPE (s,z)     [64][2][2] fp16     at 22528 | 14336
 *   page bytes     23040 | 14848       (360 | 232 B per token)
 * In general the regions are, per token, d_c c_bits / 8 and d_r r_bits / 8
 * code bytes, then one 4-byte (s, z) pair per content group and per RoPE
 * group, each region 64 tokens long, in that order (e.g. C4R4 with groups of
 * 64: 256 + 32 + 8 * 4 + 1 * 4 = 324 B per token; C2R2 with groups of 32:
 * 128 + 16 + 16 * 4 + 2 * 4 = 216 B).
 * Code order inside a token's code row (little-endian 32-bit words), the same
 * for every group size: channel c of 32-channel block g is 32 g + 8 j + 2 i + k
 * with sub-block j, pair i = 0..3, k = 0, 1:
 *   content, 4-bit: 16-byte chunk (j, l = g div 4) at byte 16 (4 l + j), word
 *     g mod 4, channel at bit 16 k + 4 i;
 *   content, 2-bit: 16-byte chunk (j, l = g div 8) at byte 16 (4 l + j), word
 *     (g mod 8) div 2, channel at bit 16 k + 8 (g mod 2) + 2 i;
 *   RoPE, 4-bit: 8-byte chunk j at byte 8 j, word g, channel at bit 16 k + 4 i;
 *   RoPE, 2-bit: 4-byte chunk j at byte 4 j (one word), channel at bit
 *     16 k + 8 g + 2 i.
 * So one 16-byte load gives the same 8 channels of 4 (or 8) blocks, and even
 * channels sit in the low half-word, odd ones in the high half-word.
 *
 * Protected tokens (sink / local buffers, bf16 [B][n][d_c + d_r], row =
 * [c_kv | k_rope]): token p of a sequence of length L is read from
 * sink[b][p] if p < n_sink, else from local[b][p % n_local] if
 * p >= L - n_local, else from its packed copy.
 */
#ifndef MLA_LOWBIT_H
#define MLA_LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_LOWBIT_OK 0
#define MLA_LOWBIT_EINVAL (-1)       /* null/misaligned pointer, bad count or shape */
#define MLA_LOWBIT_EUNSUPPORTED (-2) /* configuration outside what the kernels build */
#define MLA_LOWBIT_EWORKSPACE (-3)   /* workspace smaller than the size query says */
#define MLA_LOWBIT_ELAUNCH (-4)      /* the HIP runtime reported a launch error */
#define MLA_LOWBIT_ESCRATCH (-5)     /* shape needs more than the static scratch holds */

/* Size of the static device scratch array that mla_lowbit_decode_noalloc
 * uses in place of a caller's workspace (one copy per GPU, held until the
 * process ends). */
#define MLA_LOWBIT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Cache geometry. Supported: d_c = 512, d_r = 64, c_bits in {4, 2},
 * r_bits in {4, 2}, group in {32, 64, 128}, page_size = 64,
 * 0 <= n_sink <= 64, 0 <= n_local <= 256. The workloads use C4R4 and C2R4
 * (r_bits = 4, group = 32); the other bit widths and group sizes are
 * variants of the same writer and decode (QuantMLA abstract: INT4 or INT2
 * content with an INT4 RoPE key; 2-bit caches on the RoLaQ page). */
typedef struct mla_lowbit_config {
  int32_t d_c;       /* content latent width */
  int32_t d_r;       /* decoupled RoPE key width */
  int32_t c_bits;    /* content code bits */
  int32_t r_bits;    /* RoPE key code bits */
  int32_t group;     /* channels per (scale, zero) group */
  int32_t page_size; /* token slots per page */
  int32_t n_sink;    /* leading tokens kept in BF16 */
  int32_t n_local;   /* most recent tokens kept in BF16 (ring of n_local slots) */
} mla_lowbit_config;

/* Library version (major * 10000 + minor * 100 + patch). */
int mla_lowbit_version(void);

/* Static message for an error code (never NULL). */
const char* mla_lowbit_strerror(int code);

/* MLA_LOWBIT_OK if the kernels support `cfg`, else EINVAL / EUNSUPPORTED. */
int mla_lowbit_check_config(const mla_lowbit_config* cfg);

/* Bytes of one cache page (23040 for C4R4, 14848 for C2R4); 0 if unsupported. */
size_t mla_lowbit_page_bytes(const mla_lowbit_config* cfg);

/* Workspace bytes mla_lowbit_decode needs for this shape (depends only on
 * host-side scalars); 0 if unsupported. */
size_t mla_lowbit_decode_workspace_bytes(const mla_lowbit_config* cfg, int B, int H,
                                         int max_pages);

/*
 * Fused writer (Figure 8 caption: a packed copy for every incoming token, plus
 * the unquantized BF16 row of each protected token).
 *   n_tokens    tokens to write (>= 0; 0 is a no-op)
 *   c_kv        bf16 [n_tokens, d_c]   content latents
 *   k_rope      bf16 [n_tokens, d_r]   RoPE keys, already rotated
 *   seq_idx     int32 [n_tokens]       sequence of each token, in [0, B)
 *   pos         int32 [n_tokens]       position of each token in its sequence
 *   seq_lens    int32 [B]              sequence lengths AFTER this write
 *   page_table  int32 [B, max_pages]   physical page of each logical page
 *   pages       uint8 [num_pages, page_bytes]   packed cache (written)
 *   sink        bf16 [B, n_sink, d_c + d_r]     (written for pos < n_sink)
 *   local       bf16 [B, n_local, d_c + d_r]    (written for pos >= len - n_local)
 * Each (seq, pos) may appear at most once per call, so no ring slot is
 * written twice by one call. A token whose seq_idx is outside [0, B) or whose
 * pos is outside [0, max_pages * page_size) is dropped (nothing is written);
 * page_table entries must name pages that exist (not checked on the device).
 * A token leaving the recent window needs no call: its packed copy already
 * exists (Figure 8 caption).
 * Precondition: every c_kv / k_rope value lies in the fp16 range
 * (|x| <= 65504), since each group's zero point and scale are stored in fp16;
 * a group beyond it gets an infinite zero or scale and undefined codes.
 */
int mla_lowbit_write(const mla_lowbit_config* cfg, int n_tokens, const void* c_kv,
                     const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                     const int32_t* seq_lens, const int32_t* page_table, int B, int max_pages,
                     void* pages, void* sink, void* local, void* stream);

/*
 * Absorbed-MLA decode over the mixed BF16 / packed cache (abstract; Figure 8
 * caption; GQLA card). For every sequence b and head h, over tokens
 * p < seq_lens[b]:
 *   score[p] = softmax_scale * (q_lat[b,h] . c[p] + q_rope[b,h] . k_rope[p])
 *   out[b,h] = sum_p softmax(score)[p] * c[p]          (bf16, RNE)
 *   lse[b,h] = log(sum_p exp(score[p]))                (fp32, natural log)
 * with c / k_rope read from BF16 buffers for protected tokens and
 * dequantized otherwise. A sequence of length 0 gives out = 0, lse = -inf;
 * seq_lens[b] is clamped to [0, max_pages * page_size]. The pages of all
 * tokens p < seq_lens[b] (page_table[b][0 .. ceil(L / 64))) must exist: every
 * token has a packed copy, protected ones included.
 *   H            heads, a positive multiple of 16
 *   q_lat        bf16 [B, H, d_c];  q_rope  bf16 [B, H, d_r]
 *   out          bf16 [B, H, d_c];  lse     fp32 [B, H]
 *   workspace    device scratch of at least
 *                mla_lowbit_decode_workspace_bytes(cfg, B, H, max_pages) bytes
 * The sequence is split into page ranges processed in parallel and merged by
 * their log-sum-exp (one global softmax, Figure 8 caption).
 * Precondition (fp16 inside the kernel): q_lat, q_rope and the BF16 rows of
 * the sink / local buffers are converted to fp16 for the MFMA products. That
 * is exact for bf16 values with 2^-14 <= |x| <= 65504 (and for 0); larger
 * magnitudes overflow to infinity (undefined results), and smaller ones
 * become fp16 subnormals that keep only the bits at or above 2^-24.
 */
int mla_lowbit_decode(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                      const void* q_lat, const void* q_rope, const void* pages,
                      const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                      const void* sink, const void* local, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_lowbit_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc. Same arguments, kernels and results as mla_lowbit_decode, minus
 * the workspace: the page-range partials go to a file-scope static device
 * array of MLA_LOWBIT_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, whose address is
 * looked up once per device on the first call made with that device current.
 * The call allocates nothing, through HIP or any library.
 *   - A shape whose workspace (mla_lowbit_decode_workspace_bytes) exceeds
 *     MLA_LOWBIT_NOALLOC_SCRATCH_BYTES is refused with MLA_LOWBIT_ESCRATCH
 *     before anything is launched.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, no ordering between them) race and
 *     give undefined results; calls ordered on one stream are safe. Nothing in
 *     the array needs to start at zero (every partial a call reads was written
 *     earlier in the same call).
 *   - `stream` must belong to the current device.
 */
int mla_lowbit_decode_noalloc(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                              const void* q_lat, const void* q_rope, const void* pages,
                              const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                              const void* sink, const void* local, void* out, float* lse,
                              void* stream);

/*
 * Multi-query decode over the same cache: s_q query tokens per sequence, the
 * last s_q tokens of the cache (GQLA card on the cards page: multi-token
 * prediction verifies s_q = 2 tokens per step). Query token i (0 <= i < s_q)
 * attends causally, to tokens p < seq_lens[b] - (s_q - 1 - i); which tokens
 * come from the BF16 buffers is decided by seq_lens[b], as in
 * mla_lowbit_decode. s_q = 1 is mla_lowbit_decode.
 *   H            heads per query token, a positive multiple of 16
 *   q_lat        bf16 [B, s_q, H, d_c];  q_rope  bf16 [B, s_q, H, d_r]
 *   out          bf16 [B, s_q, H, d_c];  lse     fp32 [B, s_q, H]
 *   workspace    at least mla_lowbit_decode_workspace_bytes(cfg, B, s_q * H,
 *                max_pages) bytes
 * A query token with no token to attend to (seq_lens[b] < s_q - i) gives
 * out = 0, lse = -inf.
 */
int mla_lowbit_decode_mq(const mla_lowbit_config* cfg, int B, int s_q, int H,
                         float softmax_scale, const void* q_lat, const void* q_rope,
                         const void* pages, const int32_t* page_table, int max_pages,
                         const int32_t* seq_lens, const void* sink, const void* local, void* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One serving step (Figure 8 caption): write one new token per sequence
 * (mla_lowbit_write with n_tokens = B, seq_idx = 0..B-1, pos[b] =
 * seq_lens[b] - 1), then decode every sequence including its new token.
 * Arguments as in the two calls above; enqueued in that order on `stream`.
 */
int mla_lowbit_write_decode(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                            const void* c_kv, const void* k_rope, const int32_t* pos,
                            const void* q_lat, const void* q_rope, void* pages,
                            const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                            void* sink, void* local, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Simulated quantize-dequantize, QDQ (Figure 3 caption: the quantizer applied
 * and undone in place, as calibration and accuracy studies use it). Every
 * group of every row goes through the writer's quantizer above at cfg's bit
 * widths and comes back as x^ = q * s + z, rounded once to fp32 (a fused
 * multiply-add) and then to bf16 (nearest even). Bit-exact; no protection
 * policy applies (n_sink / n_local are ignored).
 *   c_kv, k_rope   bf16 [n_tokens, d_c], [n_tokens, d_r]  inputs
 *   out_c, out_r   bf16 [n_tokens, d_c], [n_tokens, d_r]  outputs (may alias the inputs)
 */
int mla_lowbit_qdq(const mla_lowbit_config* cfg, int n_tokens, const void* c_kv,
                   const void* k_rope, void* out_c, void* out_r, void* stream);

/*
 * Paired BF16 cache: the unquantized baseline that the low-bit decode is
 * measured against (Figure 5(b) caption: attention latency normalized to
 * paired measurements with a BF16 cache; Table 9 caption: delta =
 * t_C4R4 / t_BF16 - 1). Same paging as the packed cache (64-token pages,
 * page_table[b][pos / 64], slot pos % 64), d_c = 512, d_r = 64; a page holds
 * 64 rows of [c_kv (512) | k_rope (64)] bf16 (73728 bytes); no sink or local
 * buffers. The decode runs the same kernel skeleton as mla_lowbit_decode
 * (page ranges, or at 128 heads the length-aware chunks; one softmax,
 * log-sum-exp merge) without the unpacking: with 128 heads per query token
 * the scores are one fp16 MFMA chain over the rows converted to fp16, with
 * any other head count bf16 MFMA on the rows as stored. The product with P
 * is in fp16 in both, so the fp16-range precondition of the packed cache
 * applies:
 * |x| <= 65504 for every cached value, and values below 2^-14 keep only the
 * bits an fp16 subnormal holds.
 */
size_t mla_bf16_page_bytes(void);
size_t mla_bf16_decode_workspace_bytes(int B, int H, int max_pages);

/* Copy each token's row into its page slot; arguments as in mla_lowbit_write
 * (tokens outside [0, B) x [0, max_pages * 64) are dropped). */
int mla_bf16_write(int n_tokens, const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                   const int32_t* pos, const int32_t* page_table, int B, int max_pages,
                   void* pages, void* stream);

/* Attention over tokens p < seq_lens[b] of the BF16 cache; arguments and
 * outputs as in mla_lowbit_decode (workspace of at least
 * mla_bf16_decode_workspace_bytes(B, H, max_pages) bytes). */
int mla_bf16_decode(int B, int H, float softmax_scale, const void* q_lat, const void* q_rope,
                    const void* pages, const int32_t* page_table, int max_pages,
                    const int32_t* seq_lens, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif
