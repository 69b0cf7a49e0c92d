// C-ABI entry points (include/mla_lowbit.h): host-side validation, size
// queries and launches on the caller's stream. Nothing here allocates or
// synchronizes; the only state is the per-device address of the static
// scratch array of the no-allocation decode, looked up once.
#include <math.h>

#include <mutex>

#include "../../include/mla_lowbit.h"
#include "mla_common.h"
#include "mla_kernels.h"

using namespace mla;

namespace {

int check_cfg(const mla_lowbit_config* c) {
  if (!c) return MLA_LOWBIT_EINVAL;
  if (c->d_c != D_C || c->d_r != D_R || c->page_size != PAGE) return MLA_LOWBIT_EUNSUPPORTED;
  if (c->group != 32 && c->group != 64 && c->group != 128) return MLA_LOWBIT_EUNSUPPORTED;
  if ((c->c_bits != 4 && c->c_bits != 2) || (c->r_bits != 4 && c->r_bits != 2))
    return MLA_LOWBIT_EUNSUPPORTED;
  if (c->n_sink < 0 || c->n_sink > 64 || c->n_local < 0 || c->n_local > 256)
    return MLA_LOWBIT_EUNSUPPORTED;
  return MLA_LOWBIT_OK;
}

// Format code of a checked configuration (mla_common.h).
int fmt_of(const mla_lowbit_config* c) { return fmt_code(c->c_bits, c->r_bits, c->group); }

size_t page_bytes_of(int fmt) {
  size_t n = 0;
#define MLA_PAGE_BYTES(F) n = (size_t)PageGeom<F>::BYTES
  MLA_FOR_PACKED_FMT(fmt, MLA_PAGE_BYTES)
#undef MLA_PAGE_BYTES
  return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
bool ok_ptr4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

int write_checks(const mla_lowbit_config* cfg, int n_tokens, const void* c_kv,
                 const void* k_rope, const int32_t* pos, const int32_t* seq_lens,
                 const int32_t* page_table, int B, int max_pages, void* pages, void* sink,
                 void* local) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (n_tokens < 0 || B < 0 || max_pages < 1) return MLA_LOWBIT_EINVAL;
  if (n_tokens == 0) return MLA_LOWBIT_OK;
  if (B == 0) return MLA_LOWBIT_EINVAL;
  if (!ok_ptr(c_kv) || !ok_ptr(k_rope) || !ok_ptr4(pos) || !ok_ptr4(seq_lens) ||
      !ok_ptr4(page_table) || !ok_ptr(pages))
    return MLA_LOWBIT_EINVAL;
  if (cfg->n_sink > 0 && !ok_ptr(sink)) return MLA_LOWBIT_EINVAL;
  if (cfg->n_local > 0 && !ok_ptr(local)) return MLA_LOWBIT_EINVAL;
  return MLA_LOWBIT_OK;
}

int decode_checks(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                  const void* q_lat, const void* q_rope, const void* pages,
                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                  const void* sink, const void* local, void* out, float* lse, void* workspace,
                  size_t workspace_bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (B < 0 || H <= 0 || H % 16 != 0 || max_pages < 1) return MLA_LOWBIT_EINVAL;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_LOWBIT_EINVAL;
  if (B == 0) return MLA_LOWBIT_OK;
  if (!ok_ptr(q_lat) || !ok_ptr(q_rope) || !ok_ptr(pages) || !ok_ptr4(page_table) ||
      !ok_ptr4(seq_lens) || !ok_ptr(out) || !ok_ptr(lse) || !ok_ptr(workspace))
    return MLA_LOWBIT_EINVAL;
  if (cfg->n_sink > 0 && !ok_ptr(sink)) return MLA_LOWBIT_EINVAL;
  if (cfg->n_local > 0 && !ok_ptr(local)) return MLA_LOWBIT_EINVAL;
  if (plan_splits(B, H, max_pages).n_split > MAX_SPLITS) return MLA_LOWBIT_EUNSUPPORTED;
  if (workspace_bytes < decode_workspace_bytes(B, H, max_pages)) return MLA_LOWBIT_EWORKSPACE;
  return MLA_LOWBIT_OK;
}

DecodeArgs make_decode_args(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                            const void* q_lat, const void* q_rope, const void* pages,
                            const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                            const void* sink, const void* local, void* out, float* lse,
                            void* workspace) {
  const SplitPlan sp = plan_splits(B, H, max_pages);
  DecodeArgs a;
  a.q_lat = static_cast<const uint16_t*>(q_lat);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.pages = static_cast<const uint8_t*>(pages);
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.sink = static_cast<const uint16_t*>(sink);
  a.local = static_cast<const uint16_t*>(local);
  a.ws_lse = static_cast<float*>(workspace);
  a.ws_o = reinterpret_cast<_Float16*>(a.ws_lse + (size_t)B * sp.n_split * H);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.n_split = sp.n_split;
  a.pages_per_split = sp.pages_per_split;
  a.n_sink = cfg->n_sink;
  a.n_local = cfg->n_local;
  a.s_q = 1;
  a.h_per_q = H;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  return a;
}


}  // namespace

// Static workspace of mla_lowbit_decode_noalloc (one copy per GPU, held until
// the process ends). In host code `scratch` only names the symbol: its device
// address on the current GPU comes from hipGetSymbolAddress, looked up once
// per device, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[MLA_LOWBIT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;

// Device address of `scratch` on the current device, or null on a HIP error.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int mla_lowbit_version(void) { return 100; }

const char* mla_lowbit_strerror(int code) {
  switch (code) {
    case MLA_LOWBIT_OK: return "ok";
    case MLA_LOWBIT_EINVAL: return "invalid argument (null/misaligned pointer, count or shape)";
    case MLA_LOWBIT_EUNSUPPORTED: return "unsupported cache configuration";
    case MLA_LOWBIT_EWORKSPACE: return "workspace smaller than mla_lowbit_decode_workspace_bytes";
    case MLA_LOWBIT_ELAUNCH: return "HIP kernel launch failed";
    case MLA_LOWBIT_ESCRATCH:
      return "shape needs more workspace than the 64 MiB static scratch of the no-allocation decode";
    default: return "unknown error code";
  }
}

int mla_lowbit_check_config(const mla_lowbit_config* cfg) { return check_cfg(cfg); }

size_t mla_lowbit_page_bytes(const mla_lowbit_config* cfg) {
  if (check_cfg(cfg)) return 0;
  return page_bytes_of(fmt_of(cfg));
}

size_t mla_lowbit_decode_workspace_bytes(const mla_lowbit_config* cfg, int B, int H,
                                         int max_pages) {
  if (check_cfg(cfg) || B < 0 || H <= 0 || H % 16 != 0 || max_pages < 1) return 0;
  return decode_workspace_bytes(B, H, max_pages);
}

int mla_lowbit_write(const mla_lowbit_config* cfg, int n_tokens, const void* c_kv,
                     const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                     const int32_t* seq_lens, const int32_t* page_table, int B, int max_pages,
                     void* pages, void* sink, void* local, void* stream) {
  int rc = write_checks(cfg, n_tokens, c_kv, k_rope, pos, seq_lens, page_table, B, max_pages,
                        pages, sink, local);
  if (rc || n_tokens == 0) return rc;
  if (!ok_ptr4(seq_idx)) return MLA_LOWBIT_EINVAL;
  WriteArgs a;
  a.n_tokens = n_tokens;
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_rope = static_cast<const uint16_t*>(k_rope);
  a.seq_idx = seq_idx;
  a.pos = pos;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.B = B;
  a.max_pages = max_pages;
  a.pages = static_cast<uint8_t*>(pages);
  a.sink = static_cast<uint16_t*>(sink);
  a.local = static_cast<uint16_t*>(local);
  a.n_sink = cfg->n_sink;
  a.n_local = cfg->n_local;
  return launch_write(a, fmt_of(cfg), static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

int mla_lowbit_decode(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                      const void* q_lat, const void* q_rope, const void* pages,
                      const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                      const void* sink, const void* local, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = decode_checks(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table, max_pages,
                         seq_lens, sink, local, out, lse, workspace, workspace_bytes);
  if (rc || B == 0) return rc;
  DecodeArgs a = make_decode_args(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table,
                                  max_pages, seq_lens, sink, local, out, lse, workspace);
  return launch_decode(a, fmt_of(cfg), static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

int mla_lowbit_decode_noalloc(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                              const void* q_lat, const void* q_rope, const void* pages,
                              const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                              const void* sink, const void* local, void* out, float* lse,
                              void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (B < 0 || H <= 0 || H % 16 != 0 || max_pages < 1) return MLA_LOWBIT_EINVAL;
  if (B == 0) return decode_checks(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table,
                                   max_pages, seq_lens, sink, local, out, lse, nullptr, 0);
  const size_t need = decode_workspace_bytes(B, H, max_pages);
  if (need > MLA_LOWBIT_NOALLOC_SCRATCH_BYTES) return MLA_LOWBIT_ESCRATCH;
  // every other check first, with a stand-in workspace address, so that a bad
  // argument is reported before the device is touched
  rc = decode_checks(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table, max_pages,
                     seq_lens, sink, local, out, lse, reinterpret_cast<void*>(uintptr_t{256}),
                     MLA_LOWBIT_NOALLOC_SCRATCH_BYTES);
  if (rc) return rc;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return MLA_LOWBIT_ELAUNCH;
  DecodeArgs a = make_decode_args(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table,
                                  max_pages, seq_lens, sink, local, out, lse, ws);
  return launch_decode(a, fmt_of(cfg), static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

int mla_lowbit_decode_mq(const mla_lowbit_config* cfg, int B, int s_q, int H,
                         float softmax_scale, const void* q_lat, const void* q_rope,
                         const void* pages, const int32_t* page_table, int max_pages,
                         const int32_t* seq_lens, const void* sink, const void* local, void* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (s_q < 1 || H <= 0 || H % 16 != 0 || (int64_t)s_q * H > (1 << 20)) return MLA_LOWBIT_EINVAL;
  const int R = s_q * H;  // rows per sequence
  int rc = decode_checks(cfg, B, R, softmax_scale, q_lat, q_rope, pages, page_table, max_pages,
                         seq_lens, sink, local, out, lse, workspace, workspace_bytes);
  if (rc || B == 0) return rc;
  DecodeArgs a = make_decode_args(cfg, B, R, softmax_scale, q_lat, q_rope, pages, page_table,
                                  max_pages, seq_lens, sink, local, out, lse, workspace);
  a.s_q = s_q;
  a.h_per_q = H;
  return launch_decode(a, fmt_of(cfg), static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

int mla_lowbit_write_decode(const mla_lowbit_config* cfg, int B, int H, float softmax_scale,
                            const void* c_kv, const void* k_rope, const int32_t* pos,
                            const void* q_lat, const void* q_rope, void* pages,
                            const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                            void* sink, void* local, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int rc = write_checks(cfg, B, c_kv, k_rope, pos, seq_lens, page_table, B, max_pages, pages,
                        sink, local);
  if (rc) return rc;
  rc = decode_checks(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table, max_pages,
                     seq_lens, sink, local, out, lse, workspace, workspace_bytes);
  if (rc || B == 0) return rc;
  WriteArgs w;
  w.n_tokens = B;
  w.c_kv = static_cast<const uint16_t*>(c_kv);
  w.k_rope = static_cast<const uint16_t*>(k_rope);
  w.seq_idx = nullptr;  // token t belongs to sequence t
  w.pos = pos;
  w.seq_lens = seq_lens;
  w.page_table = page_table;
  w.B = B;
  w.max_pages = max_pages;
  w.pages = static_cast<uint8_t*>(pages);
  w.sink = static_cast<uint16_t*>(sink);
  w.local = static_cast<uint16_t*>(local);
  w.n_sink = cfg->n_sink;
  w.n_local = cfg->n_local;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_write(w, fmt_of(cfg), s) != hipSuccess) return MLA_LOWBIT_ELAUNCH;
  DecodeArgs a = make_decode_args(cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table,
                                  max_pages, seq_lens, sink, local, out, lse, workspace);
  return launch_decode(a, fmt_of(cfg), s) == hipSuccess ? MLA_LOWBIT_OK : MLA_LOWBIT_ELAUNCH;
}

int mla_lowbit_qdq(const mla_lowbit_config* cfg, int n_tokens, const void* c_kv,
                   const void* k_rope, void* out_c, void* out_r, void* stream) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (n_tokens < 0) return MLA_LOWBIT_EINVAL;
  if (n_tokens == 0) return MLA_LOWBIT_OK;
  if (!ok_ptr(c_kv) || !ok_ptr(k_rope) || !ok_ptr(out_c) || !ok_ptr(out_r))
    return MLA_LOWBIT_EINVAL;
  QdqArgs a;
  a.n_tokens = n_tokens;
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_rope = static_cast<const uint16_t*>(k_rope);
  a.out_c = static_cast<uint16_t*>(out_c);
  a.out_r = static_cast<uint16_t*>(out_r);
  return launch_qdq(a, fmt_of(cfg), static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

size_t mla_bf16_page_bytes(void) { return (size_t)PageGeom<16>::BYTES; }

size_t mla_bf16_decode_workspace_bytes(int B, int H, int max_pages) {
  if (B < 0 || H <= 0 || H % 16 != 0 || max_pages < 1) return 0;
  return decode_workspace_bytes(B, H, max_pages);
}

int mla_bf16_write(int n_tokens, const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                   const int32_t* pos, const int32_t* page_table, int B, int max_pages,
                   void* pages, void* stream) {
  if (n_tokens < 0 || B < 0 || max_pages < 1) return MLA_LOWBIT_EINVAL;
  if (n_tokens == 0) return MLA_LOWBIT_OK;
  if (B == 0) return MLA_LOWBIT_EINVAL;
  if (!ok_ptr(c_kv) || !ok_ptr(k_rope) || !ok_ptr4(seq_idx) || !ok_ptr4(pos) ||
      !ok_ptr4(page_table) || !ok_ptr(pages))
    return MLA_LOWBIT_EINVAL;
  WriteArgs a = {};
  a.n_tokens = n_tokens;
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_rope = static_cast<const uint16_t*>(k_rope);
  a.seq_idx = seq_idx;
  a.pos = pos;
  a.page_table = page_table;
  a.B = B;
  a.max_pages = max_pages;
  a.pages = static_cast<uint8_t*>(pages);
  return launch_write(a, 16, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

int mla_bf16_decode(int B, int H, float softmax_scale, const void* q_lat, const void* q_rope,
                    const void* pages, const int32_t* page_table, int max_pages,
                    const int32_t* seq_lens, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (B < 0 || H <= 0 || H % 16 != 0 || max_pages < 1) return MLA_LOWBIT_EINVAL;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_LOWBIT_EINVAL;
  if (B == 0) return MLA_LOWBIT_OK;
  if (!ok_ptr(q_lat) || !ok_ptr(q_rope) || !ok_ptr(pages) || !ok_ptr4(page_table) ||
      !ok_ptr4(seq_lens) || !ok_ptr(out) || !ok_ptr(lse) || !ok_ptr(workspace))
    return MLA_LOWBIT_EINVAL;
  if (plan_splits(B, H, max_pages).n_split > MAX_SPLITS) return MLA_LOWBIT_EUNSUPPORTED;
  if (workspace_bytes < decode_workspace_bytes(B, H, max_pages)) return MLA_LOWBIT_EWORKSPACE;
  // no protected buffers: n_sink = n_local = 0
  mla_lowbit_config cfg = {D_C, D_R, 16, 16, GROUP, PAGE, 0, 0};
  DecodeArgs a = make_decode_args(&cfg, B, H, softmax_scale, q_lat, q_rope, pages, page_table,
                                  max_pages, seq_lens, nullptr, nullptr, out, lse, workspace);
  return launch_decode(a, 16, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_LOWBIT_OK
             : MLA_LOWBIT_ELAUNCH;
}

}  // extern "C"
