// C ABI of the QSA library: host-side argument checks, then kernel launches on the
// caller's stream.  Nothing here allocates, frees or synchronizes.
#include "qsa.h"
#include "qsa_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

thread_local std::string g_last_error;

qsa_status fail(qsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

qsa_status ok() {
  g_last_error.clear();
  return QSA_OK;
}

qsa_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QSA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define QSA_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define QSA_PTR(p, name)                                                                   \
  do {                                                                                     \
    QSA_REQUIRE((p) != nullptr, QSA_ERR_INVALID_ARGUMENT, "%s must not be NULL", name);    \
    QSA_REQUIRE(aligned16(p), QSA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name); \
  } while (0)

#define QSA_OPT_PTR(p, name)                                                                 \
  do {                                                                                       \
    QSA_REQUIRE((p) == nullptr || aligned16(p), QSA_ERR_INVALID_ARGUMENT,                    \
                "%s must be 16-byte aligned", name);                                         \
  } while (0)

bool dtype_ok(qsa_dtype dt) { return dt == QSA_F32 || dt == QSA_BF16; }

}  // namespace

extern "C" {

const char* qsa_last_error(void) { return g_last_error.c_str(); }

int qsa_version(void) { return 10000; }

qsa_status qsa_compress_keys(const void* ik, const int32_t* kv_lens, float* cmp, int batch,
                             int max_len, int d_idx, int block, qsa_dtype dt,
                             hipStream_t stream) {
  QSA_REQUIRE(dtype_ok(dt), QSA_ERR_INVALID_ARGUMENT, "dt must be QSA_F32 or QSA_BF16");
  QSA_REQUIRE(batch >= 0 && max_len >= 0, QSA_ERR_INVALID_ARGUMENT,
              "batch and max_len must be >= 0 (got %d, %d)", batch, max_len);
  QSA_REQUIRE(d_idx >= 1 && block >= 1, QSA_ERR_INVALID_ARGUMENT,
              "d_idx and block must be >= 1 (got %d, %d)", d_idx, block);
  QSA_REQUIRE(d_idx == 32 || d_idx == 64 || d_idx == 128, QSA_ERR_UNSUPPORTED,
              "d_idx %d not supported (32, 64, 128)", d_idx);
  QSA_REQUIRE(block <= 1024, QSA_ERR_UNSUPPORTED, "block %d not supported (<= 1024)", block);
  if (batch == 0 || max_len / block == 0) return ok();
  QSA_PTR(ik, "ik");
  QSA_PTR(cmp, "cmp");
  return from_hip(qsa::launch_compress(ik, kv_lens, cmp, batch, max_len, d_idx, block,
                                       dt == QSA_BF16, stream),
                  "qsa_compress_keys");
}

qsa_status qsa_index_topk(const void* iq, const float* cmp, const int32_t* kv_lens, int32_t* sel,
                          float* sel_scores, int batch, int n_q, int h_idx, int d_idx,
                          int max_blocks, int block, int top_k, qsa_dtype dt,
                          hipStream_t stream) {
  QSA_REQUIRE(dtype_ok(dt), QSA_ERR_INVALID_ARGUMENT, "dt must be QSA_F32 or QSA_BF16");
  QSA_REQUIRE(batch >= 0 && n_q >= 0 && max_blocks >= 0, QSA_ERR_INVALID_ARGUMENT,
              "batch, n_q and max_blocks must be >= 0");
  QSA_REQUIRE(h_idx >= 1 && d_idx >= 1 && block >= 1, QSA_ERR_INVALID_ARGUMENT,
              "h_idx, d_idx and block must be >= 1");
  QSA_REQUIRE(top_k >= 1, QSA_ERR_INVALID_ARGUMENT, "top_k must be >= 1 (got %d)", top_k);
  QSA_REQUIRE(kv_lens != nullptr || max_blocks >= n_q / block, QSA_ERR_INVALID_ARGUMENT,
              "max_blocks %d < n_q / block = %d", max_blocks, n_q / block);
  QSA_REQUIRE(d_idx == 32 || d_idx == 64 || d_idx == 128, QSA_ERR_UNSUPPORTED,
              "d_idx %d not supported (32, 64, 128)", d_idx);
  QSA_REQUIRE(h_idx <= 64, QSA_ERR_UNSUPPORTED, "h_idx %d not supported (<= 64)", h_idx);
  QSA_REQUIRE(top_k <= qsa::kMaxTopK, QSA_ERR_UNSUPPORTED, "top_k %d not supported (<= %d)",
              top_k, qsa::kMaxTopK);
  QSA_REQUIRE(max_blocks <= qsa::kIndexMaxBlocks, QSA_ERR_UNSUPPORTED,
              "max_blocks %d not supported (<= %d)", max_blocks, qsa::kIndexMaxBlocks);
  QSA_REQUIRE(block <= 1024, QSA_ERR_UNSUPPORTED, "block %d not supported (<= 1024)", block);
  if (batch == 0 || n_q == 0) return ok();
  QSA_PTR(iq, "iq");
  QSA_PTR(sel, "sel");
  QSA_OPT_PTR(sel_scores, "sel_scores");
  if (max_blocks > 0) QSA_PTR(cmp, "cmp");
  return from_hip(qsa::launch_index_topk(iq, cmp, kv_lens, sel, sel_scores, batch, n_q, h_idx,
                                         d_idx, max_blocks, block, top_k, dt == QSA_BF16, stream),
                  "qsa_index_topk");
}

qsa_status qsa_index_topk_decode(const void* iq, const void* ik_cache, float* cmp,
                                 const int32_t* kv_lens, int32_t* sel, float* sel_scores,
                                 int batch, int max_len, int h_idx, int d_idx, int max_blocks,
                                 int block, int top_k, qsa_dtype dt, hipStream_t stream) {
  QSA_REQUIRE(dtype_ok(dt), QSA_ERR_INVALID_ARGUMENT, "dt must be QSA_F32 or QSA_BF16");
  QSA_REQUIRE(batch >= 0 && max_len >= 1 && max_blocks >= 0, QSA_ERR_INVALID_ARGUMENT,
              "batch and max_blocks must be >= 0, max_len >= 1");
  QSA_REQUIRE(h_idx >= 1 && d_idx >= 1 && block >= 1, QSA_ERR_INVALID_ARGUMENT,
              "h_idx, d_idx and block must be >= 1");
  QSA_REQUIRE(top_k >= 1, QSA_ERR_INVALID_ARGUMENT, "top_k must be >= 1 (got %d)", top_k);
  QSA_REQUIRE(d_idx == 32 || d_idx == 64 || d_idx == 128, QSA_ERR_UNSUPPORTED,
              "d_idx %d not supported (32, 64, 128)", d_idx);
  QSA_REQUIRE(h_idx <= 64, QSA_ERR_UNSUPPORTED, "h_idx %d not supported (<= 64)", h_idx);
  QSA_REQUIRE(top_k <= qsa::kMaxTopK, QSA_ERR_UNSUPPORTED, "top_k %d not supported (<= %d)",
              top_k, qsa::kMaxTopK);
  QSA_REQUIRE(max_blocks <= qsa::kIndexMaxBlocks, QSA_ERR_UNSUPPORTED,
              "max_blocks %d not supported (<= %d)", max_blocks, qsa::kIndexMaxBlocks);
  QSA_REQUIRE(block <= 1024, QSA_ERR_UNSUPPORTED, "block %d not supported (<= 1024)", block);
  if (batch == 0) return ok();
  QSA_PTR(iq, "iq");
  QSA_PTR(ik_cache, "ik_cache");
  QSA_PTR(kv_lens, "kv_lens");
  QSA_PTR(sel, "sel");
  QSA_OPT_PTR(sel_scores, "sel_scores");
  if (max_blocks > 0) QSA_PTR(cmp, "cmp");
  return from_hip(qsa::launch_index_topk_decode(iq, ik_cache, cmp, kv_lens, sel, sel_scores,
                                                batch, max_len, h_idx, d_idx, max_blocks, block,
                                                top_k, dt == QSA_BF16, stream),
                  "qsa_index_topk_decode");
}

// The three prefill calls: the whole sequence (n_q == kv_len), a chunk of the last n_q
// tokens over a common kv_len, and a batch of sequences of their own lengths kv_lens[b]
// (K/V slabs of kv_stride rows).
static qsa_status prefill_impl(const char* fn, const void* q, const void* k, const void* v,
                               const int32_t* kv_lens, const int32_t* sel, void* out, float* lse,
                               int batch, int n_q, int kv_len, int kv_stride, int h_q, int h_kv,
                               int d, int block, int top_k, float sm_scale, qsa_dtype dt,
                               hipStream_t stream) {
  QSA_REQUIRE(dtype_ok(dt), QSA_ERR_INVALID_ARGUMENT, "dt must be QSA_F32 or QSA_BF16");
  QSA_REQUIRE(batch >= 0 && n_q >= 0 && kv_len >= 0, QSA_ERR_INVALID_ARGUMENT,
              "batch, n_q and kv_len must be >= 0");
  QSA_REQUIRE(n_q <= kv_len, QSA_ERR_INVALID_ARGUMENT, "n_q %d > kv_len %d", n_q, kv_len);
  QSA_REQUIRE(h_q >= 1 && h_kv >= 1 && d >= 1 && block >= 1, QSA_ERR_INVALID_ARGUMENT,
              "h_q, h_kv, d and block must be >= 1");
  QSA_REQUIRE(top_k >= 1, QSA_ERR_INVALID_ARGUMENT, "top_k must be >= 1 (got %d)", top_k);
  QSA_REQUIRE(h_q % h_kv == 0, QSA_ERR_INVALID_ARGUMENT, "h_q %d is not a multiple of h_kv %d",
              h_q, h_kv);
  QSA_REQUIRE(std::isfinite(sm_scale), QSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  QSA_REQUIRE(d == 64 || d == 128 || d == 256, QSA_ERR_UNSUPPORTED,
              "head dim %d not supported (64, 128, 256)", d);
  QSA_REQUIRE(top_k <= qsa::kMaxTopK, QSA_ERR_UNSUPPORTED, "top_k %d not supported (<= %d)",
              top_k, qsa::kMaxTopK);
  QSA_REQUIRE(block <= 1024, QSA_ERR_UNSUPPORTED, "block %d not supported (<= 1024)", block);
  if (batch == 0 || n_q == 0) return ok();
  QSA_PTR(q, "q");
  QSA_PTR(k, "k");
  QSA_PTR(v, "v");
  QSA_PTR(sel, "sel");
  QSA_PTR(out, "out");
  QSA_OPT_PTR(lse, "lse");
  if (dt == QSA_BF16) {
    QSA_REQUIRE(qsa::prefill_bf16_supported(h_q / h_kv, d, block, top_k, kv_stride, h_kv),
                QSA_ERR_UNSUPPORTED,
                "bf16 prefill not built for group %d, d %d, block %d, top_k %d, kv_len %d, "
                "h_kv %d", h_q / h_kv, d, block, top_k, kv_stride, h_kv);
    return from_hip(qsa::launch_prefill_bf16(q, k, v, sel, out, lse, batch, n_q, kv_len, kv_lens,
                                             kv_stride, h_q, h_kv, d, block, top_k, sm_scale,
                                             stream),
                    fn);
  }
  return from_hip(qsa::launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                       static_cast<const float*>(v), sel, kv_lens,
                                       static_cast<float*>(out), lse, batch, n_q, kv_stride, kv_len,
                                       h_q, h_kv, d, block, top_k, sm_scale, stream),
                  fn);
}

qsa_status qsa_sparse_attn_prefill(const void* q, const void* k, const void* v,
                                   const int32_t* sel, void* out, float* lse, int batch, int seq,
                                   int h_q, int h_kv, int d, int block, int top_k,
                                   float sm_scale, qsa_dtype dt, hipStream_t stream) {
  return prefill_impl("qsa_sparse_attn_prefill", q, k, v, nullptr, sel, out, lse, batch, seq, seq,
                      seq, h_q, h_kv, d, block, top_k, sm_scale, dt, stream);
}

qsa_status qsa_sparse_attn_prefill_chunk(const void* q, const void* k, const void* v,
                                         const int32_t* sel, void* out, float* lse, int batch,
                                         int n_q, int kv_len, int h_q, int h_kv, int d, int block,
                                         int top_k, float sm_scale, qsa_dtype dt,
                                         hipStream_t stream) {
  return prefill_impl("qsa_sparse_attn_prefill_chunk", q, k, v, nullptr, sel, out, lse, batch,
                      n_q, kv_len, kv_len, h_q, h_kv, d, block, top_k, sm_scale, dt, stream);
}

qsa_status qsa_sparse_attn_prefill_varlen(const void* q, const void* k, const void* v,
                                          const int32_t* kv_lens, const int32_t* sel, void* out,
                                          float* lse, int batch, int n_q, int max_len, int h_q,
                                          int h_kv, int d, int block, int top_k, float sm_scale,
                                          qsa_dtype dt, hipStream_t stream) {
  QSA_REQUIRE(batch == 0 || n_q == 0 || kv_lens != nullptr, QSA_ERR_INVALID_ARGUMENT,
              "kv_lens must not be NULL");
  return prefill_impl("qsa_sparse_attn_prefill_varlen", q, k, v, kv_lens, sel, out, lse, batch,
                      n_q, max_len, max_len, h_q, h_kv, d, block, top_k, sm_scale, dt, stream);
}

qsa_status qsa_sparse_attn_decode_workspace_size(int batch, int h_q, int h_kv, int d, int block,
                                                 int top_k, size_t* bytes) {
  QSA_REQUIRE(bytes != nullptr, QSA_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  QSA_REQUIRE(batch >= 0 && h_q >= 1 && h_kv >= 1 && d >= 1 && block >= 1 && top_k >= 1,
              QSA_ERR_INVALID_ARGUMENT, "sizes must be positive (batch >= 0)");
  const int ns = qsa::decode_num_splits(batch, h_kv, block, top_k);
  *bytes = qsa::decode_workspace_bytes(batch, h_q, d, ns);
  return ok();
}

qsa_status qsa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, const int32_t* sel, void* out,
                                  float* lse, int batch, int max_len, int h_q, int h_kv, int d,
                                  int block, int top_k, float sm_scale, void* workspace,
                                  size_t workspace_bytes, qsa_dtype dt, hipStream_t stream) {
  QSA_REQUIRE(dtype_ok(dt), QSA_ERR_INVALID_ARGUMENT, "dt must be QSA_F32 or QSA_BF16");
  QSA_REQUIRE(batch >= 0 && max_len >= 0, QSA_ERR_INVALID_ARGUMENT,
              "batch and max_len must be >= 0");
  QSA_REQUIRE(h_q >= 1 && h_kv >= 1 && d >= 1 && block >= 1, QSA_ERR_INVALID_ARGUMENT,
              "h_q, h_kv, d and block must be >= 1");
  QSA_REQUIRE(top_k >= 1, QSA_ERR_INVALID_ARGUMENT, "top_k must be >= 1 (got %d)", top_k);
  QSA_REQUIRE(h_q % h_kv == 0, QSA_ERR_INVALID_ARGUMENT, "h_q %d is not a multiple of h_kv %d",
              h_q, h_kv);
  QSA_REQUIRE(std::isfinite(sm_scale), QSA_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  QSA_REQUIRE(d == 64 || d == 128 || d == 256, QSA_ERR_UNSUPPORTED,
              "head dim %d not supported (64, 128, 256)", d);
  QSA_REQUIRE(top_k <= qsa::kMaxTopK, QSA_ERR_UNSUPPORTED, "top_k %d not supported (<= %d)",
              top_k, qsa::kMaxTopK);
  QSA_REQUIRE(block <= 1024, QSA_ERR_UNSUPPORTED, "block %d not supported (<= 1024)", block);
  if (batch == 0) return ok();
  QSA_REQUIRE(max_len >= 1, QSA_ERR_INVALID_ARGUMENT, "max_len must be >= 1");
  QSA_PTR(q, "q");
  QSA_PTR(k_cache, "k_cache");
  QSA_PTR(v_cache, "v_cache");
  QSA_PTR(kv_lens, "kv_lens");
  QSA_PTR(sel, "sel");
  QSA_PTR(out, "out");
  QSA_OPT_PTR(lse, "lse");
  if (dt == QSA_BF16) {
    QSA_REQUIRE(qsa::decode_bf16_supported(h_q / h_kv, d, block, top_k, max_len, h_kv),
                QSA_ERR_UNSUPPORTED,
                "bf16 decode not built for group %d, d %d, max_len %d, h_kv %d", h_q / h_kv, d,
                max_len, h_kv);
    const int ns = qsa::decode_num_splits(batch, h_kv, block, top_k);
    const size_t need = qsa::decode_workspace_bytes(batch, h_q, d, ns);
    QSA_REQUIRE(workspace_bytes >= need, QSA_ERR_INVALID_ARGUMENT,
                "workspace_bytes %zu < required %zu", workspace_bytes, need);
    if (need > 0) QSA_PTR(workspace, "workspace");
    return from_hip(qsa::launch_decode_bf16(q, k_cache, v_cache, kv_lens, sel, out, lse, batch,
                                            max_len, h_q, h_kv, d, block, top_k, sm_scale,
                                            workspace, ns, stream),
                    "qsa_sparse_attn_decode");
  }
  return from_hip(qsa::launch_attn_f32(static_cast<const float*>(q),
                                       static_cast<const float*>(k_cache),
                                       static_cast<const float*>(v_cache), sel, kv_lens,
                                       static_cast<float*>(out), lse, batch, 1, max_len, 0, h_q,
                                       h_kv, d, block, top_k, sm_scale, stream),
                  "qsa_sparse_attn_decode");
}

qsa_status qsa_sparse_attn_decode_noalloc(const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* kv_lens,
                                          const int32_t* sel, void* out, float* lse, int batch,
                                          int max_len, int h_q, int h_kv, int d, int block,
                                          int top_k, float sm_scale, qsa_dtype dt,
                                          hipStream_t stream) {
  size_t need = 0;
  if (dt == QSA_BF16 && batch > 0 && h_q >= 1 && h_kv >= 1 && d >= 1 && block >= 1 &&
      top_k >= 1) {
    const int ns = qsa::decode_num_splits(batch, h_kv, block, top_k);
    need = qsa::decode_workspace_bytes(batch, h_q, d, ns);
    QSA_REQUIRE(need <= qsa::kDecodeScratchBytes, QSA_ERR_UNSUPPORTED,
                "qsa_sparse_attn_decode_noalloc: these sizes need %zu bytes of scratch, more "
                "than the %zu the library holds per device; use qsa_sparse_attn_decode with a "
                "workspace", need, qsa::kDecodeScratchBytes);
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = qsa::decode_scratch(&ws);
    if (e != hipSuccess) return from_hip(e, "qsa_sparse_attn_decode_noalloc (scratch address)");
  }
  return qsa_sparse_attn_decode(q, k_cache, v_cache, kv_lens, sel, out, lse, batch, max_len,
                                h_q, h_kv, d, block, top_k, sm_scale, ws, need, dt, stream);
}

}  // extern "C"
