/*
 * qsa.h -- C ABI of the QSA (Qwen Sparse Attention) library for AMD MI355X (gfx950).
 *
 * The method is the one described on the Hugging Face Transformers model page
 * "Qwen4-Exp": in the overview, several indexer query heads score compressed key
 * blocks, every query keeps its most relevant contiguous token blocks plus its own
 * incomplete trailing block (kept uncompressed), and attention runs over those tokens
 * only; the Qwen4ExpTextConfig parameters indexer_n_heads, indexer_kv_heads (one key
 * head), indexer_head_dim, indexer_budget and indexer_compress_ratio size it.
 *
 * Readings taken where the page is silent (the same ones the test oracle states):
 *   - compression is the arithmetic mean of each complete block of `block` keys;
 *   - a block's score is the sum over indexer heads of <indexer query, compressed key>;
 *   - block j is a candidate for query position p iff (j+1)*block <= p+1, so
 *     n(p) = floor((p+1)/block) candidates;
 *   - a query keeps m = min(top_k, n(p)) blocks ranked by score (descending), ties
 *     going to the lower block index (top_k = indexer_budget / indexer_compress_ratio);
 *   - the trailing tokens of p are block*n(p) .. p (none when p closes a block);
 *   - T(p) = tokens of the kept blocks + trailing tokens; softmax attention of every
 *     query head over T(p) with scale sm_scale; grouped-query attention maps query
 *     head h to key/value head h / (h_q / h_kv); one selection per token serves all
 *     query heads;
 *   - query i of a call with n_q queries over kv_len keys sits at p = kv_len - n_q + i.
 *
 * Conventions for every entry point
 *   - Tensors are row-major and contiguous; shapes are given innermost-last.
 *   - Every pointer is a caller-owned DEVICE pointer (hipMalloc'd or equivalent) unless
 *     stated otherwise; it must stay valid until `stream` has executed the call.  The
 *     library never allocates, frees or synchronizes; all work is enqueued on `stream`
 *     (0 = the null stream).  Calls on one stream execute in order.
 *   - `dt` gives the element type of all floating-point inputs and outputs of a call
 *     other than the ones documented as float (QSA_F32 = float32, QSA_BF16 = bfloat16).
 *   - Errors: arguments that can be checked on the host are checked before anything is
 *     enqueued and give QSA_ERR_INVALID_ARGUMENT; valid arguments outside what the
 *     kernels are built for give QSA_ERR_UNSUPPORTED; a failed kernel launch gives
 *     QSA_ERR_HIP.  qsa_last_error() then describes the problem.  Values that live on
 *     the device (kv_lens, sel) are not checked by the host: out-of-range values give
 *     unspecified results, but kernels never read or write outside the documented
 *     extents of their arguments.  No exception crosses this ABI.
 *   - Results are deterministic: the same inputs give bitwise-identical outputs.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID_ARGUMENT = 1,
  QSA_ERR_UNSUPPORTED = 2,
  QSA_ERR_HIP = 3
} qsa_status;

typedef enum { QSA_F32 = 0, QSA_BF16 = 1 } qsa_dtype;

/* Text describing the last failed call made by this thread ("" if none).  The string is
 * owned by the library and stays valid until the next qsa_* call on the same thread. */
const char* qsa_last_error(void);

/* Version of the library as major*10000 + minor*100 + patch. */
int qsa_version(void);

/*
 * Step 1 -- key-block compression (Qwen4-Exp page, Qwen4ExpTextConfig,
 * indexer_compress_ratio: consecutive token keys averaged into one index block; overview:
 * the incomplete trailing block stays uncompressed).
 *
 *   cmp[b, j, c] = (1/block) * sum_{s = j*block}^{j*block+block-1} ik[b, s, c]
 *
 * for every complete block j < floor(len_b / block), len_b = kv_lens[b] (or max_len if
 * kv_lens is NULL).  Entries of cmp for j >= floor(len_b / block) are left untouched.
 *
 *   ik       [batch, max_len, d_idx]  element type dt; the single indexer key head
 *   kv_lens  [batch] int32 or NULL; each value must lie in [0, max_len]
 *   cmp      [batch, max_len / block, d_idx] float32 (output, floor division)
 * Supported: d_idx in {32, 64, 128}, block in [1, 1024].  Accumulation is float32 in a
 * fixed order (the same for every call and for qsa_index_topk_decode).
 */
qsa_status qsa_compress_keys(const void* ik, const int32_t* kv_lens, float* cmp,
                             int batch, int max_len, int d_idx, int block,
                             qsa_dtype dt, hipStream_t stream);

/*
 * Steps 2 + 3 -- indexer scores and top-k block selection (Qwen4-Exp overview: multiple
 * query heads score compressed key blocks and the most relevant blocks are selected;
 * indexer_n_heads, indexer_head_dim, indexer_budget).
 *
 * Query i of sequence b sits at p = len_b - n_q + i, len_b = kv_lens[b] (or n_q if
 * kv_lens is NULL; prefill passes n_q == len_b, decode passes n_q == 1).  Its score for
 * a candidate block j < n(p) = floor((p+1)/block) is
 *
 *   S[j] = sum_h sum_c iq[b, i, h, c] * cmp[b, j, c]
 *
 * (computed in float32 as (sum_h iq[., h, .]) . cmp[j]).  The m = min(top_k, n(p))
 * blocks with the largest S are kept, ties going to the lower block index (-0 == +0).
 *
 *   iq          [batch, n_q, h_idx, d_idx]   element type dt
 *   cmp         [batch, max_blocks, d_idx]   float32 (from qsa_compress_keys)
 *   kv_lens     [batch] int32 or NULL; values <= max_blocks*block + block - 1; a value
 *               below n_q makes the rows with p < 0 padding (every slot -1)
 *   sel         [batch, n_q, top_k] int32 output: the kept block ids in ascending order,
 *               then -1 in the remaining top_k - m slots
 *   sel_scores  [batch, n_q, top_k] float32 output or NULL: S of each kept block in the
 *               same order, -INFINITY in padded slots
 * Invalid: max_blocks < floor(n_q / block) when kv_lens is NULL.
 * Supported: d_idx in {32, 64, 128}, h_idx <= 64, top_k <= 256, max_blocks <= 4096,
 * block in [1, 1024].  Non-finite inputs are not supported.
 */
qsa_status qsa_index_topk(const void* iq, const float* cmp, const int32_t* kv_lens,
                          int32_t* sel, float* sel_scores,
                          int batch, int n_q, int h_idx, int d_idx, int max_blocks,
                          int block, int top_k, qsa_dtype dt, hipStream_t stream);

/*
 * Steps 1-3 for one decode step, with the indexer state kept on the device (Qwen4-Exp
 * usage tips: cached generation keeps the QSA indexer states on the device; config:
 * indexer_compress_ratio consecutive keys are averaged into one index block).
 *
 * Sequence b has len_b = kv_lens[b] tokens; its newest token sits at p = len_b - 1 and its
 * indexer key is already stored in ik_cache[b, p].  If len_b is a positive multiple of
 * block, that token completes block j = len_b / block - 1: the call first writes
 *
 *   cmp[b, j, c] = (1/block) * sum_{s = j*block}^{j*block+block-1} ik_cache[b, s, c]
 *
 * bit-identical to what qsa_compress_keys computes for that block, then scores and selects
 * exactly like qsa_index_topk with n_q = 1.  Rows of cmp for other blocks are only read:
 * they must hold the compressed blocks of the prefix (from qsa_compress_keys or earlier
 * calls of this function).
 *
 *   iq          [batch, h_idx, d_idx]        element type dt
 *   ik_cache    [batch, max_len, d_idx]      element type dt
 *   cmp         [batch, max_blocks, d_idx]   float32, read and updated in place
 *   kv_lens     [batch] int32 (required); values in [1, min(max_len, max_blocks*block + block - 1)]
 *   sel, sel_scores  as for qsa_index_topk with n_q = 1
 * Invalid: kv_lens or ik_cache NULL.
 * Supported: as qsa_index_topk.
 */
qsa_status qsa_index_topk_decode(const void* iq, const void* ik_cache, float* cmp,
                                 const int32_t* kv_lens, int32_t* sel, float* sel_scores,
                                 int batch, int max_len, int h_idx, int d_idx, int max_blocks,
                                 int block, int top_k, qsa_dtype dt, hipStream_t stream);

/*
 * Steps 4 + 5, prefill -- attention of every prompt token over its selected tokens
 * (Qwen4-Exp overview: the selected contiguous blocks plus the uncompressed trailing
 * block; usage tips: sparse token selection feeding softmax attention; config fields
 * num_attention_heads / num_key_value_heads give grouped-query attention).
 *
 * For p in [0, seq) and query head h (key/value head g = h / (h_q / h_kv)):
 *   T(p) = U_{j in sel[b,p]} [j*block, (j+1)*block)  U  [block*floor((p+1)/block), p]
 *   out[b, p, h, :] = sum_{s in T(p)} softmax_s(sm_scale * q[b,p,h,:].k[b,s,g,:]) v[b,s,g,:]
 *   lse[b, p, h]    = log sum_{s in T(p)} exp(sm_scale * q[b,p,h,:].k[b,s,g,:])
 *
 *   q, out   [batch, seq, h_q, d]   element type dt (out may not alias any input)
 *   k, v     [batch, seq, h_kv, d]  element type dt
 *   sel      [batch, seq, top_k] int32: per row, the distinct block ids of T(p)
 *            (qsa_index_topk writes them ascending, then -1 padding); the kernels take
 *            them in any order and ignore ids outside [0, n(p))
 *   lse      [batch, seq, h_q] float32 output or NULL
 * Invalid: h_q % h_kv != 0, a non-finite sm_scale.  Any finite sm_scale is accepted (a
 * negative one ranks keys in reverse, zero gives every token of T(p) the same weight).
 * bf16 computes Q.K^T and P.V on bf16 matrix cores with float32 accumulation and float32
 * softmax (P rounded to bf16), out rounded to nearest even; f32 computes everything in
 * float32.
 * Supported: d in {64, 128, 256} (256: the model page's default attention shape);
 * top_k <= 256; block in [1, 1024].  bf16 also needs G = h_q / h_kv in {1, 2, 4, 8, 16, 32},
 * (seq + block - 1) / block <= 4096 and seq * h_kv * d < 2^32.
 */
qsa_status qsa_sparse_attn_prefill(const void* q, const void* k, const void* v,
                                   const int32_t* sel, void* out, float* lse,
                                   int batch, int seq, int h_q, int h_kv, int d,
                                   int block, int top_k, float sm_scale,
                                   qsa_dtype dt, hipStream_t stream);

/*
 * Steps 4 + 5, chunked prefill onto an existing cache -- the last n_q tokens of a sequence
 * of kv_len tokens attend over their selected tokens (Qwen4-Exp, as above; the queries are
 * the tail of the sequence, so query i sits at position p = kv_len - n_q + i, the same rule
 * qsa_index_topk applies with kv_lens[b] = kv_len).  With n_q == kv_len this is
 * qsa_sparse_attn_prefill.
 *
 *   q, out   [batch, n_q, h_q, d]     element type dt (out may not alias any input)
 *   k, v     [batch, kv_len, h_kv, d] element type dt (the whole sequence, cache included)
 *   sel      [batch, n_q, top_k] int32, as for qsa_sparse_attn_prefill
 *   lse      [batch, n_q, h_q] float32 output or NULL
 * Invalid: n_q > kv_len; as qsa_sparse_attn_prefill otherwise.
 * Supported: as qsa_sparse_attn_prefill with seq = kv_len.
 */
qsa_status qsa_sparse_attn_prefill_chunk(const void* q, const void* k, const void* v,
                                         const int32_t* sel, void* out, float* lse,
                                         int batch, int n_q, int kv_len, int h_q, int h_kv,
                                         int d, int block, int top_k, float sm_scale,
                                         qsa_dtype dt, hipStream_t stream);

/*
 * Steps 4 + 5 for a batch of sequences of different lengths (Qwen4-Exp, as above; batched
 * generation pads the shorter prompts on the left, and every query still attends only to
 * its own sequence's tokens).  Sequence b has len_b = kv_lens[b] tokens (clamped to
 * [0, max_len]); its queries are the last n_q rows of q[b], right-aligned: query row i sits
 * at p = len_b - n_q + i, the rule qsa_index_topk applies with the same kv_lens and n_q.
 * Rows with p < 0 are padding: out is 0 there and lse is -inf.  With n_q = max_b len_b and
 * kv_lens the prompt lengths this is a batched prefill of prompts of mixed length; with
 * n_q <= min_b len_b it is a chunk appended to caches of mixed length.
 *
 *   q, out   [batch, n_q, h_q, d]         element type dt (out may not alias any input)
 *   k, v     [batch, max_len, h_kv, d]    element type dt; rows >= len_b are not read
 *   kv_lens  [batch] int32 (device)
 *   sel      [batch, n_q, top_k] int32, as for qsa_sparse_attn_prefill (padding rows: -1)
 *   lse      [batch, n_q, h_q] float32 output or NULL
 * Invalid: kv_lens NULL (when batch and n_q are non-zero); n_q > max_len.
 * Supported: as qsa_sparse_attn_prefill with seq = max_len.
 */
qsa_status qsa_sparse_attn_prefill_varlen(const void* q, const void* k, const void* v,
                                          const int32_t* kv_lens, const int32_t* sel, void* out,
                                          float* lse, int batch, int n_q, int max_len, int h_q,
                                          int h_kv, int d, int block, int top_k, float sm_scale,
                                          qsa_dtype dt, hipStream_t stream);

/*
 * Bytes of device workspace qsa_sparse_attn_decode needs for these sizes (may be 0).
 * Writes the size to *bytes (a HOST pointer).
 */
qsa_status qsa_sparse_attn_decode_workspace_size(int batch, int h_q, int h_kv, int d,
                                                 int block, int top_k, size_t* bytes);

/*
 * Steps 4 + 5, decode -- one new query token per sequence attending over its selected
 * tokens of a contiguous per-sequence KV cache (Qwen4-Exp usage tips: cached generation
 * with the QSA indexer state kept on device).
 *
 * The query of sequence b sits at p = kv_lens[b] - 1; its own key/value are already in
 * the cache at that position.  T(p) and out/lse are as for prefill with n(p) =
 * floor(kv_lens[b] / block).
 *
 *   q, out            [batch, h_q, d]               element type dt
 *   k_cache, v_cache  [batch, max_len, h_kv, d]     element type dt
 *   kv_lens           [batch] int32, values in [1, max_len]
 *   sel               [batch, top_k] int32 (as for prefill; from qsa_index_topk with n_q=1)
 *   lse               [batch, h_q] float32 output or NULL
 *   workspace         device buffer of at least workspace_bytes bytes, as given by
 *                     qsa_sparse_attn_decode_workspace_size for the same sizes (NULL
 *                     allowed when that size is 0); contents need no initialization and
 *                     are scratch: two calls in flight at once must not share it
 * Invalid: h_q % h_kv != 0, workspace_bytes too small.
 * Supported: d in {64, 128, 256}; bf16 needs h_q / h_kv in {1, 2, 4, 8, 16} and
 * max_len * h_kv * d < 2^32; top_k <= 256; block in [1, 1024].
 */
qsa_status qsa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, const int32_t* sel,
                                  void* out, float* lse,
                                  int batch, int max_len, int h_q, int h_kv, int d,
                                  int block, int top_k, float sm_scale,
                                  void* workspace, size_t workspace_bytes,
                                  qsa_dtype dt, hipStream_t stream);

/*
 * qsa_sparse_attn_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as qsa_sparse_attn_decode, whose
 * workspace this call takes from a device array the library holds: 8 MiB per device, from
 * the library's load until the process ends (its address is looked up once per device, on
 * the first call with that device current).  Sizes whose workspace
 * (qsa_sparse_attn_decode_workspace_size) exceeds 8 MiB give QSA_ERR_UNSUPPORTED; nothing
 * here allocates.  All calls on one device share that array: two of them in flight at once
 * on the same device (on different streams, or from different threads without ordering)
 * race and give unspecified results.
 */
qsa_status qsa_sparse_attn_decode_noalloc(const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* kv_lens,
                                          const int32_t* sel, void* out, float* lse,
                                          int batch, int max_len, int h_q, int h_kv, int d,
                                          int block, int top_k, float sm_scale,
                                          qsa_dtype dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
