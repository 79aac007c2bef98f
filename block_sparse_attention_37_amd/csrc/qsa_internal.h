// Host-side launchers behind the C ABI (one per kernel family).  Arguments have been
// validated by the caller; each returns the HIP error of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

hipError_t launch_compress(const void* ik, const int32_t* kv_lens, float* cmp, int batch,
                           int max_len, int d_idx, int block, bool bf16, hipStream_t stream);

// Largest number of candidate blocks the index kernel can rank per query.
constexpr int kIndexMaxBlocks = 4096;
constexpr int kMaxTopK = 256;

hipError_t launch_index_topk(const void* iq, const float* cmp, const int32_t* kv_lens,
                             int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                             int d_idx, int max_blocks, int block, int top_k, bool bf16,
                             hipStream_t stream);

// Decode step of the indexer with the state update: compresses the block each sequence's
// newest token completes (from the indexer-key cache), writes it to cmp, then scores and
// selects for the one query per sequence.
hipError_t launch_index_topk_decode(const void* iq, const void* ik, float* cmp,
                                    const int32_t* kv_lens, int32_t* sel, float* sel_scores,
                                    int batch, int max_len, int h_idx, int d_idx, int max_blocks,
                                    int block, int top_k, bool bf16, hipStream_t stream);

// bf16 prefill on matrix cores.  Returns hipErrorInvalidValue for shapes it is not built for.
// A workgroup keeps a bitmap of the blocks it visits in LDS, and per visited block one bit
// per query position.
constexpr int kPrefillMaxBlocks = 4096;
bool prefill_bf16_supported(int group, int d, int block, int top_k, int kv_len, int h_kv);
// n_q query rows at positions kv_len - n_q .. kv_len - 1 over kv_len keys, where kv_len is
// kv_lens[b] clamped to [0, kv_stride] when kv_lens is given (else the common kv_len); K/V
// hold kv_stride rows per sequence; rows with a negative position are padding (zeros).
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, const int32_t* sel,
                               void* out, float* lse, int batch, int n_q, int kv_len,
                               const int32_t* kv_lens, int kv_stride, int h_q, int h_kv, int d,
                               int block, int top_k, float sm_scale, hipStream_t stream);
// The head-dim-256 instance (16-row tiles, 32-key chunks); launch_prefill_bf16 and
// prefill_bf16_supported route d = 256 here.
bool prefill_bf16_rt_supported(int group, int d, int block, int top_k, int kv_len, int h_kv);
hipError_t launch_prefill_bf16_rt(const void* q, const void* k, const void* v, const int32_t* sel,
                                  void* out, float* lse, int batch, int n_q, int kv_len,
                                  const int32_t* kv_lens, int kv_stride, int h_q, int h_kv, int d,
                                  int block, int top_k, float sm_scale, hipStream_t stream);

// float32 attention (prefill and decode) on the vector ALUs.
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, const int32_t* sel,
                           const int32_t* kv_lens, float* out, float* lse, int batch, int n_q,
                           int kv_stride_len, int seq_fixed, int h_q, int h_kv, int d, int block,
                           int top_k, float sm_scale, hipStream_t stream);

// bf16 decode on matrix cores, split over chunks of the selected tokens.
bool decode_bf16_supported(int group, int d, int block, int top_k, int max_len, int h_kv);
int decode_num_splits(int batch, int h_kv, int block, int top_k);
size_t decode_workspace_bytes(int batch, int h_q, int d, int nsplit);
// Device scratch of the decode call that takes no workspace: kDecodeScratchBytes per
// device, its address looked up once per device (hipGetSymbolAddress) with that device
// current.  Returns the lookup's error, if any.
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* kv_lens, const int32_t* sel, void* out, float* lse,
                              int batch, int max_len, int h_q, int h_kv, int d, int block,
                              int top_k, float sm_scale, void* workspace, int nsplit,
                              hipStream_t stream);

}  // namespace qsa
