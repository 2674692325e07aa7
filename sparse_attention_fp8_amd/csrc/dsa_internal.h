// Host-side declarations shared by the launch code of the DSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// production dimensions (fp8 indexer, bf16 attention)
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kHeads = 128;
constexpr int kQkDim = 576;
constexpr int kVDim = 512;
constexpr int kTopk = 2048;
constexpr int kMhaHeadDim = 128;  // MHA mode: per-head nope-key and value width
constexpr int kTopkMaxPositions = 131072;  // longest row (t + 1) the top-k kernels take
// contiguous bf16 latent caches are addressed with 32-bit byte offsets per sequence
constexpr uint64_t kMaxLatentSeqBytes = 0xFFFFFFFFull;

// Location of cache entries.  table == nullptr: contiguous caches [B, N, ...], entry
// (b, s) at row b * N + s.  Otherwise a page pool [npages, 1 << shift, ...] seen
// through the block table [B, pps]: entry (b, s) at row
// table[b * pps + (s >> shift)] * (1 << shift) + (s & ((1 << shift) - 1)); table
// entries outside [0, npages) are read as page 0 (results unspecified, no fault).
struct PageMap {
  const int32_t* table = nullptr;
  int pps = 0;
  int shift = 0;
  int npages = 0;
};

// pool row of entry s of sequence b (s < pps << shift)
__host__ __device__ __forceinline__ uint32_t paged_row(const PageMap& pm, int b, int s) {
  int pg = pm.table[(size_t)b * pm.pps + (s >> pm.shift)];
  pg = (pg >= 0 && pg < pm.npages) ? pg : 0;
  return ((uint32_t)pg << pm.shift) | (uint32_t)(s & ((1 << pm.shift) - 1));
}

// Words the fp8 indexer launch sets to zero (from its first block) for the top-k
// launch that follows it: the per-row counts of the many-blocks-per-row top-k.
struct ClearWords {
  uint32_t* ptr = nullptr;
  int n = 0;
};

hipError_t launch_indexer_fp8(const dsa_rows& rows, const uint8_t* q_idx, const float* q_scale,
                              const float* w, const uint8_t* k_idx, const float* k_scale,
                              float* scores, int64_t ld, hipStream_t stream,
                              const PageMap& pm = PageMap(), ClearWords clear = ClearWords(),
                              uint32_t* rowmm = nullptr);
// Whether launch_indexer_fp8 runs the tiled (prefill) kernel for these rows.  Only that
// kernel accepts rowmm: two words per row (2 r: max, 2 r + 1: ~min, as order-preserving
// float keys) that must start at zero and that it raises with atomic maxima to the
// extremes of the row's non-NaN scores at positions <= its own.
bool indexer_uses_tiles(const dsa_rows& rows);

hipError_t launch_indexer_f32(const dsa_rows& rows, const dsa_dims& dims, const float* q_idx,
                              const float* w, const float* k_idx, float* scores, int64_t ld,
                              hipStream_t stream);

// Workspace of the top-k launch for these rows (0 when one block per row runs).
size_t topk_workspace_bytes(const dsa_rows& rows);
// The words of that workspace that must be zero when the top-k launch starts
// (none when one block per row runs).
ClearWords topk_counts(const dsa_rows& rows, void* workspace);
// counts_cleared: an earlier launch on the stream has zeroed topk_counts(rows, ws);
// otherwise the launch zeroes them itself first.
// rowmm (only when topk_streams_rows): the extremes the tiled indexer left for these
// rows (see indexer_uses_tiles); the launch reads them and sets them back to zero.
hipError_t launch_topk(const dsa_rows& rows, int topk, const float* scores, int64_t ld,
                       int32_t* indices, void* workspace, hipStream_t stream,
                       bool counts_cleared = false, uint32_t* rowmm = nullptr);
// Whether launch_topk runs one block per row with rows longer than its registers hold
// (streamed from memory once per pass).
bool topk_streams_rows(const dsa_rows& rows);
// Sets n words to zero (a fill kernel, so a captured stream records no memset node).
hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t stream);

// Number of splits of each row's selected set used by the bf16 attention for R rows.
int attn_num_splits(int num_rows, int topk);
size_t attn_workspace_bytes(int num_rows, const dsa_dims& dims);

hipError_t launch_attn_bf16(const dsa_rows& rows, const void* q, const void* latent,
                            const int32_t* indices, float softmax_scale, void* out, float* lse,
                            void* workspace, hipStream_t stream, const PageMap& pm = PageMap());

// Reads the calling device's index-domain flag (1 once an attention kernel met an
// index entry past its row's position), then clears it.  Synchronises the device.
hipError_t read_index_domain_flag(uint32_t* seen);

hipError_t launch_attn_f32(const dsa_rows& rows, const dsa_dims& dims, const float* q,
                           const float* latent, const int32_t* indices, float softmax_scale,
                           float* out, float* lse, hipStream_t stream);

size_t project_workspace_bytes(int num_rows, int d_model);

hipError_t launch_project(const dsa_rows& rows, int d_model, const uint16_t* h, const uint16_t* wq,
                          const uint16_t* wk, const uint16_t* wc, const uint16_t* ww, uint8_t* q_idx,
                          float* q_scale, float* w, uint8_t* k_idx, float* k_scale,
                          uint16_t* latent, void* workspace, hipStream_t stream,
                          const PageMap& pm = PageMap());

size_t indexer_loss_workspace_bytes(int num_rows, int topk);
size_t indexer_loss_dense_workspace_bytes(int num_rows, int max_pos);
// Backward workspace: shared_keys accumulators for keys selected more than once
// (-1: the most the call's shape allows).
size_t indexer_backward_workspace_bytes(const dsa_rows& rows, int topk, bool dense,
                                        int64_t shared_keys);
hipError_t launch_indexer_backward_dense(const dsa_rows& rows, const uint8_t* q_idx,
                                         const float* q_scale, const float* w, const uint8_t* k_idx,
                                         const float* k_scale, const float* dscores, int64_t ld,
                                         float* dq, float* dw, float* dk, void* workspace,
                                         size_t ws_bytes, hipStream_t stream);
hipError_t launch_indexer_loss_dense(const dsa_rows& rows, const void* q, const void* latent,
                                     float softmax_scale, const float* scores, int64_t ld,
                                     float* loss, float* dscores, void* workspace,
                                     hipStream_t stream);

hipError_t launch_indexer_loss(const dsa_rows& rows, const void* q, const void* latent,
                               const int32_t* indices, const float* lse, float softmax_scale,
                               const float* scores, int64_t ld, float* loss, float* dscores,
                               void* workspace, hipStream_t stream, const PageMap& pm = PageMap());

hipError_t launch_indexer_backward(const dsa_rows& rows, const uint8_t* q_idx,
                                   const float* q_scale, const float* w, const uint8_t* k_idx,
                                   const float* k_scale, const int32_t* indices,
                                   const float* dscores, float* dq, float* dw, float* dk,
                                   void* workspace, size_t ws_bytes, hipStream_t stream);

size_t mha_workspace_bytes(int num_rows, int num_seqs, int max_pos);

hipError_t launch_mha(const dsa_rows& rows, const void* q, const void* latent, const void* w_uk,
                      const void* w_uv, const int32_t* indices, float softmax_scale, void* out,
                      float* lse, void* workspace, hipStream_t stream);

// Sets the calling thread's dsa_last_error() text and returns st.
dsa_status set_error(dsa_status st, const char* fmt, ...);

}  // namespace dsa
