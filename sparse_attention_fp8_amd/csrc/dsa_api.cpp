// C ABI of the DSA library: argument validation, workspace layout, launches.
// The steps and their sources are documented in include/dsa.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

dsa_status hip_fail(hipError_t err, const char* what) {
  return fail(DSA_E_HIP, "%s: %s", what, hipGetErrorString(err));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

dsa_status check_rows(const dsa_rows* rows) {
  if (rows == nullptr) return fail(DSA_E_INVALID, "rows is NULL");
  if (rows->num_rows < 0) return fail(DSA_E_INVALID, "num_rows < 0");
  if (rows->num_seqs < 1) return fail(DSA_E_INVALID, "num_seqs < 1");
  if (rows->max_ctx < 1) return fail(DSA_E_INVALID, "max_ctx < 1");
  if (rows->max_pos < 0 || rows->max_pos >= rows->max_ctx)
    return fail(DSA_E_INVALID, "max_pos must lie in [0, max_ctx)");
  if (rows->num_rows > 0 && (rows->row_seq == nullptr || rows->row_pos == nullptr))
    return fail(DSA_E_INVALID, "row_seq / row_pos is NULL");
  return DSA_OK;
}

// The top-k kernels take rows of at most kTopkMaxPositions candidates.
dsa_status check_topk_rows(const dsa_rows& rows) {
  if ((int64_t)rows.max_pos + 1 > dsa::kTopkMaxPositions)
    return fail(DSA_E_UNSUPPORTED, "top-k supports max_pos + 1 <= %d", dsa::kTopkMaxPositions);
  return DSA_OK;
}

// Contiguous bf16 latent caches are addressed with 32-bit byte offsets within a
// sequence: max_ctx * row bytes must fit.
dsa_status check_latent_span(const dsa_rows& rows, const dsa_dims& dims) {
  if (dims.attn_dtype == DSA_BF16 &&
      (uint64_t)rows.max_ctx * (uint64_t)dims.qk_dim * 2u > dsa::kMaxLatentSeqBytes)
    return fail(DSA_E_UNSUPPORTED, "a contiguous latent cache must stay below 4 GiB per sequence "
                "(max_ctx * %d bytes)", dims.qk_dim * 2);
  return DSA_OK;
}

bool is_production(const dsa_dims& d) {
  return d.n_idx_heads == dsa::kIdxHeads && d.idx_dim == dsa::kIdxDim &&
         d.n_heads == dsa::kHeads && d.qk_dim == dsa::kQkDim && d.v_dim == dsa::kVDim &&
         d.topk == dsa::kTopk && d.idx_dtype == DSA_FP8_E4M3FN && d.attn_dtype == DSA_BF16;
}

bool is_fp32(const dsa_dims& d) {
  return d.idx_dtype == DSA_F32 && d.attn_dtype == DSA_F32 && d.n_idx_heads >= 1 &&
         d.n_idx_heads <= 64 && d.idx_dim >= 1 && d.idx_dim <= 128 && d.n_heads >= 1 &&
         d.n_heads <= 128 && d.qk_dim >= 1 && d.qk_dim <= dsa::kQkDim && d.v_dim >= 1 &&
         d.v_dim <= d.qk_dim && d.topk >= 1 && d.topk <= dsa::kTopk;
}

dsa_status check_dims(const dsa_dims* dims) {
  if (dims == nullptr) return fail(DSA_E_INVALID, "dims is NULL");
  if (is_production(*dims) || is_fp32(*dims)) return DSA_OK;
  return fail(DSA_E_UNSUPPORTED,
              "unsupported dims (H_I=%d d_I=%d H=%d D_k=%d D_v=%d topk=%d idx_dtype=%d "
              "attn_dtype=%d)",
              dims->n_idx_heads, dims->idx_dim, dims->n_heads, dims->qk_dim, dims->v_dim,
              dims->topk, (int)dims->idx_dtype, (int)dims->attn_dtype);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Paged caches: descriptor checks and the kernels' page map.  row_bytes is the
// largest cache row a call addresses (32-bit offsets from a pool's base).
dsa_status check_pages(const dsa_rows& rows, const dsa_dims& dims, const dsa_pages* pages,
                       size_t row_bytes, dsa::PageMap* pm) {
  if (pages == nullptr) return fail(DSA_E_INVALID, "pages is NULL");
  if (!is_production(dims))
    return fail(DSA_E_UNSUPPORTED, "paged caches need the production dims (fp8 indexer, bf16 latent)");
  const int P = pages->page_size;
  if (P < 64 || P > 65536 || (P & (P - 1)) != 0)
    return fail(DSA_E_UNSUPPORTED, "page_size must be a power of two in [64, 65536]");
  if (pages->pages_per_seq < 1 || pages->num_pages < 1 || pages->block_table == nullptr)
    return fail(DSA_E_INVALID, "pages_per_seq and num_pages must be >= 1 and block_table set");
  if ((int64_t)pages->pages_per_seq * P != rows.max_ctx)
    return fail(DSA_E_INVALID, "max_ctx must equal pages_per_seq * page_size");
  if ((uint64_t)pages->num_pages * (uint64_t)P * row_bytes > 0xFFFFFFFFull)
    return fail(DSA_E_UNSUPPORTED, "a page pool must stay below 4 GiB");
  pm->table = pages->block_table;
  pm->pps = pages->pages_per_seq;
  pm->shift = __builtin_ctz((unsigned)P);
  pm->npages = pages->num_pages;
  return DSA_OK;
}

constexpr size_t kKeyRow = dsa::kIdxDim;                  // fp8 indexer key
constexpr size_t kLatentRow = dsa::kQkDim * sizeof(uint16_t);  // bf16 latent entry

// --- step launchers shared by the public calls and dsa_forward -----------------

dsa_status run_indexer(const dsa_rows& rows, const dsa_dims& dims, const void* q_idx,
                       const float* q_scale, const float* w, const void* k_idx,
                       const float* k_scale, float* scores, int64_t ld, hipStream_t stream,
                       const dsa::PageMap& pm, dsa::ClearWords clear = dsa::ClearWords(),
                       uint32_t* rowmm = nullptr) {
  hipError_t err;
  if (dims.idx_dtype == DSA_FP8_E4M3FN)
    err = dsa::launch_indexer_fp8(rows, static_cast<const uint8_t*>(q_idx), q_scale, w,
                                  static_cast<const uint8_t*>(k_idx), k_scale, scores, ld, stream,
                                  pm, clear, rowmm);
  else
    err = dsa::launch_indexer_f32(rows, dims, static_cast<const float*>(q_idx), w,
                                  static_cast<const float*>(k_idx), scores, ld, stream);
  return err == hipSuccess ? DSA_OK : hip_fail(err, "indexer launch");
}

dsa_status run_topk(const dsa_rows& rows, int topk, const float* scores, int64_t ld,
                    int32_t* indices, void* ws, hipStream_t stream, bool counts_cleared = false,
                    uint32_t* rowmm = nullptr) {
  const hipError_t err = dsa::launch_topk(rows, topk, scores, ld, indices, ws, stream,
                                          counts_cleared, rowmm);
  return err == hipSuccess ? DSA_OK : hip_fail(err, "top-k launch");
}

dsa_status run_attn(const dsa_rows& rows, const dsa_dims& dims, const void* q,
                    const void* latent, const int32_t* indices, float scale, void* out,
                    float* lse, void* ws, hipStream_t stream, const dsa::PageMap& pm) {
  hipError_t err;
  if (dims.attn_dtype == DSA_BF16)
    err = dsa::launch_attn_bf16(rows, q, latent, indices, scale, out, lse, ws, stream, pm);
  else
    err = dsa::launch_attn_f32(rows, dims, static_cast<const float*>(q),
                               static_cast<const float*>(latent), indices, scale,
                               static_cast<float*>(out), lse, stream);
  return err == hipSuccess ? DSA_OK : hip_fail(err, "attention launch");
}

size_t elem_bytes(dsa_dtype t) { return t == DSA_FP8_E4M3FN ? 1 : (t == DSA_BF16 ? 2 : 4); }

int64_t scores_ld(const dsa_rows& rows) { return (int64_t)align_up((size_t)rows.max_pos + 1, 64); }

// top-k workspace of the forward's chunks: the largest over the chunk sizes it uses
size_t forward_topk_ws(const dsa_rows& rows, int CH) {
  dsa_rows a = rows, b = rows;
  a.num_rows = CH;
  b.num_rows = rows.num_rows - (rows.num_rows - 1) / CH * CH;
  const size_t x = dsa::topk_workspace_bytes(a), y = dsa::topk_workspace_bytes(b);
  return x > y ? x : y;
}

// A chunk whose fp8 indexer runs the tiled kernel and whose top-k streams its rows
// passes each row's score extremes from the one to the other (two words per row),
// so the top-k skips its min / max pass over the scores.
bool forward_fuses_extremes(const dsa_rows& sub, const dsa_dims& dims) {
  return dims.idx_dtype == DSA_FP8_E4M3FN && dsa::indexer_uses_tiles(sub) &&
         dsa::topk_streams_rows(sub);
}

size_t forward_extremes_bytes(const dsa_rows& rows, const dsa_dims& dims, int CH) {
  dsa_rows a = rows, b = rows;
  a.num_rows = CH;
  b.num_rows = rows.num_rows - (rows.num_rows - 1) / CH * CH;
  if (!forward_fuses_extremes(a, dims) && !forward_fuses_extremes(b, dims)) return 0;
  return (size_t)CH * 2 * sizeof(uint32_t);
}

dsa_status forward_impl(const dsa_rows* rows, const dsa_dims* dims, const dsa_pages* pages,
                        const void* q_idx, const float* q_scale, const float* w, const void* k_idx,
                        const float* k_scale, const void* q, const void* latent,
                        float softmax_scale, void* out, float* lse, int32_t* indices_out,
                        int32_t chunk_rows, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if ((st = check_dims(dims)) != DSA_OK) return st;
  dsa::PageMap pm;
  if (pages != nullptr && (st = check_pages(*rows, *dims, pages, kLatentRow, &pm)) != DSA_OK)
    return st;
  if (pages == nullptr && (st = check_latent_span(*rows, *dims)) != DSA_OK) return st;
  if ((st = check_topk_rows(*rows)) != DSA_OK) return st;
  if (chunk_rows < 0) return fail(DSA_E_INVALID, "chunk_rows < 0");
  const int R = rows->num_rows;
  if (R == 0) return DSA_OK;
  if (!q_idx || !w || !k_idx || !q || !latent || !out)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (dims->idx_dtype == DSA_FP8_E4M3FN && (!q_scale || !k_scale))
    return fail(DSA_E_INVALID, "fp8 indexer needs q_scale and k_scale");
  const size_t need = dsa_forward_workspace_size(rows, dims, chunk_rows);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_E_WORKSPACE, "dsa_forward needs %zu workspace bytes, got %zu", need,
                ws_bytes);

  const int CH = (chunk_rows > 0 && chunk_rows < R) ? chunk_rows : R;
  const int64_t ld = scores_ld(*rows);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* scores = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)CH * ld * sizeof(float), 256);
  int32_t* idx_ws = reinterpret_cast<int32_t*>(ws);
  ws += align_up((size_t)CH * dims->topk * sizeof(int32_t), 256);
  void* topk_ws = ws;
  ws += align_up(forward_topk_ws(*rows, CH), 256);
  uint32_t* rowmm = reinterpret_cast<uint32_t*>(ws);
  ws += align_up(forward_extremes_bytes(*rows, *dims, CH), 256);
  bool rowmm_zero = false;  // every top-k launch leaves the words it read at zero
  void* attn_ws = ws;
  const hipStream_t s = as_stream(stream);

  const size_t qi_row = (size_t)dims->n_idx_heads * dims->idx_dim * elem_bytes(dims->idx_dtype);
  const size_t q_row = (size_t)dims->n_heads * dims->qk_dim * elem_bytes(dims->attn_dtype);
  const size_t o_row = (size_t)dims->n_heads * dims->v_dim * elem_bytes(dims->attn_dtype);
  const size_t hi = (size_t)dims->n_idx_heads;

  for (int r0 = 0; r0 < R; r0 += CH) {
    dsa_rows sub = *rows;
    sub.num_rows = (R - r0) < CH ? (R - r0) : CH;
    sub.row_seq = rows->row_seq + r0;
    sub.row_pos = rows->row_pos + r0;
    int32_t* idx = indices_out ? indices_out + (size_t)r0 * dims->topk : idx_ws;
    // the fp8 indexer clears the top-k launch's per-row counts, saving it a launch
    const dsa::ClearWords clear = dims->idx_dtype == DSA_FP8_E4M3FN
                                      ? dsa::topk_counts(sub, topk_ws) : dsa::ClearWords();
    const bool fuse = forward_fuses_extremes(sub, *dims);
    if (fuse && !rowmm_zero) {
      const hipError_t err = dsa::launch_zero_words(rowmm, 2 * CH, s);
      if (err != hipSuccess) return hip_fail(err, "workspace clear");
      rowmm_zero = true;
    }
    st = run_indexer(sub, *dims, static_cast<const uint8_t*>(q_idx) + r0 * qi_row,
                     q_scale ? q_scale + r0 * hi : nullptr, w + r0 * hi, k_idx, k_scale, scores,
                     ld, s, pm, clear, fuse ? rowmm : nullptr);
    if (st != DSA_OK) return st;
    st = run_topk(sub, dims->topk, scores, ld, idx, topk_ws, s, clear.ptr != nullptr,
                  fuse ? rowmm : nullptr);
    if (st != DSA_OK) return st;
    st = run_attn(sub, *dims, static_cast<const uint8_t*>(q) + r0 * q_row, latent, idx,
                  softmax_scale, static_cast<uint8_t*>(out) + r0 * o_row,
                  lse ? lse + (size_t)r0 * dims->n_heads : nullptr, attn_ws, s, pm);
    if (st != DSA_OK) return st;
  }
  return DSA_OK;
}

dsa_status project_impl(const dsa_rows* rows, const dsa_dims* dims, const dsa_pages* pages,
                        int32_t d_model, const void* h, const void* w_q, const void* w_k,
                        const void* w_c, const void* w_w, void* q_idx, float* q_scale, float* w,
                        void* k_idx, float* k_scale, void* latent, void* workspace,
                        size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (dims == nullptr) return fail(DSA_E_INVALID, "dims is NULL");
  if (dims->n_idx_heads != dsa::kIdxHeads || dims->idx_dim != dsa::kIdxDim ||
      dims->qk_dim != dsa::kQkDim || dims->idx_dtype != DSA_FP8_E4M3FN ||
      dims->attn_dtype != DSA_BF16)
    return fail(DSA_E_UNSUPPORTED,
                "projections support H_I=64, d_I=128, D_k=576, fp8 indexer, bf16 latent only");
  if (d_model < 64 || d_model % 64 != 0 || d_model > 65536)
    return fail(DSA_E_UNSUPPORTED, "d_model must be a positive multiple of 64, at most 65536");
  dsa::PageMap pm;
  if (pages != nullptr) {
    dsa_dims full = *dims;  // the paged check wants the whole production set
    full.n_heads = dsa::kHeads;
    full.v_dim = dsa::kVDim;
    full.topk = dsa::kTopk;
    if ((st = check_pages(*rows, full, pages, kLatentRow, &pm)) != DSA_OK) return st;
  }
  if (rows->num_rows == 0) return DSA_OK;
  if (!h || !w_q || !w_k || !w_c || !w_w || !q_idx || !q_scale || !w || !k_idx || !k_scale ||
      !latent)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  const size_t need = dsa::project_workspace_bytes(rows->num_rows, d_model);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(DSA_E_WORKSPACE, "projections need %zu workspace bytes, got %zu", need, ws_bytes);
  const hipError_t err = dsa::launch_project(
      *rows, d_model, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_q),
      static_cast<const uint16_t*>(w_k), static_cast<const uint16_t*>(w_c),
      static_cast<const uint16_t*>(w_w), static_cast<uint8_t*>(q_idx), q_scale, w,
      static_cast<uint8_t*>(k_idx), k_scale, static_cast<uint16_t*>(latent), workspace,
      as_stream(stream), pm);
  return err == hipSuccess ? DSA_OK : hip_fail(err, "projection launch");
}

}  // namespace

namespace dsa {

dsa_status set_error(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

}  // namespace dsa

extern "C" {

int32_t dsa_api_version(void) { return DSA_API_VERSION; }

const char* dsa_status_string(dsa_status status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_E_INVALID: return "DSA_E_INVALID: invalid argument";
    case DSA_E_UNSUPPORTED: return "DSA_E_UNSUPPORTED: unsupported dimensions or dtype";
    case DSA_E_WORKSPACE: return "DSA_E_WORKSPACE: workspace missing or too small";
    case DSA_E_HIP: return "DSA_E_HIP: HIP runtime error";
  }
  return "unknown dsa_status";
}

const char* dsa_last_error(void) { return g_last_error; }

dsa_status dsa_check_index_domain(int32_t* seen) {
  if (seen == nullptr) return fail(DSA_E_INVALID, "seen is NULL");
  uint32_t v = 0u;
  const hipError_t err = dsa::read_index_domain_flag(&v);
  if (err != hipSuccess) return hip_fail(err, "index-domain flag read");
  *seen = v != 0u ? 1 : 0;
  return DSA_OK;
}

dsa_status dsa_indexer_scores(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                              const float* q_scale, const float* w, const void* k_idx,
                              const float* k_scale, float* scores, int64_t ld_scores,
                              void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if ((st = check_dims(dims)) != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q_idx || !w || !k_idx || !scores) return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (dims->idx_dtype == DSA_FP8_E4M3FN && (!q_scale || !k_scale))
    return fail(DSA_E_INVALID, "fp8 indexer needs q_scale and k_scale");
  if (ld_scores < (int64_t)rows->max_pos + 1)
    return fail(DSA_E_INVALID, "ld_scores < max_pos + 1");
  return run_indexer(*rows, *dims, q_idx, q_scale, w, k_idx, k_scale, scores, ld_scores,
                     as_stream(stream), dsa::PageMap());
}

size_t dsa_topk_workspace_size(const dsa_rows* rows, int32_t topk) {
  if (check_rows(rows) != DSA_OK || topk < 1 || topk > 4096) return 0;
  return dsa::topk_workspace_bytes(*rows);
}

dsa_status dsa_topk(const dsa_rows* rows, int32_t topk, const float* scores, int64_t ld_scores,
                    int32_t* indices, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (topk < 1 || topk > 4096) return fail(DSA_E_UNSUPPORTED, "topk must lie in [1, 4096]");
  if ((st = check_topk_rows(*rows)) != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!scores || !indices) return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (ld_scores < (int64_t)rows->max_pos + 1)
    return fail(DSA_E_INVALID, "ld_scores < max_pos + 1");
  const size_t need = dsa::topk_workspace_bytes(*rows);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(DSA_E_WORKSPACE, "top-k needs %zu workspace bytes, got %zu", need, ws_bytes);
  return run_topk(*rows, topk, scores, ld_scores, indices, workspace, as_stream(stream));
}

size_t dsa_sparse_mla_attn_workspace_size(const dsa_rows* rows, const dsa_dims* dims) {
  if (check_rows(rows) != DSA_OK || check_dims(dims) != DSA_OK) return 0;
  return dsa::attn_workspace_bytes(rows->num_rows, *dims);
}

dsa_status dsa_sparse_mla_attn(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                               const void* latent, const int32_t* indices, float softmax_scale,
                               void* out, float* lse, void* workspace, size_t ws_bytes,
                               void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if ((st = check_dims(dims)) != DSA_OK) return st;
  if ((st = check_latent_span(*rows, *dims)) != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !latent || !indices || !out) return fail(DSA_E_INVALID, "NULL tensor pointer");
  const size_t need = dsa::attn_workspace_bytes(rows->num_rows, *dims);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(DSA_E_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
  return run_attn(*rows, *dims, q, latent, indices, softmax_scale, out, lse, workspace,
                  as_stream(stream), dsa::PageMap());
}

size_t dsa_forward_workspace_size(const dsa_rows* rows, const dsa_dims* dims, int32_t chunk_rows) {
  if (check_rows(rows) != DSA_OK || check_dims(dims) != DSA_OK || chunk_rows < 0) return 0;
  const int R = rows->num_rows;
  const int CH = (chunk_rows > 0 && chunk_rows < R) ? chunk_rows : R;
  if (CH == 0) return 0;
  const int64_t ld = scores_ld(*rows);
  size_t bytes = align_up((size_t)CH * ld * sizeof(float), 256);
  bytes += align_up((size_t)CH * dims->topk * sizeof(int32_t), 256);
  bytes += align_up(forward_topk_ws(*rows, CH), 256);
  bytes += align_up(forward_extremes_bytes(*rows, *dims, CH), 256);
  // the last chunk may hold fewer rows and therefore use more attention splits
  const int last = R - (R - 1) / CH * CH;
  const size_t attn = dsa::attn_workspace_bytes(CH, *dims);
  const size_t attn_last = dsa::attn_workspace_bytes(last, *dims);
  bytes += align_up(attn > attn_last ? attn : attn_last, 256);
  return bytes;
}

dsa_status dsa_forward(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                       const float* q_scale, const float* w, const void* k_idx,
                       const float* k_scale, const void* q, const void* latent,
                       float softmax_scale, void* out, float* lse, int32_t* indices_out,
                       int32_t chunk_rows, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(rows, dims, nullptr, q_idx, q_scale, w, k_idx, k_scale, q, latent,
                      softmax_scale, out, lse, indices_out, chunk_rows, workspace, ws_bytes,
                      stream);
}

dsa_status dsa_forward_paged(const dsa_rows* rows, const dsa_dims* dims, const dsa_pages* pages,
                             const void* q_idx, const float* q_scale, const float* w,
                             const void* k_pool, const float* k_scale_pool, const void* q,
                             const void* latent_pool, float softmax_scale, void* out, float* lse,
                             int32_t* indices_out, int32_t chunk_rows, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (pages == nullptr) return fail(DSA_E_INVALID, "pages is NULL");
  return forward_impl(rows, dims, pages, q_idx, q_scale, w, k_pool, k_scale_pool, q,
                      latent_pool, softmax_scale, out, lse, indices_out, chunk_rows, workspace,
                      ws_bytes, stream);
}

dsa_status dsa_indexer_scores_paged(const dsa_rows* rows, const dsa_dims* dims,
                                    const dsa_pages* pages, const void* q_idx,
                                    const float* q_scale, const float* w, const void* k_pool,
                                    const float* k_scale_pool, float* scores, int64_t ld_scores,
                                    void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if ((st = check_dims(dims)) != DSA_OK) return st;
  dsa::PageMap pm;
  if ((st = check_pages(*rows, *dims, pages, kKeyRow, &pm)) != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q_idx || !q_scale || !w || !k_pool || !k_scale_pool || !scores)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (ld_scores < (int64_t)rows->max_pos + 1)
    return fail(DSA_E_INVALID, "ld_scores < max_pos + 1");
  return run_indexer(*rows, *dims, q_idx, q_scale, w, k_pool, k_scale_pool, scores, ld_scores,
                     as_stream(stream), pm);
}

dsa_status dsa_sparse_mla_attn_paged(const dsa_rows* rows, const dsa_dims* dims,
                                     const dsa_pages* pages, const void* q,
                                     const void* latent_pool, const int32_t* indices,
                                     float softmax_scale, void* out, float* lse, void* workspace,
                                     size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if ((st = check_dims(dims)) != DSA_OK) return st;
  dsa::PageMap pm;
  if ((st = check_pages(*rows, *dims, pages, kLatentRow, &pm)) != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !latent_pool || !indices || !out) return fail(DSA_E_INVALID, "NULL tensor pointer");
  const size_t need = dsa::attn_workspace_bytes(rows->num_rows, *dims);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(DSA_E_WORKSPACE, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
  return run_attn(*rows, *dims, q, latent_pool, indices, softmax_scale, out, lse, workspace,
                  as_stream(stream), pm);
}

size_t dsa_project_append_workspace_size(const dsa_rows* rows, int32_t d_model) {
  if (check_rows(rows) != DSA_OK || d_model < 64 || d_model % 64 != 0) return 0;
  return dsa::project_workspace_bytes(rows->num_rows, d_model);
}

dsa_status dsa_project_append(const dsa_rows* rows, const dsa_dims* dims, int32_t d_model,
                              const void* h, const void* w_q, const void* w_k, const void* w_c,
                              const void* w_w, void* q_idx, float* q_scale, float* w,
                              void* k_idx, float* k_scale, void* latent, void* workspace,
                              size_t ws_bytes, void* stream) {
  return project_impl(rows, dims, nullptr, d_model, h, w_q, w_k, w_c, w_w, q_idx, q_scale, w,
                      k_idx, k_scale, latent, workspace, ws_bytes, stream);
}

dsa_status dsa_project_append_paged(const dsa_rows* rows, const dsa_dims* dims,
                                    const dsa_pages* pages, int32_t d_model, const void* h,
                                    const void* w_q, const void* w_k, const void* w_c,
                                    const void* w_w, void* q_idx, float* q_scale, float* w,
                                    void* k_pool, float* k_scale_pool, void* latent_pool,
                                    void* workspace, size_t ws_bytes, void* stream) {
  if (pages == nullptr) return fail(DSA_E_INVALID, "pages is NULL");
  return project_impl(rows, dims, pages, d_model, h, w_q, w_k, w_c, w_w, q_idx, q_scale, w,
                      k_pool, k_scale_pool, latent_pool, workspace, ws_bytes, stream);
}

size_t dsa_indexer_loss_workspace_size(const dsa_rows* rows, const dsa_dims* dims) {
  if (check_rows(rows) != DSA_OK || dims == nullptr || !is_production(*dims)) return 0;
  return dsa::indexer_loss_workspace_bytes(rows->num_rows, dims->topk);
}

dsa_status dsa_indexer_loss(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                            const void* latent, const int32_t* indices, const float* lse,
                            float softmax_scale, const float* scores, int64_t ld_scores,
                            float* loss, float* dscores, void* workspace, size_t ws_bytes,
                            void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (dims == nullptr) return fail(DSA_E_INVALID, "dims is NULL");
  if (!is_production(*dims))
    return fail(DSA_E_UNSUPPORTED, "the indexer loss supports the production dims only");
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !latent || !indices || !lse || !scores || !loss || !dscores)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (ld_scores < (int64_t)rows->max_pos + 1)
    return fail(DSA_E_INVALID, "ld_scores < max_pos + 1");
  const size_t need = dsa::indexer_loss_workspace_bytes(rows->num_rows, dims->topk);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_E_WORKSPACE, "the indexer loss needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  const hipError_t err = dsa::launch_indexer_loss(*rows, q, latent, indices, lse, softmax_scale,
                                                  scores, ld_scores, loss, dscores, workspace,
                                                  as_stream(stream));
  return err == hipSuccess ? DSA_OK : hip_fail(err, "indexer loss launch");
}

size_t dsa_indexer_loss_dense_workspace_size(const dsa_rows* rows, const dsa_dims* dims) {
  if (check_rows(rows) != DSA_OK || dims == nullptr || !is_production(*dims)) return 0;
  return dsa::indexer_loss_dense_workspace_bytes(rows->num_rows, rows->max_pos);
}

dsa_status dsa_indexer_loss_dense(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                                  const void* latent, float softmax_scale, const float* scores,
                                  int64_t ld_scores, float* loss, float* dscores, void* workspace,
                                  size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (dims == nullptr) return fail(DSA_E_INVALID, "dims is NULL");
  if (!is_production(*dims))
    return fail(DSA_E_UNSUPPORTED, "the dense indexer loss supports the production dims only");
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !latent || !scores || !loss || !dscores) return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (ld_scores < (int64_t)rows->max_pos + 1)
    return fail(DSA_E_INVALID, "ld_scores < max_pos + 1");
  const size_t need = dsa::indexer_loss_dense_workspace_bytes(rows->num_rows, rows->max_pos);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_E_WORKSPACE, "the dense indexer loss needs %zu workspace bytes, got %zu", need,
                ws_bytes);
  const hipError_t err = dsa::launch_indexer_loss_dense(*rows, q, latent, softmax_scale, scores,
                                                        ld_scores, loss, dscores, workspace,
                                                        as_stream(stream));
  return err == hipSuccess ? DSA_OK : hip_fail(err, "dense indexer loss launch");
}

namespace {
// checks shared by the two backward calls
dsa_status check_backward(const dsa_rows* rows, const dsa_dims* dims) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (dims == nullptr) return fail(DSA_E_INVALID, "dims is NULL");
  if (!is_production(*dims))
    return fail(DSA_E_UNSUPPORTED, "the indexer backward supports the production dims only");
  if ((int64_t)rows->max_pos + 1 > dsa::kTopkMaxPositions)
    return fail(DSA_E_UNSUPPORTED, "the indexer backward takes rows of up to %d positions",
                dsa::kTopkMaxPositions);
  if ((int64_t)rows->num_seqs * ((int64_t)rows->max_pos + 1) > INT32_MAX)
    return fail(DSA_E_UNSUPPORTED, "the indexer backward needs num_seqs * (max_pos + 1) < 2^31");
  return DSA_OK;
}
}  // namespace

size_t dsa_indexer_backward_workspace_size(const dsa_rows* rows, const dsa_dims* dims,
                                           int64_t shared_keys) {
  if (check_rows(rows) != DSA_OK || dims == nullptr || !is_production(*dims)) return 0;
  return dsa::indexer_backward_workspace_bytes(*rows, dims->topk, false, shared_keys);
}

size_t dsa_indexer_backward_dense_workspace_size(const dsa_rows* rows, const dsa_dims* dims,
                                                 int64_t shared_keys) {
  if (check_rows(rows) != DSA_OK || dims == nullptr || !is_production(*dims)) return 0;
  return dsa::indexer_backward_workspace_bytes(*rows, dims->topk, true, shared_keys);
}

dsa_status dsa_indexer_backward_dense(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                                      const float* q_scale, const float* w, const void* k_idx,
                                      const float* k_scale, const float* dscores,
                                      int64_t ld_dscores, float* dq, float* dw, float* dk,
                                      void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_backward(rows, dims);
  if (st != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q_idx || !q_scale || !w || !k_idx || !k_scale || !dscores || !dq || !dw || !dk)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  if (ld_dscores < (int64_t)rows->max_pos + 1)
    return fail(DSA_E_INVALID, "ld_dscores < max_pos + 1");
  const size_t need = dsa::indexer_backward_workspace_bytes(*rows, dims->topk, true, 0);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_E_WORKSPACE, "the dense indexer backward needs at least %zu workspace bytes, got %zu",
                need, ws_bytes);
  const hipError_t err = dsa::launch_indexer_backward_dense(
      *rows, static_cast<const uint8_t*>(q_idx), q_scale, w, static_cast<const uint8_t*>(k_idx),
      k_scale, dscores, ld_dscores, dq, dw, dk, workspace, ws_bytes, as_stream(stream));
  return err == hipSuccess ? DSA_OK : hip_fail(err, "dense indexer backward launch");
}

dsa_status dsa_indexer_backward(const dsa_rows* rows, const dsa_dims* dims, const void* q_idx,
                                const float* q_scale, const float* w, const void* k_idx,
                                const float* k_scale, const int32_t* indices,
                                const float* dscores, float* dq, float* dw, float* dk,
                                void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_backward(rows, dims);
  if (st != DSA_OK) return st;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q_idx || !q_scale || !w || !k_idx || !k_scale || !indices || !dscores || !dq || !dw || !dk)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  const size_t need = dsa::indexer_backward_workspace_bytes(*rows, dims->topk, false, 0);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_E_WORKSPACE, "the indexer backward needs at least %zu workspace bytes, got %zu",
                need, ws_bytes);
  const hipError_t err = dsa::launch_indexer_backward(
      *rows, static_cast<const uint8_t*>(q_idx), q_scale, w, static_cast<const uint8_t*>(k_idx),
      k_scale, indices, dscores, dq, dw, dk, workspace, ws_bytes, as_stream(stream));
  return err == hipSuccess ? DSA_OK : hip_fail(err, "indexer backward launch");
}

size_t dsa_mha_prefill_workspace_size(const dsa_rows* rows, const dsa_dims* dims) {
  if (check_rows(rows) != DSA_OK || dims == nullptr || !is_production(*dims)) return 0;
  return dsa::mha_workspace_bytes(rows->num_rows, rows->num_seqs, rows->max_pos);
}

dsa_status dsa_mha_prefill(const dsa_rows* rows, const dsa_dims* dims, const void* q,
                           const void* latent, const void* w_uk, const void* w_uv,
                           const int32_t* indices, float softmax_scale, void* out, float* lse,
                           void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_rows(rows);
  if (st != DSA_OK) return st;
  if (dims == nullptr) return fail(DSA_E_INVALID, "dims is NULL");
  if (!is_production(*dims))
    return fail(DSA_E_UNSUPPORTED, "the MHA mode supports the production dims only");
  if (rows->max_pos + 1 > 16384)
    return fail(DSA_E_UNSUPPORTED, "the MHA mode is for short prefill: max_pos + 1 <= 16384");
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !latent || !w_uk || !w_uv || !indices || !out)
    return fail(DSA_E_INVALID, "NULL tensor pointer");
  const size_t need = dsa::mha_workspace_bytes(rows->num_rows, rows->num_seqs, rows->max_pos);
  if (workspace == nullptr || ws_bytes < need)
    return fail(DSA_E_WORKSPACE, "the MHA mode needs %zu workspace bytes, got %zu", need, ws_bytes);
  const hipError_t err = dsa::launch_mha(*rows, q, latent, w_uk, w_uv, indices, softmax_scale, out,
                                         lse, workspace, as_stream(stream));
  return err == hipSuccess ? DSA_OK : hip_fail(err, "MHA-mode launch");
}

}  // extern "C"
