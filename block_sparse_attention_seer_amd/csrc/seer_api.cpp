// The extern "C" entry points of libseer: argument checks, then launches.
// No HIP call happens before every host-side check has passed.

#include <algorithm>
#include <cmath>
#include <string>

#include "seer_internal.h"

using seer::check_dims;
using seer::check_ptr;

namespace {

int fail(int code, const std::string& why) {
  seer::set_error(why);
  return code;
}

// Runs a check that fills `why`; records it on failure.
#define SEER_CHECK(call)                     \
  do {                                       \
    std::string why_;                        \
    int rc_ = call;                          \
    if (rc_ != SEER_OK) return fail(rc_, why_); \
  } while (0)

int check_select_args(const seer_dims* dims, int32_t mode, int32_t topk_blocks, float threshold,
                      int32_t max_selected) {
  const int64_t nbm = seer::nb_max(dims);
  if (nbm > seer::kMaxNBSelect)
    return fail(SEER_ERR_UNSUPPORTED, "select needs ceil(max_seq_len / block_size) <= 8192");
  if (mode == SEER_SELECT_TOPK) {
    if (topk_blocks < 0) return fail(SEER_ERR_INVALID_ARG, "topk_blocks must be >= 0");
    const int64_t need = std::min<int64_t>(static_cast<int64_t>(topk_blocks) + 1, nbm);
    if (max_selected < need)
      return fail(SEER_ERR_INVALID_ARG, "max_selected must be >= min(topk_blocks + 1, NBmax)");
  } else if (mode == SEER_SELECT_THRESHOLD || mode == SEER_SELECT_TOPP) {
    if (!(threshold >= 0.0f && threshold <= 1.0f))
      return fail(SEER_ERR_INVALID_ARG, "threshold (tau or p) must be in [0, 1]");
    if (max_selected < nbm)
      return fail(SEER_ERR_INVALID_ARG, "threshold and top-p modes need max_selected >= NBmax");
  } else {
    return fail(SEER_ERR_INVALID_ARG,
                "mode must be SEER_SELECT_TOPK, SEER_SELECT_THRESHOLD or SEER_SELECT_TOPP");
  }
  if (max_selected < 1 || max_selected > nbm)
    return fail(SEER_ERR_INVALID_ARG, "max_selected must be in [1, NBmax]");
  return SEER_OK;
}

// Workgroups per (b, h) for a gate launch that only scores: enough to put
// one on every compute unit, at most kMaxGateParts.
int gate_row_parts(const seer_dims* d) {
  int cus = 0;
  if (seer::device_cu_count(&cus) != SEER_OK) return 1;
  const int64_t pairs = static_cast<int64_t>(d->batch) * d->num_kv_heads;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(seer::kMaxGateParts, cus / pairs)));
}

int resolve_split(const seer_dims* d, int max_blocks, int num_split, int* out) {
  if (num_split < SEER_SPLIT_BALANCED || num_split > seer::kMaxSplit)
    return fail(SEER_ERR_INVALID_ARG, "num_split must be SEER_SPLIT_BALANCED (-1) or in [0, 128]");
  if (num_split > 0) {
    *out = num_split;
    return SEER_OK;
  }
  int cus = 0;
  int rc = seer::device_cu_count(&cus);
  if (rc != SEER_OK) return rc;
  *out = seer::auto_num_split(d, max_blocks, cus);
  return SEER_OK;
}

// Whether a balanced division (SEER_SPLIT_BALANCED) runs stream-K: with
// fewer (b, h) pairs than compute units.  With more, the dispatcher already
// balances fixed splits, and stream-K's extra part boundaries measured
// slower.
bool balanced_uses_stream_k(int64_t pairs) {
  int cus = 0;
  return seer::device_cu_count(&cus) == SEER_OK && pairs < cus;
}

}  // namespace

extern "C" {

int seer_kcomp_update(const seer_dims* dims, const uint16_t* k_nope, const uint16_t* w_k,
                      const int32_t* seq_lens, int32_t* kcomp_lens, uint16_t* kcomp,
                      int32_t max_new_blocks, double rope_theta, void* stream) {
  SEER_CHECK(check_dims(dims, &why_));
  SEER_CHECK(check_ptr(k_nope, 16, "k_nope", &why_));
  SEER_CHECK(check_ptr(w_k, 16, "w_k", &why_));
  SEER_CHECK(check_ptr(seq_lens, 4, "seq_lens", &why_));
  SEER_CHECK(check_ptr(kcomp_lens, 4, "kcomp_lens", &why_));
  SEER_CHECK(check_ptr(kcomp, 16, "kcomp", &why_));
  if (max_new_blocks < 1) return fail(SEER_ERR_INVALID_ARG, "max_new_blocks must be >= 1");
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(SEER_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  if (max_new_blocks > seer::nb_max(dims)) max_new_blocks = static_cast<int32_t>(seer::nb_max(dims));
  seer::PrepArgs a{};
  a.k_nope = k_nope;
  a.w_k = w_k;
  a.kcomp_lens = kcomp_lens;
  a.kcomp = kcomp;
  a.max_new_blocks = max_new_blocks;
  a.seq_lens = seq_lens;
  a.theta = rope_theta;
  int rc = seer::launch_prep(*dims, a, stream);
  if (rc != SEER_OK) return rc;
  return seer::launch_commit(*dims, seq_lens, kcomp_lens, max_new_blocks, stream);
}

size_t seer_gate_workspace_bytes(const seer_dims* dims) {
  std::string why;
  if (check_dims(dims, &why) != SEER_OK) return 0;
  return seer::gate_workspace_bytes(dims);
}

int seer_gate_scores(const seer_dims* dims, const uint16_t* q_nope, const uint16_t* w_q,
                     const uint16_t* kcomp, const int32_t* kcomp_lens, const int32_t* seq_lens,
                     double rope_theta, void* workspace, size_t workspace_bytes, float* logits,
                     void* stream) {
  SEER_CHECK(check_dims(dims, &why_));
  SEER_CHECK(check_ptr(q_nope, 16, "q_nope", &why_));
  SEER_CHECK(check_ptr(w_q, 16, "w_q", &why_));
  SEER_CHECK(check_ptr(kcomp, 16, "kcomp", &why_));
  SEER_CHECK(check_ptr(kcomp_lens, 4, "kcomp_lens", &why_));
  SEER_CHECK(check_ptr(seq_lens, 4, "seq_lens", &why_));
  SEER_CHECK(check_ptr(logits, 4, "logits", &why_));
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(SEER_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  if (workspace == nullptr || workspace_bytes < seer::gate_workspace_bytes(dims))
    return fail(SEER_ERR_WORKSPACE, "gate workspace missing or smaller than seer_gate_workspace_bytes()");
  SEER_CHECK(check_ptr(workspace, 16, "workspace", &why_));
  seer::GateArgs ga{};
  ga.q_nope = q_nope;
  ga.w_q = w_q;
  ga.q_gate = static_cast<float*>(workspace);
  ga.theta = rope_theta;
  ga.kcomp = const_cast<uint16_t*>(kcomp);  // read only: no new entries in this launch
  ga.kcomp_lens = kcomp_lens;
  ga.seq_lens = seq_lens;
  ga.logits_out = logits;
  ga.row_parts = gate_row_parts(dims);
  return seer::launch_gate(*dims, ga, stream);
}

int seer_select_blocks(const seer_dims* dims, const float* logits, const int32_t* kcomp_lens,
                       const int32_t* seq_lens, int32_t mode, int32_t topk_blocks, float threshold,
                       int32_t max_selected, int32_t* block_idx, int32_t* num_selected,
                       void* stream) {
  SEER_CHECK(check_dims(dims, &why_));
  SEER_CHECK(check_ptr(logits, 4, "logits", &why_));
  SEER_CHECK(check_ptr(kcomp_lens, 4, "kcomp_lens", &why_));
  SEER_CHECK(check_ptr(seq_lens, 4, "seq_lens", &why_));
  SEER_CHECK(check_ptr(block_idx, 4, "block_idx", &why_));
  SEER_CHECK(check_ptr(num_selected, 4, "num_selected", &why_));
  {
    const int rc = check_select_args(dims, mode, topk_blocks, threshold, max_selected);
    if (rc != SEER_OK) return rc;
  }
  seer::SelectArgs a{logits, kcomp_lens, seq_lens, mode, topk_blocks, threshold,
                     max_selected, block_idx, num_selected};
  return seer::launch_select(*dims, a, stream);
}

size_t seer_decode_workspace_bytes(const seer_dims* dims, int32_t max_blocks, int32_t num_split) {
  std::string why;
  if (check_dims(dims, &why) != SEER_OK || max_blocks < 1) return 0;
  int s = 0;
  if (resolve_split(dims, max_blocks, num_split, &s) != SEER_OK) return 0;
  const int64_t pairs = static_cast<int64_t>(dims->batch) * dims->num_kv_heads;
  const int g = dims->num_q_heads / dims->num_kv_heads;
  size_t bytes = seer::decode_workspace_bytes(pairs, s, g, dims->head_dim);
  if (num_split == SEER_SPLIT_BALANCED && balanced_uses_stream_k(pairs))
    bytes = std::max(bytes, seer::decode_sk_workspace_bytes(pairs, s, g, dims->head_dim));
  return bytes;
}

size_t seer_workspace_bytes(const seer_dims* dims, int32_t max_blocks, int32_t num_split) {
  return seer_decode_workspace_bytes(dims, max_blocks, num_split);
}

int seer_decode_num_split(const seer_dims* dims, int32_t max_blocks, int32_t num_split,
                          int32_t* num_split_out) {
  SEER_CHECK(check_dims(dims, &why_));
  if (num_split_out == nullptr) return fail(SEER_ERR_INVALID_ARG, "num_split_out is NULL");
  if (max_blocks < 1) return fail(SEER_ERR_INVALID_ARG, "max_blocks must be >= 1");
  int s = 0;
  int rc = resolve_split(dims, max_blocks, num_split, &s);
  if (rc != SEER_OK) return rc;
  *num_split_out = s;
  return SEER_OK;
}

// A paged cache: page pools and the block table (see seer_sparse_decode_paged).
struct PagedCache {
  const int32_t* block_table;
  int32_t table_stride;
  int32_t num_pages;
  int64_t page_stride;
  int64_t page_head_stride;
};

static int check_paged(const seer_dims* dims, const PagedCache& pc, std::string* why) {
  if (check_ptr(pc.block_table, 4, "block_table", why) != SEER_OK) return SEER_ERR_INVALID_ARG;
  if (pc.table_stride < 1 || pc.num_pages < 1) {
    *why = "table_stride and num_pages must be >= 1";
    return SEER_ERR_INVALID_ARG;
  }
  if (pc.page_stride < 1 || pc.page_head_stride < 0 || (pc.page_stride % 8) ||
      (pc.page_head_stride % 8)) {
    *why = "page strides must be positive multiples of 8 elements";
    return SEER_ERR_INVALID_ARG;
  }
  (void)dims;
  return SEER_OK;
}

static int decode_common(const seer_dims* dims, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* seq_lens, const int32_t* block_idx,
                         const int32_t* num_selected, int32_t max_blocks, float scale,
                         int32_t num_split, void* workspace, size_t workspace_bytes,
                         uint16_t* out, float* lse, void* stream,
                         int32_t* commit_lens = nullptr, int commit_max_new = 0,
                         const PagedCache* paged = nullptr, bool stream_k = false) {
  SEER_CHECK(check_dims(dims, &why_));
  SEER_CHECK(check_ptr(q, 16, "q", &why_));
  SEER_CHECK(check_ptr(k, 16, "k_cache", &why_));
  SEER_CHECK(check_ptr(v, 16, "v_cache", &why_));
  SEER_CHECK(check_ptr(seq_lens, 4, "seq_lens", &why_));
  SEER_CHECK(check_ptr(out, 16, "out", &why_));
  if (lse != nullptr) SEER_CHECK(check_ptr(lse, 4, "lse", &why_));
  if (!std::isfinite(scale)) return fail(SEER_ERR_INVALID_ARG, "scale must be finite");
  if (max_blocks < 1 || max_blocks > seer::nb_max(dims))
    return fail(SEER_ERR_INVALID_ARG, "max_selected must be in [1, NBmax]");
  int s = 0;
  int rc = resolve_split(dims, max_blocks, num_split, &s);
  if (rc != SEER_OK) return rc;
  const int64_t pairs = static_cast<int64_t>(dims->batch) * dims->num_kv_heads;
  const int g = dims->num_q_heads / dims->num_kv_heads;
  const size_t need = seer::decode_workspace_bytes(pairs, s, g, dims->head_dim);
  // a balanced division of a selection over a contiguous cache: stream-K
  // where there are fewer pairs than compute units
  if (num_split == SEER_SPLIT_BALANCED && block_idx != nullptr && paged == nullptr)
    stream_k = stream_k || balanced_uses_stream_k(pairs);
  // stream-K only with the workspace it needs
  stream_k = stream_k && workspace != nullptr &&
             workspace_bytes >= seer::decode_sk_workspace_bytes(pairs, s, g, dims->head_dim);
  if (stream_k) {
    SEER_CHECK(check_ptr(workspace, 256, "workspace", &why_));
  } else if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(SEER_ERR_WORKSPACE, "decode workspace missing or smaller than seer_decode_workspace_bytes()");
    SEER_CHECK(check_ptr(workspace, 256, "workspace", &why_));
  }
  seer::DecodeArgs a{q, k, v, seq_lens, block_idx, num_selected, max_blocks, scale, s,
                     workspace, out, lse, commit_lens, commit_max_new};
  a.stream_k = stream_k;
  if (paged != nullptr) {
    SEER_CHECK(check_paged(dims, *paged, &why_));
    a.block_table = paged->block_table;
    a.table_stride = paged->table_stride;
    a.num_pages = paged->num_pages;
    a.page_stride = paged->page_stride;
    a.page_head_stride = paged->page_head_stride;
  }
  return seer::launch_decode(*dims, a, stream);
}

int seer_sparse_decode(const seer_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int32_t* seq_lens, const int32_t* block_idx,
                       const int32_t* num_selected, int32_t max_selected, float scale,
                       int32_t num_split, void* workspace, size_t workspace_bytes, uint16_t* out,
                       float* lse, void* stream) {
  SEER_CHECK(check_ptr(block_idx, 4, "block_idx", &why_));
  SEER_CHECK(check_ptr(num_selected, 4, "num_selected", &why_));
  return decode_common(dims, q, k_cache, v_cache, seq_lens, block_idx, num_selected, max_selected,
                       scale, num_split, workspace, workspace_bytes, out, lse, stream);
}

int seer_dense_decode(const seer_dims* dims, const uint16_t* q, const uint16_t* k_cache,
                      const uint16_t* v_cache, const int32_t* seq_lens, float scale,
                      int32_t num_split, void* workspace, size_t workspace_bytes, uint16_t* out,
                      float* lse, void* stream) {
  std::string why;
  if (check_dims(dims, &why) != SEER_OK) return fail(check_dims(dims, &why), why);
  return decode_common(dims, q, k_cache, v_cache, seq_lens, nullptr, nullptr,
                       static_cast<int32_t>(seer::nb_max(dims)), scale, num_split, workspace,
                       workspace_bytes, out, lse, stream);
}

int seer_sparse_decode_paged(const seer_dims* dims, const uint16_t* q, const uint16_t* k_pages,
                             const uint16_t* v_pages, int64_t page_stride,
                             int64_t page_head_stride, int32_t num_pages,
                             const int32_t* block_table, int32_t table_stride,
                             const int32_t* seq_lens, const int32_t* block_idx,
                             const int32_t* num_selected, int32_t max_selected, float scale,
                             int32_t num_split, void* workspace, size_t workspace_bytes,
                             uint16_t* out, float* lse, void* stream) {
  SEER_CHECK(check_ptr(block_idx, 4, "block_idx", &why_));
  SEER_CHECK(check_ptr(num_selected, 4, "num_selected", &why_));
  const PagedCache pc{block_table, table_stride, num_pages, page_stride, page_head_stride};
  return decode_common(dims, q, k_pages, v_pages, seq_lens, block_idx, num_selected, max_selected,
                       scale, num_split, workspace, workspace_bytes, out, lse, stream, nullptr, 0,
                       &pc);
}

int seer_dense_decode_paged(const seer_dims* dims, const uint16_t* q, const uint16_t* k_pages,
                            const uint16_t* v_pages, int64_t page_stride, int64_t page_head_stride,
                            int32_t num_pages, const int32_t* block_table, int32_t table_stride,
                            const int32_t* seq_lens, float scale, int32_t num_split,
                            void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                            void* stream) {
  std::string why;
  if (check_dims(dims, &why) != SEER_OK) return fail(check_dims(dims, &why), why);
  const PagedCache pc{block_table, table_stride, num_pages, page_stride, page_head_stride};
  return decode_common(dims, q, k_pages, v_pages, seq_lens, nullptr, nullptr,
                       static_cast<int32_t>(seer::nb_max(dims)), scale, num_split, workspace,
                       workspace_bytes, out, lse, stream, nullptr, 0, &pc);
}

int seer_decode_step(const seer_dims* dims, const uint16_t* q_nope, const uint16_t* q,
                     const uint16_t* k_nope, const uint16_t* k_cache, const uint16_t* v_cache,
                     const uint16_t* w_q, const uint16_t* w_k, const int32_t* seq_lens,
                     int32_t* kcomp_lens, uint16_t* kcomp, int32_t max_new_blocks,
                     double rope_theta, int32_t mode, int32_t topk_blocks, float threshold,
                     int32_t max_selected, int32_t* block_idx, int32_t* num_selected,
                     float* logits, float scale, int32_t num_split, void* workspace,
                     size_t workspace_bytes, uint16_t* out, float* lse, void* stream) {
  SEER_CHECK(check_dims(dims, &why_));
  SEER_CHECK(check_ptr(q_nope, 16, "q_nope", &why_));
  SEER_CHECK(check_ptr(q, 16, "q", &why_));
  SEER_CHECK(check_ptr(k_nope, 16, "k_nope", &why_));
  SEER_CHECK(check_ptr(k_cache, 16, "k_cache", &why_));
  SEER_CHECK(check_ptr(v_cache, 16, "v_cache", &why_));
  SEER_CHECK(check_ptr(w_q, 16, "w_q", &why_));
  SEER_CHECK(check_ptr(w_k, 16, "w_k", &why_));
  SEER_CHECK(check_ptr(seq_lens, 4, "seq_lens", &why_));
  SEER_CHECK(check_ptr(kcomp_lens, 4, "kcomp_lens", &why_));
  SEER_CHECK(check_ptr(kcomp, 16, "kcomp", &why_));
  SEER_CHECK(check_ptr(block_idx, 4, "block_idx", &why_));
  SEER_CHECK(check_ptr(num_selected, 4, "num_selected", &why_));
  if (logits != nullptr) SEER_CHECK(check_ptr(logits, 4, "logits", &why_));
  SEER_CHECK(check_ptr(out, 16, "out", &why_));
  if (lse != nullptr) SEER_CHECK(check_ptr(lse, 4, "lse", &why_));
  if (max_new_blocks < 0) return fail(SEER_ERR_INVALID_ARG, "max_new_blocks must be >= 0");
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(SEER_ERR_INVALID_ARG, "rope_theta must be positive and finite");
  if (!std::isfinite(scale)) return fail(SEER_ERR_INVALID_ARG, "scale must be finite");
  {
    const int rc = check_select_args(dims, mode, topk_blocks, threshold, max_selected);
    if (rc != SEER_OK) return rc;
  }
  int s = 0;
  {
    const int rc = resolve_split(dims, max_selected, num_split, &s);
    if (rc != SEER_OK) return rc;
  }
  const int64_t pairs = static_cast<int64_t>(dims->batch) * dims->num_kv_heads;
  const int g = dims->num_q_heads / dims->num_kv_heads;
  size_t dec_bytes = seer::decode_workspace_bytes(pairs, s, g, dims->head_dim);
  if (workspace == nullptr || workspace_bytes < dec_bytes + seer::step_gate_bytes(dims))
    return fail(SEER_ERR_WORKSPACE, "workspace missing or smaller than seer_decode_step_workspace_bytes()");
  // Threshold and top-p keep a different number of blocks per pair.  With
  // fewer pairs than compute units, fixed splits cannot even that out, so
  // with an automatic split count their decode divides all chunks evenly
  // over the grid (stream-K) when the workspace holds its larger decode
  // region.  With more pairs the dispatcher balances the fixed splits
  // itself, and stream-K's extra part boundaries measured slower.
  bool stream_k = false;
  if ((num_split == 0 || num_split == SEER_SPLIT_BALANCED) && mode != SEER_SELECT_TOPK &&
      balanced_uses_stream_k(pairs)) {
    const size_t sk_bytes =
        std::max(dec_bytes, seer::decode_sk_workspace_bytes(pairs, s, g, dims->head_dim));
    if (workspace_bytes >= sk_bytes + seer::step_gate_bytes(dims)) {
      dec_bytes = sk_bytes;
      stream_k = true;
    }
  }
  SEER_CHECK(check_ptr(workspace, 256, "workspace", &why_));
  if (max_new_blocks > seer::nb_max(dims)) max_new_blocks = static_cast<int32_t>(seer::nb_max(dims));

  // Launch 1: per (b, h), the entries of newly completed blocks, the gate
  // query, the logits and the selection.  Launch 2: the sparse decode, which
  // also raises kcomp_lens over those entries.  More new blocks than one
  // gate launch computes (a catch-up after a prompt) take the staged update
  // first.
  int rc = SEER_OK;
  int inline_new = max_new_blocks;
  if (max_new_blocks > seer::kMaxInlineNew) {
    seer::PrepArgs pa{};
    pa.k_nope = k_nope;
    pa.w_k = w_k;
    pa.kcomp_lens = kcomp_lens;
    pa.kcomp = kcomp;
    pa.max_new_blocks = max_new_blocks;
    pa.seq_lens = seq_lens;
    pa.theta = rope_theta;
    rc = seer::launch_prep(*dims, pa, stream);
    if (rc != SEER_OK) return rc;
    rc = seer::launch_commit(*dims, seq_lens, kcomp_lens, max_new_blocks, stream);
    if (rc != SEER_OK) return rc;
    inline_new = 0;
  }
  seer::GateArgs ga{};
  ga.q_nope = q_nope;
  ga.w_q = w_q;
  // the gate's scratch first (a fixed place whatever the split count), then
  // the decode workspace
  char* ws = static_cast<char*>(workspace);
  ga.q_gate = reinterpret_cast<float*>(ws);
  ga.theta = rope_theta;
  ga.k_nope = k_nope;
  ga.w_k = w_k;
  ga.max_new = inline_new;
  ga.kcomp = kcomp;
  ga.kcomp_lens = kcomp_lens;
  ga.seq_lens = seq_lens;
  ga.logits_out = logits;
  ga.block_idx = block_idx;
  ga.num_selected = num_selected;
  ga.mode = mode;
  ga.topk = topk_blocks;
  ga.max_selected = max_selected;
  ga.tau = threshold;
  // the decode's split counters (at the start of its workspace) are zeroed
  // by the gate launch, so the workspace needs no particular contents
  if (s > 1 || stream_k)
    ga.clear_counters = reinterpret_cast<int32_t*>(ws + seer::step_gate_bytes(dims));
  rc = seer::launch_gate(*dims, ga, stream);
  if (rc != SEER_OK) return rc;
  return decode_common(dims, q, k_cache, v_cache, seq_lens, block_idx, num_selected, max_selected,
                       scale, s, ws + seer::step_gate_bytes(dims), dec_bytes, out, lse, stream,
                       inline_new > 0 ? kcomp_lens : nullptr, inline_new, nullptr, stream_k);
}

size_t seer_prefill_workspace_bytes(const seer_dims* dims) {
  std::string why;
  if (check_dims(dims, &why) != SEER_OK) return 0;
  return seer::prefill_workspace_bytes(dims);
}

int seer_prefill_attention(const seer_dims* dims, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* seq_lens, float scale,
                           void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                           float* gt, void* stream) {
  SEER_CHECK(check_dims(dims, &why_));
  SEER_CHECK(check_ptr(q, 16, "q", &why_));
  SEER_CHECK(check_ptr(k, 16, "k", &why_));
  SEER_CHECK(check_ptr(v, 16, "v", &why_));
  SEER_CHECK(check_ptr(seq_lens, 4, "seq_lens", &why_));
  SEER_CHECK(check_ptr(out, 16, "out", &why_));
  SEER_CHECK(check_ptr(lse, 4, "lse", &why_));
  if (gt != nullptr) SEER_CHECK(check_ptr(gt, 4, "gt", &why_));
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(SEER_ERR_INVALID_ARG, "scale must be finite and positive");
  if (workspace == nullptr || workspace_bytes < seer::prefill_workspace_bytes(dims))
    return fail(SEER_ERR_WORKSPACE, "prefill workspace missing or smaller than seer_prefill_workspace_bytes()");
  SEER_CHECK(check_ptr(workspace, 256, "workspace", &why_));
  const seer::PrefillArgs a{q, k, v, seq_lens, scale, workspace, out, lse, gt};
  return seer::launch_prefill(*dims, a, stream);
}

size_t seer_decode_step_workspace_bytes(const seer_dims* dims, int32_t max_selected,
                                        int32_t num_split) {
  std::string why;
  if (check_dims(dims, &why) != SEER_OK || max_selected < 1) return 0;
  size_t dec = seer_decode_workspace_bytes(dims, max_selected, num_split);
  if (num_split == 0 || num_split == SEER_SPLIT_BALANCED) {  // room for the stream-K decode
    int s = 0;
    if (resolve_split(dims, max_selected, 0, &s) != SEER_OK) return 0;
    const int64_t pairs = static_cast<int64_t>(dims->batch) * dims->num_kv_heads;
    dec = std::max(dec, seer::decode_sk_workspace_bytes(pairs, s, dims->num_q_heads / dims->num_kv_heads,
                                                        dims->head_dim));
  }
  return dec + seer::step_gate_bytes(dims);
}

}  // extern "C"
