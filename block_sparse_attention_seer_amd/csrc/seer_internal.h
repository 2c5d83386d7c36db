// Internal interfaces between the C ABI layer, the HIP-free argument checks
// and the kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/seer.h"

namespace seer {

// ----------------------------------------------------------------- limits
constexpr int kMaxGroup = 16;          // query heads per KV head (MFMA N = 16)
constexpr int kMaxNBSelect = 8192;     // blocks per sequence the select kernel holds in LDS
constexpr int kMaxSplit = 128;         // splits per (b, h) in the decode kernel
constexpr int kDecodeMergeLds = 48 * 1024;  // LDS bytes for the decode wave merge
constexpr int kMaxInlineNew = 4;       // new cache entries the gate launch computes itself
constexpr size_t kNoAllocScratchBytes = SEER_NOALLOC_SCRATCH_BYTES;  // seer_decode_step_noalloc's workspace
constexpr int kCounterBytes = 256;     // alignment of the partial outputs after the partial lse
constexpr int kPrefillTokenTile = 64;  // prefill: key tile, and the padding of the token axis
constexpr int kSkMaxPairs = 2048;      // (b, h) pairs the stream-K decode prefixes in LDS
constexpr int kSkMergeLds = 32 * 1024; // wave-merge LDS bytes that leave room for that prefix
constexpr int kMaxGateParts = 4;       // workgroups per (b, h) in a scoring-only gate launch

// ------------------------------------------------------- argument checks
// These live in a HIP-free translation unit so that a CPU-only test can
// exercise every error path.  Each returns SEER_OK or an error code and
// fills *why.
int check_dims(const seer_dims* d, std::string* why);
int check_kv(const seer_dims* d, const void* k, const char* name, std::string* why);
int check_ptr(const void* p, size_t align, const char* name, std::string* why);

int64_t nb_max(const seer_dims* d);  // ceil(Lmax / b)
size_t gate_workspace_bytes(const seer_dims* d);
// The gate queries inside the fused step's workspace, rounded up to 256 bytes.
size_t step_gate_bytes(const seer_dims* d);
// Workspace of the decode kernel for `pairs` (b, h) pairs, `num_split`
// splits and group size g: the per-split lse and outputs.
size_t decode_workspace_bytes(int64_t pairs, int num_split, int g, int head_dim);
// Workspace of the stream-K decode over a grid of pairs x num_split
// workgroups: a counter per pair and two partial slots per workgroup.
size_t decode_sk_workspace_bytes(int64_t pairs, int num_split, int g, int head_dim);
// Automatic split count given the device's compute-unit count.
int auto_num_split(const seer_dims* d, int max_blocks, int num_cus);

void set_error(const std::string& msg);
const char* last_error();

// ------------------------------------------------------ kernel launchers
// Implemented in the .hip files.  Arguments were validated by the caller.
// The staged cache update: entries kcomp_lens[b] + z, z < max_new_blocks,
// of every (b, h) whose block is complete; launch_commit then raises
// kcomp_lens.
struct PrepArgs {
  const uint16_t* k_nope;
  const uint16_t* w_k;
  const int32_t* kcomp_lens;
  uint16_t* kcomp;
  int max_new_blocks;
  const int32_t* seq_lens;
  double theta;
};
int launch_prep(const seer_dims& d, const PrepArgs& a, void* stream);
int launch_commit(const seer_dims& d, const int32_t* seq_lens, int32_t* kcomp_lens, int max_new,
                  void* stream);

// Per-(b, h) gate query and block logits, and the selection when block_idx
// != nullptr.  With max_new > 0 (at most kMaxInlineNew) the launch first
// computes the pair's entries kcomp_lens[b] .. +max_new-1 whose blocks are
// complete and scores them too; kcomp_lens itself is not raised.
struct GateArgs {
  const uint16_t* q_nope;
  const uint16_t* w_q;
  float* q_gate;           // [B, H_kv, d_gate] copy of the gate queries, or nullptr
  double theta;
  const uint16_t* k_nope;  // needed when max_new > 0
  const uint16_t* w_k;
  int max_new;
  uint16_t* kcomp;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  float* logits_out;       // or nullptr
  int32_t* block_idx;      // selection when non-null (then one row part)
  int32_t* num_selected;
  int mode, topk, max_selected;
  float tau;
  int row_parts = 1;       // workgroups per (b, h), each scoring a range of cache rows
  int32_t* clear_counters = nullptr;  // [B * H_kv] decode split counters to zero, or nullptr
};
int launch_gate(const seer_dims& d, const GateArgs& a, void* stream);

struct SelectArgs {
  const float* logits;
  const int32_t* kcomp_lens;
  const int32_t* seq_lens;
  int mode;
  int topk;
  float tau;
  int max_selected;
  int32_t* block_idx;
  int32_t* num_selected;
};
int launch_select(const seer_dims& d, const SelectArgs& a, void* stream);
float log_threshold(float tau);        // ln(tau), -inf for tau <= 0
uint32_t topp_mass_target(float p);    // ceil(p * 2^30), clamped

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* block_idx;     // nullptr = dense
  const int32_t* num_selected;  // nullptr = dense
  int max_selected;             // index row length (sparse)
  float scale;
  int num_split;
  void* workspace;              // split counters and partials (num_split > 1 or stream-K)
  uint16_t* out;
  float* lse;
  int32_t* commit_lens;         // fused step: raise kcomp_lens here (or nullptr)
  int commit_max_new;
  // paged cache (k, v are page pools) when block_table != nullptr
  const int32_t* block_table;
  int table_stride;
  int num_pages;
  int64_t page_stride;
  int64_t page_head_stride;
  // Divide the selections' chunks evenly over the grid (stream-K) instead of
  // cutting each pair into num_split ranges.  Needs a workspace of
  // decode_sk_workspace_bytes(); the launch falls back to fixed splits where
  // the stream-K kernel does not apply.
  bool stream_k = false;
};
int launch_decode(const seer_dims& d, const DecodeArgs& a, void* stream);

// Causal prefill attention with the fused ground truth (prefill.hip).
struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* seq_lens;
  float scale;
  void* workspace;  // prefill_workspace_bytes(d)
  uint16_t* out;
  float* lse;
  float* gt;        // or nullptr (attention only)
};
// Prefill workspace: V^T [B, H_kv, d, Lpad] bf16 (rounded up to 256 bytes),
// then the row maxima [B, H_q, NBmax, Lpad] float32; Lpad = Lmax rounded
// up to kPrefillTokenTile.
int64_t prefill_padded_len(const seer_dims* d);
size_t prefill_vt_bytes(const seer_dims* d);
size_t prefill_workspace_bytes(const seer_dims* d);
int launch_prefill(const seer_dims& d, const PrefillArgs& a, void* stream);

// Waves per decode workgroup chosen automatically.
// Waves per decode workgroup (8 or 4) and whether nw waves fit the LDS
// budget of the wave merge.
int decode_waves_per_group(int g, int head_dim);
bool decode_waves_fit(int nw, int g, int head_dim);

// Device query (HIP): compute units of the current device, cached.
int device_cu_count(int* out);

}  // namespace seer
