// CPU-only checks of the HIP-free argument checks of libseer
// (block_sparse_attention_seer_amd/csrc/seer_checks.cpp), built with g++ and
// the host sanitizers by tests/test_abi_host.py.  Exit status 0 = all pass.
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../block_sparse_attention_seer_amd/csrc/seer_internal.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static seer_dims good() {
  seer_dims d{};
  d.batch = 16;
  d.num_q_heads = 40;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.d_gate = 128;
  d.block_size = 64;
  d.max_seq_len = 32768;
  d.reserved = 0;
  d.kv_stride_t = 128;
  d.kv_stride_h = 32768LL * 128;
  d.kv_stride_b = 8LL * 32768 * 128;
  return d;
}

int main() {
  std::string why;
  seer_dims d = good();
  EXPECT(seer::check_dims(&d, &why) == SEER_OK);
  EXPECT(seer::check_dims(nullptr, &why) == SEER_ERR_INVALID_ARG);

  d = good(); d.num_q_heads = 41;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_INVALID_ARG);
  d = good(); d.num_q_heads = 8 * 17;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_UNSUPPORTED);
  d = good(); d.head_dim = 96;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_UNSUPPORTED);
  d = good(); d.d_gate = 32;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_UNSUPPORTED);
  d = good(); d.block_size = 32;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_UNSUPPORTED);
  d = good(); d.batch = 0;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_INVALID_ARG);
  d = good(); d.kv_stride_t = 100;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_INVALID_ARG);
  d = good(); d.kv_stride_t = 136;
  EXPECT(seer::check_dims(&d, &why) == SEER_OK);
  d = good(); d.kv_stride_t = 132;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_INVALID_ARG);
  d = good(); d.reserved = 1;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_INVALID_ARG);
  d = good(); d.max_seq_len = 1 << 24;
  EXPECT(seer::check_dims(&d, &why) == SEER_ERR_UNSUPPORTED);

  EXPECT(seer::check_ptr(nullptr, 16, "x", &why) == SEER_ERR_INVALID_ARG);
  EXPECT(seer::check_ptr(reinterpret_cast<void*>(0x1008), 16, "x", &why) == SEER_ERR_INVALID_ARG);
  EXPECT(seer::check_ptr(reinterpret_cast<void*>(0x1010), 16, "x", &why) == SEER_OK);

  d = good();
  EXPECT(seer::nb_max(&d) == 512);
  d.max_seq_len = 32769;
  EXPECT(seer::nb_max(&d) == 513);
  d = good();
  EXPECT(seer::gate_workspace_bytes(&d) == 16u * 8 * 128 * 4);
  // one split needs no workspace; otherwise counters + lse (each 256-aligned) + o
  EXPECT(seer::decode_workspace_bytes(128, 1, 5, 128) == 0);
  const size_t ws = seer::decode_workspace_bytes(128, 4, 5, 128);
  EXPECT(ws == 512 + 10240 + 128u * 4 * 5 * 128 * 4);
  EXPECT(seer::decode_workspace_bytes(3, 2, 1, 64) == 256 + 256 + 3u * 2 * 64 * 4);
  // automatic split: 8-wave workgroups when their wave merge fits 48 KiB of
  // LDS (else 4), about 8 waves per compute unit in total, no more splits
  // than leave a 64-token chunk per wave
  EXPECT(seer::decode_waves_per_group(5, 128) == 8);
  EXPECT(seer::decode_waves_per_group(12, 128) == 8);  // 48 KiB
  EXPECT(seer::decode_waves_per_group(13, 128) == 4);
  EXPECT(seer::decode_waves_per_group(16, 64) == 8);
  EXPECT(!seer::decode_waves_fit(8, 13, 128) && seer::decode_waves_fit(4, 13, 128));
  EXPECT(seer::auto_num_split(&d, 53, 256) == 2);      // 128 pairs x 2 x 8 waves
  seer_dims one = good();
  one.batch = 1;
  EXPECT(seer::auto_num_split(&one, 65, 256) == 8);    // 65 chunks: 8 per split
  EXPECT(seer::auto_num_split(&one, 3, 256) == 1);     // too few chunks to split
  seer_dims wide = good();
  wide.num_q_heads = 128;                              // g = 16: 4-wave groups
  EXPECT(seer::auto_num_split(&wide, 53, 256) == 4);

  if (failures == 0) std::printf("abi host checks: all passed\n");
  return failures == 0 ? 0 : 1;
}
