// Drives every entry point of the C ABI (include/attn.h) through its argument checks and
// parameter marshalling, on the host only: built with g++ and the address and
// undefined-behaviour sanitizers against csrc/api.cpp and the stand-in launchers of
// stubs.cpp. Prints "ALL OK" and exits 0 when every expectation holds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"
#include "internal.hpp"

namespace attn_stub {
extern attn::FwdParams last_fwd;
extern attn::BwdParams last_bwd;
extern attn::DecodeParams last_decode;
extern int launches;
}  // namespace attn_stub

static int failures = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      ++failures;                                                                 \
      fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", __FILE__, \
              __LINE__, #cond, attn_last_error_message());                        \
    }                                                                             \
  } while (0)

static void* const P = reinterpret_cast<void*>(0x100000);  // never dereferenced (aligned)
static void* const MIS = reinterpret_cast<void*>(0x100008);  // 8-byte aligned only

static attn_fwd_args_t fwd_args(int32_t dtype, int32_t d, int32_t b, int32_t hq, int32_t hkv, int32_t n) {
  attn_fwd_args_t a;
  memset(&a, 0, sizeof a);
  a.batch = b;
  a.num_q_heads = hq;
  a.num_kv_heads = hkv;
  a.seqlen_q = n;
  a.seqlen_k = n;
  a.head_dim = d;
  a.dtype = dtype;
  for (int i = 0; i < 3; ++i) {
    const int64_t qs[3] = {(int64_t)hq * n * d, (int64_t)n * d, d};
    const int64_t ks[3] = {(int64_t)hkv * n * d, (int64_t)n * d, d};
    a.q_stride[i] = qs[i];
    a.o_stride[i] = qs[i];
    a.k_stride[i] = ks[i];
    a.v_stride[i] = ks[i];
  }
  a.q_scale = a.k_scale = a.v_scale = 1.0f;
  return a;
}

static void test_fwd() {
  attn_fwd_args_t a = fwd_args(ATTN_BF16, 128, 2, 8, 2, 1000);
  int before = attn_stub::launches;
  EXPECT(attn_fwd(&a, P, P, P, P, nullptr, nullptr) == ATTN_SUCCESS);
  EXPECT(attn_stub::launches == before + 1);
  EXPECT(attn_stub::last_fwd.group == 4);
  EXPECT(attn_stub::last_fwd.q_tiles == 4);  // ceil(1000 / 256)
  EXPECT(fabsf(attn_stub::last_fwd.scale_log2 - (float)(1.4426950408889634 / sqrt(128.0))) < 1e-6f);
  // causal with a window, softcap and LSE
  a.causal = 1;
  a.window = 64;
  a.softcap = 30.0f;
  EXPECT(attn_fwd(&a, P, P, P, P, (float*)P, nullptr) == ATTN_SUCCESS);
  EXPECT(attn_stub::last_fwd.cap_out > 0.0f);
  // failures: each leaves a message and launches nothing
  before = attn_stub::launches;
  attn_fwd_args_t bad = a;
  bad.window = 16;
  bad.causal = 0;
  EXPECT(attn_fwd(&bad, P, P, P, P, nullptr, nullptr) == ATTN_ERROR_INVALID_VALUE);
  EXPECT(strlen(attn_last_error_message()) > 0);
  bad = a;
  bad.num_q_heads = 7;  // not a multiple of num_kv_heads (2)
  EXPECT(attn_fwd(&bad, P, P, P, P, nullptr, nullptr) == ATTN_ERROR_INVALID_VALUE);
  bad = a;
  bad.head_dim = 80;
  EXPECT(attn_fwd(&bad, P, P, P, P, nullptr, nullptr) == ATTN_ERROR_NOT_SUPPORTED);
  EXPECT(attn_fwd(&a, MIS, P, P, P, nullptr, nullptr) == ATTN_ERROR_NOT_SUPPORTED);
  EXPECT(attn_fwd(&a, nullptr, P, P, P, nullptr, nullptr) == ATTN_ERROR_INVALID_VALUE);
  EXPECT(attn_fwd(nullptr, P, P, P, P, nullptr, nullptr) == ATTN_ERROR_INVALID_VALUE);
  bad = a;
  bad.q_stride[1] = 7;  // not 16-byte granular
  EXPECT(attn_fwd(&bad, P, P, P, P, nullptr, nullptr) != ATTN_SUCCESS);
  bad = a;
  bad.softmax_scale = NAN;
  EXPECT(attn_fwd(&bad, P, P, P, P, nullptr, nullptr) != ATTN_SUCCESS);
  EXPECT(attn_stub::launches == before);
  // ragged batches and fp8 / fp32 inputs
  attn_fwd_args_t r = fwd_args(ATTN_F16, 64, 3, 4, 4, 300);
  r.cu_seqlens_q = (const int32_t*)P;
  r.cu_seqlens_k = (const int32_t*)P;
  r.q_stride[0] = r.k_stride[0] = r.v_stride[0] = r.o_stride[0] = 0;
  r.q_stride[1] = r.k_stride[1] = r.v_stride[1] = r.o_stride[1] = 64;
  r.q_stride[2] = r.k_stride[2] = r.v_stride[2] = r.o_stride[2] = 4 * 64;
  EXPECT(attn_fwd(&r, P, P, P, P, (float*)P, nullptr) == ATTN_SUCCESS);
  attn_fwd_args_t f8 = fwd_args(ATTN_FP8_E4M3, 128, 1, 4, 4, 512);
  f8.q_scale = 0.5f;
  EXPECT(attn_fwd(&f8, P, P, P, P, nullptr, nullptr) == ATTN_SUCCESS);
  f8.v_scale = 0.0f;
  EXPECT(attn_fwd(&f8, P, P, P, P, nullptr, nullptr) == ATTN_ERROR_INVALID_VALUE);
  attn_fwd_args_t f32 = fwd_args(ATTN_F32, 32, 2, 4, 4, 64);
  EXPECT(attn_fwd(&f32, P, P, P, P, (float*)P, nullptr) == ATTN_SUCCESS);
}

static void test_paged_prefill() {
  attn_fwd_paged_args_t a;
  memset(&a, 0, sizeof a);
  a.num_seqs = 8;
  a.num_q_heads = 32;
  a.num_kv_heads = 8;
  a.head_dim = 128;
  a.page_size = 16;
  a.max_pages_per_seq = 1024;
  a.num_pages = 5000;
  a.max_seqlen_q = 2048;
  a.dtype = ATTN_BF16;
  a.causal = 1;
  const size_t ws = attn_fwd_paged_workspace_size(&a);
  EXPECT(ws == (size_t)8 * 1024 * 16 * 8 * 128 * 2 * 2);
  EXPECT(attn_fwd_paged(&a, P, P, P, (const int32_t*)P, (const int32_t*)P, (const int32_t*)P, P, nullptr, P, ws,
                        nullptr) == ATTN_SUCCESS);
  EXPECT(attn_fwd_paged(&a, P, P, P, (const int32_t*)P, (const int32_t*)P, (const int32_t*)P, P, nullptr, nullptr, 0,
                        nullptr) == ATTN_SUCCESS);
  EXPECT(attn_fwd_paged(&a, P, P, P, (const int32_t*)P, (const int32_t*)P, (const int32_t*)P, P, nullptr, P, ws - 1,
                        nullptr) == ATTN_ERROR_WORKSPACE_TOO_SMALL);
  a.page_size = 32;
  EXPECT(attn_fwd_paged_workspace_size(&a) == 0);
  EXPECT(attn_fwd_paged(&a, P, P, P, (const int32_t*)P, (const int32_t*)P, (const int32_t*)P, P, nullptr, nullptr, 0,
                        nullptr) != ATTN_SUCCESS);
}

static void test_bwd() {
  attn_bwd_args_t a;
  memset(&a, 0, sizeof a);
  a.batch = 1;
  a.num_q_heads = 32;
  a.num_kv_heads = 8;
  a.seqlen_q = 4096;
  a.seqlen_k = 4096;
  a.head_dim = 128;
  a.dtype = ATTN_BF16;
  a.causal = 1;
  const size_t ws = attn_bwd_workspace_size(&a);
  EXPECT(ws > 0);
  EXPECT(attn_bwd(&a, P, P, P, P, P, (const float*)P, P, P, P, P, ws, nullptr) == ATTN_SUCCESS);
  EXPECT(attn_stub::last_bwd.group == 4);
  EXPECT(attn_bwd(&a, P, P, P, P, P, (const float*)P, P, P, P, P, ws - 16, nullptr) == ATTN_ERROR_WORKSPACE_TOO_SMALL);
  a.head_dim = 96;
  EXPECT(attn_bwd_workspace_size(&a) == 0);
  EXPECT(attn_bwd(&a, P, P, P, P, P, (const float*)P, P, P, P, P, ws, nullptr) != ATTN_SUCCESS);
}

static attn_decode_args_t dec_args() {
  attn_decode_args_t a;
  memset(&a, 0, sizeof a);
  a.num_seqs = 64;
  a.num_q_heads = 32;
  a.num_kv_heads = 8;
  a.head_dim = 128;
  a.page_size = 16;
  a.max_pages_per_seq = 2048;
  a.max_seq_len = 32768;
  a.q_dtype = ATTN_BF16;
  a.kv_dtype = ATTN_BF16;
  return a;
}

static void test_decode() {
  attn_decode_args_t a = dec_args();
  int32_t len = 0, n = 0;
  EXPECT(attn_decode_plan(&a, &len, &n) == ATTN_SUCCESS);
  EXPECT(len == 1024 && n == 32);
  const size_t ws = attn_decode_paged_workspace_size(&a);
  EXPECT(ws == (size_t)64 * 32 * n * 128 * 4 + (size_t)64 * 32 * n * 4);
  EXPECT(attn_decode_paged(&a, P, P, P, nullptr, nullptr, (const int32_t*)P, (const int32_t*)P, P, (float*)P, P, ws,
                           nullptr) == ATTN_SUCCESS);
  EXPECT(attn_stub::last_decode.split_len == 1024 && attn_stub::last_decode.max_splits == 32);
  EXPECT(attn_stub::last_decode.part_lse == attn_stub::last_decode.part_o + (size_t)64 * 32 * 32 * 128);
  EXPECT(attn_decode_paged(&a, P, P, P, nullptr, nullptr, (const int32_t*)P, (const int32_t*)P, P, nullptr, P, ws - 1,
                           nullptr) == ATTN_ERROR_WORKSPACE_TOO_SMALL);
  // the allocation-free form: the same plan, partials in the library's scratch
  EXPECT(attn_decode_paged_noalloc(&a, P, P, P, nullptr, nullptr, (const int32_t*)P, (const int32_t*)P, P, nullptr,
                                   nullptr) == ATTN_SUCCESS);
  attn_decode_args_t big = a;
  big.num_seqs = 512;
  EXPECT(attn_decode_paged_noalloc(&big, P, P, P, nullptr, nullptr, (const int32_t*)P, (const int32_t*)P, P, nullptr,
                                   nullptr) == ATTN_ERROR_WORKSPACE_TOO_SMALL);
  // fp8 KV needs both scales
  attn_decode_args_t f8 = a;
  f8.kv_dtype = ATTN_FP8_E4M3;
  EXPECT(attn_decode_paged(&f8, P, P, P, nullptr, nullptr, (const int32_t*)P, (const int32_t*)P, P, nullptr, P,
                           attn_decode_paged_workspace_size(&f8), nullptr) == ATTN_ERROR_INVALID_VALUE);
  EXPECT(attn_decode_paged(&f8, P, P, P, (const float*)P, (const float*)P, (const int32_t*)P, (const int32_t*)P, P,
                           nullptr, P, attn_decode_paged_workspace_size(&f8), nullptr) == ATTN_SUCCESS);
  // forced splits, and bad arguments
  for (int s : {1, 2, 7, 9, 31, 313}) {
    attn_decode_args_t f = a;
    f.num_splits = s;
    EXPECT(attn_decode_plan(&f, &len, &n) == ATTN_SUCCESS);
    EXPECT(len % 16 == 0 && len <= 4096 && (int64_t)len * n >= f.max_seq_len);
  }
  attn_decode_args_t bad = a;
  bad.num_q_heads = 30;
  EXPECT(attn_decode_plan(&bad, &len, &n) == ATTN_ERROR_INVALID_VALUE);
  bad = a;
  bad.max_seq_len = 40000;
  EXPECT(attn_decode_paged_workspace_size(&bad) == 0);
  EXPECT(attn_decode_paged(&a, nullptr, P, P, nullptr, nullptr, (const int32_t*)P, (const int32_t*)P, P, nullptr, P,
                           ws, nullptr) == ATTN_ERROR_INVALID_VALUE);
}

static void test_probes_and_strings() {
  EXPECT(attn_probe_mfma((const uint32_t*)P, 256, 10, 0, (uint64_t*)P, (float*)P, nullptr) == ATTN_SUCCESS);
  EXPECT(attn_probe_mfma((const uint32_t*)P, 0, 10, 0, (uint64_t*)P, (float*)P, nullptr) != ATTN_SUCCESS);
  EXPECT(attn_probe_hbm_read(P, (size_t)32768 * 64, 64, (uint32_t*)P, nullptr) == ATTN_SUCCESS);
  EXPECT(attn_probe_hbm_read(P, 1000, 64, (uint32_t*)P, nullptr) != ATTN_SUCCESS);
  EXPECT(attn_flush_caches(P, 1 << 20, nullptr) == ATTN_SUCCESS);
  EXPECT(attn_flush_caches(P, 15, nullptr) != ATTN_SUCCESS);
  EXPECT(strcmp(attn_status_string(ATTN_SUCCESS), "ATTN_SUCCESS") == 0);
  EXPECT(strcmp(attn_status_string((attn_status_t)99), "ATTN_STATUS_UNKNOWN") == 0);
  EXPECT(attn_abi_version() == 100);
}

int main() {
  test_fwd();
  test_paged_prefill();
  test_bwd();
  test_decode();
  test_probes_and_strings();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("ALL OK\n");
  return 0;
}
