// Host-only stand-ins for the kernel launchers of the HIP library, so that the C ABI's
// argument checking and marshalling (csrc/api.cpp) can be built with g++ and the address
// and undefined-behaviour sanitizers, and run without a GPU. Each launcher records the
// parameters it was given and launches nothing.
#include <string.h>

#include "internal.hpp"

namespace attn_stub {
attn::FwdParams last_fwd;
attn::BwdParams last_bwd;
attn::DecodeParams last_decode;
int launches = 0;
}  // namespace attn_stub

extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "hipError"; }

namespace attn {
static unsigned char fake_scratch[256];

hipError_t launch_fwd(const FwdParams& p, int, int, hipStream_t) {
  attn_stub::last_fwd = p;
  ++attn_stub::launches;
  return hipSuccess;
}
hipError_t launch_fwd_paged(const FwdParams& p, int, int, hipStream_t) {
  attn_stub::last_fwd = p;
  ++attn_stub::launches;
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const FwdParams& p, int, hipStream_t) {
  attn_stub::last_fwd = p;
  ++attn_stub::launches;
  return hipSuccess;
}
int fwd_block_rows(int dtype, int head_dim, int64_t, int64_t) { return dtype == 0 ? 128 : (head_dim == 128 ? 256 : 256); }
int fwd_paged_block_rows(int) { return 256; }
int fwd_fp8_block_rows() { return 128; }
hipError_t launch_gather_kv_pages(const void*, const void*, const int32_t*, const int32_t*, void*, void*, int, int, int,
                                  int, hipStream_t) {
  ++attn_stub::launches;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdParams& p, int, int, hipStream_t) {
  attn_stub::last_bwd = p;
  ++attn_stub::launches;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeParams& p, int, int, hipStream_t) {
  attn_stub::last_decode = p;
  ++attn_stub::launches;
  return hipSuccess;
}
// the cooperative decode kernel's residency for fp8 KV with an even Hkv and at most 16
// query heads per KV head (two 64 KiB workgroups per CU at Hkv 8), none otherwise
int decode_coop_slots_per_cu(int kv_dtype, int num_q_heads, int num_kv_heads) {
  if (kv_dtype != 3 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  const int co = (num_kv_heads & -num_kv_heads) < 8 ? (num_kv_heads & -num_kv_heads) : 8;
  if (num_q_heads / num_kv_heads > 16 || co < 2) return 0;
  const int by_lds = 160 * 1024 / (2 * co * 2 * 16 * 128);
  return by_lds < 32 / co ? by_lds : 32 / co;
}
int device_cus() { return 256; }
hipError_t decode_scratch(void** ptr) {
  *ptr = fake_scratch;
  return hipSuccess;
}
hipError_t launch_probe_mfma(const uint32_t*, int, int, int, uint64_t*, float*, hipStream_t) {
  ++attn_stub::launches;
  return hipSuccess;
}
hipError_t launch_probe_hbm_read(const void*, int64_t, int, uint32_t*, hipStream_t) {
  ++attn_stub::launches;
  return hipSuccess;
}
hipError_t launch_flush(void*, int64_t, hipStream_t) {
  ++attn_stub::launches;
  return hipSuccess;
}
}  // namespace attn
