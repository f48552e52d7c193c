// C ABI of the attention library: argument validation, routing, split planning and
// launch. Every check runs on the host before any HIP call; nothing here allocates,
// copies or synchronises, so a call costs one or two kernel launches.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "../../include/attn.h"
#include "internal.hpp"

static_assert(ATTN_DECODE_NOALLOC_MAX_WORKSPACE == attn::kDecodeScratchBytes,
              "the header states the scratch size the library is built with");

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

attn_status_t ok() {
  g_last_error.clear();
  return ATTN_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) {
  switch (dtype) {
    case ATTN_F32: return 4;
    case ATTN_F16: return 2;
    case ATTN_BF16: return 2;
    case ATTN_FP8_E4M3: return 1;
    default: return 0;
  }
}

// head dims with a prefill kernel: 16-bit inputs 32, 64, 96, 128, 192, 256; fp32 32, 64, 128
bool head_dim_ok(int d, bool sixteen_bit) {
  if (d == 32 || d == 64 || d == 128) return true;
  return sixteen_bit && (d == 96 || d == 192 || d == 256);
}

float resolve_scale(float s, int head_dim) {
  return s > 0.0f ? s : (float)(1.0 / sqrt((double)head_dim));
}

constexpr double kLog2eD = 1.4426950408889634;
constexpr int kPageSize = 16;
constexpr int kMaxSplitTokens = 4096;

attn_status_t check_strides(const char* name, const int64_t st[3], int esize, int64_t min_token) {
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(ATTN_ERROR_INVALID_VALUE, "%s_stride[%d] is negative", name, i);
    if ((st[i] * esize) % 16 != 0)
      return fail(ATTN_ERROR_NOT_SUPPORTED, "%s_stride[%d]=%lld elements is not a multiple of 16 bytes",
                  name, i, (long long)st[i]);
  }
  if (st[2] >= (int64_t)1 << 24)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "%s token stride %lld is 2^24 elements or more", name,
                (long long)st[2]);
  if (st[2] < min_token)
    return fail(ATTN_ERROR_INVALID_VALUE, "%s token stride %lld is smaller than head_dim", name,
                (long long)st[2]);
  return ATTN_SUCCESS;
}

}  // namespace

extern "C" {

int32_t attn_abi_version(void) { return 100; }

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_SUCCESS: return "ATTN_SUCCESS";
    case ATTN_ERROR_INVALID_VALUE: return "ATTN_ERROR_INVALID_VALUE";
    case ATTN_ERROR_NOT_SUPPORTED: return "ATTN_ERROR_NOT_SUPPORTED";
    case ATTN_ERROR_WORKSPACE_TOO_SMALL: return "ATTN_ERROR_WORKSPACE_TOO_SMALL";
    case ATTN_ERROR_LAUNCH_FAILED: return "ATTN_ERROR_LAUNCH_FAILED";
    default: return "ATTN_STATUS_UNKNOWN";
  }
}

const char* attn_last_error_message(void) { return g_last_error.c_str(); }

attn_status_t attn_fwd(const attn_fwd_args_t* a, const void* q, const void* k, const void* v, void* o,
                       float* lse, void* stream) {
  if (a == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "args is NULL");
  if (a->batch < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(ATTN_ERROR_INVALID_VALUE, "batch, num_q_heads and num_kv_heads must be >= 1");
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(ATTN_ERROR_INVALID_VALUE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (a->seqlen_q < 0 || a->seqlen_k < 0)
    return fail(ATTN_ERROR_INVALID_VALUE, "sequence lengths must be >= 0");
  if (a->dtype != ATTN_F32 && a->dtype != ATTN_F16 && a->dtype != ATTN_BF16 && a->dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "dtype %d is not F32, F16, BF16 or FP8_E4M3", a->dtype);
  const bool fp8 = a->dtype == ATTN_FP8_E4M3;
  if (fp8 ? a->head_dim != 128 : !head_dim_ok(a->head_dim, a->dtype != ATTN_F32))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "head_dim %d is not one of %s", a->head_dim,
                fp8 ? "128" : a->dtype != ATTN_F32 ? "32, 64, 96, 128, 192, 256" : "32, 64, 128");
  if (fp8 && a->cu_seqlens_q != nullptr)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "fp8 inputs take dense batches only");
  if (fp8 && !(a->q_scale > 0.0f && a->k_scale > 0.0f && a->v_scale > 0.0f && !isinf(a->q_scale) &&
               !isinf(a->k_scale) && !isinf(a->v_scale)))
    return fail(ATTN_ERROR_INVALID_VALUE, "fp8 inputs need finite q_scale, k_scale and v_scale > 0");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  if (a->window > 0 && !a->causal)
    return fail(ATTN_ERROR_INVALID_VALUE, "a sliding window requires causal = 1");
  if (!(a->softcap == a->softcap) || !(a->softmax_scale == a->softmax_scale) || isinf(a->softcap) ||
      isinf(a->softmax_scale))
    return fail(ATTN_ERROR_INVALID_VALUE, "softcap and softmax_scale must be finite");
  if ((a->cu_seqlens_q == nullptr) != (a->cu_seqlens_k == nullptr))
    return fail(ATTN_ERROR_INVALID_VALUE, "cu_seqlens_q and cu_seqlens_k must both be set or both NULL");
  if (a->num_q_heads > 65535 || a->batch > 65535)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_q_heads and batch are limited to 65535");
  if (a->seqlen_q == 0) return ok();  // nothing to compute
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return fail(ATTN_ERROR_INVALID_VALUE, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "q, k, v and o must be 16-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(ATTN_ERROR_INVALID_VALUE, "lse must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(a->sinks) & 3u) return fail(ATTN_ERROR_INVALID_VALUE, "sinks must be 4-byte aligned");
  const int es = elem_size(a->dtype);
  attn_status_t st;
  if ((st = check_strides("q", a->q_stride, es, a->head_dim)) != ATTN_SUCCESS) return st;
  if ((st = check_strides("k", a->k_stride, es, a->head_dim)) != ATTN_SUCCESS) return st;
  if ((st = check_strides("v", a->v_stride, es, a->head_dim)) != ATTN_SUCCESS) return st;
  if ((st = check_strides("o", a->o_stride, fp8 ? 2 : es, a->head_dim)) != ATTN_SUCCESS) return st;

  attn::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = a->q_stride[i];
    p.ks[i] = a->k_stride[i];
    p.vs[i] = a->v_stride[i];
    p.os[i] = a->o_stride[i];
  }
  p.batch = a->batch;
  p.hq = a->num_q_heads;
  p.hkv = a->num_kv_heads;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.nq = a->seqlen_q;
  p.nk = a->seqlen_k;
  p.causal = a->causal;
  p.window = a->window > 0 ? a->window : 0;
  // fp8: the Q and K scales multiply the scores (folded into the exponent's scale), the V
  // scale the output (folded into the normalisation)
  const double scale = resolve_scale(a->softmax_scale, a->head_dim) *
                       (fp8 ? (double)a->q_scale * (double)a->k_scale : 1.0);
  p.scale_log2 = (float)(scale * kLog2eD);
  if (a->softcap > 0.0f) {
    p.cap_in = (float)(scale / (double)a->softcap);
    p.cap_out = (float)((double)a->softcap * kLog2eD);
  } else {
    p.cap_in = 0.0f;
    p.cap_out = 0.0f;
  }
  p.o_scale = fp8 ? a->v_scale : 1.0f;
  const int bm = fp8 ? attn::fwd_fp8_block_rows()
                     : attn::fwd_block_rows(a->dtype, a->head_dim, a->seqlen_q, (int64_t)a->batch * a->num_q_heads);
  p.q_tiles = (a->seqlen_q + bm - 1) / bm;
  p.sinks = a->sinks;

  hipError_t e = fp8 ? attn::launch_fwd_fp8(p, a->head_dim, static_cast<hipStream_t>(stream))
                     : attn::launch_fwd(p, a->dtype, a->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

static attn_status_t check_fwd_paged_args(const attn_fwd_paged_args_t* a) {
  if (a == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "args is NULL");
  if (a->num_seqs < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(ATTN_ERROR_INVALID_VALUE, "num_seqs, num_q_heads and num_kv_heads must be >= 1");
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(ATTN_ERROR_INVALID_VALUE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (!head_dim_ok(a->head_dim, true))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "head_dim %d is not one of 32, 64, 96, 128, 192, 256", a->head_dim);
  if (a->dtype != ATTN_F16 && a->dtype != ATTN_BF16)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "dtype %d is not F16 or BF16", a->dtype);
  if (a->page_size != kPageSize) return fail(ATTN_ERROR_NOT_SUPPORTED, "page_size must be 16");
  if (a->max_pages_per_seq < 1 || a->num_pages < 1)
    return fail(ATTN_ERROR_INVALID_VALUE, "max_pages_per_seq and num_pages must be >= 1");
  if (a->max_pages_per_seq > (1 << 26))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "max_pages_per_seq is limited to 2^26");
  if (a->max_seqlen_q < 0) return fail(ATTN_ERROR_INVALID_VALUE, "max_seqlen_q must be >= 0");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  if (a->window > 0 && !a->causal)
    return fail(ATTN_ERROR_INVALID_VALUE, "a sliding window requires causal = 1");
  if (!(a->softcap == a->softcap) || !(a->softmax_scale == a->softmax_scale) || isinf(a->softcap) ||
      isinf(a->softmax_scale))
    return fail(ATTN_ERROR_INVALID_VALUE, "softcap and softmax_scale must be finite");
  if (a->num_q_heads > 65535 || a->num_seqs > 65535)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_q_heads and num_seqs are limited to 65535");
  if ((int64_t)a->num_kv_heads * a->head_dim >= (int64_t)1 << 24)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_kv_heads * head_dim must be below 2^24");
  if ((int64_t)a->num_q_heads * a->head_dim >= (int64_t)1 << 24)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_q_heads * head_dim must be below 2^24");
  if (reinterpret_cast<uintptr_t>(a->sinks) & 3u) return fail(ATTN_ERROR_INVALID_VALUE, "sinks must be 4-byte aligned");
  return ATTN_SUCCESS;
}

// The gathered-key route (head_dim 128): the workspace holds K and V of every sequence in a
// slot of max_pages_per_seq * page_size tokens each.
static size_t fwd_paged_gather_bytes(const attn_fwd_paged_args_t* a) {
  if (a->head_dim != 128) return 0;
  const size_t half = (size_t)a->num_seqs * a->max_pages_per_seq * kPageSize * a->num_kv_heads * a->head_dim *
                      (size_t)elem_size(a->dtype);
  return 2 * ((half + 255) & ~(size_t)255);
}

size_t attn_fwd_paged_workspace_size(const attn_fwd_paged_args_t* a) {
  if (check_fwd_paged_args(a) != ATTN_SUCCESS) return 0;
  return fwd_paged_gather_bytes(a);
}

attn_status_t attn_fwd_paged(const attn_fwd_paged_args_t* a, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table, const int32_t* cu_seqlens_q,
                             const int32_t* seq_lens_k, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  attn_status_t st0 = check_fwd_paged_args(a);
  if (st0 != ATTN_SUCCESS) return st0;
  const size_t need = fwd_paged_gather_bytes(a);
  const bool gather = workspace != nullptr && need > 0;
  if (gather && workspace_bytes < need)
    return fail(ATTN_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need);
  if (gather && (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(ATTN_ERROR_INVALID_VALUE, "workspace must be 256-byte aligned");
  if (gather && (int64_t)a->num_seqs * a->max_pages_per_seq * kPageSize >= ((int64_t)1 << 31))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_seqs * max_pages_per_seq * page_size must be below 2^31");
  if (a->max_seqlen_q == 0) return ok();  // nothing to compute
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || o == nullptr || block_table == nullptr ||
      cu_seqlens_q == nullptr || seq_lens_k == nullptr)
    return fail(ATTN_ERROR_INVALID_VALUE,
                "q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "q, k_cache, v_cache and o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens_k) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(ATTN_ERROR_INVALID_VALUE, "block_table, cu_seqlens_q, seq_lens_k and lse must be 4-byte aligned");

  const int64_t D = a->head_dim, tok_k = (int64_t)a->num_kv_heads * D, tok_q = (int64_t)a->num_q_heads * D;
  attn::FwdParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o = o;
  p.lse = lse;
  p.cu_q = cu_seqlens_q;
  p.cu_k = nullptr;
  p.qs[0] = 0, p.qs[1] = D, p.qs[2] = tok_q;
  p.os[0] = 0, p.os[1] = D, p.os[2] = tok_q;
  p.ks[0] = kPageSize * tok_k, p.ks[1] = D, p.ks[2] = tok_k;
  p.vs[0] = kPageSize * tok_k, p.vs[1] = D, p.vs[2] = tok_k;
  p.batch = a->num_seqs;
  p.hq = a->num_q_heads;
  p.hkv = a->num_kv_heads;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.nq = a->max_seqlen_q;
  p.nk = a->max_pages_per_seq * kPageSize;
  p.causal = a->causal;
  p.window = a->window > 0 ? a->window : 0;
  const double scale = resolve_scale(a->softmax_scale, a->head_dim);
  p.scale_log2 = (float)(scale * kLog2eD);
  if (a->softcap > 0.0f) {
    p.cap_in = (float)(scale / (double)a->softcap);
    p.cap_out = (float)((double)a->softcap * kLog2eD);
  }
  const int bm = attn::fwd_paged_block_rows(a->head_dim);
  p.q_tiles = (a->max_seqlen_q + bm - 1) / bm;
  p.block_table = block_table;
  p.seq_lens_k = seq_lens_k;
  p.max_pages = a->max_pages_per_seq;
  p.num_pages = a->num_pages;
  p.sinks = a->sinks;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (gather) {
    // pages -> per-sequence slots, then the ragged kernel reads the slots
    char* wk = static_cast<char*>(workspace);
    char* wv = wk + need / 2;
    e = attn::launch_gather_kv_pages(k_cache, v_cache, block_table, seq_lens_k, wk, wv, a->num_seqs,
                                     a->max_pages_per_seq, a->num_pages,
                                     (int)(kPageSize * tok_k * elem_size(a->dtype)), hs);
    if (e == hipSuccess) {
      p.k = wk;
      p.v = wv;
      p.ks[0] = p.vs[0] = 0;
      p.block_table = nullptr;
      const int bm = attn::fwd_block_rows(a->dtype, a->head_dim, a->max_seqlen_q, (int64_t)a->num_seqs * a->num_q_heads);
      p.q_tiles = (a->max_seqlen_q + bm - 1) / bm;
      e = attn::launch_fwd(p, a->dtype, a->head_dim, hs);
    }
  } else {
    e = attn::launch_fwd_paged(p, a->dtype, a->head_dim, hs);
  }
  if (e != hipSuccess)
    return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

static attn_status_t check_bwd_args(const attn_bwd_args_t* a) {
  if (a == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "args is NULL");
  if (a->batch < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(ATTN_ERROR_INVALID_VALUE, "batch, num_q_heads and num_kv_heads must be >= 1");
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(ATTN_ERROR_INVALID_VALUE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (a->seqlen_q < 0 || a->seqlen_k < 1)
    return fail(ATTN_ERROR_INVALID_VALUE, "seqlen_q must be >= 0 and seqlen_k >= 1");
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "backward head_dim %d is not 64 or 128", a->head_dim);
  if (a->seqlen_q > 65535 * 128 || a->seqlen_k > (1 << 24))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "backward sequence lengths are limited to 8388480 / 2^24");
  if (a->dtype != ATTN_F16 && a->dtype != ATTN_BF16)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "backward dtype %d is not F16 or BF16", a->dtype);
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  if (a->window > 0 && !a->causal)
    return fail(ATTN_ERROR_INVALID_VALUE, "a sliding window requires causal = 1");
  if (!(a->softcap == a->softcap) || !(a->softmax_scale == a->softmax_scale) || isinf(a->softcap) ||
      isinf(a->softmax_scale))
    return fail(ATTN_ERROR_INVALID_VALUE, "softcap and softmax_scale must be finite");
  if (a->num_q_heads > 65535 || a->batch > 65535)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_q_heads and batch are limited to 65535");
  return ATTN_SUCCESS;
}

// Delta [B, Hq, Nq] and LSE2 [B, Hq, Nq] (each rounded up to 256 bytes), then fp32 dK and
// dV [chunks][B, Hkv, Nk, D] (a multiple of 256 bytes), then the int32 run order of the
// dK / dV items
static size_t bwd_delta_bytes(const attn_bwd_args_t* a) {
  return ((size_t)a->batch * a->num_q_heads * (size_t)a->seqlen_q * sizeof(float) + 255) & ~(size_t)255;
}

static size_t bwd_partial_bytes(const attn_bwd_args_t* a, int chunks) {
  return 2 * (size_t)chunks * a->batch * a->num_kv_heads * (size_t)a->seqlen_k * a->head_dim * sizeof(float);
}

// Sized for the largest split (kBwdMaxChunks), whatever the mask: the same buffer serves a
// causal and a full call of the same shapes.
size_t attn_bwd_workspace_size(const attn_bwd_args_t* a) {
  if (check_bwd_args(a) != ATTN_SUCCESS) return 0;
  return 2 * bwd_delta_bytes(a) + bwd_partial_bytes(a, attn::kBwdMaxChunks) +
         (size_t)attn::bwd_order_entries(a->seqlen_k, attn::kBwdMaxChunks) * sizeof(int32_t);
}

attn_status_t attn_bwd(const attn_bwd_args_t* a, const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, void* stream) {
  attn_status_t st = check_bwd_args(a);
  if (st != ATTN_SUCCESS) return st;
  if (a->seqlen_q == 0) return ok();
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr || lse == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr || workspace == nullptr)
    return fail(ATTN_ERROR_INVALID_VALUE, "every tensor pointer and the workspace must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) || !aligned16(lse))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "tensors, lse and workspace must be 16-byte aligned");
  const size_t need = attn_bwd_workspace_size(a);
  if (workspace_bytes < need)
    return fail(ATTN_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  attn::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = static_cast<float*>(workspace);
  p.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_delta_bytes(a));
  attn::bwd_plan(a->num_q_heads / a->num_kv_heads, a->seqlen_q, a->seqlen_k, a->causal, a->window > 0 ? a->window : 0,
                 a->batch * a->num_kv_heads, &p.chunks, &p.chunk_steps);
  p.dk32 = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * bwd_delta_bytes(a));
  p.dv32 = p.dk32 + (size_t)p.chunks * a->batch * a->num_kv_heads * (size_t)a->seqlen_k * a->head_dim;
  p.order = attn::bwd_order_entries(a->seqlen_k, p.chunks) > 0
                ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + 2 * bwd_delta_bytes(a) +
                                             bwd_partial_bytes(a, attn::kBwdMaxChunks))
                : nullptr;
  p.batch = a->batch;
  p.hq = a->num_q_heads;
  p.hkv = a->num_kv_heads;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.nq = a->seqlen_q;
  p.nk = a->seqlen_k;
  p.causal = a->causal;
  p.window = a->window > 0 ? a->window : 0;
  const double scale = resolve_scale(a->softmax_scale, a->head_dim);
  p.scale = (float)scale;
  p.scale_log2 = (float)(scale * kLog2eD);
  if (a->softcap > 0.0f) {
    p.cap_in = (float)(scale / (double)a->softcap);
    p.cap_out = (float)((double)a->softcap * kLog2eD);
  }
  hipError_t e = attn::launch_bwd(p, a->dtype, a->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

static attn_status_t check_decode_args(const attn_decode_args_t* a) {
  if (a == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "args is NULL");
  if (a->num_seqs < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(ATTN_ERROR_INVALID_VALUE, "num_seqs, num_q_heads and num_kv_heads must be >= 1");
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(ATTN_ERROR_INVALID_VALUE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (a->num_seqs > 0 && a->num_kv_heads > 0 && (int64_t)a->num_kv_heads * ((a->num_q_heads / a->num_kv_heads + 15) / 16) > 65535)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_kv_heads * ceil(group / 16) is limited to 65535");
  if (a->head_dim != 128) return fail(ATTN_ERROR_NOT_SUPPORTED, "decode supports head_dim 128 only");
  if (a->page_size != kPageSize) return fail(ATTN_ERROR_NOT_SUPPORTED, "page_size must be 16");
  if (a->max_pages_per_seq < 1) return fail(ATTN_ERROR_INVALID_VALUE, "max_pages_per_seq must be >= 1");
  if (a->max_seq_len < 1) return fail(ATTN_ERROR_INVALID_VALUE, "max_seq_len must be >= 1");
  if ((int64_t)a->max_seq_len > (int64_t)a->max_pages_per_seq * kPageSize)
    return fail(ATTN_ERROR_INVALID_VALUE, "max_seq_len %d exceeds max_pages_per_seq * page_size",
                a->max_seq_len);
  if (a->q_dtype != ATTN_BF16 && a->q_dtype != ATTN_F16)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "q_dtype must be BF16 or F16");
  const bool kv_ok = a->kv_dtype == ATTN_FP8_E4M3 || a->kv_dtype == a->q_dtype;
  if (!kv_ok) return fail(ATTN_ERROR_NOT_SUPPORTED, "kv_dtype must equal q_dtype or be FP8_E4M3");
  if (a->num_splits < 0) return fail(ATTN_ERROR_INVALID_VALUE, "num_splits must be >= 0");
  if (a->num_seqs > 65535 || a->num_kv_heads > 65535)
    return fail(ATTN_ERROR_NOT_SUPPORTED, "num_seqs and num_kv_heads are limited to 65535");
  if (!(a->softmax_scale == a->softmax_scale) || isinf(a->softmax_scale))
    return fail(ATTN_ERROR_INVALID_VALUE, "softmax_scale must be finite");
  if (reinterpret_cast<uintptr_t>(a->sinks) & 3u) return fail(ATTN_ERROR_INVALID_VALUE, "sinks must be 4-byte aligned");
  return ATTN_SUCCESS;
}

attn_status_t attn_decode_plan(const attn_decode_args_t* a, int32_t* split_len, int32_t* max_splits) {
  attn_status_t st = check_decode_args(a);
  if (st != ATTN_SUCCESS) return st;
  int64_t len;
  const int coop = attn::decode_coop_slots_per_cu(a->kv_dtype, a->num_q_heads, a->num_kv_heads);
  if (a->num_splits > 0) {
    const int64_t per = ((int64_t)a->max_seq_len + a->num_splits - 1) / a->num_splits;
    len = (per + kPageSize - 1) / kPageSize * kPageSize;
  } else if (coop > 0) {
    // The cooperative kernel runs one workgroup per (split, sequence), all KV heads in it.
    // With the lengths taken as half the maximum on average and every sequence's last
    // split partial, the splits are sized for about three quarters of the workgroups the
    // device holds at once: one round of long splits, with room for lengths above the
    // average (a second round of full splits doubles the time; many short splits pay the
    // pipeline fill of each). At least 256 tokens; then spread evenly over the maximum.
    const double slots = 0.75 * coop * attn::device_cus();
    const double room = slots - 0.5 * a->num_seqs;
    const double want = room > 0 ? (double)a->num_seqs * 0.5 * a->max_seq_len / room : (double)kMaxSplitTokens;
    len = std::max<int64_t>(256, (int64_t)std::ceil(want));
    if (len > kMaxSplitTokens) len = kMaxSplitTokens;
    const int64_t n = ((int64_t)a->max_seq_len + len - 1) / len;
    len = (((int64_t)a->max_seq_len + n - 1) / n + kPageSize - 1) / kPageSize * kPageSize;
  } else {
    // Two aims, with the sequences' lengths taken as half the maximum on average:
    // (1) about kDecodeItems single-wave work items (splits x KV heads), so short
    //     splits keep a small batch busy: the shortest power of two reaching it;
    // (2) partial results (fp32 O and LSE per query head, written, then read by the
    //     combine) small next to the split's K/V bytes: at least 512 * G / kv_bytes
    //     tokens for G query heads per KV head. This matters where many query heads
    //     share a KV head (MQA: G = 32 makes 256-token splits move 25% extra bytes).
    //     It is taken only while the split grid keeps at least kDecodeMinWaves waves
    //     (a wave takes up to two head tiles of 16 query heads).
    constexpr int64_t kDecodeItems = 8192, kDecodeMinWaves = 384;
    const int64_t seqs_heads = (int64_t)a->num_seqs * a->num_kv_heads;
    const int64_t want = seqs_heads * a->max_seq_len / (2 * kDecodeItems);
    len = 256;
    while (len < want && len < kMaxSplitTokens) len *= 2;
    const int64_t group = a->num_q_heads / a->num_kv_heads;
    const int64_t tiles = group > 16 ? (group + 31) / 32 : 1;  // waves per KV head and split
    const int64_t kv_bytes = a->kv_dtype == ATTN_FP8_E4M3 ? 1 : 2;
    const int64_t partial_len = 512 * group / kv_bytes;
    while (len < partial_len && len < kMaxSplitTokens &&
           seqs_heads * tiles * a->max_seq_len / (2 * (2 * len)) >= kDecodeMinWaves)
      len *= 2;
  }
  if (len > kMaxSplitTokens) len = kMaxSplitTokens;  // the split kernel's page window
  const int64_t n = ((int64_t)a->max_seq_len + len - 1) / len;
  if (split_len) *split_len = (int32_t)len;
  if (max_splits) *max_splits = (int32_t)n;
  return ok();
}

size_t attn_decode_paged_workspace_size(const attn_decode_args_t* a) {
  int32_t len = 0, n = 0;
  if (attn_decode_plan(a, &len, &n) != ATTN_SUCCESS) return 0;
  const size_t slots = (size_t)a->num_seqs * a->num_q_heads * n;
  const size_t o_bytes = slots * a->head_dim * sizeof(float);
  const size_t l_bytes = (slots * sizeof(float) + 15) / 16 * 16;
  return o_bytes + l_bytes;
}

// Checks of the decode call's tensors (not of the workspace), on the host.
static attn_status_t check_decode_tensors(const attn_decode_args_t* a, const void* q, const void* k_cache,
                                          const void* v_cache, const float* k_scale, const float* v_scale,
                                          const int32_t* block_table, const int32_t* seq_lens, const void* o,
                                          const float* lse) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || o == nullptr)
    return fail(ATTN_ERROR_INVALID_VALUE, "q, k_cache, v_cache, block_table, seq_lens and o must be non-NULL");
  const bool fp8 = a->kv_dtype == ATTN_FP8_E4M3;
  if (fp8 && (k_scale == nullptr || v_scale == nullptr))
    return fail(ATTN_ERROR_INVALID_VALUE, "fp8 KV needs k_scale and v_scale");
  if (!fp8 && (k_scale != nullptr || v_scale != nullptr))
    return fail(ATTN_ERROR_INVALID_VALUE, "k_scale / v_scale are only accepted with fp8 KV");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERROR_NOT_SUPPORTED, "q, caches and o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(ATTN_ERROR_INVALID_VALUE, "block_table, seq_lens and lse must be 4-byte aligned");
  return ATTN_SUCCESS;
}

// The decode launch on a checked call with a workspace of at least the planned size.
static attn_status_t decode_launch(const attn_decode_args_t* a, int32_t split_len, int32_t max_splits,
                                   const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                   void* o, float* lse, void* workspace, void* stream);

attn_status_t attn_decode_paged(const attn_decode_args_t* a, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  int32_t split_len = 0, max_splits = 0;
  attn_status_t st = attn_decode_plan(a, &split_len, &max_splits);
  if (st != ATTN_SUCCESS) return st;
  st = check_decode_tensors(a, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o, lse);
  if (st != ATTN_SUCCESS) return st;
  if (workspace == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "workspace must be non-NULL");
  if (!aligned16(workspace)) return fail(ATTN_ERROR_NOT_SUPPORTED, "workspace must be 16-byte aligned");
  const size_t need = attn_decode_paged_workspace_size(a);
  if (workspace_bytes < need)
    return fail(ATTN_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return decode_launch(a, split_len, max_splits, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o,
                       lse, workspace, stream);
}

attn_status_t attn_decode_paged_noalloc(const attn_decode_args_t* a, const void* q, const void* k_cache,
                                        const void* v_cache, const float* k_scale, const float* v_scale,
                                        const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                        void* stream) {
  int32_t split_len = 0, max_splits = 0;
  attn_status_t st = attn_decode_plan(a, &split_len, &max_splits);
  if (st != ATTN_SUCCESS) return st;
  st = check_decode_tensors(a, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o, lse);
  if (st != ATTN_SUCCESS) return st;
  const size_t need = attn_decode_paged_workspace_size(a);
  if (need > attn::kDecodeScratchBytes)
    return fail(ATTN_ERROR_WORKSPACE_TOO_SMALL,
                "these arguments need %zu bytes of partial results; the built-in scratch holds %zu "
                "(use attn_decode_paged with a workspace)",
                need, (size_t)attn::kDecodeScratchBytes);
  void* scratch = nullptr;
  hipError_t e = attn::decode_scratch(&scratch);
  if (e != hipSuccess)
    return fail(ATTN_ERROR_LAUNCH_FAILED, "locating the decode scratch failed: %s", hipGetErrorString(e));
  return decode_launch(a, split_len, max_splits, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, o,
                       lse, scratch, stream);
}

static attn_status_t decode_launch(const attn_decode_args_t* a, int32_t split_len, int32_t max_splits,
                                   const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                                   const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                   void* o, float* lse, void* workspace, void* stream) {

  attn::DecodeParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  const size_t slots = (size_t)a->num_seqs * a->num_q_heads * max_splits;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = p.part_o + slots * a->head_dim;
  p.o = o;
  p.lse = lse;
  p.num_seqs = a->num_seqs;
  p.hq = a->num_q_heads;
  p.hkv = a->num_kv_heads;
  p.group = a->num_q_heads / a->num_kv_heads;
  p.head_tiles = (p.group + 15) / 16;
  p.max_pages = a->max_pages_per_seq;
  p.split_len = split_len;
  p.sinks = a->sinks;
  p.max_splits = max_splits;
  p.scale_log2 = (float)(resolve_scale(a->softmax_scale, a->head_dim) * kLog2eD);
  hipError_t e = attn::launch_decode(p, a->q_dtype, a->kv_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

attn_status_t attn_probe_mfma(const uint32_t* operands, int32_t workgroups, int32_t iters, int32_t valu_mix,
                              uint64_t* clocks, float* sink, void* stream) {
  if (operands == nullptr || clocks == nullptr || sink == nullptr)
    return fail(ATTN_ERROR_INVALID_VALUE, "operands, clocks and sink must be non-NULL");
  if (workgroups < 1 || workgroups > 65535 || iters < 1 || (valu_mix != 0 && valu_mix != 1))
    return fail(ATTN_ERROR_INVALID_VALUE, "workgroups in [1, 65535], iters >= 1 and valu_mix 0 or 1 required");
  if ((reinterpret_cast<uintptr_t>(operands) & 3u) || (reinterpret_cast<uintptr_t>(clocks) & 7u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(ATTN_ERROR_INVALID_VALUE, "operands and sink must be 4-byte, clocks 8-byte aligned");
  hipError_t e = attn::launch_probe_mfma(operands, workgroups, iters, valu_mix, clocks, sink,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

attn_status_t attn_probe_hbm_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "buf and sink must be non-NULL");
  if (workgroups < 1 || workgroups > 65535) return fail(ATTN_ERROR_INVALID_VALUE, "workgroups in [1, 65535]");
  if (bytes == 0 || bytes % ((size_t)workgroups * 32768u) != 0)
    return fail(ATTN_ERROR_INVALID_VALUE, "bytes must be a non-zero multiple of 32768 * workgroups");
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(ATTN_ERROR_INVALID_VALUE, "buf must be 16-byte and sink 4-byte aligned");
  hipError_t e = attn::launch_probe_hbm_read(buf, (int64_t)bytes, workgroups, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

attn_status_t attn_flush_caches(void* buf, size_t bytes, void* stream) {
  if (buf == nullptr) return fail(ATTN_ERROR_INVALID_VALUE, "buf must be non-NULL");
  if (bytes == 0 || bytes % 16 != 0 || !aligned16(buf))
    return fail(ATTN_ERROR_INVALID_VALUE, "buf must be 16-byte aligned and bytes a non-zero multiple of 16");
  hipError_t e = attn::launch_flush(buf, (int64_t)bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERROR_LAUNCH_FAILED, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
