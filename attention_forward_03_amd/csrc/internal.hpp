// Host-side kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// One prefill launch. Pointers are device pointers; strides are in elements for
// the [batch, head, token] dimensions (head_dim contiguous).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_q;  // null for dense batches
  const int32_t* cu_k;
  int64_t qs[3], ks[3], vs[3], os[3];
  int32_t batch, hq, hkv, group;
  int32_t nq, nk;       // dense lengths, or the upper bounds for ragged batches
  int32_t causal, window;
  float scale_log2;     // softmax scale * log2(e)
  float cap_in;         // softcap: multiplier of the raw dot product inside tanh (scale / c)
  float cap_out;        // softcap: c * log2(e); 0 = off
  int32_t q_tiles;      // query tiles per sequence
  // paged keys (chunked prefill): k / v are caches [pages, 16, Hkv, D]; ks[0] / vs[0] are
  // the page strides and ks[2] / vs[2] the token strides; sequence b has seq_lens_k[b]
  // keys in the pages that row b of block_table [batch, max_pages] names. For the ragged
  // kernels (cu_q set, block_table NULL) a non-NULL seq_lens_k means: sequence b's keys
  // are tokens [b * max_pages * 16, + seq_lens_k[b]) of the packed k / v (gathered pages)
  const int32_t* block_table;
  const int32_t* seq_lens_k;
  int32_t max_pages, num_pages;
  const float* sinks;   // per query head sink logit (natural log), or NULL
  float o_scale;        // fp8 inputs: the value scale, applied with the normalisation
  int32_t pair_items;   // 16-bit compiler-built kernel: a workgroup per pair of query tiles
};

// One backward launch (dense, contiguous [B, H, N, D] tensors, 16-bit).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;     // [B, Hq, Nq], natural log, as the forward writes it
  void* dq;
  void* dk;
  void* dv;
  float* delta;         // workspace [B, Hq, Nq]
  float* lse2;          // workspace [B, Hq, Nq]: lse * log2(e)
  float* dk32;          // workspace [chunks][B, Hkv, Nk, D] fp32 partial dK, then dv32 alike
  float* dv32;
  int32_t* order;       // workspace [bwd_order_entries]: the (key block, chunk) items of a
                        // unit, longest first; NULL: run them in index order
  int32_t chunk_steps, chunks;  // dK / dV work split, from bwd_plan
  int32_t kblocks;              // 128-key blocks per (sequence, KV head), set by the launcher
  int32_t batch, hq, hkv, group, nq, nk, causal, window;
  float scale;          // softmax scale
  float scale_log2;     // scale * log2(e)
  float cap_in, cap_out;  // softcap as for the forward (cap_out = 0: off)
};

hipError_t launch_bwd(const BwdParams& p, int dtype, int head_dim, hipStream_t stream);

// Split of the dK / dV work. A workgroup owns a block of kBwdKeyBlock keys and walks the
// (query head of its group, kBwdQueryTile-row query tile) steps that reach them; those steps,
// at most group * ceil(nq / kBwdQueryTile) per block, are cut into `chunks` (<= kBwdMaxChunks) runs of
// `steps`, each a work item with an fp32 partial dK / dV of its own. Items are kept no
// longer than one CU's share of all the steps (kBwdPlanCUs CUs), so that the longest-first
// order balances them (with the dQ items that follow in the same launch), and split no
// further: every extra chunk costs a partial written and summed.
constexpr int kBwdKeyBlock = 128;
constexpr int kBwdQueryTile = 32;
constexpr int kBwdPlanCUs = 256;
constexpr int kBwdMaxChunks = 4;
inline void bwd_plan(int group, int nq, int nk, int causal, int window, int units, int* chunks, int* steps) {
  const int max_steps = group * ((nq + kBwdQueryTile - 1) / kBwdQueryTile);
  // all steps of one unit (the query-tile range of each key block, as the kernels count it)
  int64_t total = 0;
  const int delta = nk - nq;
  for (int kb0 = 0; kb0 < nk; kb0 += kBwdKeyBlock) {
    const int kb1 = nk < kb0 + kBwdKeyBlock ? nk : kb0 + kBwdKeyBlock;
    int q_lo = causal ? (kb0 - delta > 0 ? kb0 - delta : 0) : 0;
    const int q_hi = window > 0 ? (nq < kb1 - 1 - delta + window ? nq : kb1 - 1 - delta + window) : nq;
    q_lo = (q_lo / kBwdQueryTile) * kBwdQueryTile;
    if (q_hi > q_lo) total += (int64_t)((q_hi - q_lo + kBwdQueryTile - 1) / kBwdQueryTile) * group;
  }
  total *= units;
  int c = total > 0 ? (int)(((int64_t)max_steps * kBwdPlanCUs + total - 1) / total) : 1;
  c = c < 1 ? 1 : (c > kBwdMaxChunks ? kBwdMaxChunks : c);
  if (c > max_steps) c = max_steps > 0 ? max_steps : 1;
  *chunks = c;
  *steps = (max_steps + c - 1) / c;
  if (*steps < 1) *steps = 1;
}

// Entries of the dK / dV run-order table: one per (128-key block, chunk); 0 when the table
// would exceed kBwdOrderMax entries (the items then run in index order).
constexpr int64_t kBwdOrderMax = 32768;
inline int64_t bwd_order_entries(int nk, int chunks) {
  const int64_t n = (int64_t)((nk + kBwdKeyBlock - 1) / kBwdKeyBlock) * chunks;
  return n <= kBwdOrderMax ? n : 0;
}

// One paged-decode launch (split kernel + combine kernel).
struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* part_o;        // [S, Hq, max_splits, D]
  float* part_lse;      // [S, Hq, max_splits], log2 domain
  void* o;
  float* lse;
  int32_t num_seqs, hq, hkv, group, max_pages;
  int32_t head_tiles;   // ceil(group / 16): query-head tiles of 16 per KV head
  int32_t split_len, max_splits;
  float scale_log2;
  const float* sinks;   // per query head sink logit (natural log), or NULL
};

// Block-rows of the prefill kernels for a given dtype/head_dim (the host needs it
// to size the grid).
// query rows per workgroup of the dense / ragged prefill (units = sequences x query heads)
int fwd_block_rows(int dtype, int head_dim, int64_t nq, int64_t units);

hipError_t launch_fwd(const FwdParams& p, int dtype, int head_dim, hipStream_t stream);
// chunked prefill over a paged cache (16-bit inputs)
hipError_t launch_fwd_paged(const FwdParams& p, int dtype, int head_dim, hipStream_t stream);
int fwd_paged_block_rows(int head_dim);
// fp8 e4m3 dense prefill (head_dim 128, bf16 output)
int fwd_fp8_block_rows();
hipError_t launch_fwd_fp8(const FwdParams& p, int head_dim, hipStream_t stream);
// page-by-page copy of K and V into per-sequence slots of max_pages * 16 tokens
hipError_t launch_gather_kv_pages(const void* k_cache, const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, void* ws_k, void* ws_v, int num_seqs, int max_pages,
                                  int num_pages, int page_bytes, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int q_dtype, int kv_dtype, hipStream_t stream);
// Workgroups of the cooperative decode split kernel (one per split and sequence, all KV
// heads) that one CU holds at once, or 0 when these heads take the one-wave kernel.
int decode_coop_slots_per_cu(int kv_dtype, int num_q_heads, int num_kv_heads);
// Compute units of the current device (256 when there is none).
int device_cus();
// Bytes of the device scratch array behind attn_decode_paged_noalloc (per GPU): the
// header's ATTN_DECODE_NOALLOC_MAX_WORKSPACE.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
// Device address of that array on the current device (looked up once per device).
hipError_t decode_scratch(void** ptr);

hipError_t launch_probe_mfma(const uint32_t* operands, int workgroups, int iters, int valu_mix, uint64_t* clocks,
                             float* sink, hipStream_t stream);
hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, int workgroups, uint32_t* sink, hipStream_t stream);
hipError_t launch_flush(void* buf, int64_t bytes, hipStream_t stream);

}  // namespace attn
