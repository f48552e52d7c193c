// Pieces shared by the prefill kernels (16-bit, fp32 and fp8 translation units).
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace attn {
namespace {

struct RowRange {
  int wend, wbeg;  // keys any row of the wave may see: [wbeg, wend)
  int fend, fbeg;  // keys every row of the wave sees:  [fbeg, fend)
};

// Work item of workgroup w: (query tile, query head, sequence). Workgroups are dealt to
// the 8 XCDs round-robin (w % 8), and each XCD has its own L2. The unit of placement is a
// (sequence, KV head) pair: all query tiles of all query heads that read one KV head run on
// one XCD and share its L2 copy of K and V, and unit j goes to XCD j % 8, so every XCD
// gets a slice of every sequence (a ragged or chunked batch stays balanced across XCDs).
// When the unit count is not a multiple of 8 the work index is taken XCD-major instead.
struct WorkItem {
  int qt, h, b;
};
__device__ __forceinline__ WorkItem work_item(int w, int nblk, int q_tiles, int hq, int hkv, int batch) {
  const int G = hq / hkv;
  const int per = G * q_tiles;  // items per unit
  const int units = batch * hkv;
  int j, rem;
  if ((units & 7) == 0) {
    const int i = w >> 3;
    j = (w & 7) + 8 * (i / per);
    rem = i % per;
  } else {
    const int u = (nblk & 7) == 0 ? (w & 7) * (nblk >> 3) + (w >> 3) : w;
    j = u / per;
    rem = u % per;
  }
  WorkItem r;
  r.b = j / hkv;
  r.h = (j % hkv) * G + rem / q_tiles;
  r.qt = rem % q_tiles;
  return r;
}

__device__ __forceinline__ RowRange wave_key_range(const FwdParams& p, int w0, int Lk, int delta) {
  RowRange r;
  r.wend = p.causal ? min(Lk, w0 + 32 + delta) : Lk;
  r.wbeg = p.window > 0 ? max(0, w0 + delta - p.window + 1) : 0;
  r.fend = p.causal ? min(Lk, w0 + delta + 1) : Lk;
  r.fbeg = p.window > 0 ? max(0, w0 + 31 + delta - p.window + 1) : 0;
  return r;
}

// Final normalisation of a row whose probabilities 2^(s - m) over its keys sum to lt (m in
// log2 units): 1 / denominator for O and the natural-log LSE. The attention sink (a per
// query head logit that joins the denominator with no value) adds 2^(sink - M) at the
// common reference M = max(m, sink). Without a sink a row with no key gets O = 0 and
// LSE = -inf; with one, O = 0 and LSE = the sink.
struct RowNorm {
  float inv, lse;
};
__device__ __forceinline__ RowNorm row_norm(float lt, float m, const float* sinks, int h) {
  if (sinks == nullptr) return {lt > 0.0f ? 1.0f / lt : 0.0f, lt > 0.0f ? (m + fast_log2(lt)) * kLn2 : kNegInf};
  const float s2 = sinks[h] * kLog2e;
  const float M = lt > 0.0f ? fmaxf(m, s2) : s2;
  const float f = lt > 0.0f ? fast_exp2(m - M) : 0.0f;
  const float l2 = lt * f + fast_exp2(s2 - M);
  return {l2 > 0.0f ? f / l2 : 0.0f, l2 > 0.0f ? (M + fast_log2(l2)) * kLn2 : kNegInf};
}

// Lanes l and l^32 hold the two halves of a query row's keys; they exchange through the
// LDS crossbar (ds_bpermute).
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, xor_shuffle(x, 32)); }
__device__ __forceinline__ float pair_sum(float x) { return x + xor_shuffle(x, 32); }

// Probabilities are formed against a reference max that may trail the true running max
// by up to this many binary orders of magnitude; the accumulator is rescaled only when
// a tile would exceed it (p <= 2^8, far from overflow). The result is unchanged: the
// same reference max is used for P, for l and for the final LSE.
constexpr float kRescaleSlack = 8.0f;

}  // namespace
}  // namespace attn
