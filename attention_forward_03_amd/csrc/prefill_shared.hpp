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

// Lanes l and l^32 hold the two halves of a query row's keys; they exchange by a swap of
// the wave's 32-lane halves (v_permlane32_swap: one vector instruction, no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Probabilities are formed against a reference max that may trail the true running max
// by up to this many binary orders of magnitude; the accumulator is rescaled only when
// a tile would exceed it (p <= 2^8, far from overflow). The result is unchanged: the
// same reference max is used for P, for l and for the final LSE.
constexpr float kRescaleSlack = 8.0f;

// ----------------------------------------------------------------- 16-bit inputs ----
// K and V tiles live in LDS row-major with 16-byte chunks XOR-swizzled per row (no
// padding), filled straight from global memory by direct-to-LDS loads: each load
// instruction moves 64 lanes x 16 bytes into one contiguous 1 KiB LDS block, and the
// swizzle is applied by choosing which global chunk each lane fetches.
//   K reads (A operand of S^T): 16 consecutive rows at one chunk -> 16 bank groups.
//   V reads use the transposing LDS read: in each 16-lane group, lane i receives element
//   i%4 of the 4-element rows addressed by lanes i/4 + 4e (e = 0..3). Lanes address 4
//   consecutive head-dim entries of 4 keys, so every lane ends up with 4 keys of one
//   head-dim entry: exactly the A operand of O^T = V^T . P^T, with no transposition on
//   the way into LDS. A 4-key x 4-chunk read hits 16 distinct bank groups.
// Head dims that are not a power of two (96, 192) use LDS rows of the next power of two
// (128, 256): the extra chunks of a row are padding that no read touches.

template <int D>
struct Swizzle {
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  __device__ static __forceinline__ int k(int row, int c) {
    if constexpr (CPR >= 16) return c ^ (row & 15);
    else return c ^ ((row / (16 / CPR)) % CPR);
  }
  __device__ static __forceinline__ int v(int row, int c) {
    if constexpr (D >= 128) return c ^ ((row & 3) << 2);
    else if constexpr (D == 64) return c ^ (((row >> 1) & 1) << 2);
    else return c;
  }
};

// LDS row width (elements) for head dim D
constexpr int lds_row(int D) { return D <= 32 ? 32 : D <= 64 ? 64 : D <= 128 ? 128 : 256; }

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}


}  // namespace
}  // namespace attn
