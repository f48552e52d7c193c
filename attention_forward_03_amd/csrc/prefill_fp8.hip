// fp8 (OCP e4m3) dense prefill for gfx950, head_dim 128: both products on the
// 32x32x64 fp8 matrix cores, output bf16.
//
// fp8 inputs are a scenario axis of "Ask, Don't Equip: Question-Driven Coding Agents for
// Deep Kernel Optimization" (section 研究动机); Q, K and V are e4m3 codes with one scale
// per tensor (value = code * scale). The scales of Q and K fold into the exponent's
// scale, the scale of V into the final normalisation. The tiling and the online softmax
// are those of the 16-bit kernel (the recurrence of the page "Agent 帮我写 CUDA：一个
// Softmax Attention 算子的开发全记录", section 四): 4 waves of 32 query rows (three
// workgroups per CU: three waves per SIMD, so one wave's softmax runs beside the products
// of the others), 64-key K / V tiles double-buffered in LDS by direct-to-LDS loads, both
// products transposed:
//   S^T = K . Q^T   A = K rows from LDS (32 bytes of one key per lane), B = Q in registers;
//   O^T = V^T . P^T A = V^T from the 8-bit transposing LDS read, B = P rounded to e4m3
//                   straight from the S^T accumulators; the row sums add the rounded P.
// Lane layouts (measured): the 32x32x64 fp8 product gives its result in the layout of the
// other 32x32 products (register r of lane l: row 8(r/4) + 4(l/32) + r%4, column l%32),
// and A and B pair byte j of lane half h with the same k, so any assignment of k to
// (half, byte) that A and B share is valid. ds_read_b64_tr_b8 hands lane i of each
// 16-lane group byte i%8 of the 8-byte rows addressed by lanes i/8 + 2e (e = 0..7).
//
// P takes byte 16 kb + r of its operand from register r of score block kb, i.e. key
// 32 kb + 8(r/4) + 4h + r%4 for lane half h. The V^T operand must hold the same keys in
// the same order: read r (0..3) of a lane pair (2e, 2e+1) addresses key
// 32(r/2) + 16(r%2) + 8(e/4) + 4h + e%4, the even lane head-dim entries d0..d0+7 and the
// odd lane d0+8..d0+15, so lane i of the group ends with 8 keys of head-dim entry
// d0 + i: exactly its row of V^T.
//
// LDS rows are 128 bytes; 16-byte chunk c of key row k sits at chunk c ^ g(k), where g
// takes bits 1-3 of k with the lower two swapped. With 64 four-byte banks (256 bytes, 16
// chunk slots, per cycle) a row pair k, k ^ 1 spans the 16 slots, so:
//   a K read (16 lanes per cycle: 16 consecutive keys at one chunk) has 8 keys of each
//   parity, whose g values are all distinct;
//   a V read (32 lanes per cycle: keys {0..3, 8..11} + 4h at chunks 2db and 2db + 1) has
//   4 keys of each parity per chunk, whose g values take one of each pair {2i, 2i + 1},
//   so the two chunks fill disjoint slots. (g = (k >> 1) & 7 put both chunks on the same
//   8 slots: two extra cycles per transposing read, as the counters showed.)
// g depends on bits 1-3 only, so keys 16 apart share it.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "prefill_shared.hpp"

namespace attn {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int sw8(int key, int c) {
  const int x = (key >> 1) & 7;
  return c ^ ((x & 4) | ((x & 1) << 1) | ((x >> 1) & 1));
}

// four floats -> four e4m3 codes (round to nearest even), first in the low byte
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  // the first conversion writes the low half; its high half (the old value, any register)
  // is then written by the second
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p));
}

constexpr int kD = 128;
constexpr int kNW = 4;
constexpr int kBN = 64;
// P = 2^(s - m + kPOff) with the reference m at most kSlack8 below the row max: P <= 2^8,
// inside e4m3's 448, and the row's largest P >= 2^6, so probabilities down to 2^-12 of it
// stay normal e4m3 numbers (3-bit mantissa; below 2^-6 the format only has absolute
// steps of 2^-9)
constexpr float kSlack8 = 2.0f;
constexpr float kPOff = 6.0f;

__global__ __launch_bounds__(kNW * 64, 3) void fwd_fp8_kernel(const FwdParams p) {
  constexpr int D = kD, NW = kNW, BN = kBN;
  constexpr int BM = NW * 32;
  constexpr int TILE = BN * D;  // bytes per K or V tile
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE];
  uint8_t* const k_lds = smem;             // [2][BN][128 B]
  uint8_t* const v_lds = smem + 2 * TILE;  // [2][BN][128 B]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS load addresses stay scalar
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const WorkItem wi = work_item(blockIdx.x, gridDim.x, p.q_tiles, p.hq, p.hkv, p.batch);
  const int h = wi.h, b = wi.b;
  const int qt = p.causal ? p.q_tiles - 1 - wi.qt : wi.qt;

  int q_off = 0, k_off = 0, Lq = p.nq, Lk = p.nk;
  if (p.cu_q != nullptr) {
    q_off = p.cu_q[b];
    Lq = p.cu_q[b + 1] - q_off;
    k_off = p.cu_k[b];
    Lk = p.cu_k[b + 1] - k_off;
  }
  const int r0 = qt * BM;
  if (r0 >= Lq) return;
  const int hk = h / p.group;
  const int delta = Lk - Lq;
  const bool ragged = p.cu_q != nullptr;
  const uint8_t* qg = static_cast<const uint8_t*>(p.q) + (ragged ? 0 : (int64_t)b * p.qs[0]) +
                      (int64_t)h * p.qs[1] + (int64_t)q_off * p.qs[2];
  const uint8_t* kg = static_cast<const uint8_t*>(p.k) + (ragged ? 0 : (int64_t)b * p.ks[0]) +
                      (int64_t)hk * p.ks[1] + (int64_t)k_off * p.ks[2];
  const uint8_t* vg = static_cast<const uint8_t*>(p.v) + (ragged ? 0 : (int64_t)b * p.vs[0]) +
                      (int64_t)hk * p.vs[1] + (int64_t)k_off * p.vs[2];
  uint16_t* og = static_cast<uint16_t*>(p.o) + (ragged ? 0 : (int64_t)b * p.os[0]) +
                 (int64_t)h * p.os[1] + (int64_t)q_off * p.os[2];
  const int64_t qs2 = p.qs[2], os2 = p.os[2];
  const int ks2 = (int)p.ks[2], vs2 = (int)p.vs[2];  // bytes per token; host keeps 64 * stride < 2^31

  const int r1 = min(Lq, r0 + BM);
  const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
  int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
  kbeg = (kbeg / BN) * BN;
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const int w0 = r0 + wave * 32;
  const bool wave_live = w0 < Lq;
  const int qrow = w0 + l32;
  const RowRange rr = wave_key_range(p, w0, Lk, delta);
  const int key_lo = p.window > 0 ? qrow + delta - p.window + 1 : 0;
  const int key_hi = p.causal ? min(Lk, qrow + delta + 1) : Lk;
  const uint32_t key_n = (uint32_t)max(key_hi - key_lo, 0);

  // Q: product t covers head-dim bytes [64 t, 64 t + 64); lane half hi holds [64 t + 32 hi, +32)
  i32x8_t qf[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u32x4_t x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
    if (qrow < Lq) {
      const uint8_t* src = qg + qrow * qs2 + 64 * t + 32 * hi;
      x0 = load_global<u32x4_t>(src);
      x1 = load_global<u32x4_t>(src + 16);
    }
    qf[t] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  // direct-to-LDS loads of 8 rows (1 KiB) each: load i of wave w fills LDS block
  // w + NW i (rows 8 (w + NW i) .. +7) of a tile; lane position lane % 8 of row
  // 8 (w + NW i) + lane / 8 holds memory chunk sw8(row, lane % 8)
  constexpr int LPW = BN / (8 * NW);  // loads per wave per K or V tile
  static_assert(BN % (8 * NW) == 0, "every wave loads whole 8-row blocks");
  int ld_row[LPW], ld_k[LPW], ld_v[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    ld_row[i] = (wave + NW * i) * 8 + lane / 8;
    ld_k[i] = ld_row[i] * ks2 + sw8(ld_row[i], lane % 8) * 16;
    ld_v[i] = ld_row[i] * vs2 + sw8(ld_row[i], lane % 8) * 16;
  }
  auto load_rows = [&](const uint8_t* gbase, int stride, const int* off, int kt, uint8_t* dst)
                       __attribute__((always_inline)) {
    const uint8_t* g = gbase + (int64_t)kt * stride;
    if (kt + BN <= Lk) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) load_lds16(g, (uint32_t)off[i], dst + (wave + NW * i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        // tail rows re-read the last key
        const int shift = min(ld_row[i], Lk - 1 - kt) - ld_row[i];
        load_lds16(g, (uint32_t)(off[i] + shift * stride), dst + (wave + NW * i) * 1024);
      }
    }
  };

  // K reads: row l32 of score block kb, chunks 4 t + 2 hi and 4 t + 2 hi + 1 of product t
  int rd_k[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) rd_k[t][c2] = l32 * D + sw8(l32, 4 * t + 2 * hi + c2) * 16;
  // V^T reads: read r of head-dim block db
  const int grp = lane >> 4, j16 = lane & 15, e = j16 >> 1, par = j16 & 1;
  // (the swizzle term is the same for the four reads of a lane, whose keys differ by
  // multiples of 16, so read r sits at a fixed offset from read 0)
  int rd_v[NDB];
  {
    const int key0 = 8 * (e >> 2) + 4 * hi + (e & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) rd_v[db] = key0 * D + sw8(key0, 2 * db + (grp & 1)) * 16 + 8 * par;
  }
  auto rd_v_ofs = [](int r) { return (32 * (r >> 1) + 16 * (r & 1)) * D; };
  // all-ones A operand (e4m3 1.0) of the row-sum product, kept in registers
  i32x8_t ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = 0x38383838;
  asm volatile("" : "+v"(ones));

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  // m: the row's reference (log2 units); thr: the raw score above which a tile moves it,
  // (m + kSlack8) / sc; neg_mu: -(m - kPOff), the exponent offset of P (0 while m = -inf)
  float m = kNegInf, l = 0.0f, thr = kNegInf, neg_mu = 0.0f;
  const f32x16_t zero16 = {};
  f32x16_t s[NKB];

  auto needs = [&](int it) {
    const int kt = kbeg + it * BN;
    return wave_live && kt < rr.wend && kt + BN > rr.wbeg;
  };
  // S^T = K . Q^T: product j = (kb, t) takes its K fragment from a ring that the reads two
  // products ahead fill (program order fixed by scheduling fences)
  auto scores = [&](const uint8_t* kl) __attribute__((always_inline)) {
    constexpr int NS = NKB * 2, RA = 2;
    auto frag = [&](int j) __attribute__((always_inline)) {
      const int kb = j >> 1, t = j & 1;
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(kl + kb * 32 * D + rd_k[t][0]);
      const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(kl + kb * 32 * D + rd_k[t][1]);
      return i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    i32x8_t ring[RA + 1];
#pragma unroll
    for (int j = 0; j < RA; ++j) ring[j] = frag(j);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      if (j + RA < NS) ring[(j + RA) % (RA + 1)] = frag(j + RA);
      const int kb = j >> 1, t = j & 1;
      s[kb] = mfma_fp8(ring[j % (RA + 1)], qf[t], t == 0 ? zero16 : s[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto softmax_pv = [&](int it, const uint8_t* vl) __attribute__((always_inline)) {
    const int kt = kbeg + it * BN;
    // O^T += V^T . P^T (below): product db takes its V^T fragment (four transposing reads)
    // from a ring that the reads two products ahead fill
    constexpr int VA = 2;
    auto vfrag = [&](int db) __attribute__((always_inline)) {
      i32x8_t a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const i32x2_t w = lds_read_tr8(vl + rd_v[db] + rd_v_ofs(r));
        a[2 * r] = w[0];
        a[2 * r + 1] = w[1];
      }
      return a;
    };
    i32x8_t vr[VA + 1];
    float sc = p.scale_log2;
    if (p.cap_out > 0.0f) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = p.cap_out * tanh_via_exp2(s[kb][r] * p.cap_in);
      sc = 1.0f;
    }
    if (!(kt >= rr.fbeg && kt + BN <= rr.fend)) {
      const uint32_t base = (uint32_t)(kt + hi * 4 - key_lo);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (base + (uint32_t)(kb * 32 + (r >> 2) * 8 + (r & 3)) >= key_n) s[kb][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    // a lane's half-row max against the threshold: the row max is formed only when some
    // row moves its reference
    if (__any(mx > thr)) {
      const float m_new = fmaxf(m, pair_max(mx) * sc);
      const float alpha = fast_exp2(m - (m_new == kNegInf ? 0.0f : m_new));
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m = m_new;
      thr = (m + kSlack8) / sc;
      neg_mu = (m == kNegInf) ? 0.0f : kPOff - m;
    }
    // P in e4m3, byte 16 kb + r <- s[kb][r]
    i32x8_t pf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = fast_exp2(__builtin_fmaf(s[kb][4 * q4 + i], sc, neg_mu));
        pf[4 * kb + q4] = pack4_fp8(x[0], x[1], x[2], x[3]);
      }
#pragma unroll
    for (int db = 0; db < VA; ++db) vr[db] = vfrag(db);
    {
      // the row sum of the rounded P from the matrix core: the all-ones A operand puts the
      // column sums of P^T (all 64 keys of the tile) in every row of the result;
      // lanes l and l^32 hold the same query column and their sums are added at the end,
      // so each takes half (exact)
      const f32x16_t ts = mfma_fp8(ones, pf, zero16);
      l += 0.5f * ts[0];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      __builtin_amdgcn_sched_barrier(0);
      if (db + VA < NDB) vr[(db + VA) % (VA + 1)] = vfrag(db + VA);
      o[db] = mfma_fp8(vr[db % (VA + 1)], pf, o[db]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  auto tile = [&](auto bufc, int it) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    const int kt = kbeg + it * BN;
    if (it + 1 < ntiles) {
      load_rows(kg, ks2, ld_k, kt + BN, k_lds + (BUF ^ 1) * TILE);
      load_rows(vg, vs2, ld_v, kt + BN, v_lds + (BUF ^ 1) * TILE);
    }
    if (needs(it)) {
      scores(k_lds + BUF * TILE);
      softmax_pv(it, v_lds + BUF * TILE);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  settle_global_loads();
  if (ntiles > 0) {
    load_rows(kg, ks2, ld_k, kbeg, k_lds);
    load_rows(vg, vs2, ld_v, kbeg, v_lds);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntiles) tile(std::integral_constant<int, 1>{}, it + 1);
  }

  if (!wave_live) return;
  // l sums 2^(s - (m - kPOff))
  const RowNorm nrm = row_norm(pair_sum(l), m == kNegInf ? m : m - kPOff, p.sinks, h);
  const float inv = nrm.inv * p.o_scale;
  if (qrow < Lq) {
    uint16_t* orow = og + qrow * os2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hi * 4;
        const u32x2_t w = {pack2<true>(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv),
                           pack2<true>(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + d) = w;
      }
    if (hi == 0 && p.lse != nullptr) {
      const int64_t idx = ragged ? (int64_t)h * p.cu_q[p.batch] + q_off + qrow
                                 : ((int64_t)b * p.hq + h) * p.nq + qrow;
      p.lse[idx] = nrm.lse;
    }
  }
}

}  // namespace

int fwd_fp8_block_rows() { return kNW * 32; }

hipError_t launch_fwd_fp8(const FwdParams& p, int head_dim, hipStream_t st) {
  if (head_dim != kD) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)p.q_tiles * p.hq * p.batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_fp8_kernel, dim3((unsigned)blocks), dim3(kNW * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace attn
