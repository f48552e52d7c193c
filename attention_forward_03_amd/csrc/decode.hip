// Split-KV paged decode for gfx950: one query token per sequence, keys in a
// block-table KV cache, the key range of each sequence cut into splits that run in
// separate workgroups, then merged by an LSE-weighted combine.
//
// Split kernel: one wave per (split, KV head g, sequence s); for fp8 KV with at most 16
// query heads per KV head, the waves of up to 8 KV heads of one (split, sequence) form a
// workgroup that loads whole pages contiguously into a shared LDS stage (the head-strided
// row segments a lone wave reads cost 16% of the page stream's rate). The G = Hq/Hkv query
// heads that share KV head g are processed together, so every K/V byte is read
// once; beyond 16 heads per KV head (MQA-like groups) a wave takes two tiles of 16 query
// heads, which share every K and V fragment read (more than 32 heads: adjacent workgroups
// take further pairs of tiles). Work runs page by page (16 tokens = one page):
//   scores  S^T[key][query] = K . Q^T on the 16x16x32 matrix core, K loaded straight
//           from the page into the A operand (lane l: token slot l%16, 64 contiguous
//           bytes of head_dim at 32*(l/16)); Q (zero beyond G) is the B operand;
//   softmax online-softmax update per query column (max over the 4 lanes that hold
//           a column via two lane swaps); alpha = 2^(m_old - m_new);
//   values  O^T += V^T . P^T on the 16x16x16 16-bit matrix core, V^T read with the
//           transposing LDS read (16- or 8-bit; fp8 codes widen exactly to 16 bits).
// The split writes its normalised partial output and its log2-domain LSE to the
// workspace. Combine kernel: one wave per (sequence, query head) merges the
// ceil(L_s / split_len) partials: LSE = log sum_k 2^{lse_k}, O = sum_k
// 2^{lse_k - LSE} O_k. Split-KV decode over a paged cache and the fp8 KV precision
// are scenario axes of "Ask, Don't Equip: Question-Driven Coding Agents for Deep
// Kernel Optimization", section 研究动机.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kMaxSplitPages = 256;  // the host plans splits of at most 4096 tokens
#ifndef ATTN_DECODE_HEAD_MAJOR
#define ATTN_DECODE_HEAD_MAJOR 1
#endif

enum KvKind { KV_BF16 = 0, KV_F16 = 1, KV_FP8 = 2 };

// Four OCP e4m3 codes (one dword, code 0 in the low byte) -> four 16-bit values in
// two dwords, in the same order, by the packed scaled conversion at scale 1. Exact:
// every finite e4m3 value (|x| <= 448, smallest subnormal 2^-9) is representable in
// both bf16 and f16, and a unit scale leaves it unchanged.
template <bool BF16>
__device__ __forceinline__ u32x2_t fp8x4_to_16(int codes) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
  u32x2_t r;
  if constexpr (BF16) {
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
    r[0] = __builtin_bit_cast(uint32_t, lo);
    r[1] = __builtin_bit_cast(uint32_t, hi);
  } else {
    const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, false);
    const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, true);
    r[0] = __builtin_bit_cast(uint32_t, lo);
    r[1] = __builtin_bit_cast(uint32_t, hi);
  }
  return r;
}

// Eight codes (two dwords) -> eight 16-bit values (a 128-bit operand of a 16-bit product).
template <bool BF16>
__device__ __forceinline__ u32x4_t fp8x8_to_16(u32x2_t codes) {
  const u32x2_t a = fp8x4_to_16<BF16>((int)codes[0]);
  const u32x2_t b = fp8x4_to_16<BF16>((int)codes[1]);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

// Maximum and sum over the four lanes col, col+16, col+32, col+48 (the lanes that hold one
// query column of a 16x16 result) by the gfx950 lane-swap instructions, with no LDS round
// trip: swapping the odd 16-lane rows of x with the even rows of a copy of x pairs lane l
// with l^16, and swapping the upper 32 lanes with the lower 32 pairs l with l^32.
__device__ __forceinline__ float max_over_column(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_column(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;

__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

typedef __attribute__((ext_vector_type(2))) int i32x2_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
__device__ __forceinline__ i32x2_t lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p));
}

// 16x16x16 matrix-core product on 16-bit inputs (4 per lane): lane l supplies row l%16 of
// A and column l%16 of B, k-slots 4*(l/16) .. +3; result register r of lane l is row
// 4*(l/16) + r, column l%16.
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
}

// Pages of one split stream through an LDS ring of NST stages per wave, filled by
// direct-to-LDS loads issued NST-1 pages ahead (each load instruction moves 1 KiB of
// whole token rows, so global accesses are fully coalesced). A stage holds the page's
// K rows then its V rows, row-major with 16-byte chunks XOR-swizzled per row:
//   K: the score operand reads (16 token rows at one chunk) hit 16 bank groups;
//   V (16-bit): the transposing reads of the P.V operand (16 rows x 2 chunks) hit each
//      bank group twice, the minimum for 512 bytes.
template <int KV>
struct PageLayout {
  static constexpr int ELT = KV == KV_FP8 ? 1 : 2;           // bytes per element
  static constexpr int ROW = kD * ELT;                       // bytes per token row
  static constexpr int CPR = ROW / 16;                       // 16-byte chunks per row
  static constexpr int HALF = kPage * ROW;                   // bytes of K (or V) per page
  static constexpr int STAGE = 2 * HALF;
  static constexpr int ROWS_PER_LOAD = 1024 / ROW;
  static constexpr int LOADS = kPage / ROWS_PER_LOAD;        // per K (or V) page
  __device__ static __forceinline__ int k_slot(int row, int c) {
    return c ^ ((row / (16 / CPR)) % CPR);
  }
  __device__ static __forceinline__ int v_slot(int row, int c) {
    if constexpr (KV == KV_FP8) return c ^ ((row / 2) % CPR);
    else return c ^ (2 * (row % 8));
  }
};

// HT: query-head tiles of 16 per wave (2 when a KV head has more than 16 query heads:
// both tiles then share every K and V fragment read, and each page is streamed once).
// CO: waves per workgroup. CO = 1: each wave streams its own KV head's rows of a page,
// Hkv row segments of 128 or 256 bytes at a stride of Hkv rows. CO = Hkv > 1: the
// workgroup holds the Hkv waves of one (split, sequence); wave w loads a contiguous
// 1/Hkv slice of the whole page (K, then V) into a shared stage, which keeps the memory
// stream sequential, and then reads its own head's rows from it (one barrier before
// the stage is refilled, one after its loads land). The stage keeps the page's layout;
// the 16-byte chunk slots are XOR-swizzled within each row as in the one-wave layout,
// and for 8-bit KV the even/odd head pair is swapped on odd rows, so the 16 rows of one
// head still cover all 16 bank groups.
template <int KV, bool QBF16, int NST, int HT, int CO>
__global__ __launch_bounds__(64 * CO) void decode_split_kernel(const DecodeParams p) {
  using PL = PageLayout<KV>;
  constexpr bool KBF16 = (KV == KV_FP8) ? QBF16 : (KV == KV_BF16);
  static_assert(KV == KV_FP8 || KBF16 == QBF16, "16-bit K must match the query type");
  static_assert(CO == 1 || (HT == 1 && (KV != KV_FP8 || CO % 2 == 0)), "shared stages hold one tile per head");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NST * CO * PL::STAGE];
  constexpr int RS = CO * PL::ROW;       // stage bytes between token rows
  constexpr int KHALF = CO * PL::HALF;   // stage bytes of K (or V)

#if ATTN_DECODE_HEAD_MAJOR
  // the KV heads of one split are adjacent workgroups: the slices of each physical page
  // that belong to different heads are fetched at about the same time
  const int gt = CO > 1 ? (int)(blockIdx.y * CO + (threadIdx.x >> 6)) : (int)blockIdx.x;
  const int split = CO > 1 ? blockIdx.x : blockIdx.y;
#else
  const int split = blockIdx.x;
  const int gt = CO > 1 ? (int)(blockIdx.y * CO + (threadIdx.x >> 6)) : (int)blockIdx.y;
#endif
  const int wave_tiles = (p.head_tiles + HT - 1) / HT;
  const int g = gt / wave_tiles;  // KV head
  int h0[HT], G[HT];              // first query head and query heads of each tile (G may be 0)
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const int tile = HT * (gt % wave_tiles) + t;
    h0[t] = g * p.group + 16 * tile;
    G[t] = max(0, min(16, p.group - 16 * tile));
  }
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;   // query column (head h0[t] + col when col < G[t]) / token slot
  const int quad = lane >> 4;  // token slots 4*quad .. 4*quad+3 of the score tile

  const int L = p.seq_lens[s];
  const int t0 = split * p.split_len;
  if (t0 >= L || split >= p.max_splits) return;  // (the grid may hold one more split column)
  const int t1 = min(L, t0 + p.split_len);

  // Q as the B operand of the score product: k-step ks, slot group quad <-> head_dim
  // 32*quad + 8*ks .. +7.
  u32x4_t qf[HT][4];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)s * p.hq + h0[t] + col) * kD + 32 * quad;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[t][ks] = u32x4_t{0, 0, 0, 0};
      if (col < G[t]) qf[t][ks] = load_global<u32x4_t>(qrow + 8 * ks);
    }
  }

  const int64_t tok_bytes = (int64_t)p.hkv * PL::ROW;  // bytes between token slots
  const int64_t page_bytes = kPage * tok_bytes;
  // CO > 1: the workgroup's KV heads are g0 .. g0+CO-1, this wave's is g0 + wv
  const int wv = CO > 1 ? (int)(threadIdx.x >> 6) : 0;
  const int g0 = CO > 1 ? (int)blockIdx.y * CO : g;  // from the block index: wave-uniform
  const uint8_t* kc = static_cast<const uint8_t*>(p.k_cache) + (int64_t)g0 * PL::ROW;
  const uint8_t* vc = static_cast<const uint8_t*>(p.v_cache) + (int64_t)g0 * PL::ROW;
  // stage offset of row r of this wave's head
  auto row_at = [&](int r) __attribute__((always_inline)) {
    const int h = CO == 1 ? 0 : (KV == KV_FP8 ? wv ^ (r & 1) : wv);
    return r * RS + h * PL::ROW;
  };
  const int32_t* bt = p.block_table + (int64_t)s * p.max_pages;
  float ksc = 1.0f, vsc = 1.0f;
  if constexpr (KV == KV_FP8) {
    ksc = p.k_scale[g];
    vsc = p.v_scale[g];
  }
  const float sl2 = p.scale_log2 * ksc;

  // per-lane load pattern: load i of a half-page fills stage bytes lds_blk(i) .. +1023,
  // lane l the 16-byte slot l of it; the slot's token row, head and chunk give the
  // global chunk it holds (the slot and head permutations are their own inverses)
  int ld_row[PL::LOADS], ld_k[PL::LOADS], ld_v[PL::LOADS];
#pragma unroll
  for (int i = 0; i < PL::LOADS; ++i) {
    const int pos = (wv * PL::LOADS + i) * 64 + lane;  // 16-byte slot within the stage half
    const int row = pos / (CO * PL::CPR);
    const int hs = (pos / PL::CPR) % CO;
    const int h = CO == 1 ? 0 : (KV == KV_FP8 ? hs ^ (row & 1) : hs);
    const int slot = pos % PL::CPR;
    ld_row[i] = row;
    ld_k[i] = row * (int)tok_bytes + h * PL::ROW + PL::k_slot(row, slot) * 16;
    ld_v[i] = row * (int)tok_bytes + h * PL::ROW + PL::v_slot(row, slot) * 16;
  }

  const int pg0 = t0 / kPage;
  const int pg1 = (t1 + kPage - 1) / kPage;
  // The split's block-table entries, lane i holding entry pg0 + i + 64 * c (a split spans
  // at most kMaxSplitPages pages); read with one vector load per 64 pages up front.
  int btv[kMaxSplitPages / 64];
#pragma unroll
  for (int c = 0; c < kMaxSplitPages / 64; ++c) {
    const int e = pg0 + lane + 64 * c;
    btv[c] = (64 * c < pg1 - pg0 && e < pg1) ? bt[e] : 0;
  }
  // Each register is read at the uniform lane first and the scalar results are selected:
  // selecting among the registers before the read lets the compiler index the array
  // dynamically, which puts it in scratch memory (a memory round trip per page).
  auto phys_page = [&](int idx) __attribute__((always_inline)) {  // idx = pg - pg0, uniform
    int v = __builtin_amdgcn_readlane(btv[0], idx & 63);
#pragma unroll
    for (int c = 1; c < kMaxSplitPages / 64; ++c) {
      const int w = __builtin_amdgcn_readlane(btv[c], idx & 63);
      v = idx >= 64 * c ? w : v;
    }
    return v;
  };
  auto issue = [&](int pg) __attribute__((always_inline)) {
    uint8_t* st = ring + ((pg - pg0) % NST) * CO * PL::STAGE + wv * PL::LOADS * 1024;
    const int64_t base = (int64_t)phys_page(pg - pg0) * page_bytes;
    const int valid = t1 - pg * kPage;  // rows past the end re-read the last valid row
#pragma unroll
    for (int i = 0; i < PL::LOADS; ++i) {
      const int shift = valid >= kPage ? 0 : (min(ld_row[i], valid - 1) - ld_row[i]) * (int)tok_bytes;
      load_lds16_stream(kc + base, (uint32_t)(ld_k[i] + shift), st + i * 1024);
      load_lds16_stream(vc + base, (uint32_t)(ld_v[i] + shift), st + KHALF + i * 1024);
    }
  };

  f32x4_t o[HT][8];
  float m[HT], l[HT];
#pragma unroll
  for (int t = 0; t < HT; ++t) {
#pragma unroll
    for (int c = 0; c < 8; ++c) o[t][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[t] = kNegInf;
    l[t] = 0.0f;
  }

  settle_global_loads();
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (pg0 + i < pg1) issue(pg0 + i);

  for (int pg = pg0; pg < pg1; ++pg) {
    if constexpr (CO > 1 && NST >= 3) {
      // one barrier per page: this wave's loads of page pg are done once at most those of
      // the NST-2 later pages remain; after the barrier every wave's are, and every wave
      // is done with page pg-1, whose stage the next issue refills
      if (pg + NST - 2 < pg1) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PL::LOADS * (NST - 2)) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (pg + NST - 1 < pg1) issue(pg + NST - 1);
    } else {
    // every wave is done reading the stage the next issue refills
    if constexpr (CO > 1) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (pg + NST - 1 < pg1) {
      issue(pg + NST - 1);
      // the loads of this page are complete once at most those of the NST-1 later pages
      // remain outstanding
      if constexpr (2 * PL::LOADS * (NST - 1) <= 63) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PL::LOADS * (NST - 1)) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // every wave's loads of this page have landed
    if constexpr (CO > 1) asm volatile("s_barrier" ::: "memory");
    }
    const uint8_t* kst = ring + ((pg - pg0) % NST) * CO * PL::STAGE;
    const uint8_t* vst = kst + KHALF;

    // scores S^T[slot][query] = K . Q^T, each K fragment feeding every tile
    f32x4_t sc[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) sc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (KV == KV_FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // 16 codes = head_dim 32*quad + 16*j .. +15 of token slot `col`
        const int c = 2 * quad + j;
        const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(kst + row_at(col) + PL::k_slot(col, c) * 16);
        const u32x4_t k0 = fp8x8_to_16<QBF16>(u32x2_t{raw[0], raw[1]});
        const u32x4_t k1 = fp8x8_to_16<QBF16>(u32x2_t{raw[2], raw[3]});
#pragma unroll
        for (int t = 0; t < HT; ++t) {
          sc[t] = mfma16x16x32<QBF16>(k0, qf[t][2 * j], sc[t]);
          sc[t] = mfma16x16x32<QBF16>(k1, qf[t][2 * j + 1], sc[t]);
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = 4 * quad + ks;
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kst + row_at(col) + PL::k_slot(col, c) * 16);
#pragma unroll
        for (int t = 0; t < HT; ++t) sc[t] = mfma16x16x32<QBF16>(a, qf[t][ks], sc[t]);
      }
    }
    const int tb = pg * kPage + 4 * quad;  // token of register r is tb + r
    const bool partial = (pg + 1) * kPage > t1;
    float pr[HT][4];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (partial && tb + r >= t1) sc[t][r] = kNegInf;
        mx = fmaxf(mx, sc[t][r]);
      }
      mx = max_over_column(mx);
      // The reference max may trail the running max by up to 2^8; the accumulator is
      // rescaled only when a page would exceed that (every page holds at least one valid
      // token, so the new max is finite).
      const float mxs = mx * sl2;
      if (__any(mxs > m[t] + 8.0f)) {
        const float m_new = fmaxf(m[t], mxs);
        const float alpha = fast_exp2(m[t] - m_new);
        l[t] *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[t][c] *= alpha;
        m[t] = m_new;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[t][r] = fast_exp2(sc[t][r] * sl2 - m[t]);
    }

    if constexpr (KV == KV_FP8) {
      // P packed to 16 bit as the B operand (keys 4*quad .. +3 of this lane's column); the
      // row sum is taken over the same rounded values
      u32x2_t pb[HT];
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        pb[t] = u32x2_t{pack2<QBF16>(pr[t][0], pr[t][1]), pack2<QBF16>(pr[t][2], pr[t][3])};
        l[t] += (lo16<QBF16>(pb[t][0]) + hi16<QBF16>(pb[t][0])) + (lo16<QBF16>(pb[t][1]) + hi16<QBF16>(pb[t][1]));
      }
      // O^T += V^T . P^T on the 16-bit 16x16x16 product. The 8-bit transposing read gives
      // lane i of a 16-lane group byte i%8 of the 8-byte rows addressed by lanes i/8 + 2e:
      // lane pair (2e, 2e+1) of quad q addresses key 4q + e%4 (each key twice), the even lane
      // head_dim entries 16 db .. +7 and the odd lane 16 db + 8 .. +15, so the low dword of
      // lane i holds keys 4q .. 4q+3 of head_dim 16 db + i, in the order P's registers hold
      // them; the e4m3 codes widen exactly to 16 bits.
      const int vkey = 4 * quad + ((col >> 1) & 3);
      const int vpar = col & 1;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const i32x2_t w = lds_read_tr8(vst + row_at(vkey) + PL::v_slot(vkey, db) * 16 + 8 * vpar);
        const u32x2_t vw = fp8x4_to_16<QBF16>(w[0]);
#pragma unroll
        for (int t = 0; t < HT; ++t) o[t][db] = mfma16x16x16<KBF16>(vw, pb[t], o[t][db]);
      }
    } else {
      // P packed to 16 bit as the B operand (keys 4*quad .. +3 of this lane's column);
      // the row sum is taken over the same rounded values
      u32x2_t pb[HT];
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        pb[t] = u32x2_t{pack2<QBF16>(pr[t][0], pr[t][1]), pack2<QBF16>(pr[t][2], pr[t][3])};
        l[t] += (lo16<QBF16>(pb[t][0]) + hi16<QBF16>(pb[t][0])) + (lo16<QBF16>(pb[t][1]) + hi16<QBF16>(pb[t][1]));
      }
      // O^T += V^T . P^T, 16 head_dim entries per product: the transposing read gives lane
      // l the 4 keys 4*quad .. +3 of head_dim 16*db + col
      const int vr = 4 * quad + (col >> 2);
      const int vc2 = (col & 3);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int c = 2 * db + (vc2 >> 1);
        const u32x2_t a = lds_read_tr16(vst + row_at(vr) + PL::v_slot(vr, c) * 16 + (vc2 & 1) * 8);
#pragma unroll
        for (int t = 0; t < HT; ++t) o[t][db] = mfma16x16x16<KBF16>(a, pb[t], o[t][db]);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < HT; ++t) {
    const float lt = sum_over_column(l[t]);
    if (col < G[t]) {
      const int h = h0[t] + col;
      const int64_t slot = ((int64_t)s * p.hq + h) * p.max_splits + split;
      float* dst = p.part_o + slot * kD;
      const float inv = vsc / lt;
      // block db, row r holds head_dim 16*db + 4*quad + r
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<f32x4_t*>(dst + 16 * db + 4 * quad) = o[t][db] * inv;
      if (quad == 0) p.part_lse[slot] = m[t] + fast_log2(lt);
    }
  }
}

template <bool QBF16>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeParams p) {
  const int s = blockIdx.x / p.hq;
  const int h = blockIdx.x % p.hq;
  const int lane = threadIdx.x;
  const int L = p.seq_lens[s];
  // the split grid covers max_splits pieces; lengths beyond max_seq_len are clamped to it
  const int n = min((L + p.split_len - 1) / p.split_len, p.max_splits);
  const int64_t base = ((int64_t)s * p.hq + h) * p.max_splits;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + ((int64_t)s * p.hq + h) * kD + 2 * lane;
  if (n <= 0) {
    *reinterpret_cast<uint32_t*>(orow) = 0u;
    if (lane == 0 && p.lse != nullptr) p.lse[(int64_t)s * p.hq + h] = p.sinks != nullptr ? p.sinks[h] : kNegInf;
    return;
  }
  const float* lse2 = p.part_lse + base;
  // the attention sink (a per-head logit with no value) is one more term of the merge
  const float sink2 = p.sinks != nullptr ? p.sinks[h] * kLog2e : kNegInf;

  float mx = sink2;
  for (int k = lane; k < n; k += 64) mx = fmaxf(mx, lse2[k]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, xor_shuffle(mx, off));

  f32x2_t acc = {0.0f, 0.0f};
  float wsum = p.sinks != nullptr ? fast_exp2(sink2 - mx) : 0.0f;
  const float* po = p.part_o + base * kD + 2 * lane;
  for (int k = 0; k < n; ++k) {
    const float w = fast_exp2(lse2[k] - mx);
    wsum += w;
    const f32x2_t x = load_global<f32x2_t>(po + (int64_t)k * kD);
    acc[0] += w * x[0];
    acc[1] += w * x[1];
  }
  const float inv = 1.0f / wsum;
  *reinterpret_cast<uint32_t*>(orow) = pack2<QBF16>(acc[0] * inv, acc[1] * inv);
  if (lane == 0 && p.lse != nullptr) p.lse[(int64_t)s * p.hq + h] = (mx + fast_log2(wsum)) * kLn2;
}

#ifndef ATTN_DECODE_STAGES
#define ATTN_DECODE_STAGES 2
#endif
#ifndef ATTN_DECODE_STAGES_FP8
#define ATTN_DECODE_STAGES_FP8 2
#endif
// LDS ring depth per wave: fewer stages leave room for more resident waves, which on
// this memory system pays more than a deeper prefetch per wave (measured).
constexpr int kStages16 = ATTN_DECODE_STAGES;     // 16-bit KV, 8 KiB per stage
constexpr int kStages8 = ATTN_DECODE_STAGES_FP8;  // fp8 KV, 4 KiB per stage

#ifndef ATTN_DECODE_COOP
#define ATTN_DECODE_COOP 1
#endif
// KV kinds whose split kernel runs as one workgroup of Hkv waves per (split, sequence)
// (bit 0: fp8; bit 1: 16-bit) when Hkv is 2, 4 or 8 and a KV head has at most 16 query heads.
constexpr int kCoopKinds = ATTN_DECODE_COOP;
#ifndef ATTN_DECODE_COOP_WAVES
#define ATTN_DECODE_COOP_WAVES 8
#endif
constexpr int kCoopWaves = ATTN_DECODE_COOP_WAVES;  // at most this many KV heads per workgroup
#ifndef ATTN_DECODE_STAGES_COOP
#define ATTN_DECODE_STAGES_COOP 2
#endif
constexpr int kStagesCoop = ATTN_DECODE_STAGES_COOP;  // whole-page stages per workgroup

// The hardware deals workgroups to the 8 XCDs round-robin by linear index, here split +
// width * (head group + ... * sequence). With an even width the XCD of a split hardly moves
// from one sequence to the next (a multiple of 8: split j of every sequence on XCD j % 8),
// and the early splits, which every sequence has, pile onto a few XCDs. An odd width (one
// more split column, whose workgroups find no keys and end at once) deals the splits of
// each index over all 8 XCDs: the fp8 decode workload 0.426 -> 0.38 ms at 16 splits.
template <int KV, bool QBF16, int NST, int CO>
hipError_t launch_coop(const DecodeParams& p, hipStream_t st) {
  const int width = p.max_splits | 1;
  hipLaunchKernelGGL((decode_split_kernel<KV, QBF16, NST, 1, CO>), dim3(width, p.hkv / CO, p.num_seqs), dim3(64 * CO),
                     0, st, p);
  return hipGetLastError();
}

template <int KV, bool QBF16>
hipError_t launch(const DecodeParams& p, hipStream_t st) {
  const bool two = p.head_tiles >= 2;  // more than 16 query heads per KV head
  const int wave_tiles = two ? (p.head_tiles + 1) / 2 : p.head_tiles;
  constexpr int nst = KV == KV_FP8 ? kStages8 : kStages16;
  const int co = min(p.hkv & -p.hkv, kCoopWaves);  // a power of two that divides Hkv
  const bool coop = (kCoopKinds & (KV == KV_FP8 ? 1 : 2)) && p.head_tiles == 1 && co >= 2;
  if (coop) {
    // a 16-bit page of 8 heads is 64 KiB: two stages fill most of the 160 KiB
    constexpr int cst = KV == KV_FP8 ? kStagesCoop : 2;
    const hipError_t e = co == 8   ? launch_coop<KV, QBF16, cst, 8>(p, st)
                         : co == 4 ? launch_coop<KV, QBF16, cst, 4>(p, st)
                                   : launch_coop<KV, QBF16, cst, 2>(p, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<QBF16>), dim3(p.num_seqs * p.hq), dim3(64), 0, st, p);
    return hipGetLastError();
  }
#if ATTN_DECODE_HEAD_MAJOR
  // With a multiple of 8 head columns each XCD takes whole columns; an odd split width
  // then changes which of the XCD's CUs the splits of consecutive sequences meet (a
  // multiple of 8 kept split j on the same CUs): -1.6% on the decode workload, -9.5% on
  // 64 short sequences. With fewer columns (MQA) the even width measured faster.
  const int cols = p.hkv * wave_tiles;
  dim3 grid(cols, cols % 8 == 0 ? p.max_splits | 1 : p.max_splits, p.num_seqs);
#else
  dim3 grid(p.max_splits, p.hkv * wave_tiles, p.num_seqs);
#endif
  if (two)
    hipLaunchKernelGGL((decode_split_kernel<KV, QBF16, nst, 2, 1>), grid, dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<KV, QBF16, nst, 1, 1>), grid, dim3(64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<QBF16>), dim3(p.num_seqs * p.hq), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Per-split partial results of the allocation-free decode entry point: a file-scope
// device array, one copy per GPU, held until the process ends. Its name is only a
// host-side stand-in for the symbol; kernels receive the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// kv_dtype: 1 = f16, 2 = bf16, 3 = fp8 e4m3. The same choice of kernel as launch() below;
// the count is the LDS limit of the workgroup's page stages (at most 32 waves per CU).
int decode_coop_slots_per_cu(int kv_dtype, int num_q_heads, int num_kv_heads) {
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  const bool fp8 = kv_dtype == 3;
  const int group = num_q_heads / num_kv_heads;
  const int co = min(num_kv_heads & -num_kv_heads, kCoopWaves);
  if (!(kCoopKinds & (fp8 ? 1 : 2)) || group > 16 || co < 2) return 0;
  const int stages = fp8 ? kStagesCoop : 2;
  const int lds = stages * co * 2 * kPage * kD * (fp8 ? 1 : 2);
  return max(1, min(160 * 1024 / lds, 32 / co));
}

// q_dtype: 1 = f16, 2 = bf16; kv_dtype: 1 = f16, 2 = bf16, 3 = fp8 e4m3
hipError_t launch_decode(const DecodeParams& p, int q_dtype, int kv_dtype, hipStream_t st) {
  const bool qbf = q_dtype == 2;
  if (kv_dtype == 3) return qbf ? launch<KV_FP8, true>(p, st) : launch<KV_FP8, false>(p, st);
  if (kv_dtype == 2 && qbf) return launch<KV_BF16, true>(p, st);
  if (kv_dtype == 1 && !qbf) return launch<KV_F16, false>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
