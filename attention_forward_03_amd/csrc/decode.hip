// Split-KV paged decode for gfx950: one query token per sequence, keys in a
// block-table KV cache, the key range of each sequence cut into splits that run in
// separate workgroups, then merged by an LSE-weighted combine.
//
// Split kernel: one wave per (split, KV head g, sequence s). The G = Hq/Hkv query
// heads that share KV head g are processed together, so every K/V byte is read
// once. Work runs page by page (16 tokens = one page):
//   scores  S^T[key][query] = K . Q^T on the 16x16x32 matrix core, K loaded straight
//           from the page into the A operand (lane l: token slot l%16, 64 contiguous
//           bytes of head_dim at 32*(l/16)); Q (zero beyond G) is the B operand;
//   softmax online-softmax update per query column (max over the 4 lanes that hold
//           a column via two xor exchanges); alpha = 2^(m_old - m_new);
//   values  O^T += V^T . P^T on the 16x16x4 fp32 matrix core: lane l loads 8
//           head_dim entries of one token row (16 lanes cover a 256-byte row) and
//           feeds entry c to product c, whose output row i is head_dim 8*i + c.
// The split writes its normalised partial output and its log2-domain LSE to the
// workspace. Combine kernel: one wave per (sequence, query head) merges the
// ceil(L_s / split_len) partials: LSE = log sum_k 2^{lse_k}, O = sum_k
// 2^{lse_k - LSE} O_k. Split-KV decode over a paged cache and the fp8 KV precision
// are scenario axes of "Ask, Don't Equip: Question-Driven Coding Agents for Deep
// Kernel Optimization", section 研究动机.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;

enum KvKind { KV_BF16 = 0, KV_F16 = 1, KV_FP8 = 2 };

// Eight OCP e4m3 codes (two dwords) -> eight 16-bit values (a 128-bit operand of a
// 16-bit product). Exact: every finite e4m3 value (|x| <= 448, smallest subnormal
// 2^-9) is representable in both bf16 and f16.
template <bool BF16>
__device__ __forceinline__ u32x4_t fp8x8_to_16(u32x2_t codes) {
  u32x4_t r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[w], false);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[w], true);
    r[2 * w] = pack2<BF16>(a[0], a[1]);
    r[2 * w + 1] = pack2<BF16>(c[0], c[1]);
  }
  return r;
}

template <int KV, bool QBF16>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
  constexpr bool KBF16 = (KV == KV_FP8) ? QBF16 : (KV == KV_BF16);
  static_assert(KV == KV_FP8 || KBF16 == QBF16, "16-bit K must match the query type");
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane & 15;   // query column (head g*G + col when col < G)
  const int quad = lane >> 4;  // key slots 4*quad .. 4*quad+3 / head_dim block 32*quad

  const int L = p.seq_lens[s];
  const int t0 = split * p.split_len;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + p.split_len);
  const int G = p.group;

  // Q as the B operand: k-step ks, slot group quad <-> head_dim 32*quad + 8*ks .. +7.
  u32x4_t qf[4];
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)s * p.hq + g * G + col) * kD + 32 * quad;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qf[ks] = u32x4_t{0, 0, 0, 0};
    if (col < G) qf[ks] = load_global<u32x4_t>(qrow + 8 * ks);
  }

  const int64_t tok_stride = (int64_t)p.hkv * kD;        // elements between token slots
  const int64_t page_stride = kPage * tok_stride;
  const int32_t* bt = p.block_table + (int64_t)s * p.max_pages;
  float ksc = 1.0f, vsc = 1.0f;
  if constexpr (KV == KV_FP8) {
    ksc = p.k_scale[g];
    vsc = p.v_scale[g];
  }
  const float sl2 = p.scale_log2 * ksc;

  f32x4_t o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kNegInf, l = 0.0f;

  // Registers of one page: K operand (4 k-steps) and 4 V rows of 8 entries.
  using KRaw = typename std::conditional<KV == KV_FP8, u32x2_t, u32x4_t>::type;
  KRaw kr[4], kn[4];
  KRaw vr[4], vn[4];
  auto load_page = [&](int pg, KRaw (&kk)[4], KRaw (&vv)[4]) {
    const int64_t phys = bt[pg];
    const int64_t kbase = phys * page_stride + (int64_t)col * tok_stride + (int64_t)g * kD + 32 * quad;
    const int64_t vbase = phys * page_stride + (int64_t)g * kD + 8 * col;
    if constexpr (KV == KV_FP8) {
      const uint8_t* kc = static_cast<const uint8_t*>(p.k_cache);
      const uint8_t* vc = static_cast<const uint8_t*>(p.v_cache);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = load_global<u32x2_t>(kc + kbase + 8 * ks);
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[r] = load_global<u32x2_t>(vc + vbase + (4 * quad + r) * tok_stride);
    } else {
      const uint16_t* kc = static_cast<const uint16_t*>(p.k_cache);
      const uint16_t* vc = static_cast<const uint16_t*>(p.v_cache);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = load_global<u32x4_t>(kc + kbase + 8 * ks);
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[r] = load_global<u32x4_t>(vc + vbase + (4 * quad + r) * tok_stride);
    }
  };

  const int pg0 = t0 / kPage;
  const int pg1 = (t1 + kPage - 1) / kPage;
  load_page(pg0, kr, vr);
  for (int pg = pg0; pg < pg1; ++pg) {
    if (pg + 1 < pg1) load_page(pg + 1, kn, vn);
    // scores
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t a;
      if constexpr (KV == KV_FP8) a = fp8x8_to_16<QBF16>(kr[ks]);
      else a = kr[ks];
      sc = mfma16x16x32<QBF16>(a, qf[ks], sc);
    }
    const int tb = pg * kPage + 4 * quad;  // token of register r is tb + r
    const bool partial = (pg + 1) * kPage > t1;
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (partial && tb + r >= t1) sc[r] = kNegInf;
      mx = fmaxf(mx, sc[r]);
    }
    mx = fmaxf(mx, xor_shuffle(mx, 16));
    mx = fmaxf(mx, xor_shuffle(mx, 32));
    const float m_new = fmaxf(m, mx * sl2);  // every page holds at least one valid token
    const float alpha = fast_exp2(m - m_new);
    float pr[4];
    float rs = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = fast_exp2(sc[r] * sl2 - m_new);
      rs += pr[r];
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] *= alpha;
    // values: row r of this lane is token tb + r; zero the rows past the end (the
    // cache tail may hold anything, and 0 * NaN would poison the sum)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float vf[8];
      if constexpr (KV == KV_FP8) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)vr[r][w], false);
          const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)vr[r][w], true);
          vf[4 * w + 0] = a[0];
          vf[4 * w + 1] = a[1];
          vf[4 * w + 2] = c[0];
          vf[4 * w + 3] = c[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vf[2 * w] = lo16<KBF16>(vr[r][w]);
          vf[2 * w + 1] = hi16<KBF16>(vr[r][w]);
        }
      }
      if (partial && tb + r >= t1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) vf[c] = 0.0f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[c], pr[r], o[c], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = kn[i];
      vr[i] = vn[i];
    }
  }

  float lt = l + xor_shuffle(l, 16);
  lt += xor_shuffle(lt, 32);
  if (col < G) {
    const int h = g * G + col;
    const int64_t slot = ((int64_t)s * p.hq + h) * p.max_splits + split;
    float* dst = p.part_o + slot * kD + 32 * quad;
    const float inv = vsc / lt;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      *reinterpret_cast<f32x4_t*>(dst + 8 * rr) =
          f32x4_t{o[0][rr] * inv, o[1][rr] * inv, o[2][rr] * inv, o[3][rr] * inv};
      *reinterpret_cast<f32x4_t*>(dst + 8 * rr + 4) =
          f32x4_t{o[4][rr] * inv, o[5][rr] * inv, o[6][rr] * inv, o[7][rr] * inv};
    }
    if (quad == 0) p.part_lse[slot] = m + fast_log2(lt);
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
    if (lane == 0 && p.lse != nullptr) p.lse[(int64_t)s * p.hq + h] = kNegInf;
    return;
  }
  const float* lse2 = p.part_lse + base;

  float mx = kNegInf;
  for (int k = lane; k < n; k += 64) mx = fmaxf(mx, lse2[k]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, xor_shuffle(mx, off));

  f32x2_t acc = {0.0f, 0.0f};
  float wsum = 0.0f;
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

template <int KV, bool QBF16>
hipError_t launch(const DecodeParams& p, hipStream_t st) {
  dim3 grid(p.max_splits, p.hkv, p.num_seqs);
  hipLaunchKernelGGL((decode_split_kernel<KV, QBF16>), grid, dim3(64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<QBF16>), dim3(p.num_seqs * p.hq), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// q_dtype: 1 = f16, 2 = bf16; kv_dtype: 1 = f16, 2 = bf16, 3 = fp8 e4m3
hipError_t launch_decode(const DecodeParams& p, int q_dtype, int kv_dtype, hipStream_t st) {
  const bool qbf = q_dtype == 2;
  if (kv_dtype == 3) return qbf ? launch<KV_FP8, true>(p, st) : launch<KV_FP8, false>(p, st);
  if (kv_dtype == 2 && qbf) return launch<KV_BF16, true>(p, st);
  if (kv_dtype == 1 && !qbf) return launch<KV_F16, false>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace attn
