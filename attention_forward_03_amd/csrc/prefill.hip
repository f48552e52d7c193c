// Fused attention forward (prefill) kernels for gfx950.
//
// O = softmax(Q K^T * scale [+ mask]) V, one workgroup per (query tile, query head,
// sequence). K/V tiles stream through double-buffered LDS; the scores and the
// probabilities never leave registers. The online-softmax state per query row
// (running max m, denominator l, output accumulator) is rescaled by
// alpha = 2^(m_old - m_new) whenever the max grows, which is the recurrence of the
// page "Agent 帮我写 CUDA：一个 Softmax Attention 算子的开发全记录", section 四
// (tiled-attention core idea), evaluated in base 2 with the scale folded into the
// exponent argument. The split into a Q.K^T matrix-unit stage, a softmax row stage
// on the vector unit and a P.V matrix-unit stage follows the QK / Softmax / PV
// stage table of the PTO FlashAttention cost-model post ("为什么 PTO 适合 Agent
// 来优化").
//
// Both products are computed transposed so that each lane owns one query row:
//   S^T = K . Q^T   (A = K tile from LDS, B = Q held in registers)
//   O^T = V^T . P^T (A = V^T tile from LDS, B = P straight from the S^T registers)
// In the 32x32 matrix-core result layout a lane holds one column (= one query) and
// 16 rows (= keys, or head-dim entries), so the row max / row sum are lane-local
// except for one exchange with lane l^32, and alpha is a per-lane scalar.
#include "common.hpp"
#include "internal.hpp"

namespace attn {
namespace {

// Position of key k inside its 16-key group in the transposed V tile. The middle two
// groups of four are swapped: the eight keys a lane contributes to one P.V k-step
// (keys {0-3, 8-11} for lanes 0-31, {4-7, 12-15} for lanes 32-63, as produced by the
// S^T result layout) then sit contiguously and load with one 128-bit LDS read.
__device__ __forceinline__ int vt_pos(int k) {
  const int grp = (k >> 2) & 3;
  const int sw = ((grp & 1) << 1) | (grp >> 1);
  return (k & ~15) | (sw << 2) | (k & 3);
}

struct RowRange {
  int wend, wbeg;  // keys any row of the wave may see: [wbeg, wend)
  int fend, fbeg;  // keys every row of the wave sees:  [fbeg, fend)
};

__device__ __forceinline__ RowRange wave_key_range(const FwdParams& p, int w0, int Lk, int delta) {
  RowRange r;
  r.wend = p.causal ? min(Lk, w0 + 32 + delta) : Lk;
  r.wbeg = p.window > 0 ? max(0, w0 + delta - p.window + 1) : 0;
  r.fend = p.causal ? min(Lk, w0 + delta + 1) : Lk;
  r.fbeg = p.window > 0 ? max(0, w0 + 31 + delta - p.window + 1) : 0;
  return r;
}

// Softcap, mask and online-softmax update of one key tile for one lane's query row.
// s[] holds raw dot products on entry and unnormalised probabilities on exit.
template <int NKB>
__device__ __forceinline__ float softmax_tile(const FwdParams& p, f32x16_t (&s)[NKB], float& m,
                                              float& l, bool full, int kt, int qrow, int Lk,
                                              int delta, int hi) {
  float sc = p.scale_log2;
  if (p.cap_out > 0.0f) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = p.cap_out * tanh_via_exp2(s[kb][r] * p.cap_in);
    sc = 1.0f;
  }
  if (!full) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kt + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
        bool ok = j < Lk;
        if (p.causal) ok = ok && (j <= qrow + delta);
        if (p.window > 0) ok = ok && (j > qrow + delta - p.window);
        if (!ok) s[kb][r] = kNegInf;
      }
  }
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, xor_shuffle(mx, 32));
  const float m_new = fmaxf(m, mx * sc);
  const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
  const float alpha = fast_exp2(m - m_use);
  float rs = 0.0f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(s[kb][r] * sc - m_use);
      s[kb][r] = e;
      rs += e;
    }
  l = l * alpha + rs;
  m = m_new;
  return alpha;
}

// ----------------------------------------------------------------- 16-bit inputs ----

template <int D, int NW, int BN, bool BF16>
__global__ __launch_bounds__(NW * 64) void fwd_mfma16_kernel(const FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KLD = D + 8;   // padded K row: consecutive rows shift by 16 bytes
  constexpr int VLD = BN + 8;  // padded V^T row
  constexpr int KT = BN * KLD;
  constexpr int VT = D * VLD;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int NPS = BN / 16;
  constexpr int KCH = BN * D / 8;
  constexpr int KCH_T = (KCH + NT - 1) / NT;
  constexpr int VU = (BN / 4) * (D / 8);
  constexpr int VU_T = (VU + NT - 1) / NT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT + VT)];
  uint16_t* const k_lds = smem;
  uint16_t* const v_lds = smem + 2 * KT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int qt = blockIdx.x;
  if (p.causal) qt = p.q_tiles - 1 - qt;  // longest rows first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
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
  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (ragged ? 0 : (int64_t)b * p.qs[0]) +
                       (int64_t)h * p.qs[1] + (int64_t)q_off * p.qs[2];
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (ragged ? 0 : (int64_t)b * p.ks[0]) +
                       (int64_t)hk * p.ks[1] + (int64_t)k_off * p.ks[2];
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (ragged ? 0 : (int64_t)b * p.vs[0]) +
                       (int64_t)hk * p.vs[1] + (int64_t)k_off * p.vs[2];
  uint16_t* og = static_cast<uint16_t*>(p.o) + (ragged ? 0 : (int64_t)b * p.os[0]) +
                 (int64_t)h * p.os[1] + (int64_t)q_off * p.os[2];
  const int64_t qs2 = p.qs[2], ks2 = p.ks[2], vs2 = p.vs[2], os2 = p.os[2];

  // Key range of the whole block, aligned down to the tile grid.
  const int r1 = min(Lq, r0 + BM);
  const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
  int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
  kbeg = (kbeg / BN) * BN;
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const int w0 = r0 + wave * 32;
  const bool wave_live = w0 < Lq;
  const int qrow = w0 + l32;
  const RowRange rr = wave_key_range(p, w0, Lk, delta);

  u32x4_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = u32x4_t{0, 0, 0, 0};
    if (qrow < Lq) qf[ks] = load_global<u32x4_t>(qg + qrow * qs2 + ks * 16 + hi * 8);
  }

  u32x4_t kreg[KCH_T];
  u32x4_t vreg[VU_T][4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KCH_T; ++i) {
      const int c = tid + i * NT;
      kreg[i] = u32x4_t{0, 0, 0, 0};
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / (D / 8), col = c % (D / 8);
        const int key = kt + row;
        if (key < Lk) kreg[i] = load_global<u32x4_t>(kg + key * ks2 + col * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VU_T; ++i) {
      const int u = tid + i * NT;
      if (VU % NT == 0 || u < VU) {
        const int kq = u % (BN / 4), dc = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt + kq * 4 + r;
          vreg[i][r] = u32x4_t{0, 0, 0, 0};
          if (key < Lk) vreg[i][r] = load_global<u32x4_t>(vg + key * vs2 + dc * 8);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kl = k_lds + buf * KT;
    uint16_t* vl = v_lds + buf * VT;
#pragma unroll
    for (int i = 0; i < KCH_T; ++i) {
      const int c = tid + i * NT;
      if (KCH % NT == 0 || c < KCH) {
        const int row = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<u32x4_t*>(kl + row * KLD + col * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VU_T; ++i) {
      const int u = tid + i * NT;
      if (VU % NT == 0 || u < VU) {
        const int kq = u % (BN / 4), dc = u / (BN / 4);
        const int pos = vt_pos(kq * 4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // column 2w gathers the low halves of dword w of the four rows, 2w+1 the high halves
          const u32x2_t even = {__builtin_amdgcn_perm(vreg[i][1][w], vreg[i][0][w], 0x05040100u),
                                __builtin_amdgcn_perm(vreg[i][3][w], vreg[i][2][w], 0x05040100u)};
          const u32x2_t odd = {__builtin_amdgcn_perm(vreg[i][1][w], vreg[i][0][w], 0x07060302u),
                               __builtin_amdgcn_perm(vreg[i][3][w], vreg[i][2][w], 0x07060302u)};
          *reinterpret_cast<u32x2_t*>(vl + (dc * 8 + 2 * w) * VLD + pos) = even;
          *reinterpret_cast<u32x2_t*>(vl + (dc * 8 + 2 * w + 1) * VLD + pos) = odd;
        }
      }
    }
  };

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = kNegInf, l = 0.0f;

  if (ntiles > 0) {
    load_tile(kbeg);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int kt = kbeg + it * BN;
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(kt + BN);
    if (wave_live && kt < rr.wend && kt + BN > rr.wbeg) {
      const uint16_t* kl = k_lds + buf * KT;
      const uint16_t* vl = v_lds + buf * VT;
      f32x16_t s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kl + (kb * 32 + l32) * KLD + ks * 16 + hi * 8);
          s[kb] = mfma32x32x16<BF16>(a, qf[ks], s[kb]);
        }
      }
      const bool full = kt >= rr.fbeg && kt + BN <= rr.fend;
      const float alpha = softmax_tile<NKB>(p, s, m, l, full, kt, qrow, Lk, delta, hi);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      u32x4_t pf[NPS];
#pragma unroll
      for (int t = 0; t < NPS; ++t) {
        const int kb = t >> 1, base = (t & 1) * 8;
        pf[t] = u32x4_t{pack2<BF16>(s[kb][base + 0], s[kb][base + 1]),
                        pack2<BF16>(s[kb][base + 2], s[kb][base + 3]),
                        pack2<BF16>(s[kb][base + 4], s[kb][base + 5]),
                        pack2<BF16>(s[kb][base + 6], s[kb][base + 7])};
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int t = 0; t < NPS; ++t) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vl + (db * 32 + l32) * VLD + t * 16 + hi * 8);
          o[db] = mfma32x32x16<BF16>(a, pf[t], o[db]);
        }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const float lt = l + xor_shuffle(l, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (qrow < Lq) {
    uint16_t* orow = og + qrow * os2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hi * 4;
        const u32x2_t w = {pack2<BF16>(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv),
                           pack2<BF16>(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(orow + d) = w;
      }
    if (hi == 0 && p.lse != nullptr) {
      const int64_t idx = ragged ? (int64_t)h * p.cu_q[p.batch] + q_off + qrow
                                 : ((int64_t)b * p.hq + h) * p.nq + qrow;
      p.lse[idx] = lt > 0.0f ? (m + fast_log2(lt)) * kLn2 : kNegInf;
    }
  }
}

// ------------------------------------------------------------------ fp32 inputs ----
// 32x32x2 fp32 matrix-core products. Q.K^T contracts over head_dim with lanes 0-31
// taking the first half of D and lanes 32-63 the second; P.V contracts over keys in
// the order the S^T result registers hold them, and V is read row-major (each lane
// needs a single element per product, so no transposition is required).

template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64) void fwd_f32_kernel(const FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int LD = D + 4;
  constexpr int TS = BN * LD;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;  // products per P.V k-step; output row i holds d = NDB*i + db
  constexpr int HD = D / 2;
  constexpr int CH = BN * D / 4;
  constexpr int CH_T = (CH + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) float smem[4 * TS];
  float* const k_lds = smem;
  float* const v_lds = smem + 2 * TS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int qt = blockIdx.x;
  if (p.causal) qt = p.q_tiles - 1 - qt;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
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
  const float* qg = static_cast<const float*>(p.q) + (ragged ? 0 : (int64_t)b * p.qs[0]) +
                    (int64_t)h * p.qs[1] + (int64_t)q_off * p.qs[2];
  const float* kg = static_cast<const float*>(p.k) + (ragged ? 0 : (int64_t)b * p.ks[0]) +
                    (int64_t)hk * p.ks[1] + (int64_t)k_off * p.ks[2];
  const float* vg = static_cast<const float*>(p.v) + (ragged ? 0 : (int64_t)b * p.vs[0]) +
                    (int64_t)hk * p.vs[1] + (int64_t)k_off * p.vs[2];
  float* og = static_cast<float*>(p.o) + (ragged ? 0 : (int64_t)b * p.os[0]) +
              (int64_t)h * p.os[1] + (int64_t)q_off * p.os[2];
  const int64_t qs2 = p.qs[2], ks2 = p.ks[2], vs2 = p.vs[2], os2 = p.os[2];

  const int r1 = min(Lq, r0 + BM);
  const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
  int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
  kbeg = (kbeg / BN) * BN;
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const int w0 = r0 + wave * 32;
  const bool wave_live = w0 < Lq;
  const int qrow = w0 + l32;
  const RowRange rr = wave_key_range(p, w0, Lk, delta);

  float qf[HD];
#pragma unroll
  for (int j = 0; j < HD / 4; ++j) {
    f32x4_t x = {0.0f, 0.0f, 0.0f, 0.0f};
    if (qrow < Lq) x = load_global<f32x4_t>(qg + qrow * qs2 + hi * HD + j * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[j * 4 + e] = x[e];
  }

  f32x4_t kreg[CH_T], vreg[CH_T];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH_T; ++i) {
      const int c = tid + i * NT;
      kreg[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      vreg[i] = kreg[i];
      if (CH % NT == 0 || c < CH) {
        const int row = c / (D / 4), col = c % (D / 4);
        const int key = kt + row;
        if (key < Lk) {
          kreg[i] = load_global<f32x4_t>(kg + key * ks2 + col * 4);
          vreg[i] = load_global<f32x4_t>(vg + key * vs2 + col * 4);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH_T; ++i) {
      const int c = tid + i * NT;
      if (CH % NT == 0 || c < CH) {
        const int row = c / (D / 4), col = c % (D / 4);
        *reinterpret_cast<f32x4_t*>(k_lds + buf * TS + row * LD + col * 4) = kreg[i];
        *reinterpret_cast<f32x4_t*>(v_lds + buf * TS + row * LD + col * 4) = vreg[i];
      }
    }
  };

  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = kNegInf, l = 0.0f;

  if (ntiles > 0) {
    load_tile(kbeg);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int kt = kbeg + it * BN;
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(kt + BN);
    if (wave_live && kt < rr.wend && kt + BN > rr.wbeg) {
      const float* kl = k_lds + buf * TS;
      const float* vl = v_lds + buf * TS;
      f32x16_t s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
        for (int j = 0; j < HD / 4; ++j) {
          const f32x4_t a = *reinterpret_cast<const f32x4_t*>(kl + (kb * 32 + l32) * LD + hi * HD + j * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[j * 4 + e], s[kb], 0, 0, 0);
        }
      }
      const bool full = kt >= rr.fbeg && kt + BN <= rr.fend;
      const float alpha = softmax_tile<NKB>(p, s, m, l, full, kt, qrow, Lk, delta, hi);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const float* vrow = vl + key * LD + NDB * l32;
          if constexpr (NDB == 4) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(vrow);
#pragma unroll
            for (int db = 0; db < 4; ++db)
              o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[db], s[kb][r], o[db], 0, 0, 0);
          } else if constexpr (NDB == 2) {
            const f32x2_t x = *reinterpret_cast<const f32x2_t*>(vrow);
#pragma unroll
            for (int db = 0; db < 2; ++db)
              o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[db], s[kb][r], o[db], 0, 0, 0);
          } else {
            o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[0], s[kb][r], o[0], 0, 0, 0);
          }
        }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const float lt = l + xor_shuffle(l, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (qrow < Lq) {
    float* orow = og + qrow * os2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = (r >> 2) * 8 + hi * 4 + (r & 3);
      if constexpr (NDB == 4) {
        *reinterpret_cast<f32x4_t*>(orow + 4 * i) =
            f32x4_t{o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv};
      } else if constexpr (NDB == 2) {
        *reinterpret_cast<f32x2_t*>(orow + 2 * i) = f32x2_t{o[0][r] * inv, o[1][r] * inv};
      } else {
        orow[i] = o[0][r] * inv;
      }
    }
    if (hi == 0 && p.lse != nullptr) {
      const int64_t idx = ragged ? (int64_t)h * p.cu_q[p.batch] + q_off + qrow
                                 : ((int64_t)b * p.hq + h) * p.nq + qrow;
      p.lse[idx] = lt > 0.0f ? (m + fast_log2(lt)) * kLn2 : kNegInf;
    }
  }
}

constexpr int kNW16 = 4;   // waves per workgroup, 16-bit inputs
constexpr int kBN16 = 64;  // keys per tile, 16-bit inputs
constexpr int kNW32 = 4;
constexpr int kBN32 = 32;

template <int D, bool BF16>
hipError_t launch16(const FwdParams& p, hipStream_t st) {
  dim3 grid(p.q_tiles, p.hq, p.batch);
  hipLaunchKernelGGL((fwd_mfma16_kernel<D, kNW16, kBN16, BF16>), grid, dim3(kNW16 * 64), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch32(const FwdParams& p, hipStream_t st) {
  dim3 grid(p.q_tiles, p.hq, p.batch);
  hipLaunchKernelGGL((fwd_f32_kernel<D, kNW32, kBN32>), grid, dim3(kNW32 * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int fwd_block_rows(int dtype, int /*head_dim*/) {
  return dtype == 0 ? kNW32 * 32 : kNW16 * 32;
}

// dtype: 0 = f32, 1 = f16, 2 = bf16 (attn_dtype_t values)
hipError_t launch_fwd(const FwdParams& p, int dtype, int head_dim, hipStream_t st) {
  switch (dtype * 1000 + head_dim) {
    case 32: return launch32<32>(p, st);
    case 64: return launch32<64>(p, st);
    case 128: return launch32<128>(p, st);
    case 1032: return launch16<32, false>(p, st);
    case 1064: return launch16<64, false>(p, st);
    case 1128: return launch16<128, false>(p, st);
    case 2032: return launch16<32, true>(p, st);
    case 2064: return launch16<64, true>(p, st);
    case 2128: return launch16<128, true>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
