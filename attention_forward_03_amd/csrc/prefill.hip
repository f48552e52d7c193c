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
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "prefill_shared.hpp"

namespace attn {
namespace {

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

// One workgroup = NW waves; each wave owns 32 query rows and walks all key tiles of the
// workgroup's range. K and V tiles are double-buffered: the loads of tile j+1 are issued
// before tile j is computed and waited for at the per-tile barrier.
//
// PAGED: chunked prefill. Sequence b's queries are its last Nq_b positions (packed rows
// cu_q[b] ...) and its Nk_b = seq_lens_k[b] keys sit in 16-token cache pages named by
// row b of the block table, so the causal offset is Nk_b - Nq_b as in the dense case.
// Key tiles start at multiples of 16, and one direct-to-LDS load covers at most 16 rows,
// so each load reads inside a single page: its base is the page (a wave-uniform address)
// and each lane adds its token slot. The page ids of a tile are read one tile ahead.
//
// Head dim 256 runs two workgroups per CU: 256 registers, with a few values of the item
// set-up spilled (one workgroup per CU measured 9% slower).
template <int D, int NW, int BN, bool BF16, bool PAGED = false>
__global__ __launch_bounds__(NW * 64, (NW == 8 && D == 96 ? 1 : 2)) void fwd_mfma16_kernel(const FwdParams p) {
  constexpr int BM = NW * 32;
  constexpr int DP = lds_row(D);  // LDS row width
  constexpr int TILE = BN * DP;   // elements per K or V tile in LDS
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int NPS = BN / 16;
  constexpr int CPR = D / 8;    // chunks of a row in memory
  constexpr int CPRP = DP / 8;  // chunks of a row in LDS
  constexpr int ROWS_PER_LOAD = 64 / CPRP;
  constexpr int LOADS = BN / ROWS_PER_LOAD;  // load instructions per tile (K or V)
  constexpr int LPW = (LOADS + NW - 1) / NW;  // per wave
  static_assert(BN % 32 == 0 && D % 32 == 0 && BN % ROWS_PER_LOAD == 0, "tile shape");
  static_assert(!PAGED || (BN % 16 == 0 && ROWS_PER_LOAD <= 16), "a paged load stays in one page");
  using SW = Swizzle<DP>;
  // the memory chunk held at LDS chunk position `slot` of a row; padding positions hold a
  // copy of chunk 0 (loaded, never read)
  auto src_k = [](int row, int slot) { const int c = SW::k(row, slot); return c < CPR ? c : 0; };
  auto src_v = [](int row, int slot) { const int c = SW::v(row, slot); return c < CPR ? c : 0; };

  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TILE];
  uint16_t* const k_lds = smem;             // [2][BN][DP]
  uint16_t* const v_lds = smem + 2 * TILE;  // [2][BN][DP]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: load addresses stay scalar
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // The work of one query tile; a workgroup runs one, or (p.pair_items) a pair of tiles of
  // one (sequence, head) whose causal key ranges add up to the same length for every pair:
  // tile q_tiles - 1 - x and tile x.
  auto run_item = [&](const int qt, const int h, const int b) __attribute__((always_inline)) {
    int q_off = 0, k_off = 0, Lq = p.nq, Lk = p.nk;
    if (PAGED || p.cu_q != nullptr) {
      q_off = p.cu_q[b];
      Lq = p.cu_q[b + 1] - q_off;
    }
    if constexpr (PAGED) {
      Lk = min(max(p.seq_lens_k[b], 0), p.max_pages * 16);  // a bad length cannot leave the table row
    } else if (p.cu_q != nullptr) {
      k_off = p.cu_k[b];
      Lk = p.cu_k[b + 1] - k_off;
    }
    const int r0 = qt * BM;
    if (r0 >= Lq) return;
    const int hk = h / p.group;
    const int delta = Lk - Lq;
    const bool ragged = PAGED || p.cu_q != nullptr;
    const uint16_t* qg = static_cast<const uint16_t*>(p.q) + (ragged ? 0 : (int64_t)b * p.qs[0]) +
                         (int64_t)h * p.qs[1] + (int64_t)q_off * p.qs[2];
    const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (int64_t)hk * p.ks[1] +
                         (PAGED ? 0 : (ragged ? 0 : (int64_t)b * p.ks[0]) + (int64_t)k_off * p.ks[2]);
    const uint16_t* vg = static_cast<const uint16_t*>(p.v) + (int64_t)hk * p.vs[1] +
                         (PAGED ? 0 : (ragged ? 0 : (int64_t)b * p.vs[0]) + (int64_t)k_off * p.vs[2]);
    uint16_t* og = static_cast<uint16_t*>(p.o) + (ragged ? 0 : (int64_t)b * p.os[0]) +
                   (int64_t)h * p.os[1] + (int64_t)q_off * p.os[2];
    const int64_t qs2 = p.qs[2], os2 = p.os[2];
    const int ks2 = (int)p.ks[2], vs2 = (int)p.vs[2];  // host guarantees 64 * stride < 2^31

    const int r1 = min(Lq, r0 + BM);
    const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
    int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
    kbeg = (kbeg / BN) * BN;
    const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

    const int w0 = r0 + wave * 32;
    const bool wave_live = w0 < Lq;
    const int qrow = w0 + l32;
    const RowRange rr = wave_key_range(p, w0, Lk, delta);
    // this lane's allowed keys: [key_lo, key_lo + key_n)
    const int key_lo = p.window > 0 ? qrow + delta - p.window + 1 : 0;
    const int key_hi = p.causal ? min(Lk, qrow + delta + 1) : Lk;
    const uint32_t key_n = (uint32_t)max(key_hi - key_lo, 0);

    u32x4_t qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = u32x4_t{0, 0, 0, 0};
      if (qrow < Lq) qf[ks] = load_global<u32x4_t>(qg + qrow * qs2 + ks * 16 + hi * 8);
    }

    // Per-lane constant offsets (elements). Direct-to-LDS loads: load n of this wave fills
    // LDS block i = wave + n * NW (rows i*ROWS_PER_LOAD ...) of a tile. Both swizzles repeat
    // every 16 rows, so loads n and n + LP (LP * RSTEP a multiple of 16 rows) differ by whole
    // rows: LP offsets per lane serve every load, the rest is a scalar row step.
    constexpr int RSTEP = NW * ROWS_PER_LOAD;
    static_assert(RSTEP % 16 == 0 || 16 % RSTEP == 0, "swizzle period");
    constexpr int LP = RSTEP >= 16 ? 1 : (16 / RSTEP < LPW ? 16 / RSTEP : LPW);
    int ld_row0[LP], ld_k[LP], ld_v[LP];
#pragma unroll
    for (int n = 0; n < LP; ++n) {
      const int i = wave + n * NW;
      const int row = i * ROWS_PER_LOAD + lane / CPRP;
      const int slot = lane % CPRP;
      ld_row0[n] = row;
      ld_k[n] = row * ks2 + src_k(row, slot) * 8;
      ld_v[n] = row * vs2 + src_v(row, slot) * 8;
    }
    auto ld_row = [&](int n) __attribute__((always_inline)) { return ld_row0[n % LP] + (n / LP) * (LP * RSTEP); };
    // K reads: chunk 2*ks + hi of row kb*32 + l32 (the swizzle does not depend on kb). In
    // 256-element rows the swizzle (an XOR of the chunk with row & 15) leaves the chunk's
    // bit 4 alone, so fragment ks + 8 lies 128 elements after fragment ks: 8 offsets serve.
    constexpr int NKR = DP >= 256 ? 8 : NKS;
    int rd_k[NKR];
#pragma unroll
    for (int ks = 0; ks < NKR; ++ks) rd_k[ks] = l32 * DP + SW::k(l32, 2 * ks + hi) * 8;
    auto k_ofs = [&](int ks) __attribute__((always_inline)) { return rd_k[ks % NKR] + (ks / NKR) * 128; };
    // V transposing reads: rows t*16 + vrow (+8), head-dim block db; likewise in 256-element
    // rows block db + 4 lies 128 elements after block db
    const int grp = lane >> 4, gi = lane & 15;
    const int vrow = 4 * hi + (gi >> 2);
    constexpr int NVR = DP >= 256 ? 4 : NDB;
    int rd_v[NVR];
#pragma unroll
    for (int db = 0; db < NVR; ++db) {
      const int c = db * 4 + (grp & 1) * 2 + ((gi & 3) >> 1);
      rd_v[db] = vrow * DP + SW::v(vrow, c) * 8 + (gi & 1) * 4;
    }
    auto v_ofs = [&](int db) __attribute__((always_inline)) { return rd_v[db % NVR] + (db / NVR) * 128; };

    // Direct-to-LDS loads of one K or V tile. In the tail tile, rows past the last key
    // re-read the last key (always in bounds); the mask gives them zero weight.
    auto load_rows = [&](const uint16_t* gbase, int stride, const int (&off)[LP], int kt,
                         uint16_t* dst) __attribute__((always_inline)) {
      const uint16_t* g = gbase + (int64_t)kt * stride;
      if (kt + BN <= Lk) {
#pragma unroll
        for (int n = 0; n < LPW; ++n) {
          const int i = wave + n * NW;
          if (LOADS % NW == 0 || i < LOADS)
            load_lds16(g, (uint32_t)(off[n % LP] + (n / LP) * (LP * RSTEP) * stride) * 2u, dst + i * 512);
        }
      } else {
#pragma unroll
        for (int n = 0; n < LPW; ++n) {
          const int i = wave + n * NW;
          if (LOADS % NW == 0 || i < LOADS) {
            // rows past the last key re-read it (off[n % LP] addresses row ld_row0[n % LP])
            const int shift = min(ld_row(n), Lk - 1 - kt) - ld_row0[n % LP];
            load_lds16(g, (uint32_t)(off[n % LP] + shift * stride) * 2u, dst + i * 512);
          }
        }
      }
    };
    // Paged form: load n of a tile reads page pg[n]; its rows past the last key re-read the
    // last key. The page ids come from the block table (clamped to the cache, so a bad
    // entry gives wrong values, never an access outside the cache).
    // read through the constant address space: the table does not change during the launch,
    // so its wave-uniform entries come in by scalar loads (which the loop's memory-clobbering
    // direct-to-LDS loads would otherwise turn into vector loads with a wait on every load)
    typedef __attribute__((address_space(4))) const int32_t const_i32_t;
    const_i32_t* bt = PAGED ? (const_i32_t*)(p.block_table + (int64_t)b * p.max_pages) : nullptr;
    const int last_page = (Lk - 1) >> 4, last_slot = (Lk - 1) & 15;
    int ld_col_k[LPW], ld_col_v[LPW];
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      ld_col_k[n] = src_k(ld_row(n), lane % CPRP) * 8;
      ld_col_v[n] = src_v(ld_row(n), lane % CPRP) * 8;
    }
    auto page_ids = [&](int kt, int (&pg)[LPW]) __attribute__((always_inline)) {
#pragma unroll
      for (int n = 0; n < LPW; ++n) {
        // a wave-uniform index (the compiler cannot see that tid >> 6 is)
        const int P = __builtin_amdgcn_readfirstlane((kt + (wave + n * NW) * ROWS_PER_LOAD) >> 4);
        pg[n] = bt[min(P, last_page)];
      }
    };
    auto load_rows_paged = [&](const uint16_t* gbase, int64_t pstride, int stride, const int (&col)[LPW],
                               const int (&pg)[LPW], int kt, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int n = 0; n < LPW; ++n) {
        const int i = wave + n * NW;
        if (LOADS % NW == 0 || i < LOADS) {
          const int P = (kt + i * ROWS_PER_LOAD) >> 4;
          const int slot = ld_row(n) & 15;
          const int se = P < last_page ? slot : (P == last_page ? min(slot, last_slot) : last_slot);
          const int page = min(max(pg[n], 0), p.num_pages - 1);
          load_lds16(gbase + (int64_t)page * pstride, (uint32_t)(se * stride + col[n]) * 2u, dst + i * 512);
        }
      }
    };
    int pg_next[LPW] = {};

    f32x16_t o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    // m: the row's reference (log2 units); thr: the raw score above which a tile moves it,
    // (m + kRescaleSlack) / sc; neg_mu: -m, the exponent offset of P (0 while m = -inf)
    float m = kNegInf, l = 0.0f, thr = kNegInf, neg_mu = 0.0f;
    const f32x16_t zero16 = {};
    f32x16_t s[NKB];

    auto needs = [&](int it) {
      const int kt = kbeg + it * BN;
      return wave_live && kt < rr.wend && kt + BN > rr.wbeg;
    };
    // S^T = K Q^T: product j = (kb, ks) takes its K fragment from a ring that the reads four
    // products ahead fill (program order fixed by scheduling fences, so the fragments of a
    // whole tile are never held at once)
    auto scores = [&](const uint16_t* kl) __attribute__((always_inline)) {
      constexpr int NS = NKB * NKS, RA = D == 256 ? 2 : 4;
      auto frag = [&](int j) __attribute__((always_inline)) {
        return *reinterpret_cast<const u32x4_t*>(kl + (j / NKS) * 32 * DP + k_ofs(j % NKS));
      };
      u32x4_t ring[RA + 1];
#pragma unroll
      for (int j = 0; j < RA && j < NS; ++j) ring[j] = frag(j);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        if (j + RA < NS) ring[(j + RA) % (RA + 1)] = frag(j + RA);
        const int kb = j / NKS, ks = j % NKS;
        s[kb] = mfma32x32x16<BF16>(ring[j % (RA + 1)], qf[ks], ks == 0 ? zero16 : s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // softcap / mask / online-softmax update of tile `it` (in s), then O^T += V^T . P^T
    auto softmax_pv = [&](int it, const uint16_t* vl) __attribute__((always_inline)) {
      const int kt = kbeg + it * BN;
      float sc = p.scale_log2;
      if (p.cap_out > 0.0f) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = p.cap_out * tanh_via_exp2(s[kb][r] * p.cap_in);
        sc = 1.0f;
      }
      if (!(kt >= rr.fbeg && kt + BN <= rr.fend)) {
        // key kt + kb*32 + (r/4)*8 + hi*4 + r%4 is allowed iff it lies in [key_lo, key_lo + key_n)
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
        // rows with no allowed key yet keep m = -inf (their l and O are still zero)
        const float alpha = fast_exp2(m - (m_new == kNegInf ? 0.0f : m_new));
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m = m_new;
        thr = (m + kRescaleSlack) / sc;
        neg_mu = (m == kNegInf) ? 0.0f : -m;
      }
      u32x4_t pf[NPS];
#pragma unroll
      for (int t = 0; t < NPS; ++t) {
        const int kb = t >> 1, base = (t & 1) * 8;
        float e[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) e[x] = fast_exp2(__builtin_fmaf(s[kb][base + x], sc, neg_mu));
        pf[t] = u32x4_t{pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]), pack2<BF16>(e[4], e[5]),
                        pack2<BF16>(e[6], e[7])};
        // row sum in fp32 adds: a packed dot product would hold the matrix core up
        l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
      // O^T += V^T P^T: product j = (t, db) takes its V fragment from a ring that the
      // transposing reads two products ahead fill
      constexpr int NV = NPS * NDB;
      auto vfrag = [&](int j) __attribute__((always_inline)) {
        const int t = j / NDB, db = j % NDB;
        const u32x2_t lo = lds_read_tr16(vl + t * 16 * DP + v_ofs(db));
        const u32x2_t up = lds_read_tr16(vl + (t * 16 + 8) * DP + v_ofs(db));
        return u32x4_t{lo[0], lo[1], up[0], up[1]};
      };
      u32x4_t vr[3];
      vr[0] = vfrag(0);
      if (NV > 1) vr[1] = vfrag(1);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        if (j + 2 < NV) vr[(j + 2) % 3] = vfrag(j + 2);
        o[j % NDB] = mfma32x32x16<BF16>(vr[j % 3], pf[j / NDB], o[j % NDB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    auto tile = [&](auto bufc, int it) __attribute__((always_inline)) {
      constexpr int BUF = decltype(bufc)::value;  // it % 2
      const int kt = kbeg + it * BN;
      if (it + 1 < ntiles) {
        if constexpr (PAGED) {
          load_rows_paged(kg, p.ks[0], ks2, ld_col_k, pg_next, kt + BN, k_lds + (BUF ^ 1) * TILE);
          load_rows_paged(vg, p.vs[0], vs2, ld_col_v, pg_next, kt + BN, v_lds + (BUF ^ 1) * TILE);
          if (it + 2 < ntiles) page_ids(kt + 2 * BN, pg_next);
        } else {
          load_rows(kg, ks2, ld_k, kt + BN, k_lds + (BUF ^ 1) * TILE);
          load_rows(vg, vs2, ld_v, kt + BN, v_lds + (BUF ^ 1) * TILE);
        }
      }
      if (needs(it)) {
        scores(k_lds + BUF * TILE);
        softmax_pv(it, v_lds + BUF * TILE);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };

    settle_global_loads();
    if constexpr (PAGED) {
      if (ntiles > 0) {
        int pg[LPW];
        page_ids(kbeg, pg);
        if (ntiles > 1) page_ids(kbeg + BN, pg_next);
        load_rows_paged(kg, p.ks[0], ks2, ld_col_k, pg, kbeg, k_lds);
        load_rows_paged(vg, p.vs[0], vs2, ld_col_v, pg, kbeg, v_lds);
      }
    } else {
      if (ntiles > 0) {
        load_rows(kg, ks2, ld_k, kbeg, k_lds);
        load_rows(vg, vs2, ld_v, kbeg, v_lds);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
      tile(std::integral_constant<int, 0>{}, it);
      if (it + 1 < ntiles) tile(std::integral_constant<int, 1>{}, it + 1);
    }

    if (!wave_live) return;
    const RowNorm nrm = row_norm(pair_sum(l), m, p.sinks, h);
    const float inv = nrm.inv;
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
        p.lse[idx] = nrm.lse;
      }
    }
  };  // run_item

  // (an item ends with a barrier after its last LDS read, so the next one may load at once)
  const int units = p.pair_items ? (p.q_tiles + 1) / 2 : p.q_tiles;
  const WorkItem wi = work_item(blockIdx.x, gridDim.x, units, p.hq, p.hkv, p.batch);
  const int qa = p.causal ? p.q_tiles - 1 - wi.qt : wi.qt;  // longest rows first
  const int n_items = p.pair_items && wi.qt != qa ? 2 : 1;
  for (int i = 0; i < n_items; ++i) run_item(i == 0 ? qa : wi.qt, wi.h, wi.b);
}

// ------------------------------------------- 16-bit inputs, 64 query rows per wave ----
// head_dim 128. Each wave owns two 32-row blocks of queries, so every K or V fragment read
// from LDS feeds two matrix-core products: half the LDS reads per flop of the 32-row
// kernel, at the price of one wave per SIMD (the accumulators and Q fragments of two row
// blocks take 192 AGPRs). With a single wave there is no other wave to hide the softmax
// behind the matrix cores, so the wave overlaps them itself, in program order: keys are
// taken in sub-tiles of 32, and phase X(i) issues, alternately, the products of
// S(i+1) = K Q^T and of O^T += V^T P(i-1)^T while the vector unit forms
// P(i) = 2^(S(i) sc - m) and its row sums.
//
// The reference max m. The recurrence of the tiled-attention section of the page keeps O
// scaled to the running max; any fixed reference gives the same O / l as long as no
// 2^(s sc - m) overflows the 16-bit P (or loses all its bits to underflow). So each row
// takes as its reference the max of its first sub-tile that has an unmasked key (O and l
// are still zero then), and it stays: no rescale of O ever. A later score may exceed the
// reference by up to a slack (15 for fp16 P, whose range ends at 2^16; 40 for bf16). A
// pass in which that fails for some row flags the workgroup; it then takes the exact row
// maxima in a pass of S products only and runs the attention pass again against them.
// Q is scaled by sc (the softmax scale in log2 units) once, when it is loaded, and each
// sub-tile's S product starts from -m instead of 0, so the product delivers s sc - m and
// P = 2^S takes a single instruction per score. With a softcap, Q is scaled by the
// argument factor of the cap's exponential instead, and the cap's last FMA subtracts m.
// Tiles of 64 keys with no mask, once every row of the wave has its reference, take a
// body without row maxima: the max of each phase's row sums stands guard (a P past the
// slack makes its sum pass it). The others take a body with the mask and the row maxima,
// checked after every phase, that also fixes the first references.
//
// K and V arrive in 64-key tiles by range-checked buffer loads straight into LDS, spread
// over the first phase of each tile, three LDS buffers each and one barrier per tile; the
// tile loop is unrolled over the three buffers so that every LDS address is a lane
// register plus an immediate.
// The loop is one inline-asm statement written by gen_prefill_r2.py (register map and
// schedule fixed there); this function computes its inputs.
#include "prefill_r2_clobbers.inc"

template <bool BF16, int MODE>
__global__ __launch_bounds__(256, 1) void fwd_r2_kernel(const FwdParams p) {
  constexpr int D = 128, BN = 64, RB = 2, NW = 4;
  constexpr int BM = NW * 32 * RB;
  constexpr int TILE = BN * D;
  using SW = Swizzle<D>;
  // K x3, V x3, then the redo flag
  __shared__ __attribute__((aligned(1024))) uint16_t smem[6 * TILE + 2];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_void_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const WorkItem wi = work_item(blockIdx.x, gridDim.x, p.q_tiles, p.hq, p.hkv, p.batch);
  const int h = wi.h, b = wi.b;
  const int qt = p.causal ? p.q_tiles - 1 - wi.qt : wi.qt;

  int q_off = 0, k_off = 0, Lq = p.nq, Lk = p.nk;
  if (p.cu_q != nullptr) {
    q_off = p.cu_q[b];
    Lq = p.cu_q[b + 1] - q_off;
    if (p.seq_lens_k != nullptr) {
      // keys gathered from a paged cache: sequence b's slot of max_pages * 16 tokens
      k_off = b * p.max_pages * 16;
      Lk = min(max(p.seq_lens_k[b], 0), p.max_pages * 16);
    } else {
      k_off = p.cu_k[b];
      Lk = p.cu_k[b + 1] - k_off;
    }
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
  const int64_t qs2 = p.qs[2], os2 = p.os[2];
  const int ks2 = (int)p.ks[2], vs2 = (int)p.vs[2];

  const int r1 = min(Lq, r0 + BM);
  const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
  int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
  kbeg = (kbeg / BN) * BN;
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const int w0 = r0 + wave * 32 * RB;
  int qrow[RB];
  uint32_t khi[RB], key_n[RB];
  const uint16_t* qa[RB];
  uint16_t* oa[RB];
  float* la[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qrow[rb] = w0 + rb * 32 + l32;
    const int key_lo = p.window > 0 ? qrow[rb] + delta - p.window + 1 : 0;
    const int key_hi = p.causal ? min(Lk, qrow[rb] + delta + 1) : Lk;
    key_n[rb] = (uint32_t)max(key_hi - key_lo, 0);
    khi[rb] = (uint32_t)(hi * 4 - key_lo);
    qa[rb] = qg + min(qrow[rb], Lq - 1) * qs2 + hi * 8;  // rows past Lq read the last row (never stored)
    oa[rb] = og + qrow[rb] * os2 + hi * 4;
    la[rb] = p.lse;
    if (p.lse != nullptr)
      la[rb] = p.lse + (ragged ? (int64_t)h * p.cu_q[p.batch] + q_off + qrow[rb]
                               : ((int64_t)b * p.hq + h) * p.nq + qrow[rb]);
  }
  if (ntiles == 0) {  // no allowed key for any row: O = 0, LSE = -inf (the sink with one)
    const float lse0 = p.sinks != nullptr ? p.sinks[h] : kNegInf;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (qrow[rb] < Lq) {
        // the lane's 4 entries (offset hi * 4) of each 8-entry chunk of the row
#pragma unroll
        for (int c = 0; c < D / 8; ++c)
          *reinterpret_cast<u32x2_t*>(oa[rb] + c * 8) = u32x2_t{0, 0};
        if (hi == 0 && p.lse != nullptr) *la[rb] = lse0;
      }
    return;
  }
  // byte offsets of this lane's 16 bytes in load 0 of a tile (rows wave*4 + lane/16),
  // columns swizzled as the reads expect; load n adds 16 rows
  const int ld_row0 = wave * 4 + lane / 16;
  const uint32_t ld_k0 = (uint32_t)(ld_row0 * ks2 + SW::k(ld_row0, lane % 16) * 8) * 2u;
  const uint32_t ld_v0 = (uint32_t)(ld_row0 * vs2 + SW::v(ld_row0, lane % 16) * 8) * 2u;
  // keys that every row of this wave may see: a 64-key tile inside [wlo, whi) needs no mask
  const int wlast = min(w0 + 32 * RB - 1, Lq - 1);
  const int wlo = p.window > 0 ? max(0, wlast + delta - p.window + 1) : 0;
  const int whi = p.causal ? max(0, min(Lk, w0 + delta + 1)) : Lk;
  const uint32_t k_rd = (uint32_t)(l32 * D + SW::k(l32, hi) * 8) * 2u;
  const int grp = lane >> 4, gi = lane & 15;
  const int vrow = 4 * hi + (gi >> 2);
  const uint32_t v_rd =
      (uint32_t)(vrow * D + SW::v(vrow, (grp & 1) * 2 + ((gi & 3) >> 1)) * 8 + (gi & 1) * 4) * 2u;
  // wave-uniform inputs of the statement, made visibly uniform for the SGPR constraints
  auto uni = [](auto x) __attribute__((always_inline)) {
    if constexpr (sizeof(x) == 8) {
      const uint64_t w = __builtin_bit_cast(uint64_t, x);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)w);
      const uint32_t hi32 = __builtin_amdgcn_readfirstlane((uint32_t)(w >> 32));
      return __builtin_bit_cast(decltype(x), ((uint64_t)hi32 << 32) | lo);
    } else {
      return __builtin_bit_cast(decltype(x), __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, x)));
    }
  };
  const float sc = uni(MODE == 2 ? 1.0f : fmaxf(p.scale_log2, 1.17549435e-38f));  // > 0: its reciprocal is taken
  const float cap_in = uni(p.cap_in), cap_c = uni(p.cap_out);
  const float sink2 = uni(p.sinks != nullptr ? p.sinks[h] * kLog2e : kNegInf);
  const int has_lse = uni((int)(p.lse != nullptr));
  const uint16_t* const kg_u = uni(kg);
  const uint16_t* const vg_u = uni(vg);
  const int ks2_u = uni(ks2), vs2_u = uni(vs2), Lk_u = uni(Lk), kbeg_u = uni(kbeg), ntiles_u = uni(ntiles);
  const int Lq_u = uni(Lq), wlo_u = uni(wlo), whi_u = uni(whi);
  const uint32_t lds_u = uni(lds0);

#define ATTN_R2_INPUTS                                                                                        \
  "{v[0:1]}"(qa[0]), "{v[2:3]}"(qa[1]), "{v[4:5]}"(oa[0]), "{v[6:7]}"(oa[1]), "{v[8:9]}"(la[0]),              \
      "{v[10:11]}"(la[1]), "{v12}"(khi[0]), "{v13}"(khi[1]), "{v14}"(key_n[0]), "{v15}"(key_n[1]),            \
      "{v16}"(qrow[0]), "{v17}"(qrow[1]), "{v19}"(ld_k0), "{v20}"(ld_v0), "{v21}"(k_rd),                      \
      "{v22}"(v_rd), "{s[40:41]}"(kg_u), "{s[42:43]}"(vg_u), "{s44}"(ks2_u), "{s45}"(vs2_u), "{s46}"(Lk_u),   \
      "{s47}"(kbeg_u), "{s48}"(ntiles_u), "{s49}"(sc), "{s50}"(cap_in), "{s51}"(cap_c),                         \
      "{s52}"(sink2), "{s53}"(wave), "{s54}"(Lq_u), "{s55}"(has_lse), "{s56}"(lds_u), "{s57}"(wlo_u),             \
      "{s58}"(whi_u)
  if constexpr (BF16 && MODE == 0) {
    asm volatile(
#include "prefill_r2_bf16_m0.inc"
        : : ATTN_R2_INPUTS : ATTN_R2_CLOBBERS);
  } else if constexpr (BF16 && MODE == 1) {
    asm volatile(
#include "prefill_r2_bf16_m1.inc"
        : : ATTN_R2_INPUTS : ATTN_R2_CLOBBERS);
  } else if constexpr (BF16) {
    asm volatile(
#include "prefill_r2_bf16_m2.inc"
        : : ATTN_R2_INPUTS : ATTN_R2_CLOBBERS);
  } else if constexpr (MODE == 0) {
    asm volatile(
#include "prefill_r2_f16_m0.inc"
        : : ATTN_R2_INPUTS : ATTN_R2_CLOBBERS);
  } else if constexpr (MODE == 1) {
    asm volatile(
#include "prefill_r2_f16_m1.inc"
        : : ATTN_R2_INPUTS : ATTN_R2_CLOBBERS);
  } else {
    asm volatile(
#include "prefill_r2_f16_m2.inc"
        : : ATTN_R2_INPUTS : ATTN_R2_CLOBBERS);
  }
#undef ATTN_R2_INPUTS
}

// Persistent form of the same kernel: one workgroup per CU runs a list of work items one
// after another inside the statement. Between items the next item's first K / V tiles are
// issued before the current item's O is normalised and stored, and the next item's Q
// fragments load into spare AGPRs while the current item's last P.V products run; the
// per-item cost of a fresh workgroup (Q load, first tiles, dispatch) is thereby overlapped.
// Workgroup w (on XCD w % 8) takes, in round j, item x + 8 p with x = w % 8 and p = j * n + c
// (c = w / 8 of n = G / 8 workgroups per XCD) in even rounds, j * n + n - 1 - c in odd
// ones: items keep the XCD placement of work_item(), and under a causal mask, where item
// lengths fall with the item index inside a (sequence, KV head) unit, a workgroup's long
// and short items alternate. Wave 0 writes the workgroup's item table into LDS (one
// record per item, the layout gen_prefill_r2.py documents); items whose rows see no key
// get O = 0 here and no record.
constexpr int kMaxItemsPerWG = 64;

struct ItemRec {
  uint64_t q, o, lse, k, v;
  int32_t r0, lq, lk, kbeg, ntiles;
  float sink2;
};
static_assert(sizeof(ItemRec) == 64, "an item record is 16 dwords");

template <bool BF16, int MODE>
__global__ __launch_bounds__(256, 1) void fwd_r2p_kernel(const FwdParams p, int total_items) {
  constexpr int D = 128, BN = 64, RB = 2, NW = 4;
  constexpr int BM = NW * 32 * RB;
  constexpr int TILE = BN * D;
  using SW = Swizzle<D>;
  // K x3, V x3, two redo-flag slots (16 bytes), the item table, the items without keys
  __shared__ __attribute__((aligned(1024))) uint16_t smem[6 * TILE + 8 + 2 * kMaxItemsPerWG * 32];
  ItemRec* const table = reinterpret_cast<ItemRec*>(smem + 6 * TILE + 8);
  ItemRec* const empty = table + kMaxItemsPerWG;
  __shared__ int n_items, n_empty;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_void_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool ragged = p.cu_q != nullptr;

  if (wave == 0) {
    const int G = gridDim.x, nloc = G >> 3, x = blockIdx.x & 7, c = blockIdx.x >> 3;
    const int item = x + 8 * (lane * nloc + ((lane & 1) ? nloc - 1 - c : c));
    ItemRec r{};
    bool work = false, none = false;
    if (item < total_items) {
      const WorkItem wi = work_item(item, total_items, p.q_tiles, p.hq, p.hkv, p.batch);
      const int h = wi.h, b = wi.b;
      const int qt = p.causal ? p.q_tiles - 1 - wi.qt : wi.qt;
      int q_off = 0, k_off = 0, Lq = p.nq, Lk = p.nk;
      if (ragged) {
        q_off = p.cu_q[b];
        Lq = p.cu_q[b + 1] - q_off;
        if (p.seq_lens_k != nullptr) {
          k_off = b * p.max_pages * 16;
          Lk = min(max(p.seq_lens_k[b], 0), p.max_pages * 16);
        } else {
          k_off = p.cu_k[b];
          Lk = p.cu_k[b + 1] - k_off;
        }
      }
      const int r0 = qt * BM;
      if (r0 < Lq) {
        const int hk = h / p.group;
        const int delta = Lk - Lq;
        const int r1 = min(Lq, r0 + BM);
        const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
        int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
        kbeg = (kbeg / BN) * BN;
        const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
        const int64_t qe = (ragged ? 0 : (int64_t)b * p.qs[0]) + (int64_t)h * p.qs[1] + (int64_t)q_off * p.qs[2];
        const int64_t oe = (ragged ? 0 : (int64_t)b * p.os[0]) + (int64_t)h * p.os[1] + (int64_t)q_off * p.os[2];
        const int64_t ke = (ragged ? 0 : (int64_t)b * p.ks[0]) + (int64_t)hk * p.ks[1] + (int64_t)k_off * p.ks[2];
        const int64_t ve = (ragged ? 0 : (int64_t)b * p.vs[0]) + (int64_t)hk * p.vs[1] + (int64_t)k_off * p.vs[2];
        r.q = (uint64_t)(uintptr_t)p.q + 2 * (uint64_t)qe;
        r.o = (uint64_t)(uintptr_t)p.o + 2 * (uint64_t)oe;
        r.k = (uint64_t)(uintptr_t)p.k + 2 * (uint64_t)ke;
        r.v = (uint64_t)(uintptr_t)p.v + 2 * (uint64_t)ve;
        r.lse = p.lse == nullptr ? 0
                                 : (uint64_t)(uintptr_t)(p.lse + (ragged ? (int64_t)h * p.cu_q[p.batch] + q_off
                                                                         : ((int64_t)b * p.hq + h) * p.nq));
        r.r0 = r0;
        r.lq = Lq;
        r.lk = Lk;
        r.kbeg = kbeg;
        r.ntiles = ntiles;
        work = ntiles > 0;
        none = ntiles == 0;
        // the sink in log2 units, -inf for none (the epilogue's added terms are then exact
        // no-ops); an item without keys keeps it in natural-log units: its LSE
        const float sink = p.sinks != nullptr ? p.sinks[h] : kNegInf;
        r.sink2 = none ? sink : sink * kLog2e;
      }
    }
    const uint64_t wm = __ballot(work), nm = __ballot(none);
    const uint64_t below = (1ull << lane) - 1ull;
    if (work) table[__popcll(wm & below)] = r;
    if (none) empty[__popcll(nm & below)] = r;
    if (lane == 0) {
      n_items = __popcll(wm);
      n_empty = __popcll(nm);
    }
  }
  __syncthreads();
  // items whose rows see no key: O = 0, LSE = -inf (the sink with one); thread t owns row t
  for (int e = 0; e < n_empty; ++e) {
    const ItemRec r = empty[e];
    const int row = r.r0 + tid;
    if (row < r.lq) {
      uint16_t* orow = reinterpret_cast<uint16_t*>((uintptr_t)r.o) + (int64_t)row * p.os[2];
#pragma unroll
      for (int c = 0; c < D / 8; ++c) *reinterpret_cast<u32x4_t*>(orow + c * 8) = u32x4_t{0, 0, 0, 0};
      if (r.lse != 0) reinterpret_cast<float*>((uintptr_t)r.lse)[row] = r.sink2;
    }
  }
  const int n = n_items;
  if (n == 0) return;

  const int ks2 = (int)p.ks[2], vs2 = (int)p.vs[2];
  const int ld_row0 = wave * 4 + lane / 16;
  const uint32_t ld_k0 = (uint32_t)(ld_row0 * ks2 + SW::k(ld_row0, lane % 16) * 8) * 2u;
  const uint32_t ld_v0 = (uint32_t)(ld_row0 * vs2 + SW::v(ld_row0, lane % 16) * 8) * 2u;
  const uint32_t k_rd = (uint32_t)(l32 * D + SW::k(l32, hi) * 8) * 2u;
  const int grp = lane >> 4, gi = lane & 15;
  const int vrow = 4 * hi + (gi >> 2);
  const uint32_t v_rd =
      (uint32_t)(vrow * D + SW::v(vrow, (grp & 1) * 2 + ((gi & 3) >> 1)) * 8 + (gi & 1) * 4) * 2u;
  const uint32_t lane_row = (uint32_t)(wave * 64 + l32);
  const uint32_t lane_hi = (uint32_t)hi;
  auto uni = [](auto x) __attribute__((always_inline)) {
    return __builtin_bit_cast(decltype(x), __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, x)));
  };
  const float sc = uni(MODE == 2 ? 1.0f : fmaxf(p.scale_log2, 1.17549435e-38f));
  const float cap_in = uni(p.cap_in), cap_c = uni(p.cap_out);
  const int has_lse = uni((int)(p.lse != nullptr));
  const int ks2_u = uni(ks2), vs2_u = uni(vs2);
  const uint32_t lds_u = uni(lds0);
  const int n_u = uni(n);
  const uint32_t table_u = uni(lds0 + (uint32_t)((6 * TILE + 8) * 2));
  const int win_u = uni(p.window), causal_u = uni(p.causal);
  const int qrow_b = uni((int)(p.qs[2] * 2)), orow_b = uni((int)(p.os[2] * 2));

#define ATTN_R2P_INPUTS                                                                                        \
  "{v19}"(ld_k0), "{v20}"(ld_v0), "{v21}"(k_rd), "{v22}"(v_rd), "{v249}"(lane_row), "{v250}"(lane_hi),          \
      "{s44}"(ks2_u), "{s45}"(vs2_u), "{s49}"(sc), "{s50}"(cap_in), "{s51}"(cap_c), "{s53}"(wave),             \
      "{s55}"(has_lse), "{s56}"(lds_u), "{s30}"(n_u), "{s31}"(table_u), "{s32}"(win_u), "{s33}"(causal_u),     \
      "{s34}"(qrow_b), "{s35}"(orow_b)
  if constexpr (BF16 && MODE == 0) {
    asm volatile(
#include "prefill_r2p_bf16_m0.inc"
        : : ATTN_R2P_INPUTS : ATTN_R2P_CLOBBERS);
  } else if constexpr (BF16 && MODE == 1) {
    asm volatile(
#include "prefill_r2p_bf16_m1.inc"
        : : ATTN_R2P_INPUTS : ATTN_R2P_CLOBBERS);
  } else if constexpr (BF16) {
    asm volatile(
#include "prefill_r2p_bf16_m2.inc"
        : : ATTN_R2P_INPUTS : ATTN_R2P_CLOBBERS);
  } else if constexpr (MODE == 0) {
    asm volatile(
#include "prefill_r2p_f16_m0.inc"
        : : ATTN_R2P_INPUTS : ATTN_R2P_CLOBBERS);
  } else if constexpr (MODE == 1) {
    asm volatile(
#include "prefill_r2p_f16_m1.inc"
        : : ATTN_R2P_INPUTS : ATTN_R2P_CLOBBERS);
  } else {
    asm volatile(
#include "prefill_r2p_f16_m2.inc"
        : : ATTN_R2P_INPUTS : ATTN_R2P_CLOBBERS);
  }
#undef ATTN_R2P_INPUTS
}

// ------------------------------------------------------------------ fp32 inputs ----
// 32x32x2 fp32 matrix-core products. Q.K^T contracts over head_dim with lanes 0-31
// taking the first half of D and lanes 32-63 the second; P.V contracts over keys in
// the order the S^T result registers hold them, and V is read row-major (each lane
// needs a single element per product, so no transposition is required).

template <int D, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 2) void fwd_f32_kernel(const FwdParams p) {
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
  const RowNorm nrm = row_norm(l + xor_shuffle(l, 32), m, p.sinks, h);
  const float inv = nrm.inv;
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
      p.lse[idx] = nrm.lse;
    }
  }
}

#ifndef ATTN_PREFILL_WAVES
#define ATTN_PREFILL_WAVES 8
#endif
#ifndef ATTN_PREFILL_KEYS
#define ATTN_PREFILL_KEYS 64
#endif
constexpr int kNW16 = ATTN_PREFILL_WAVES;  // waves per workgroup, 16-bit inputs
constexpr int kBN16 = ATTN_PREFILL_KEYS;   // keys per tile, 16-bit inputs
// head dims 192 and 256: 4 waves of 32 rows on 32-key tiles, two workgroups per CU (two
// waves per SIMD: one wave's softmax runs beside another's products; at 256 with the read
// and load offsets reduced to fit 256 registers). Head dim 96: the 8-wave, 64-key form of
// the smaller head dims, one 256-row workgroup per CU at two waves per SIMD (with causal
// pairing the 4-wave, 128-row form also ran two per CU, and streamed each K/V tile for half
// the rows: 0.120 -> 0.112 ms).
constexpr int nw16(int D) { return D >= 192 ? 4 : kNW16; }
constexpr int bn16(int D) { return D >= 192 ? 32 : kBN16; }
constexpr int kNW32 = 4;
constexpr int kBN32 = 32;

// Head dims 32 and 64 take 4-wave workgroups (128 rows) when 8-wave ones (256 rows) would
// not give every CU a workgroup: small batches then still spread over the whole chip
// (B=2 H=8, N <= 2048: +18-23%), while larger grids keep the 8-wave form, whose K/V
// tiles serve twice the rows (N = 4096: 4% ahead at D = 64).
bool small_grid16(int head_dim, int64_t nq, int64_t units) {
  return head_dim <= 64 && (nq + 255) / 256 * units < 256;
}

#ifndef ATTN_PREFILL_PERSISTENT
#define ATTN_PREFILL_PERSISTENT 1
#endif


template <bool BF16>
hipError_t launch_r2p(const FwdParams& p, int items, int grid, hipStream_t st) {
  if (p.cap_out > 0.0f) {
    hipLaunchKernelGGL((fwd_r2p_kernel<BF16, 2>), dim3(grid), dim3(256), 0, st, p, items);
  } else if (p.causal || p.window > 0 || p.cu_q != nullptr || p.nk % 64 != 0) {
    hipLaunchKernelGGL((fwd_r2p_kernel<BF16, 1>), dim3(grid), dim3(256), 0, st, p, items);
  } else {
    hipLaunchKernelGGL((fwd_r2p_kernel<BF16, 0>), dim3(grid), dim3(256), 0, st, p, items);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch16(const FwdParams& p, hipStream_t st) {
  const int64_t blocks = (int64_t)p.q_tiles * p.hq * p.batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if constexpr (D == 128) {
    // dense batches with more items than compute units: the persistent form, one workgroup
    // per CU (a multiple of 8, the XCD count), while each takes at most kMaxItemsPerWG items.
    // Ragged batches keep one workgroup per item: their item lengths follow the sequence
    // lengths, which the hardware's dispatch of workgroups to free CUs balances better than
    // a fixed assignment (the ragged GQA workload ran 17% slower in the persistent form).
    const int64_t cus = (int64_t)(device_cus() / 8 * 8);
    if (ATTN_PREFILL_PERSISTENT && p.cu_q == nullptr && cus >= 8 && blocks > cus && blocks <= cus * kMaxItemsPerWG)
      return launch_r2p<BF16>(p, (int)blocks, (int)cus, st);
    const dim3 grid((unsigned)blocks), block(256);
    if (p.cap_out > 0.0f) {
      hipLaunchKernelGGL((fwd_r2_kernel<BF16, 2>), grid, block, 0, st, p);
    } else if (p.causal || p.window > 0 || p.cu_q != nullptr || p.nk % 64 != 0) {
      hipLaunchKernelGGL((fwd_r2_kernel<BF16, 1>), grid, block, 0, st, p);
    } else {
      hipLaunchKernelGGL((fwd_r2_kernel<BF16, 0>), grid, block, 0, st, p);
    }
    return hipGetLastError();
  } else {
    if constexpr (D <= 64) {
      if (small_grid16(D, p.nq, (int64_t)p.batch * p.hq)) {
        hipLaunchKernelGGL((fwd_mfma16_kernel<D, 4, bn16(D), BF16>), dim3((unsigned)blocks), dim3(4 * 64), 0, st, p);
        return hipGetLastError();
      }
    }
    // causal dense batches: a workgroup takes a long and a short query tile of one
    // (sequence, head), so that every workgroup has the same work
    FwdParams pp = p;
    pp.pair_items = p.causal && p.window == 0 && p.cu_q == nullptr ? 1 : 0;
    const int64_t grid = pp.pair_items ? (int64_t)((p.q_tiles + 1) / 2) * p.hq * p.batch : blocks;
    hipLaunchKernelGGL((fwd_mfma16_kernel<D, nw16(D), bn16(D), BF16>), dim3((unsigned)grid), dim3(nw16(D) * 64), 0,
                       st, pp);
    return hipGetLastError();
  }
}

template <int D>
hipError_t launch32(const FwdParams& p, hipStream_t st) {
  dim3 grid(p.q_tiles, p.hq, p.batch);
  hipLaunchKernelGGL((fwd_f32_kernel<D, kNW32, kBN32>), grid, dim3(kNW32 * 64), 0, st, p);
  return hipGetLastError();
}

// Copy of each sequence's pages of K and V into its slot of max_pages * 16 tokens in a
// token-major workspace [S * max_pages * 16, Hkv, D]. A page of 16 tokens is one
// contiguous block in the cache and in the workspace, so the copy streams whole pages
// (nontemporal reads: the cache is read once). Workgroup (j, s) copies page j of sequence
// s if the sequence has that many pages. Page ids are clamped to the cache.
__global__ __launch_bounds__(256) void gather_kv_pages_kernel(const u32x4_t* __restrict__ kc,
                                                              const u32x4_t* __restrict__ vc,
                                                              const int32_t* __restrict__ bt,
                                                              const int32_t* __restrict__ seq_lens,
                                                              u32x4_t* __restrict__ wk, u32x4_t* __restrict__ wv,
                                                              int max_pages, int num_pages, int page16) {
  const int j = blockIdx.x, sq = blockIdx.y;
  const int L = min(max(seq_lens[sq], 0), max_pages * 16);
  if (j * 16 >= L) return;
  const int page = min(max(bt[(int64_t)sq * max_pages + j], 0), num_pages - 1);
  const u32x4_t* ks = kc + (int64_t)page * page16;
  const u32x4_t* vs = vc + (int64_t)page * page16;
  const int64_t dst = ((int64_t)sq * max_pages + j) * page16;
  for (int i = threadIdx.x; i < page16; i += 256) {
    const u32x4_t a = __builtin_nontemporal_load(ks + i);
    const u32x4_t c = __builtin_nontemporal_load(vs + i);
    wk[dst + i] = a;
    wv[dst + i] = c;
  }
}

template <int D, bool BF16>
hipError_t launch16_paged(const FwdParams& p, hipStream_t st) {
  const int64_t blocks = (int64_t)p.q_tiles * p.hq * p.batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_mfma16_kernel<D, nw16(D), bn16(D), BF16, true>), dim3((unsigned)blocks),
                     dim3(nw16(D) * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (one persistent prefill workgroup each; the decode
// plan sizes its splits by them).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

int fwd_paged_block_rows(int head_dim) { return nw16(head_dim) * 32; }

hipError_t launch_gather_kv_pages(const void* k_cache, const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, void* ws_k, void* ws_v, int num_seqs, int max_pages,
                                  int num_pages, int page_bytes, hipStream_t st) {
  hipLaunchKernelGGL(gather_kv_pages_kernel, dim3(max_pages, num_seqs), dim3(256), 0, st,
                     static_cast<const u32x4_t*>(k_cache), static_cast<const u32x4_t*>(v_cache), block_table,
                     seq_lens, static_cast<u32x4_t*>(ws_k), static_cast<u32x4_t*>(ws_v), max_pages, num_pages,
                     page_bytes / 16);
  return hipGetLastError();
}

// dtype: 1 = f16, 2 = bf16
hipError_t launch_fwd_paged(const FwdParams& p, int dtype, int head_dim, hipStream_t st) {
  switch (dtype * 1000 + head_dim) {
    case 1032: return launch16_paged<32, false>(p, st);
    case 1064: return launch16_paged<64, false>(p, st);
    case 1096: return launch16_paged<96, false>(p, st);
    case 1128: return launch16_paged<128, false>(p, st);
    case 1192: return launch16_paged<192, false>(p, st);
    case 1256: return launch16_paged<256, false>(p, st);
    case 2032: return launch16_paged<32, true>(p, st);
    case 2064: return launch16_paged<64, true>(p, st);
    case 2096: return launch16_paged<96, true>(p, st);
    case 2128: return launch16_paged<128, true>(p, st);
    case 2192: return launch16_paged<192, true>(p, st);
    case 2256: return launch16_paged<256, true>(p, st);
    default: return hipErrorInvalidValue;
  }
}

int fwd_block_rows(int dtype, int head_dim, int64_t nq, int64_t units) {
  if (dtype == 0) return kNW32 * 32;
  if (head_dim == 128) return 256;
  if (small_grid16(head_dim, nq, units)) return 4 * 32;
  return nw16(head_dim) * 32;
}

// dtype: 0 = f32, 1 = f16, 2 = bf16 (attn_dtype_t values)
hipError_t launch_fwd(const FwdParams& p, int dtype, int head_dim, hipStream_t st) {
  switch (dtype * 1000 + head_dim) {
    case 32: return launch32<32>(p, st);
    case 64: return launch32<64>(p, st);
    case 128: return launch32<128>(p, st);
    case 1032: return launch16<32, false>(p, st);
    case 1064: return launch16<64, false>(p, st);
    case 1096: return launch16<96, false>(p, st);
    case 1128: return launch16<128, false>(p, st);
    case 1192: return launch16<192, false>(p, st);
    case 1256: return launch16<256, false>(p, st);
    case 2032: return launch16<32, true>(p, st);
    case 2064: return launch16<64, true>(p, st);
    case 2096: return launch16<96, true>(p, st);
    case 2128: return launch16<128, true>(p, st);
    case 2192: return launch16<192, true>(p, st);
    case 2256: return launch16<256, true>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
