// Attention backward (dQ, dK, dV) for gfx950, 16-bit inputs, head_dim 64 or 128.
//
// The backward pass is named as the next step by "Ask, Don't Equip: Question-Driven Coding
// Agents for Deep Kernel Optimization" (section 局限与改进) and not defined there; these
// kernels compute the derivatives of the forward definition with the saved LSE, the
// recomputation scheme that the online softmax of the page "Agent 帮我写 CUDA：一个
// Softmax Attention 算子的开发全记录" (section 四) makes possible (P is rebuilt tile by
// tile from S and the row LSE, never stored):
//   P = exp(S - LSE)   dV = P^T dO   dP = dO V^T   dS = P (dP - Delta) * scale
//   (times 1 - tanh^2 under a softcap)   dQ = dS K   dK = dS^T Q,   Delta = rowsum(dO O).
// Three launches:
//   bwd_delta_kernel   -Delta and LSE log2(e) per query row (fp32); extra workgroups build
//                      the run order of the dK / dV items (longest first);
//   bwd_main_kernel    the dK / dV items, then the dQ items:
//     dK / dV item     a workgroup owns 128 keys of one KV head (4 waves of 32) and one of
//                      at most 4 equal chunks of the (query head of its group, query tile)
//                      steps that reach them, so a causal problem (where early keys meet
//                      far more queries than late ones) stays balanced; each chunk stores
//                      its fp32 partial dK, dV in a slot of its own;
//     dQ item          a workgroup owns 128 query rows (4 waves of 32) and walks the key
//                      tiles, like the forward;
//   bwd_convert_kernel adds a key's slots in a fixed order and rounds to the output type
//                      (no atomics: the result is repeatable bit for bit).
// Every product is a 32x32x16 matrix-core product with the layouts of the forward
// kernels: results are kept transposed when that puts P or dS straight into a B operand
// (dV^T = dO^T P, dK^T = Q^T dS, dQ^T = K^T dS^T), and the transposed A operands (dO^T,
// Q^T, K^T) come from row-major LDS tiles through the transposing LDS read. Q, dO and K
// tiles are read both by rows and transposed, so every tile takes one swizzle that suits
// both (BwdSwizzle) and the transposing reads apply it to their own rows; it depends on
// the row only through bits that a step of 16 rows leaves unchanged.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "prefill_shared.hpp"

namespace attn {
namespace {

// Swizzle of the tiles read both by rows (16-byte chunks, 32 rows) and by the transposing
// read (8 bytes of each of 8 rows x 4 chunks per instruction). At D = 128 (16 chunks per
// row) the forward's row swizzle c ^ (row & 15) sends a transposing read to 8 of the 16
// chunk positions: a 2-way bank conflict, and each 16-lane group of it (4 rows x 2
// chunks) reaches only 4. XOR-ing the chunk with the row's low four bits rotated left by
// one still maps a chunk column of 16 rows onto all 16 positions (row reads stay
// conflict-free), and puts the 4 rows of a 16-lane group on bits 1 and 2 of the position
// and the group's half of the wave on bit 3: 8 positions per group, 16 per instruction.
template <int D>
struct BwdSwizzle {
  __device__ static __forceinline__ int k(int row, int c) {
    if constexpr (D == 128) {
      const int r = row & 15;
      return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    } else {
      return Swizzle<D>::k(row, c);
    }
  }
};

constexpr int kBwdNW = 4;   // waves per workgroup (one per SIMD: the accumulators are large)
constexpr int kBwdBQ = kBwdQueryTile;  // query rows per step of the dK / dV items
static_assert(kBwdNW * 32 == kBwdKeyBlock, "a dK / dV workgroup owns one block of keys");

// One direct-to-LDS load of 4 bytes per lane: lane l's dword from base + voff (bytes) to
// LDS address lds_base + 4 l (the 4-byte form of load_lds16).
__device__ __forceinline__ void load_lds4(const void* base, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// x, opaque to the optimiser (kept in a register of its own, not folded into addresses)
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Direct-to-LDS loads (16 and 4 bytes per lane) to a wave-uniform LDS byte address.
__device__ __forceinline__ void load_lds16_at(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void load_lds4_at(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Direct-to-LDS load of one row-major tile of ROWS rows x D (16-bit) into LDS, swizzled
// as BwdSwizzle<D>; rows past `valid` re-read the last valid row (the masks zero them).
template <int D, int ROWS>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int RPL = 64 / CPR;            // rows per load instruction
  static constexpr int LOADS = ROWS / RPL;        // per tile
  static constexpr int LPW = LOADS / kBwdNW;      // per wave
  static_assert(LOADS % kBwdNW == 0, "tile loads split evenly over the waves");
  int row[LPW], off[LPW];
  __device__ void init(int wave, int lane, int stride) {
    using SW = BwdSwizzle<D>;
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      const int i = wave + n * kBwdNW;
      row[n] = i * RPL + lane / CPR;
      off[n] = row[n] * stride + SW::k(row[n], lane % CPR) * 8;
    }
  }
  // rows r0 .. r0 + ROWS - 1 of `base`, of which those < valid exist
  __device__ void load(const uint16_t* base, int stride, int r0, int valid, uint16_t* dst, int wave) const {
    const uint16_t* g = base + (int64_t)r0 * stride;
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      const int i = wave + n * kBwdNW;
      const int shift = r0 + row[n] < valid ? 0 : (valid - 1 - r0) - row[n];
      load_lds16(g, (uint32_t)(off[n] + shift * stride) * 2u, dst + i * 512);
    }
  }
};

// The query tiles (of kBwdBQ rows) that reach any key of the block starting at kb0: the
// first tile's row and the count (causal: rows >= key - (Nk - Nq); window: rows < key + W
// - (Nk - Nq), as the forward's mask).
struct BwdQueryRange {
  int q_lo, nqt;
};
__device__ __forceinline__ BwdQueryRange bwd_query_range(const BwdParams& p, int kb0) {
  const int delta = p.nk - p.nq;
  const int kb1 = min(p.nk, kb0 + kBwdNW * 32);
  int q_lo = p.causal ? max(0, kb0 - delta) : 0;
  const int q_hi = p.window > 0 ? min(p.nq, kb1 - 1 - delta + p.window) : p.nq;
  q_lo = (q_lo / kBwdBQ) * kBwdBQ;
  return {q_lo, q_hi > q_lo ? (q_hi - q_lo + kBwdBQ - 1) / kBwdBQ : 0};
}

// The number of dK / dV chunks that hold a partial for keys of block kb0 (one: the
// item writes dK and dV in the output type itself).
__device__ __forceinline__ int bwd_chunks_of(const BwdParams& p, int kb0) {
  const int all = bwd_query_range(p, kb0).nqt * p.group;
  return min(p.chunks, (all + p.chunk_steps - 1) / p.chunk_steps);
}

// Steps (query head, query tile) of dK / dV item `item` (= key block * chunks + chunk).
__device__ __forceinline__ int bwd_item_steps(const BwdParams& p, int item) {
  const int all = bwd_query_range(p, (item / p.chunks) * (kBwdNW * 32)).nqt * p.group;
  return min(max(all - (item % p.chunks) * p.chunk_steps, 0), p.chunk_steps);
}

// Run order of the dK / dV items of a unit (every unit has the same items): longest first,
// so that the dispatcher, which starts workgroups in grid order as CUs free up, fills the
// tail with short items (causal problems mix full chunks with short and empty ones). Item
// i's place is the number of items with a larger key, plus those with an equal key and a
// smaller index (a permutation, the same on every run); the key is the step count scaled
// to 0..255. One thread per item; each workgroup first writes all keys into LDS. Runs in
// the extra workgroups ob of the Delta kernel.
__device__ __forceinline__ void bwd_order_block(const BwdParams& p, int ob, uint8_t* keys) {
  const int n = p.kblocks * p.chunks;
  for (int i = threadIdx.x; i < n; i += 256)
    keys[i] = (uint8_t)(bwd_item_steps(p, i) * 255 / p.chunk_steps);
  __syncthreads();
  const int i = ob * 256 + threadIdx.x;
  if (i >= n) return;
  const int ki = keys[i];
  int place = 0;
  for (int j = 0; j < n; ++j) {
    const int kj = keys[j];
    place += (kj > ki) | ((kj == ki) & (j < i));
  }
  p.order[place] = i;
}

// ------------------------------------------------------------------------- Delta ----
// Delta = sum_d dO O in fp32 (both read as 16-bit), and LSE2 = LSE log2(e) of the row. D/8 consecutive lanes share a row, each
// reading 16 bytes of it, so every load instruction of a wave covers 64 / (D/8) whole rows
// of contiguous memory; the lanes of a row add their partial sums by lane exchanges.
// Workgroups from delta_blocks on build the dK / dV run order instead.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const BwdParams p, int delta_blocks) {
  constexpr int LPR = D / 8;        // lanes per row
  constexpr int RPB = 256 / LPR;    // rows per workgroup
  // the order's keys, one byte per item (the launch sizes this LDS to the item count)
  extern __shared__ __attribute__((aligned(16))) uint8_t keys[];
  if ((int)blockIdx.x >= delta_blocks) {
    bwd_order_block(p, (int)blockIdx.x - delta_blocks, keys);
    return;
  }
  const int64_t rows = (int64_t)p.batch * p.hq * p.nq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4_t a = load_global<u32x4_t>(static_cast<const uint16_t*>(p.o) + row * D + 8 * c);
    const u32x4_t b = load_global<u32x4_t>(static_cast<const uint16_t*>(p.dout) + row * D + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += lo16<BF16>(a[w]) * lo16<BF16>(b[w]) + hi16<BF16>(a[w]) * hi16<BF16>(b[w]);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += xor_shuffle(acc, off);
  if (row < rows && c == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// 32x32x16 products written out, with the accumulator in VGPRs and the B operand in AGPRs
// (the compiler would give a product's result an AGPR, which the vector work cannot read,
// and copy it out score by score). The compiler does not see these as matrix products, so
// it keeps no wait states for them: their A operands come from LDS reads and their B
// operands from AGPRs written once per item (no vector-ALU write just before), their
// results are read by other instructions only a phase later (beyond the 12 wait states
// of that hazard), and a chain's next product takes its predecessor's result as srcC,
// which is forwarded. A host test checks every such distance in the compiled kernels.
template <bool BF16>
__device__ __forceinline__ void mfma_v_first(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
template <bool BF16>
__device__ __forceinline__ void mfma_v_acc(f32x16_t& d, const u32x4_t& a, const u32x4_t& b) {
  if constexpr (BF16)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// --------------------------------------------------------------------- dK and dV ----
// Wave w of the workgroup owns keys kb0 + 32 w .. +31 and sums their dK^T and dV^T over the
// steps (query head, query tile of 32 rows) of its item. A step's Q and dO tiles and its
// rows' LSE (base 2) and Delta are staged in LDS:
//   S = Q K^T          A = Q rows (LDS), B = K^T (the wave's keys, registers)
//   P = 2^(S sc - LSE2)                                 lane: key column, 16 query rows
//   dP = dO V^T        A = dO rows (LDS), B = V^T (registers)
//   dS = P (dP - Delta) [(1 - t^2)]      (the softmax scale multiplies dK once, at the end)
//   dV^T += dO^T P     A = dO^T (transposing LDS read), B = P (16-bit)
//   dK^T += Q^T dS     A = Q^T (transposing LDS read), B = dS (16-bit)
// The steps are software pipelined: step i computes S and dP of step i + 1 beside the
// exponentials of its own P, then its dV products beside its dS, then its dK products, so
// the matrix cores of the one wave per SIMD have independent work while the vector unit
// runs. Only tiles that cut the mask or the sequence ends test pairs one by one. The
// workgroup meets at a barrier once per two steps; eight staging buffers let the loads of
// a pair of steps start two pairs ahead.
template <int D, bool BF16, bool CAP>
__device__ __forceinline__ void bwd_dkdv_item(const BwdParams& p, int w, uint16_t* smem, float* stats) {
  constexpr int BQ = kBwdBQ;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int TILE = BQ * D;
  constexpr int NBUF = 8;
  using SW = BwdSwizzle<D>;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;             // rows per load instruction
  constexpr int LPW = BQ / RPL / kBwdNW;    // tile load instructions per wave
  static_assert(BQ % (RPL * kBwdNW) == 0, "tile loads split evenly over the waves");
  constexpr int NV = 2 * LPW + 2;           // direct-to-LDS loads per wave per step
  // LDS: smem holds buffer i's Q tile at element 2 i TILE and its dO tile at 2 i TILE + TILE
  // (each [BQ][D]); stats, per buffer, LSE2 then Delta, each [4 waves][64] floats (a wave
  // loads rows 8 w .. 8 w + 7 into the first 8 entries of its slot)
  // LDS reads take a buffer's offset as the instruction's immediate, which reaches 64 KB:
  // buffers from HB on are read from lane offsets 64 KB higher
  constexpr int HB = 32768 / (2 * TILE);
  static_assert(HB * 2 * TILE == 32768 || NBUF * 2 * TILE <= 32768, "buffers split at 64 KB");

  // (wave is uniform over the wave; readfirstlane lets the compiler branch on it)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  // Workgroup w runs place w / units of the run order for unit w % units (units = sequences
  // x KV heads): the longest items of every unit come first. With a multiple of 8 units,
  // all items of a unit run on one XCD (workgroup w runs on XCD w % 8) and share its L2
  // copy of the unit's Q and dO.
  const int units = p.batch * p.hkv;
  const int unit = w % units;
  const int item = p.order != nullptr ? p.order[w / units] : w / units;
  const int g = unit % p.hkv, b = unit / p.hkv;
  const int kb0 = (item / p.chunks) * (kBwdNW * 32);
  const int chunk = item % p.chunks;
  const int Lq = p.nq, Lk = p.nk, delta = Lk - Lq;
  const int kw0 = kb0 + wave * 32;  // this wave's first key
  const int key = kw0 + l32;        // this lane's key column

  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.hkv + g) * Lk * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.hkv + g) * Lk * D;
  // K^T and V^T as B operands: lane holds head-dim entries 16 ks + 8 hi .. +7 of its key
  u32x4_t kf[NKS], vf[NKS];
  {
    const int kr = min(key, Lk - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = load_global<u32x4_t>(kg + (int64_t)kr * D + ks * 16 + hi * 8);
      vf[ks] = load_global<u32x4_t>(vg + (int64_t)kr * D + ks * 16 + hi * 8);
    }
  }
  // the query rows that see any key of the block
  const BwdQueryRange qr = bwd_query_range(p, kb0);
  const int q_lo = qr.q_lo, nqt = qr.nqt;
  const int G = p.group;
  const int all_steps = nqt * G;  // (head, query tile) pairs, head-major
  // key - query offsets a pair may have: key <= query + delta (causal), key > query + delta -
  // window (window), key < Lk; with key_rel = key - hi*4 the test is on u = key_rel - row
  const int key_rel = key - hi * 4;
  const int hi_u = key < Lk ? (p.causal ? delta + 1 : 0x40000000) : -0x40000000;
  const int lo_u = p.window > 0 ? delta - p.window + 1 : -0x40000000;
  const int st0 = chunk * p.chunk_steps;
  if (st0 >= all_steps) return;  // (uniform over the workgroup)
  const int steps = min(all_steps, st0 + p.chunk_steps);

  int rd_q[NKS], rd_q_hi[NKS];  // row l32, chunk 2 ks + hi
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    rd_q[ks] = l32 * D + SW::k(l32, 2 * ks + hi) * 8;
    rd_q_hi[ks] = opaque_int(rd_q[ks] + 32768);
  }
  const int grp = lane >> 4, gi = lane & 15;
  const int vrow = 4 * hi + (gi >> 2);
  int rd_t[2][NDB], rd_t_hi[2][NDB];  // transposing reads of rows t*16 + 8*half + vrow (add t*16*D)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int c = db * 4 + (grp & 1) * 2 + ((gi & 3) >> 1);
      const int row = 8 * hf + vrow;
      rd_t[hf][db] = row * D + SW::k(row, c) * 8 + (gi & 1) * 4;
      rd_t_hi[hf][db] = opaque_int(rd_t[hf][db] + 32768);
    }

  f32x16_t dv[NDB], dk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[db][r] = dk[db][r] = 0.0f;
  const f32x16_t zero16 = {};

  // ---- loads. Tile load n of this wave moves rows RPL (wave + n kBwdNW) .. + RPL - 1 of a
  // tile: lane l takes 16 bytes of row RPL (wave + n kBwdNW) + l / CPR into the swizzled
  // LDS tile at byte 1024 (wave + n kBwdNW) + 16 l.
  const uint32_t lds_q = (uint32_t)(uintptr_t)(const lds_void_t*)smem;
  const uint32_t lds_do = lds_q + (uint32_t)(TILE * 2);
  const uint32_t lds_st = (uint32_t)(uintptr_t)(const lds_void_t*)stats;
  int trow[LPW];      // tile row of load n
  uint32_t toff[LPW]; // its byte offset in global memory from the tile's first row
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    trow[n] = RPL * (wave + n * kBwdNW) + lane / CPR;
    toff[n] = (uint32_t)(trow[n] * D + SW::k(trow[n], lane % CPR) * 8) * 2u;
  }
  // The loads of the steps run in order: the head and first row of the next one to load
  int ld_head = g * G + st0 / max(nqt, 1), ld_q0 = q_lo + (st0 % max(nqt, 1)) * BQ;
  auto load_next = [&](int buf) __attribute__((always_inline)) {
    const int64_t row0 = ((int64_t)b * p.hq + ld_head) * Lq;
    const uint16_t* qt = static_cast<const uint16_t*>(p.q) + (row0 + ld_q0) * D;
    const uint16_t* dt = static_cast<const uint16_t*>(p.dout) + (row0 + ld_q0) * D;
    const uint32_t lq = lds_q + (uint32_t)(buf * 4 * TILE), ld = lds_do + (uint32_t)(buf * 4 * TILE);
    if (ld_q0 + BQ <= Lq) {
#pragma unroll
      for (int n = 0; n < LPW; ++n) {
        load_lds16_at(qt, toff[n], lq + 1024u * (uint32_t)(wave + n * kBwdNW));
        load_lds16_at(dt, toff[n], ld + 1024u * (uint32_t)(wave + n * kBwdNW));
      }
    } else {
      // rows past the sequence end re-read its last row (the pair test zeroes them)
#pragma unroll
      for (int n = 0; n < LPW; ++n) {
        const int shift = ld_q0 + trow[n] < Lq ? 0 : (Lq - 1 - ld_q0) - trow[n];
        const uint32_t off = toff[n] + (uint32_t)(shift * D * 2);
        load_lds16_at(qt, off, lq + 1024u * (uint32_t)(wave + n * kBwdNW));
        load_lds16_at(dt, off, ld + 1024u * (uint32_t)(wave + n * kBwdNW));
      }
    }
    const uint32_t voff = (uint32_t)min(ld_q0 + 8 * wave + (lane & 7), Lq - 1) * 4u;
    load_lds4_at(p.lse2 + row0, voff, lds_st + (uint32_t)((((buf * 2 + 0) * kBwdNW + wave) * 64) * 4));
    load_lds4_at(p.delta + row0, voff, lds_st + (uint32_t)((((buf * 2 + 1) * kBwdNW + wave) * 64) * 4));
    ld_q0 += BQ;
    if (ld_q0 >= q_lo + nqt * BQ) {
      ld_q0 = q_lo;
      ++ld_head;
    }
  };
  // waits until at most n steps' loads remain in flight (n <= 3)
  auto wait_loads = [&](int n) __attribute__((always_inline)) {
    if (n >= 3) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * NV) : "memory");
    } else if (n == 2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NV) : "memory");
    } else if (n == 1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // P of score r of a step in two stages: the exponent (and under a softcap 1 - t^2), then
  // the power of two with the pair test
  auto prob_a = [&](float sr, float lse2, float& t2r) __attribute__((always_inline)) {
    if constexpr (CAP) {
      const float t = tanh_via_exp2(sr * p.cap_in);
      t2r = 1.0f - t * t;
      return fmaf(p.cap_out, t, -lse2);
    } else {
      return fmaf(sr, p.scale_log2, -lse2);
    }
  };
  auto prob_b = [&](float xe, auto maskc, int q0, int r) __attribute__((always_inline)) {
    const float e = fast_exp2(xe);
    if constexpr (decltype(maskc)::value) {
      // query q0 + (r/4)*8 + hi*4 + r%4 sees this lane's key iff u = key - (that query) lies
      // in [lo_u, hi_u) (the causal / window offsets relative to the diagonal)
      const int u = key_rel - q0 - ((r >> 2) * 8 + (r & 3));
      const bool ok = (u < hi_u) & (u >= lo_u) & (q0 + (r >> 2) * 8 + hi * 4 + (r & 3) < Lq);
      return ok ? e : 0.0f;
    } else {
      return e;
    }
  };
  // a step's tile of this wave needs the pair test unless every pair is allowed: all its
  // rows and keys exist, its last key is at or before the first row's diagonal (causal),
  // and its first key is inside the last row's window
  auto masked_tile = [&](int q0) {
    bool full = q0 + BQ <= Lq && kw0 + 32 <= Lk;
    if (p.causal) full = full && kw0 + 31 <= q0 + delta;
    if (p.window > 0) full = full && kw0 > q0 + BQ - 1 + delta - p.window;
    return !full;
  };

  // the pipeline's start: steps st0 .. st0 + 5 in flight. Step st0's S and dP, and its P,
  // once steps st0 .. st0 + 3 have arrived (the wait for them also covers the K and V
  // fragments, loaded first)
  const int first = min(steps - st0, 6);
  for (int i = 0; i < min(first, 4); ++i) load_next(i);
  settle_global_loads();
  for (int i = 4; i < first; ++i) load_next(i);
  __syncthreads();
  constexpr int NP = 2 * NKS;         // products of S and dP (phase X)
  constexpr int NT = 4 * NDB;         // products of dV and dK (phase Y)
  constexpr int RA = 4;               // row fragments read ahead
  constexpr int E1 = 16 / NP;         // dS entries per phase-X product
  constexpr int E2 = 16 / NT;         // P entries per phase-Y product
  int cur_head_t = st0 % max(nqt, 1);  // query tile index of the step being computed
  auto tile_q0 = [&](int t) { return q_lo + t * BQ; };
  f32x16_t s = zero16, dp = zero16;  // P and dP of the current step (fp32)
  u32x4_t pb[2];                     // its P as 16-bit B operands
  float t2[16];                      // its 1 - t^2 (softcap)
  {
    u32x4_t qa[NKS], da[NKS];
    f32x4_t lse[4];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qa[ks] = *reinterpret_cast<const u32x4_t*>(smem + rd_q[ks]);
      da[ks] = *reinterpret_cast<const u32x4_t*>(smem + TILE + rd_q[ks]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lse[j] = *reinterpret_cast<const f32x4_t*>(stats + (0 * kBwdNW + j) * 64 + 4 * hi);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      s = mfma32x32x16<BF16>(qa[ks], kf[ks], s);
      dp = mfma32x32x16<BF16>(da[ks], vf[ks], dp);
    }
    const int q0 = tile_q0(cur_head_t);
    const bool masked = masked_tile(q0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float xe = prob_a(s[r], lse[r >> 2][r & 3], t2[r]);
      s[r] = masked ? prob_b(xe, std::true_type{}, q0, r) : prob_b(xe, std::false_type{}, q0, r);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) pb[t][j] = pack2<BF16>(s[8 * t + 2 * j], s[8 * t + 2 * j + 1]);
  }
  // row fragment k of the step staged in buffer buf: k even feeds the S chain (Q rows), k
  // odd the dP chain (dO rows)
  auto row_frag = [&](int buf, int k) __attribute__((always_inline)) {
    const int qo = (buf < HB ? buf : buf - HB) * 2 * TILE;
    return *reinterpret_cast<const u32x4_t*>(smem + (buf < HB ? rd_q[k >> 1] : rd_q_hi[k >> 1]) + qo +
                                             (k & 1 ? TILE : 0));
  };
  u32x4_t fr[RA + 1];
#pragma unroll
  for (int k = 0; k < RA; ++k) fr[k] = row_frag(1 % NBUF, k);
  f32x4_t del[4];  // Delta of the current step's rows
#pragma unroll
  for (int j = 0; j < 4; ++j) del[j] = *reinterpret_cast<const f32x4_t*>(stats + (1 * kBwdNW + j) * 64 + 4 * hi);

  // One step (buffer BUF). Phase X: the S and dP products of step st + 1 (buffer BUF + 1)
  // beside dS of step st. Phase Y: the dV and dK products of step st beside P of step st + 1.
  // The program order is fixed per product by scheduling fences: each product comes with
  // the LDS reads of a later one and a share of the vector work, skewed over the products
  // so that no instruction waits on the one before it. The row fragments of the next step's
  // phase X are read at the end of phase Y (buffer BUF + 2, which the barriers have made
  // complete), and the transposing reads of phase Y at the end of phase X.
  auto step = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;  // (st - st0) % NBUF
    constexpr int NXT = (BUF + 1) % NBUF;
    constexpr int QO = (BUF < HB ? BUF : BUF - HB) * 2 * TILE;
    // LSE2 of the next step's rows (lane rows 8 j + 4 hi + i, loaded by wave j into
    // entries 4 hi ..; first needed in phase Y); Delta of this step's rows came in at the
    // end of the step before
    f32x4_t lsn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      lsn[j] = *reinterpret_cast<const f32x4_t*>(stats + ((NXT * 2 + 0) * kBwdNW + j) * 64 + 4 * hi);
    if (++cur_head_t == nqt) cur_head_t = 0;
    const int q0n = tile_q0(cur_head_t);  // the next step's first row
    f32x16_t sn, dpn;
    u32x4_t sb[2], pbn[2];
    float t2n[16];
    // ---- phase X
#pragma unroll
    for (int k = 0; k < NP + 2; ++k) {
      __builtin_amdgcn_sched_barrier(0);
      if (k < NP) {
        if (k + RA < NP) fr[(k + RA) % (RA + 1)] = row_frag(NXT, k + RA);
        f32x16_t& acc = k & 1 ? dpn : sn;
        const u32x4_t& kv = k & 1 ? vf[k >> 1] : kf[k >> 1];
        if (k < 2)
          mfma_v_first<BF16>(acc, fr[k % (RA + 1)], kv);
        else
          mfma_v_acc<BF16>(acc, fr[k % (RA + 1)], kv);
      }
      // dS = P (dP - Delta) [(1 - t^2)]: dP - Delta of product k's share, the product of
      // k - 1's, packing of k - 2's
#pragma unroll
      for (int e = 0; e < E1; ++e) {
        if (k < NP) {
          const int r = k * E1 + e;
          dp[r] = dp[r] - del[r >> 2][r & 3];
        }
        if (k >= 1 && k - 1 < NP) {
          const int r = (k - 1) * E1 + e;
          float ds = s[r] * dp[r];
          if constexpr (CAP) ds *= t2[r];
          s[r] = ds;
        }
        if (k >= 2) {
          const int r = (k - 2) * E1 + e;
          if (r & 1) sb[r >> 3][(r & 7) >> 1] = pack2<BF16>(s[r - 1], s[r]);
        }
      }
      if (k < NP && k + RA < NP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase Y: product i takes its A operand from the ring slot that the transposing
    // reads two products earlier filled; P of step st + 1 without the pair test
    auto tr_frag = [&](int i) __attribute__((always_inline)) {
      const int off = QO + (i < 2 * NDB ? TILE : 0) + ((i / NDB) & 1) * 16 * D;
      const int b0 = BUF < HB ? rd_t[0][i % NDB] : rd_t_hi[0][i % NDB];
      const int b1 = BUF < HB ? rd_t[1][i % NDB] : rd_t_hi[1][i % NDB];
      const u32x2_t lo = lds_read_tr16(smem + b0 + off);
      const u32x2_t up = lds_read_tr16(smem + b1 + off);
      return u32x4_t{lo[0], lo[1], up[0], up[1]};
    };
    {
      float xe[16];
      u32x4_t ring[3];
      ring[0] = tr_frag(0);
      ring[1] = tr_frag(1);
#pragma unroll
      for (int i = 0; i < NT + 2; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i < NT) {
          if (i + 2 < NT) ring[(i + 2) % 3] = tr_frag(i + 2);
          const int db = i % NDB, t = (i / NDB) & 1;
          if (i < 2 * NDB)
            dv[db] = mfma32x32x16<BF16>(ring[i % 3], pb[t], dv[db]);
          else
            dk[db] = mfma32x32x16<BF16>(ring[i % 3], sb[t], dk[db]);
        }
        // P of step st + 1: its dP taken over and the exponent of product i's share, the
        // power of i - 1's, packing of i - 2's
#pragma unroll
        for (int e = 0; e < E2; ++e) {
          if (i < NT) {
            const int r = i * E2 + e;
            dp[r] = dpn[r];
            xe[r] = prob_a(sn[r], lsn[r >> 2][r & 3], t2n[r]);
          }
          if (i >= 1 && i - 1 < NT) {
            const int r = (i - 1) * E2 + e;
            s[r] = prob_b(xe[r], std::false_type{}, q0n, r);
          }
          if (i >= 2) {
            const int r = (i - 2) * E2 + e;
            if (r & 1) pbn[r >> 3][(r & 7) >> 1] = pack2<BF16>(s[r - 1], s[r]);
          }
        }
        if (i < NT) {
          if (i + 2 < NT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // a next tile that cuts the mask: its excluded pairs set to 0 after the fact (their
    // powers may be inf; the selection drops them)
    if (masked_tile(q0n)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int u = key_rel - q0n - ((r >> 2) * 8 + (r & 3));
        const bool ok = (u < hi_u) & (u >= lo_u) & (q0n + (r >> 2) * 8 + hi * 4 + (r & 3) < Lq);
        s[r] = ok ? s[r] : 0.0f;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) pbn[t][j] = pack2<BF16>(s[8 * t + 2 * j], s[8 * t + 2 * j + 1]);
    }
    pb[0] = pbn[0];
    pb[1] = pbn[1];
    if constexpr (CAP) {
#pragma unroll
      for (int r = 0; r < 16; ++r) t2[r] = t2n[r];
    }
    // row fragments of the next step's phase X (buffer BUF + 2), Delta of the next step's
    // rows (buffer BUF + 1)
#pragma unroll
    for (int k = 0; k < RA; ++k) fr[k] = row_frag((BUF + 2) % NBUF, k);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      del[j] = *reinterpret_cast<const f32x4_t*>(stats + ((NXT * 2 + 1) * kBwdNW + j) * 64 + 4 * hi);
  };
  // a pair of steps (st, st + 1) in buffers B0, B0 + 1: the loads of st + 6 and st + 7 go
  // into the buffers of the previous pair (which every wave has finished); at the end the
  // steps up to st + 5 must have arrived (the next pair reads buffers up to its first step
  // + 3), so those of st + 6 and st + 7 may stay in flight
  auto pair = [&](auto b0c, int st) __attribute__((always_inline)) {
    constexpr int B0 = decltype(b0c)::value;
    if (st + 6 < steps) load_next((B0 + 6) % NBUF);
    if (st + 7 < steps) load_next((B0 + 7) % NBUF);
    step(std::integral_constant<int, B0>{});
    if (st + 1 < steps) step(std::integral_constant<int, (B0 + 1) % NBUF>{});
    wait_loads(min(2, steps - (st + 6)));
    __syncthreads();
  };
  for (int st = st0; st < steps; st += NBUF) {
    pair(std::integral_constant<int, 0>{}, st);
    if (st + 2 < steps) pair(std::integral_constant<int, 2>{}, st + 2);
    if (st + 4 < steps) pair(std::integral_constant<int, 4>{}, st + 4);
    if (st + 6 < steps) pair(std::integral_constant<int, 6>{}, st + 6);
  }

  if (key >= Lk) return;
  // dK^T / dV^T: lane column = key, register r of block db = head-dim 32 db + 8 (r/4) + 4 hi + r%4
  const float sc = p.scale;
  if (bwd_chunks_of(p, kb0) == 1) {
    uint16_t* dkr = static_cast<uint16_t*>(p.dk) + (((int64_t)b * p.hkv + g) * Lk + key) * D;
    uint16_t* dvr = static_cast<uint16_t*>(p.dv) + (((int64_t)b * p.hkv + g) * Lk + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + g4 * 8 + hi * 4;
        *reinterpret_cast<u32x2_t*>(dkr + d) = u32x2_t{pack2<BF16>(dk[db][g4 * 4 + 0] * sc, dk[db][g4 * 4 + 1] * sc),
                                                       pack2<BF16>(dk[db][g4 * 4 + 2] * sc, dk[db][g4 * 4 + 3] * sc)};
        *reinterpret_cast<u32x2_t*>(dvr + d) = u32x2_t{pack2<BF16>(dv[db][g4 * 4 + 0], dv[db][g4 * 4 + 1]),
                                                       pack2<BF16>(dv[db][g4 * 4 + 2], dv[db][g4 * 4 + 3])};
      }
    return;
  }
  const int64_t slot = (int64_t)chunk * p.batch * p.hkv * Lk * D;
  float* dkr = p.dk32 + slot + (((int64_t)b * p.hkv + g) * Lk + key) * D;
  float* dvr = p.dv32 + slot + (((int64_t)b * p.hkv + g) * Lk + key) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + hi * 4;
      *reinterpret_cast<f32x4_t*>(dkr + d) = f32x4_t{dk[db][g4 * 4 + 0] * sc, dk[db][g4 * 4 + 1] * sc,
                                                      dk[db][g4 * 4 + 2] * sc, dk[db][g4 * 4 + 3] * sc};
      *reinterpret_cast<f32x4_t*>(dvr + d) =
          f32x4_t{dv[db][g4 * 4 + 0], dv[db][g4 * 4 + 1], dv[db][g4 * 4 + 2], dv[db][g4 * 4 + 3]};
    }
}


// Sum of a key's partial dK / dV slots in chunk order -> the output type (4 entries per
// thread), for key blocks of two or more chunks
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_convert_kernel(const BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nkv = (int64_t)p.batch * p.hkv * p.nk * D;
  if (4 * i >= nkv) return;
  const int key = (int)((4 * i / D) % p.nk);
  const int n = bwd_chunks_of(p, (key / (kBwdNW * 32)) * (kBwdNW * 32));
  if (n == 1) return;  // written by its dK / dV item (none: zero)
  f32x4_t u = {0.0f, 0.0f, 0.0f, 0.0f}, w = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < n; ++c) {
    u += load_global<f32x4_t>(p.dk32 + c * nkv + 4 * i);
    w += load_global<f32x4_t>(p.dv32 + c * nkv + 4 * i);
  }
  *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.dk) + 4 * i) =
      u32x2_t{pack2<BF16>(u[0], u[1]), pack2<BF16>(u[2], u[3])};
  *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.dv) + 4 * i) =
      u32x2_t{pack2<BF16>(w[0], w[1]), pack2<BF16>(w[2], w[3])};
}

// ---------------------------------------------------------------------------- dQ ----
// Wave w owns query rows r0 + 32 w .. +31 and walks the key tiles of 64 (K and V staged in
// LDS, four buffers loaded three tiles ahead). Per tile:
//   S^T = K Q^T        A = K rows (LDS), B = Q (registers)     lane: query column, keys
//   P^T = 2^(S^T sc - LSE2)
//   dP^T = V dO^T      A = V rows (LDS), B = dO (registers)
//   dS^T = P^T (dP^T - Delta) [(1 - t^2)]   (the softmax scale multiplies dQ at the end)
//   dQ^T += K^T dS^T   A = K^T (transposing LDS read), B = dS^T (16-bit)
// Pipelined like the dK / dV kernel: tile i computes S and dP of tile i + 1 beside its own
// exponentials, then its dQ products beside its dS; only tiles that cut the mask test
// pairs one by one.
template <int D, bool BF16, bool CAP>
__device__ __forceinline__ void bwd_dq_item(const BwdParams& p, int h, int yt, int b, uint16_t* smem) {
  constexpr int BN = 64;
  constexpr int NKS = D / 16, NDB = D / 32, NKB = BN / 32, NPS = BN / 16;
  constexpr int TILE = BN * D;
  constexpr int NBUF = 4;
  using SW = BwdSwizzle<D>;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;           // rows per load instruction
  constexpr int LPW = BN / RPL / kBwdNW;  // tile load instructions per wave
  static_assert(BN % (RPL * kBwdNW) == 0, "tile loads split evenly over the waves");
  constexpr int NV = 2 * LPW;             // direct-to-LDS loads per wave per tile
  // LDS: buffer i holds the K tile at element 2 i TILE, the V tile at 2 i TILE + TILE (each
  // [BN][D])
  // LDS reads take a buffer's offset as the instruction's immediate (at most 64 KB): buffers
  // from HB on are read from lane offsets 64 KB higher
  constexpr int HB = 32768 / (2 * TILE) < NBUF ? 32768 / (2 * TILE) : NBUF;
  static_assert(HB == NBUF || HB * 2 * TILE == 32768, "buffers split at 64 KB");

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  // every head's longest (causal) query tiles first: items run head-fastest, then tile, then
  // sequence (the forward's per-XCD placement measured 7% slower here)
  const int ntile = (p.nq + kBwdNW * 32 - 1) / (kBwdNW * 32);
  const int r0 = (p.causal ? ntile - 1 - yt : yt) * (kBwdNW * 32);
  const int Lq = p.nq, Lk = p.nk, delta = Lk - Lq;
  const int hk = h / p.group;
  const int qw0 = r0 + wave * 32;  // this wave's first query row
  const int qrow = qw0 + l32;
  const bool row_ok = qrow < Lq;
  const int qr = min(qrow, Lq - 1);

  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.hkv + hk) * Lk * D;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.hkv + hk) * Lk * D;
  const int64_t rowi = ((int64_t)b * p.hq + h) * Lq + qr;
  u32x4_t qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = load_global<u32x4_t>(static_cast<const uint16_t*>(p.q) + rowi * D + ks * 16 + hi * 8);
    df[ks] = load_global<u32x4_t>(static_cast<const uint16_t*>(p.dout) + rowi * D + ks * 16 + hi * 8);
  }
  const float lse2 = p.lse2[rowi];
  const float dl = p.delta[rowi];
  const float lse_use = (row_ok && lse2 != kNegInf) ? lse2 : __builtin_inff();  // P = 0 for such rows

  // keys any row of the workgroup sees
  const int r1 = min(Lq, r0 + kBwdNW * 32);
  const int kend = p.causal ? min(Lk, r1 + delta) : Lk;
  int kbeg = p.window > 0 ? max(0, r0 + delta - p.window + 1) : 0;
  kbeg = (kbeg / BN) * BN;
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
  const int key_lo = p.window > 0 ? qrow + delta - p.window + 1 : 0;
  const int key_hi = p.causal ? min(Lk, qrow + delta + 1) : Lk;
  const uint32_t key_n = (uint32_t)max(key_hi - key_lo, 0);
  // a tile needs the pair test unless every key of it is allowed for every row of the wave
  // (rows past the sequence end have P = 0 through lse_use)
  const int full_hi = p.causal ? min(Lk, qw0 + delta + 1) : Lk;         // keys below it: all rows
  const int full_lo = p.window > 0 ? qw0 + 31 + delta - p.window + 1 : 0;  // keys from it: all rows
  auto masked_tile = [&](int kt) { return !(kt + BN <= full_hi && kt >= full_lo); };

  int rd_k[NKS], rd_k_hi[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    rd_k[ks] = l32 * D + SW::k(l32, 2 * ks + hi) * 8;
    rd_k_hi[ks] = opaque_int(rd_k[ks] + 32768);
  }
  const int grp = lane >> 4, gi = lane & 15;
  const int vrow = 4 * hi + (gi >> 2);
  int rd_t[2][NDB], rd_t_hi[2][NDB];  // transposing reads of rows t*16 + 8*half + vrow (add t*16*D)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int c = db * 4 + (grp & 1) * 2 + ((gi & 3) >> 1);
      const int row = 8 * hf + vrow;
      rd_t[hf][db] = row * D + SW::k(row, c) * 8 + (gi & 1) * 4;
      rd_t_hi[hf][db] = opaque_int(rd_t[hf][db] + 32768);
    }

  f32x16_t dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;
  const f32x16_t zero16 = {};

  // ---- loads: tile load n of this wave moves rows RPL (wave + n kBwdNW) .. + RPL - 1 of a
  // tile into the swizzled LDS tile at byte 1024 (wave + n kBwdNW) + 16 lane
  const uint32_t lds_k = (uint32_t)(uintptr_t)(const lds_void_t*)smem;
  int trow[LPW];
  uint32_t toff[LPW];
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    trow[n] = RPL * (wave + n * kBwdNW) + lane / CPR;
    toff[n] = (uint32_t)(trow[n] * D + SW::k(trow[n], lane % CPR) * 8) * 2u;
  }
  auto load_tile = [&](int it, int buf) __attribute__((always_inline)) {
    const int kt = kbeg + it * BN;
    const uint16_t* kt_g = kg + (int64_t)kt * D;
    const uint16_t* vt_g = vg + (int64_t)kt * D;
    const uint32_t lk = lds_k + (uint32_t)(buf * 4 * TILE), lv = lk + (uint32_t)(2 * TILE);
    if (kt + BN <= Lk) {
#pragma unroll
      for (int n = 0; n < LPW; ++n) {
        load_lds16_at(kt_g, toff[n], lk + 1024u * (uint32_t)(wave + n * kBwdNW));
        load_lds16_at(vt_g, toff[n], lv + 1024u * (uint32_t)(wave + n * kBwdNW));
      }
    } else {
      // rows past the sequence end re-read its last row (the pair test zeroes them)
#pragma unroll
      for (int n = 0; n < LPW; ++n) {
        const int shift = kt + trow[n] < Lk ? 0 : (Lk - 1 - kt) - trow[n];
        const uint32_t off = toff[n] + (uint32_t)(shift * D * 2);
        load_lds16_at(kt_g, off, lk + 1024u * (uint32_t)(wave + n * kBwdNW));
        load_lds16_at(vt_g, off, lv + 1024u * (uint32_t)(wave + n * kBwdNW));
      }
    }
  };

  // P^T of a score of a tile (without the pair test), and under a softcap dS^T directly
  auto prob1 = [&](float sr, float dpr) __attribute__((always_inline)) {
    float e;
    if constexpr (CAP) {
      const float t = tanh_via_exp2(sr * p.cap_in);
      e = fast_exp2(fmaf(p.cap_out, t, -lse_use));
      e *= (dpr - dl) * (1.0f - t * t);
    } else {
      e = fast_exp2(fmaf(sr, p.scale_log2, -lse_use));
    }
    return e;
  };

  // the pipeline's start: tiles 0 .. 2 in flight; S^T and dP^T of tile 0 once 0 and 1 arrived
  // (the wait for them also covers the row's Q, dO, LSE2 and Delta, loaded first)
  for (int i = 0; i < min(ntiles, 2); ++i) load_tile(i, i);
  settle_global_loads();
  if (ntiles > 2) load_tile(2, 2);
  __syncthreads();
  f32x16_t s[NKB], dp[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s[kb] = zero16;
    dp[kb] = zero16;
  }
  if (ntiles > 0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(smem + kb * 32 * D + rd_k[ks]);
        const u32x4_t va = *reinterpret_cast<const u32x4_t*>(smem + TILE + kb * 32 * D + rd_k[ks]);
        s[kb] = mfma32x32x16<BF16>(ka, qf[ks], s[kb]);
        dp[kb] = mfma32x32x16<BF16>(va, df[ks], dp[kb]);
      }
  }

  auto tile = [&](auto bufc, int it) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;  // it % NBUF
    constexpr int NXT = (BUF + 1) % NBUF;
    constexpr int NP = 2 * NKS * NKB;  // products of S^T and dP^T (phase 1)
    constexpr int NT = NPS * NDB;      // products of dQ^T (phase 2)
    constexpr int RA = 4;              // row fragments read ahead in phase 1
    constexpr int E1 = 16 * NKB / NP;  // scores turned into P per phase-1 product
    constexpr int KO = (BUF < HB ? BUF : BUF - HB) * 2 * TILE;
    constexpr int KN = (NXT < HB ? NXT : NXT - HB) * 2 * TILE;
    const int kt = kbeg + it * BN;
    // buffer (BUF + 3) % NBUF was last read in tile it - 1, which every wave has finished
    if (it + 3 < ntiles) load_tile(it + 3, (BUF + 3) % NBUF);
    // row fragment k of tile it + 1 (buffer NXT, complete since the end of tile it - 1;
    // stale after the last tile, its products then dropped): block kb = k / (2 NKS), even k
    // feed the S^T chain (K rows), odd k the dP^T chain (V rows)
    auto row_frag = [&](int k) __attribute__((always_inline)) {
      const int kb = k / (2 * NKS), ks = (k % (2 * NKS)) >> 1;
      return *reinterpret_cast<const u32x4_t*>(smem + (NXT < HB ? rd_k[ks] : rd_k_hi[ks]) + KN +
                                               (k & 1 ? TILE : 0) + kb * 32 * D);
    };
    u32x4_t fr[RA + 1];
#pragma unroll
    for (int k = 0; k < RA; ++k) fr[k] = row_frag(k);
    const uint32_t base = (uint32_t)(kt + hi * 4 - key_lo);
    f32x16_t sn[NKB], dpn[NKB];
    // phase 1: S^T and dP^T of tile it + 1 beside P^T of tile it (program order fixed per
    // product by scheduling fences)
    {
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        if (k + RA < NP) fr[(k + RA) % (RA + 1)] = row_frag(k + RA);
        const int kb = k / (2 * NKS), ks = (k % (2 * NKS)) >> 1;
        f32x16_t& acc = k & 1 ? dpn[kb] : sn[kb];
        const u32x4_t& bq = k & 1 ? df[ks] : qf[ks];
        if (ks == 0)
          mfma_v_first<BF16>(acc, fr[k % (RA + 1)], bq);
        else
          mfma_v_acc<BF16>(acc, fr[k % (RA + 1)], bq);
#pragma unroll
        for (int e = 0; e < E1; ++e) {
          const int x = k * E1 + e, xb = x >> 4, xr = x & 15;
          s[xb][xr] = prob1(s[xb][xr], dp[xb][xr]);
        }
        if (k + RA < NP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // a tile that cuts the mask: its excluded pairs set to 0 after the fact (a select, so an
    // inf power is dropped). Key kt + kb*32 + (r/4)*8 + hi*4 + r%4 is allowed iff it lies in
    // [key_lo, key_lo + key_n)
    if (masked_tile(kt)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = base + (uint32_t)(kb * 32 + (r >> 2) * 8 + (r & 3)) < key_n;
          s[kb][r] = ok ? s[kb][r] : 0.0f;
        }
    }
    // phase 2: dQ^T += K^T dS^T over the tile's four 16-key steps t; the dS of step t + 1
    // is computed and packed beside the products of step t
    auto ds_pack = [&](int t) __attribute__((always_inline)) {
      const int kb = t >> 1, o8 = (t & 1) * 8;
      if constexpr (!CAP) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s[kb][o8 + j] = s[kb][o8 + j] * (dp[kb][o8 + j] - dl);
      }
      return u32x4_t{pack2<BF16>(s[kb][o8 + 0], s[kb][o8 + 1]), pack2<BF16>(s[kb][o8 + 2], s[kb][o8 + 3]),
                     pack2<BF16>(s[kb][o8 + 4], s[kb][o8 + 5]), pack2<BF16>(s[kb][o8 + 6], s[kb][o8 + 7])};
    };
    auto tr_frag = [&](int i) __attribute__((always_inline)) {
      const int t = i / NDB, db = i % NDB;
      const int off = KO + t * 16 * D;
      const int b0 = BUF < HB ? rd_t[0][db] : rd_t_hi[0][db];
      const int b1 = BUF < HB ? rd_t[1][db] : rd_t_hi[1][db];
      const u32x2_t lo = lds_read_tr16(smem + b0 + off);
      const u32x2_t up = lds_read_tr16(smem + b1 + off);
      return u32x4_t{lo[0], lo[1], up[0], up[1]};
    };
    u32x4_t ring[3], pbs[NPS];
    ring[0] = tr_frag(0);
    ring[1] = tr_frag(1);
    pbs[0] = ds_pack(0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < NT) ring[(i + 2) % 3] = tr_frag(i + 2);
      const int t = i / NDB, db = i % NDB;
      dq[db] = mfma32x32x16<BF16>(ring[i % 3], pbs[t], dq[db]);
      // dS of step t + 1, a share beside each product of step t, packed beside the last
      if (t + 1 < NPS) {
        const int kb = (t + 1) >> 1, o8 = ((t + 1) & 1) * 8;
        if constexpr (!CAP) {
#pragma unroll
          for (int j = db * (8 / NDB); j < (db + 1) * (8 / NDB); ++j)
            s[kb][o8 + j] = s[kb][o8 + j] * (dp[kb][o8 + j] - dl);
        }
        if (db == NDB - 1)
          pbs[t + 1] = u32x4_t{pack2<BF16>(s[kb][o8 + 0], s[kb][o8 + 1]), pack2<BF16>(s[kb][o8 + 2], s[kb][o8 + 3]),
                               pack2<BF16>(s[kb][o8 + 4], s[kb][o8 + 5]), pack2<BF16>(s[kb][o8 + 6], s[kb][o8 + 7])};
      }
      if (i + 2 < NT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = sn[kb];
      dp[kb] = dpn[kb];
    }
    // tile it + 2 is complete once at most the loads of tile it + 3 remain
    if (it + 3 < ntiles) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NV) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += NBUF) {
    tile(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntiles) tile(std::integral_constant<int, 1>{}, it + 1);
    if (it + 2 < ntiles) tile(std::integral_constant<int, 2>{}, it + 2);
    if (it + 3 < ntiles) tile(std::integral_constant<int, 3>{}, it + 3);
  }

  if (!row_ok) return;
  uint16_t* dqr = static_cast<uint16_t*>(p.dq) + (((int64_t)b * p.hq + h) * Lq + qrow) * D;
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = db * 32 + g4 * 8 + hi * 4;
      *reinterpret_cast<u32x2_t*>(dqr + d) =
          u32x2_t{pack2<BF16>(dq[db][g4 * 4 + 0] * sc, dq[db][g4 * 4 + 1] * sc),
                  pack2<BF16>(dq[db][g4 * 4 + 2] * sc, dq[db][g4 * 4 + 3] * sc)};
    }
}

// ------------------------------------------------------------------------ main ----
// One launch runs the dK / dV items (longest first) and then the dQ items: the dQ items
// start on the CUs that the dK / dV tail frees. Both kinds use one LDS allocation.
template <int D>
struct BwdLds {
  static constexpr int kv_tiles = 2 * 8 * kBwdBQ * D * 2;      // bytes: 8 Q and dO buffers
  static constexpr int kv = kv_tiles + 8 * 2 * kBwdNW * 64 * 4;  // and their LSE2 / Delta
  static constexpr int dq = 2 * 4 * 64 * D * 2;                // 4 K and V buffers
  static constexpr int bytes = kv > dq ? kv : dq;
};

template <int D, bool BF16, bool CAP>
__global__ __launch_bounds__(kBwdNW * 64, 1) void bwd_main_kernel(const BwdParams p, int kv_items) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[BwdLds<D>::bytes];
  const int w = blockIdx.x;
  if (w < kv_items) {
    bwd_dkdv_item<D, BF16, CAP>(p, w, reinterpret_cast<uint16_t*>(lds),
                                reinterpret_cast<float*>(lds + BwdLds<D>::kv_tiles));
  } else {
    const int j = w - kv_items;
    const int ntile = (p.nq + kBwdNW * 32 - 1) / (kBwdNW * 32);
    bwd_dq_item<D, BF16, CAP>(p, j % p.hq, (j / p.hq) % ntile, j / (p.hq * ntile), reinterpret_cast<uint16_t*>(lds));
  }
}

template <int D, bool BF16>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.batch * p.hq * p.nq;
  constexpr int kDeltaRows = 256 / (D / 8);  // rows per workgroup of bwd_delta_kernel
  BwdParams q = p;
  q.kblocks = (p.nk + kBwdNW * 32 - 1) / (kBwdNW * 32);
  const int64_t kv_items = (int64_t)q.kblocks * p.chunks * p.hkv * p.batch;
  const int64_t dq_items = (int64_t)p.hq * ((p.nq + kBwdNW * 32 - 1) / (kBwdNW * 32)) * p.batch;
  const int64_t delta_blocks = (rows + kDeltaRows - 1) / kDeltaRows;
  const int64_t order_blocks = q.order != nullptr ? ((int64_t)q.kblocks * p.chunks + 255) / 256 : 0;
  if (kv_items + dq_items > 0x7fffffff || delta_blocks + order_blocks > 0x7fffffff)
    return hipErrorInvalidConfiguration;
  const size_t keys_bytes = q.order != nullptr ? (((size_t)q.kblocks * p.chunks + 15) & ~(size_t)15) : 0;
  hipLaunchKernelGGL((bwd_delta_kernel<D, BF16>), dim3((unsigned)(delta_blocks + order_blocks)), dim3(256), keys_bytes,
                     st, q, (int)delta_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(kv_items + dq_items));
  if (p.cap_out > 0.0f)
    hipLaunchKernelGGL((bwd_main_kernel<D, BF16, true>), grid, dim3(kBwdNW * 64), 0, st, q, (int)kv_items);
  else
    hipLaunchKernelGGL((bwd_main_kernel<D, BF16, false>), grid, dim3(kBwdNW * 64), 0, st, q, (int)kv_items);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nkv4 = (int64_t)p.batch * p.hkv * p.nk * D / 4;  // float4s per accumulator slot
  hipLaunchKernelGGL((bwd_convert_kernel<D, BF16>), dim3((unsigned)((nkv4 + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// dtype: 1 = f16, 2 = bf16
hipError_t launch_bwd(const BwdParams& p, int dtype, int head_dim, hipStream_t st) {
  switch (dtype * 1000 + head_dim) {
    case 1064: return launch_bwd_t<64, false>(p, st);
    case 1128: return launch_bwd_t<128, false>(p, st);
    case 2064: return launch_bwd_t<64, true>(p, st);
    case 2128: return launch_bwd_t<128, true>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
