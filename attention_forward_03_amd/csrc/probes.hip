// Measurement probes for gfx950: the figures a roofline needs on this machine, taken on
// the machine (clocks are not locked, so the published peaks are upper bounds only).
//
// The roofline of the page "Agent 帮我写 CUDA：一个 Softmax Attention 算子的开发全记录"
// (section 七, the arithmetic-intensity table and its ridge point) places a kernel
// between a compute peak and a memory-bandwidth peak; these kernels measure both:
//   mfma_probe_kernel   back-to-back 32x32x16 bf16 matrix products, one wave per SIMD,
//                       on operand bits the caller supplies (the power the matrix cores
//                       draw, hence the clock they hold, depends on the data), optionally
//                       with the softmax's vector work beside them; each workgroup
//                       reports its shader-clock cycles and 100 MHz reference ticks;
//   hbm_read_kernel     a streaming read of a buffer with 16-byte nontemporal loads;
//   flush_kernel        a streaming write of zeros, to evict the caches between timed
//                       launches.
#include "common.hpp"
#include "internal.hpp"

namespace attn {
namespace {

#define ATTN_PROBE_CLOBBER                                                                              \
  "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", \
      "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23", "v24", "v25", "v26", "v27", "v28", "v29",   \
      "v30", "v31", "v32", "v33", "v34", "v35", "v36", "v37", "v38", "v39", "v40", "v41", "v42", "v43",   \
      "v44", "v45", "v46", "v47", "scc"
#define ATTN_M0 "v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], v[36:39], v[0:15]\n\t"
#define ATTN_M1 "v_mfma_f32_32x32x16_bf16 v[16:31], v[32:35], v[36:39], v[16:31]\n\t"
// the vector work of the attention loop per product: an exp2, a row-sum add and half a
// pack of two probabilities to bf16 (each exp2 result is read one product later)
#define ATTN_MIX0 "v_exp_f32 v40, v46\n\tv_add_f32 v42, v41, v42\n\tv_cvt_pk_bf16_f32 v44, v41, v45\n\t"
#define ATTN_MIX1 "v_exp_f32 v41, v47\n\tv_add_f32 v43, v40, v43\n\t"
#define ATTN_X4(x) x x x x
#define ATTN_PROBE_INIT                                                                         \
  "v_mov_b32 v32, %[a0]\n\tv_mov_b32 v33, %[a1]\n\tv_mov_b32 v34, %[a2]\n\tv_mov_b32 v35, %[a3]\n\t" \
  "v_mov_b32 v36, %[b0]\n\tv_mov_b32 v37, %[b1]\n\tv_mov_b32 v38, %[b2]\n\tv_mov_b32 v39, %[b3]\n\t" \
  "v_and_b32 v46, 0x3f7fffff, %[a0]\n\tv_and_b32 v47, 0x3f7fffff, %[b0]\n\t"                         \
  "v_mov_b32 v40, 0\n\tv_mov_b32 v41, 0\n\tv_mov_b32 v42, 0\n\tv_mov_b32 v43, 0\n\tv_mov_b32 v45, 0\n\t" \
  "v_mov_b32 v0, 0\n\tv_mov_b32 v16, 0\n\ts_mov_b32 %[cnt], %[iters]\n\ts_nop 1\n\t"
// a matrix-product result is read 16 wait states after the last product at the earliest
#define ATTN_PROBE_FINI "s_nop 7\n\ts_nop 7\n\tv_add_f32 %[acc], v0, v16\n\tv_add_f32 %[acc], %[acc], v42\n\t"

template <int MIX>
__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const uint32_t* __restrict__ operands, int iters,
                                                           uint64_t* __restrict__ clocks,
                                                           float* __restrict__ sink) {
  const int t = threadIdx.x;
  const uint32_t* src = operands + 8 * t;
  const uint32_t a0 = src[0], a1 = src[1], a2 = src[2], a3 = src[3];
  const uint32_t b0 = src[4], b1 = src[5], b2 = src[6], b3 = src[7];
  const int n = __builtin_amdgcn_readfirstlane(iters);
  float acc;
  int cnt;
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  // 32 products per trip, two independent accumulator chains; the operands stay in
  // fixed registers for the whole loop
  if constexpr (MIX == 0) {
    asm volatile(ATTN_PROBE_INIT "L_probe_%=:\n\t" ATTN_X4(ATTN_X4(ATTN_M0 ATTN_M1))
                 "s_sub_u32 %[cnt], %[cnt], 1\n\ts_cmp_lg_u32 %[cnt], 0\n\ts_cbranch_scc1 L_probe_%=\n\t" ATTN_PROBE_FINI
                 : [acc] "=&v"(acc), [cnt] "=&s"(cnt)
                 : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3), [b0] "v"(b0), [b1] "v"(b1),
                   [b2] "v"(b2), [b3] "v"(b3), [iters] "s"(n)
                 : ATTN_PROBE_CLOBBER);
  } else {
    asm volatile(ATTN_PROBE_INIT "L_probe_%=:\n\t" ATTN_X4(ATTN_X4(ATTN_M0 ATTN_MIX0 ATTN_M1 ATTN_MIX1))
                 "s_sub_u32 %[cnt], %[cnt], 1\n\ts_cmp_lg_u32 %[cnt], 0\n\ts_cbranch_scc1 L_probe_%=\n\t" ATTN_PROBE_FINI
                 : [acc] "=&v"(acc), [cnt] "=&s"(cnt)
                 : [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3), [b0] "v"(b0), [b1] "v"(b1),
                   [b2] "v"(b2), [b3] "v"(b3), [iters] "s"(n)
                 : ATTN_PROBE_CLOBBER);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 256 + t] = acc;
  if (t == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Workgroup w reads bytes [w * per, (w + 1) * per); 8 loads of 16 bytes per lane in flight.
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4_t* __restrict__ p, int64_t per16,
                                                      uint32_t* __restrict__ sink) {
  const u32x4_t* b = p + per16 * blockIdx.x;
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < per16; i += 256 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(b + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // one word per workgroup keeps the loads live
  acc ^= __shfl_xor(acc, 1, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void flush_kernel(u32x4_t* __restrict__ p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(u32x4_t{0, 0, 0, 0}, p + i);
}

}  // namespace

hipError_t launch_probe_mfma(const uint32_t* operands, int workgroups, int iters, int valu_mix, uint64_t* clocks,
                             float* sink, hipStream_t st) {
  if (valu_mix) {
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(workgroups), dim3(256), 0, st, operands, iters, clocks, sink);
  } else {
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(workgroups), dim3(256), 0, st, operands, iters, clocks, sink);
  }
  return hipGetLastError();
}

hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, int workgroups, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(workgroups), dim3(256), 0, st, static_cast<const u32x4_t*>(buf),
                     bytes / 16 / workgroups, sink);
  return hipGetLastError();
}

hipError_t launch_flush(void* buf, int64_t bytes, hipStream_t st) {
  hipLaunchKernelGGL(flush_kernel, dim3(2048), dim3(256), 0, st, static_cast<u32x4_t*>(buf), bytes / 16);
  return hipGetLastError();
}

}  // namespace attn
