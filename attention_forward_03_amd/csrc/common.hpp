// Device-side building blocks shared by the prefill and decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 32x32x16 matrix-core product on 16-bit inputs packed eight to a 128-bit register
// quad. Lane l supplies row (l % 32) of A and column (l % 32) of B, k-slots
// 8*(l/32) .. 8*(l/32)+7; the 32x32 fp32 result sits in 16 registers per lane:
// register r of lane l is row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// 16x16x32 matrix-core product on 16-bit inputs. Lane l supplies row (l % 16) of
// A and column (l % 16) of B, k-slots 8*(l/16) .. +7; result register r of lane
// l is row 4*(l/16) + r, column l % 16.
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Two floats -> two 16-bit values (round to nearest even), packed low-first.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  f32x2_t v = {x, y};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
}

// The two 16-bit halves of a dword, widened to float.
template <bool BF16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (BF16) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(f16x2_t, w)[0];
}
template <bool BF16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (BF16) return __builtin_bit_cast(float, w & 0xffff0000u);
  else return (float)__builtin_bit_cast(f16x2_t, w)[1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh(x) = 1 - 2 / (e^{2x} + 1); saturates to +-1 without overflow trouble
// (e^{2x} = inf gives 1, e^{2x} = 0 gives -1).
__device__ __forceinline__ float tanh_via_exp2(float x) {
  const float e = fast_exp2(x * (2.0f * kLog2e));
  return 1.0f - 2.0f * fast_rcp(e + 1.0f);
}

__device__ __forceinline__ float xor_shuffle(float v, int mask) { return __shfl_xor(v, mask, 64); }

typedef __attribute__((address_space(3))) void lds_void_t;

// One direct-to-LDS load: every lane moves 16 bytes from global address base + voff
// (bytes) to LDS address lds_base + 16 * lane (lds_base must be wave-uniform).
// Written as inline asm: with the compiler builtin for this load, every later
// transposing LDS read (ds_read_b64_tr_b16) is made to wait for all loads still in
// flight, which would serialise the K/V prefetch with the P.V product. Completion is
// awaited explicitly (s_waitcnt vmcnt) by the callers. M0 carries the LDS base; the
// statement lists it as clobbered, so the compiler keeps no value of its own there.
__device__ __forceinline__ void load_lds16(const void* base, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// The same load with the nontemporal hint: for data read once (the paged KV cache in
// decode), which then does not displace reused lines from the caches. A streaming read
// of HBM measured 7.0 TB/s with the hint against 6.2 TB/s without on MI355X.
__device__ __forceinline__ void load_lds16_stream(const void* base, uint32_t voff, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base),
               "s"(lds)
               : "memory", "m0");
}

// Wait (visibly to the compiler) for this wave's ordinary global loads, so that the
// hot loops that follow start with no compiler-tracked load outstanding and no wait
// for them is placed inside the loop (where it would also stall on prefetches).
__device__ __forceinline__ void settle_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <typename T>
__device__ __forceinline__ T load_global(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

}  // namespace attn
