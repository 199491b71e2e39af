// Device-side helpers shared by the gfx950 kernels: vector types, matrix-core
// wrappers, bf16 conversion, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define WAVE 64

// Round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return to_bf16(x); }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

// 16-byte aligned load/store of raw bytes.
struct alignas(16) Vec16 { uint32_t w[4]; };

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// 16x16 matrix-core family used by attention: D[i][j] += sum_k A[i][k] B[k][j],
// lane l feeds row/column l%16 and the k-slot group l/16; output lane l holds
// D[(l/16)*4 + r][l%16], r = 0..3.
template <typename T> struct Mfma16;
template <> struct Mfma16<bf16> {
  static constexpr int KL = 8;  // values per lane per instruction (k = 32)
  typedef bf16x8 frag;
  static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma16<float> {
  static constexpr int KL = 1;  // k = 4
  typedef float frag;
  static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 32x32 family used by the GEMM: lane l feeds row/column l%32 and k-slot group
// l/32; output lane l holds D[(r/4)*8 + (l/32)*4 + r%4][l%32], r = 0..15.
template <typename T> struct Mfma32;
template <> struct Mfma32<bf16> {
  static constexpr int KL = 8;  // k = 16
  typedef bf16x8 frag;
  static __device__ __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma32<float> {
  static constexpr int KL = 1;  // k = 2
  typedef float frag;
  static __device__ __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Global -> LDS copy of 16 bytes per lane in the buffer (MUBUF) form: lane i's
// bytes, read at base + voffset_i, land at lds + 16 i (lds wave-uniform).
// The compiler tracks this form as a plain vector-memory load, so LDS reads
// issued while it is in flight keep exact wait counts; the global (FLAT) form
// of the same copy is treated as a possible LDS access and turns every later
// LDS wait into a wait for all outstanding LDS operations.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
extern "C" __device__ void mt_raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) void* lds,
                                                  int size, int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
// descriptor of the bytes from base on: no stride, no range limit, the gfx9
// data-format word
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);
  r[2] = -1;
  r[3] = 0x00020000;
  return r;
}
__device__ __forceinline__ void copy16_to_lds(const void* base, uint32_t voffset, void* lds) {
  mt_raw_buffer_load_lds(buffer_rsrc(base), (__attribute__((address_space(3))) void*)lds, 16, (int)voffset, 0, 0, 0);
}
