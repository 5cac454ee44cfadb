// Device-side helpers shared by the gfx950 kernels: bf16 conversion and
// 4-wide vector access to bf16 / fp32 buffers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muonh {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Global-memory (address space 1) access: pointers read from descriptor
// tables are generic, and generic accesses compile to flat_* instructions,
// which also count against the LDS wait counter.
#define MUONH_GLOBAL __attribute__((address_space(1)))

template <typename V>
__device__ __forceinline__ V ld_global(const void* p) {
  return *(const MUONH_GLOBAL V*)(p);  // C-style cast: generic -> global address space
}
template <typename V>
__device__ __forceinline__ void st_global(void* p, V v) {
  *(MUONH_GLOBAL V*)(p) = v;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> packed bf16x2 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t h;
  h[0] = (__bf16)a;
  h[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// 4 consecutive elements of type T <-> 4 floats.  The *_nt forms are
// non-temporal (streaming) accesses for data a kernel touches once (the
// elementwise kernels' W, M, G and u streams), so they do not displace
// cached data; the Newton-Schulz operands use the ordinary forms.
template <typename T> struct Vec4;
template <> struct Vec4<uint16_t> {
  static __device__ __forceinline__ f32x4_t widen(u32x2_t v) {
    f32x4_t r;
    r[0] = __uint_as_float(v[0] << 16);
    r[1] = __uint_as_float(v[0] & 0xffff0000u);
    r[2] = __uint_as_float(v[1] << 16);
    r[3] = __uint_as_float(v[1] & 0xffff0000u);
    return r;
  }
  static __device__ __forceinline__ f32x4_t load(const uint16_t* p) {
    return widen(ld_global<u32x2_t>(p));
  }
  static __device__ __forceinline__ f32x4_t load_nt(const uint16_t* p) {
    return widen(__builtin_nontemporal_load((const MUONH_GLOBAL u32x2_t*)p));
  }
  static __device__ __forceinline__ void store(uint16_t* p, f32x4_t v) {
    u32x2_t o;
    o[0] = pack_bf16x2(v[0], v[1]);
    o[1] = pack_bf16x2(v[2], v[3]);
    st_global<u32x2_t>(p, o);
  }
  static __device__ __forceinline__ void store1(uint16_t* p, float v) {
    st_global<uint16_t>(p, f32_to_bf16(v));
  }
};
template <> struct Vec4<float> {
  static __device__ __forceinline__ f32x4_t load(const float* p) {
    return ld_global<f32x4_t>(p);
  }
  static __device__ __forceinline__ void store(float* p, f32x4_t v) {
    st_global<f32x4_t>(p, v);
  }
  static __device__ __forceinline__ f32x4_t load_nt(const float* p) {
    return __builtin_nontemporal_load((const MUONH_GLOBAL f32x4_t*)p);
  }
  static __device__ __forceinline__ void store_nt(float* p, f32x4_t v) {
    __builtin_nontemporal_store(v, (MUONH_GLOBAL f32x4_t*)p);
  }
  static __device__ __forceinline__ void store1(float* p, float v) { st_global<float>(p, v); }
};

}  // namespace muonh
