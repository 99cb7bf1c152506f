// Device-side helpers shared by the gfx950 kernels of libkda: bf16 packing,
// vector loads, and the bf16 MFMA wrappers with their lane layouts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Element type tags: 0 = bf16 storage, 1 = fp32 storage.
template <int DT> struct Elem;
template <> struct Elem<0> {
  typedef uint16_t T;
  __device__ __forceinline__ static float cvt(T x) { return bf16_bits_to_f32(x); }
  __device__ __forceinline__ static float ld(const T* p, size_t i) { return bf16_bits_to_f32(p[i]); }
  __device__ __forceinline__ static void st(T* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }
  // v as it reads back after a store
  __device__ __forceinline__ static float round(float v) { return bf16_bits_to_f32(f32_to_bf16_bits(v)); }
  // 8 consecutive values starting at p[i] (i multiple of 8, 16-byte aligned)
  __device__ __forceinline__ static void ld8(const T* p, size_t i, float* out) {
    uint4 u = *reinterpret_cast<const uint4*>(p + i);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = __uint_as_float(w[j] << 16);
      out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void ld4(const T* p, size_t i, float* out) {
    uint2 u = *reinterpret_cast<const uint2*>(p + i);
    out[0] = __uint_as_float(u.x << 16);
    out[1] = __uint_as_float(u.x & 0xffff0000u);
    out[2] = __uint_as_float(u.y << 16);
    out[3] = __uint_as_float(u.y & 0xffff0000u);
  }
  __device__ __forceinline__ static void st4(T* p, size_t i, const float* v) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(p + i) = u;
  }
  __device__ __forceinline__ static void st8(T* p, size_t i, const float* v) {
    uint4 u;
    u.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    u.z = (uint32_t)f32_to_bf16_bits(v[4]) | ((uint32_t)f32_to_bf16_bits(v[5]) << 16);
    u.w = (uint32_t)f32_to_bf16_bits(v[6]) | ((uint32_t)f32_to_bf16_bits(v[7]) << 16);
    *reinterpret_cast<uint4*>(p + i) = u;
  }
};
template <> struct Elem<1> {
  typedef float T;
  __device__ __forceinline__ static float cvt(T x) { return x; }
  __device__ __forceinline__ static float ld(const T* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void st(T* p, size_t i, float v) { p[i] = v; }
  __device__ __forceinline__ static float round(float v) { return v; }
  __device__ __forceinline__ static void ld8(const T* p, size_t i, float* out) {
    float4 a = *reinterpret_cast<const float4*>(p + i);
    float4 b = *reinterpret_cast<const float4*>(p + i + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  __device__ __forceinline__ static void ld4(const T* p, size_t i, float* out) {
    float4 a = *reinterpret_cast<const float4*>(p + i);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  }
  __device__ __forceinline__ static void st4(T* p, size_t i, const float* v) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ static void st8(T* p, size_t i, const float* v) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// 8 consecutive elements kept as loaded (packed bf16 or fp32) until converted,
// so a load issued early holds as few registers as possible
template <int DT> struct Raw8;
template <> struct Raw8<0> {
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t* p, size_t i) { u = *reinterpret_cast<const uint4*>(p + i); }
  // all eight values replaced by +0 unless ok (a select on the raw words: NaN cannot pass)
  __device__ __forceinline__ void keep(bool ok) {
    u.x = ok ? u.x : 0u; u.y = ok ? u.y : 0u; u.z = ok ? u.z : 0u; u.w = ok ? u.w : 0u;
  }
  __device__ __forceinline__ void to_float(float* out) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = __uint_as_float(w[j] << 16);
      out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<1> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p, size_t i) {
    a = *reinterpret_cast<const float4*>(p + i);
    b = *reinterpret_cast<const float4*>(p + i + 4);
  }
  // one value in all eight places
  __device__ __forceinline__ void fill(float x) { a = make_float4(x, x, x, x); b = a; }
  __device__ __forceinline__ void keep(bool ok) {
    a.x = ok ? a.x : 0.f; a.y = ok ? a.y : 0.f; a.z = ok ? a.z : 0.f; a.w = ok ? a.w : 0.f;
    b.x = ok ? b.x : 0.f; b.y = ok ? b.y : 0.f; b.z = ok ? b.z : 0.f; b.w = ok ? b.w : 0.f;
  }
  __device__ __forceinline__ void to_float(float* out) const {
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16, D = A(16x32) * B(32x16) + C, one wavefront of 64 lanes.
// Lane l holds  A[row = l%16][k = 8*(l/16) .. +7],  B[k = 8*(l/16) .. +7][col = l%16],
// and D[row = 4*(l/16) .. +3][col = l%16].  (Verified on gfx950 with a probe.)
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[i];
  return r;
}
// Split fp32 values into a bf16 high part and a bf16 residual: v ~= hi + lo with
// about 16 significant bits, so products on the bf16 MFMA keep near-fp32 accuracy.
// Pairs are converted by one instruction each, and the high parts are widened back by
// a shift and a mask of the packed word (round to nearest even either way).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const bf16x2 h = __builtin_convertvector((f32x2){v[i], v[i + 1]}, bf16x2);
    const uint32_t u = __builtin_bit_cast(uint32_t, h);
    const bf16x2 l = __builtin_convertvector(
        (f32x2){v[i] - __uint_as_float(u << 16), v[i + 1] - __uint_as_float(u & 0xffff0000u)}, bf16x2);
    hi[i] = h[0]; hi[i + 1] = h[1];
    lo[i] = l[0]; lo[i + 1] = l[1];
  }
}
__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)0.0f;
  return r;
}
__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// Two 16x16 products computed transposed, so lane l holds columns 4 (l/16) .. +3 of row
// l%16 of column tiles 2s (t0) and 2s + 1 (t1), become the A-operand fragment of k step s
// (lane l: columns 32 s + 8 (l/16) .. +7 of row l%16) with two cross-lane swaps per
// register: the 32-lane swap pairs the tiles' halves, the 16-lane swap interleaves them.
__device__ __forceinline__ void pair_to_afrag(const f32x4& t0, const f32x4& t1, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(t0[i]), __float_as_uint(t1[i]), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
    out[i] = __uint_as_float(b[0]);
    out[4 + i] = __uint_as_float(b[1]);
  }
}
// x shifted down by n lanes inside each row of 16 lanes (lanes below n read 0)
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, false));
}


}  // namespace kda
