// kda_device.hpp -- device-side building blocks shared by the KDA kernels
// (gfx950 / CDNA4).  Wavefront = 64 lanes; matrix products use the CDNA4
// MFMA instructions with fp32 accumulation.
//
// Fragment convention used by every matrix product in this library.
//   A 16x16 output tile in "C layout": lane l holds rows 4*(l/16)+j (j=0..3)
//   of column l%16 (floatx4).  For a reduction slab of 16 (or 32) indices,
//   lane group g = l/16 supplies the indices {4g..4g+3} (and {16+4g..16+4g+3}).
//   A and B operands are built in that same index order -- from LDS rows with
//   two 4-element reads, or directly from C-layout registers -- so that the
//   product of two operands sums over every index of the slab exactly once,
//   whatever the instruction's internal index order is (it is the same for
//   A and B).  This lets results stay in registers between products.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(f16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return static_cast<f16>(x); }

// Per-type operand fragments and MFMA wrappers.
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  typedef bf16x4 F16;   // operand fragment of a 16-index slab
  typedef bf16x8 F32;   // operand fragment of a 32-index slab
  static __device__ __forceinline__ F16 frag16(floatx4 a) {
    F16 r; r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3]; return r;
  }
  static __device__ __forceinline__ F32 frag32(floatx4 a, floatx4 b) {
    F32 r;
    r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
    r[4] = (bf16)b[0]; r[5] = (bf16)b[1]; r[6] = (bf16)b[2]; r[7] = (bf16)b[3];
    return r;
  }
  // two 4-element (8-byte) LDS reads at p and p+16
  static __device__ __forceinline__ F32 lds32(const bf16* p) {
    F16 lo = *reinterpret_cast<const F16*>(p);
    F16 hi = *reinterpret_cast<const F16*>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ F16 lds16(const bf16* p) { return *reinterpret_cast<const F16*>(p); }
  static __device__ __forceinline__ floatx4 mma32(F32 a, F32 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma16(F16 a, F16 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<f16> {
  typedef f16x4 F16;
  typedef f16x8 F32;
  static __device__ __forceinline__ F16 frag16(floatx4 a) {
    F16 r; r[0] = (_Float16)a[0]; r[1] = (_Float16)a[1]; r[2] = (_Float16)a[2]; r[3] = (_Float16)a[3]; return r;
  }
  static __device__ __forceinline__ F32 frag32(floatx4 a, floatx4 b) {
    F32 r;
    r[0] = (_Float16)a[0]; r[1] = (_Float16)a[1]; r[2] = (_Float16)a[2]; r[3] = (_Float16)a[3];
    r[4] = (_Float16)b[0]; r[5] = (_Float16)b[1]; r[6] = (_Float16)b[2]; r[7] = (_Float16)b[3];
    return r;
  }
  static __device__ __forceinline__ F32 lds32(const _Float16* p) {
    F16 lo = *reinterpret_cast<const F16*>(p);
    F16 hi = *reinterpret_cast<const F16*>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ F16 lds16(const _Float16* p) { return *reinterpret_cast<const F16*>(p); }
  static __device__ __forceinline__ floatx4 mma32(F32 a, F32 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma16(F16 a, F16 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  typedef floatx4 F16;
  typedef floatx8 F32;
  static __device__ __forceinline__ F16 frag16(floatx4 a) { return a; }
  static __device__ __forceinline__ F32 frag32(floatx4 a, floatx4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ F32 lds32(const float* p) {
    floatx4 lo = *reinterpret_cast<const floatx4*>(p);
    floatx4 hi = *reinterpret_cast<const floatx4*>(p + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  static __device__ __forceinline__ F16 lds16(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
  // fp32 products: one 16x16x4 instruction per index of the lane's group.
  static __device__ __forceinline__ floatx4 mma16(F16 a, F16 b, floatx4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ floatx4 mma32(F32 a, F32 b, floatx4 c) {
    c = mma16(__builtin_shufflevector(a, a, 0, 1, 2, 3), __builtin_shufflevector(b, b, 0, 1, 2, 3), c);
    c = mma16(__builtin_shufflevector(a, a, 4, 5, 6, 7), __builtin_shufflevector(b, b, 4, 5, 6, 7), c);
    return c;
  }
};

// 16-byte global vector of T (8 bf16 or 4 fp32)
struct alignas(16) Vec16 { uint32_t w[4]; };

template <typename T> struct VecTraits { static constexpr int N = 16 / sizeof(T); };

template <typename T>
__device__ __forceinline__ void vec_to_f32(const Vec16& v, float* out) {
  const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
  for (int i = 0; i < VecTraits<T>::N; ++i) out[i] = to_f32(e[i]);
}

__device__ __forceinline__ Vec16 ldg16(const void* p) {
  return *reinterpret_cast<const Vec16*>(p);
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// Matrix-operand types of the chunked forward, per input type T.
//   TL: products whose operands carry gate factors of the whole chunk or the
//       recurrent state (Kg Kd^T, Qg Kd^T, Qg S, W S) -- bf16 for bf16 inputs,
//       whose 8-bit exponent covers factors up to e^+-80 and any state size.
//   TF: products of bounded operands (forward substitution with L and the
//       diagonal-block inverses, Tril(Qg Kd^T) Delta, Kb^T Delta) -- fp16 for
//       bf16 inputs: 3 more mantissa bits at the same MFMA rate.
// fp32 inputs keep every operand in fp32.
template <typename T> struct Operands;
template <> struct Operands<bf16> { typedef bf16 TL; typedef f16 TF; };
template <> struct Operands<float> { typedef float TL; typedef float TF; };

}  // namespace kda
