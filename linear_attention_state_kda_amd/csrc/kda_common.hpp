// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// * Scalar types and round-to-nearest-even casts (bf16/fp16 casts lower to
//   the hardware's RNE convert instructions).
// * 16x16 MFMA tiles with fp32 accumulation: the 16-bit products
//   (16x16x32, used by the 16-bit prefill, which lays out its own fragments)
//   and the fp32 fragments of the general chunk form (16x16x4 over K-blocks
//   of 16, one 16-byte fragment per lane).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- casts

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

// Four consecutive elements of T <-> fp32.
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef floatx4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<f16> { typedef f16x4 type; };

template <typename T>
__device__ __forceinline__ floatx4 load4(const T* p) {
  typename Vec4<T>::type x = *reinterpret_cast<const typename Vec4<T>::type*>(p);
  return floatx4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}
template <typename T>
__device__ __forceinline__ void store4(T* p, floatx4 v) {
  typename Vec4<T>::type x;
  x[0] = from_f32<T>(v[0]);
  x[1] = from_f32<T>(v[1]);
  x[2] = from_f32<T>(v[2]);
  x[3] = from_f32<T>(v[3]);
  *reinterpret_cast<typename Vec4<T>::type*>(p) = x;
}

// ---------------------------------------------------------------- math

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------- fragments

// 8 x 16-bit fragment type of the 16x16x32 MFMAs.
template <typename TOp> struct OpTraits;
template <> struct OpTraits<bf16> { typedef bf16x8 frag; };
template <> struct OpTraits<f16> { typedef f16x8 frag; };

template <int N> struct f32frag { float v[N]; };

// 16x16 MFMA products, fp32 accumulate.
__device__ __forceinline__ floatx4 mma(floatx4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(floatx4 c, f16x8 a, f16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
template <int N>
__device__ __forceinline__ floatx4 mma(floatx4 c, const f32frag<N>& a, const f32frag<N>& b) {
#pragma unroll
  for (int j = 0; j < N; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// fp32 fragments (general chunk form): a K-block of 16, lane l = 16 g + r
// holding indices 4g .. 4g+3 of its row, so the 16x16x4 MFMA e contracts
// over the indices 4g + e.  frag_load reads them from a K-contiguous row
// (already offset to the lane's row); reg_frag takes them from an fp32
// accumulator tile, whose lane l holds column l%16 at rows 4(l/16)+i: the
// accumulator of one product is the B fragment of the next one as it stands.
typedef f32frag<4> F32Frag;
__device__ __forceinline__ F32Frag frag_load(const float* row, int kb, int g) {
  const floatx4 x = *reinterpret_cast<const floatx4*>(row + kb * 16 + 4 * g);
  return F32Frag{{x[0], x[1], x[2], x[3]}};
}
__device__ __forceinline__ F32Frag reg_frag(floatx4 acc) { return F32Frag{{acc[0], acc[1], acc[2], acc[3]}}; }

// Buffer resource (V#) for raw byte-addressed buffer loads and stores: base
// address, byte range (accesses at offsets >= num_bytes read 0 / are dropped),
// stride 0.  The third dword is the gfx9-family default data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

__device__ __forceinline__ void set_err(int32_t* dev_err, uint32_t bits) {
  if (dev_err) atomicOr(reinterpret_cast<unsigned int*>(dev_err), bits);
}

}  // namespace kda
