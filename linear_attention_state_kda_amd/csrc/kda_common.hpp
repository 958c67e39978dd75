// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// * Scalar types and round-to-nearest-even casts (bf16/fp16 casts lower to
//   the hardware's RNE convert instructions).
// * 16x16 MFMA tiles with fp32 accumulation.  A "fragment" is what one lane
//   feeds into a 16 x 16 x KB product: KB/4 consecutive elements of a K-block
//   stored in a permuted order (see pos_in_block).  Because the same
//   permutation is used for both operands, any permutation gives the plain
//   contraction; the one chosen here makes the fp32 accumulator tile of one
//   product (lane l holds column l%16, rows 4*(l/16)+i) directly usable as the
//   B fragment of the next product, with no data movement.
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

// K-block size used by an operand type: 32 for the 16-bit 16x16x32 MFMAs,
// any multiple of 4 (16 or 32 here) for fp32 16x16x4.
template <typename TOp> struct OpTraits;
template <> struct OpTraits<bf16> { static constexpr int KB = 32; typedef bf16x8 frag; };
template <> struct OpTraits<f16> { static constexpr int KB = 32; typedef f16x8 frag; };

template <int N> struct f32frag { float v[N]; };

// Storage position of index `idx` (0 <= idx < KB) inside a K-block.
// KB == 32: lane group g (lanes 16g..16g+15) owns positions 8g..8g+7 which
// hold indices {4g..4g+3} and {16+4g..16+4g+3}; KB == 16: identity.
template <int KB>
__host__ __device__ constexpr int pos_in_block(int idx) {
  return KB == 16 ? idx
                  : (idx < 16 ? ((idx >> 2) << 3) + (idx & 3)
                              : (((idx - 16) >> 2) << 3) + 4 + (idx & 3));
}
template <int KB>
__host__ __device__ constexpr int pos_of(int idx) {
  return (idx / KB) * KB + pos_in_block<KB>(idx % KB);
}

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

// Fragment loads from a K-contiguous row (row pointer already offset to the
// lane's row).  kb = K-block index, g = lane / 16.
template <typename TOp, int KB> struct Frag;
template <> struct Frag<bf16, 32> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type load(const bf16* row, int kb, int g) {
    return *reinterpret_cast<const bf16x8*>(row + kb * 32 + 8 * g);
  }
};
template <> struct Frag<f16, 32> {
  typedef f16x8 type;
  __device__ __forceinline__ static type load(const f16* row, int kb, int g) {
    return *reinterpret_cast<const f16x8*>(row + kb * 32 + 8 * g);
  }
};
template <int KB> struct Frag<float, KB> {
  typedef f32frag<KB / 4> type;
  __device__ __forceinline__ static type load(const float* row, int kb, int g) {
    type f;
    const float* p = row + kb * KB + (KB / 4) * g;
#pragma unroll
    for (int j = 0; j < KB / 4; j += 4) {
      floatx4 x = *reinterpret_cast<const floatx4*>(p + j);
      f.v[j] = x[0]; f.v[j + 1] = x[1]; f.v[j + 2] = x[2]; f.v[j + 3] = x[3];
    }
    return f;
  }
};

// B fragment built from accumulator tiles held in registers: the K-block
// covers two consecutive 16-row tiles (KB == 32) or one (KB == 16).
template <typename TOp, int KB> struct RegFrag;
template <> struct RegFrag<bf16, 32> {
  __device__ __forceinline__ static bf16x8 make(floatx4 lo, floatx4 hi) {
    bf16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = (bf16)lo[i]; f[4 + i] = (bf16)hi[i]; }
    return f;
  }
};
template <> struct RegFrag<f16, 32> {
  __device__ __forceinline__ static f16x8 make(floatx4 lo, floatx4 hi) {
    f16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = (f16)lo[i]; f[4 + i] = (f16)hi[i]; }
    return f;
  }
};
template <> struct RegFrag<float, 32> {
  __device__ __forceinline__ static f32frag<8> make(floatx4 lo, floatx4 hi) {
    f32frag<8> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
    return f;
  }
};
template <> struct RegFrag<float, 16> {
  __device__ __forceinline__ static f32frag<4> make(floatx4 lo, floatx4 /*unused*/) {
    f32frag<4> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = lo[i];
    return f;
  }
};

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
