// Fused conv-state update for gfx950: the short-convolution half of the KDA
// state tuple.  ("State semantics deep water", sec. 2: clearing or copying
// the conv-state slots of many tensors, given one pointer, stride and
// feature length per tensor, in one launch rather than one launch per
// tensor; the conv state is a sliding window moved by an offset copy.
// RecoverSSM summary, implementation breakdown steps 2 and 4: decode under
// speculation keeps an extended window, and the commit compacts the conv
// history to the accepted length.)
//
// Every conv tensor holds per slot `rows` positions of `dim` channels,
// position-major, its first `keep` rows being the history carried between
// steps.  One op (dst, src, shift) applies to all tensors of the call:
// src = -1 clears every row of dst; otherwise rows [0, keep) of dst become
// rows [shift, shift + keep) of src.  Bits are moved, never converted.
//
// One workgroup per (op, tensor).  Each thread owns 16-byte columns of the
// rows and walks the rows in increasing order, loading a batch of rows (of
// up to kCols of its columns) before storing it: in every column a row is
// read before it is written, so src == dst (the in-place compaction) needs
// no staging and no barrier.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kBatch = 4;   // rows loaded before they are stored ...
constexpr int kCols = 2;    // ... for this many of a thread's columns at once

__device__ __forceinline__ ConvDesc pick(const ConvSet& cs, int j) {
  switch (j) {   // constant indices only, so the argument is never copied to be indexed
    case 1: return cs.t[1];
    case 2: return cs.t[2];
    case 3: return cs.t[3];
    case 4: return cs.t[4];
    case 5: return cs.t[5];
    case 6: return cs.t[6];
    case 7: return cs.t[7];
    default: return cs.t[0];
  }
}

__global__ __launch_bounds__(kT) void kda_conv_update_kernel(ConvSet cs, const int32_t* __restrict__ dst_slot,
                                                             const int32_t* __restrict__ src_slot,
                                                             const int32_t* __restrict__ shift_in, int n_ops,
                                                             int32_t* __restrict__ dev_err) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int op = blockIdx.x / cs.n, j = blockIdx.x % cs.n;
  if (op >= n_ops) return;
  const int d = dst_slot[op], s = src_slot[op], n = shift_in[op];
  // the op is checked against the bounds common to every tensor, so all of
  // them skip it together
  const bool bad_slot = d < 0 || (int64_t)d >= cs.min_slots || s < -1 || (int64_t)s >= cs.min_slots;
  const bool bad_shift = s >= 0 && (n < 0 || n > cs.max_shift);
  if (bad_slot || bad_shift) {
    if (threadIdx.x == 0 && j == 0) set_err(dev_err, bad_slot ? 1u : 16u);
    return;
  }
  if (s == d && n == 0) return;   // in place and not moved
  const ConvDesc c = pick(cs, j);
  const int pieces = c.dim * c.elem_bytes / 16;   // 16-byte columns per row
  u32x4* const db = reinterpret_cast<u32x4*>(c.base + (int64_t)d * c.slot_stride);
  if (s < 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int e = threadIdx.x; e < c.rows * pieces; e += kT) db[e] = z;
    return;
  }
  const u32x4* const sb = reinterpret_cast<const u32x4*>(c.base + (int64_t)s * c.slot_stride) + (int64_t)n * pieces;
  for (int col0 = threadIdx.x; col0 < pieces; col0 += kT * kCols) {
    for (int r0 = 0; r0 < c.keep; r0 += kBatch) {
      u32x4 v[kCols][kBatch];
#pragma unroll
      for (int q = 0; q < kCols; ++q)
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (col0 + q * kT < pieces && r0 + b < c.keep) v[q][b] = sb[(r0 + b) * pieces + col0 + q * kT];
#pragma unroll
      for (int q = 0; q < kCols; ++q)
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
          if (col0 + q * kT < pieces && r0 + b < c.keep) db[(r0 + b) * pieces + col0 + q * kT] = v[q][b];
    }
  }
}

}  // namespace

hipError_t launch_conv_update(const ConvArgs& a, hipStream_t st) {
  if (a.n_ops == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.n_ops * a.set.n;
  hipLaunchKernelGGL(kda_conv_update_kernel, dim3((unsigned)blocks), dim3(kT), 0, st, a.set, a.dst_slot,
                     a.src_slot, a.shift, a.n_ops, a.dev_err);
  return hipGetLastError();
}

}  // namespace kda
