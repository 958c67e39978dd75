// Indexed whole-state copy for gfx950: rollback restores the state saved at
// the verify point and a fork gives each candidate its own copy; both are
// exact block copies of a fixed-size state (state-semantics page, secs. 2-3).
// One launch covers every (src, dst) pair, as the fused slot copy of sec. 2
// does, so many small copies are not launch-bound.
//
// Grid: blocks_per_pair consecutive blocks per pair; each thread moves 4 x 16
// bytes with non-temporal loads issued before the stores.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kVec = 4;                   // 16-byte vectors per thread per block
constexpr int64_t kBlockBytes = kT * kVec * 16;

// Pairs that share a source (a fork: one checkpoint to several children)
// are copied by the blocks of the group's first valid pair: each part of
// the source is read once and written to every destination of the group.
// Groups are formed within windows of kT consecutive pairs, so a block looks
// at no more than kT entries of the lists and the launch stays linear in
// n_pairs; a source whose pairs fall in several windows is read once per
// window.
__global__ __launch_bounds__(kT) void kda_copy_kernel(uint8_t* __restrict__ pool, int64_t n_slots,
                                                      int64_t slot_bytes, int blocks_per_pair,
                                                      const int32_t* __restrict__ src_slot,
                                                      const int32_t* __restrict__ dst_slot,
                                                      int n_pairs, int32_t* __restrict__ dev_err) {
  __shared__ int s_dst[kT];
  __shared__ int s_n, s_follower;
  const int pair = blockIdx.x / blocks_per_pair;
  const int part = blockIdx.x % blocks_per_pair;
  if (pair >= n_pairs) return;
  auto slot_ok = [&](int x) { return x >= 0 && (int64_t)x < n_slots; };
  const int s = src_slot[pair], d = dst_slot[pair];
  if (!slot_ok(s) || !slot_ok(d)) {
    if (part == 0 && threadIdx.x == 0) set_err(dev_err, 1u);
    return;
  }
  const int w0 = pair / kT * kT, w1 = min(w0 + kT, n_pairs);   // this pair's window
  // an earlier valid pair of the window with the same source leads the group
  if (threadIdx.x == 0) {
    s_follower = 0;
    s_n = 0;
  }
  __syncthreads();
  const int q = w0 + threadIdx.x;
  const int sq = q < w1 ? src_slot[q] : -1;
  if (q < pair && sq == s && slot_ok(dst_slot[q])) s_follower = 1;
  __syncthreads();
  if (s_follower) return;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* sp = reinterpret_cast<const u32x4*>(pool + (int64_t)s * slot_bytes);
  const int64_t n16 = slot_bytes / 16;
  const int64_t base = (int64_t)part * (kT * kVec) + threadIdx.x;
  u32x4 buf[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int64_t e = base + (int64_t)i * kT;
    if (e < n16) buf[i] = __builtin_nontemporal_load(sp + e);
  }
  // the group's destinations in the window (a pair whose destination is its
  // source is a no-op)
  if (q >= pair && sq == s) {
    const int dq = dst_slot[q];
    if (slot_ok(dq) && dq != s) s_dst[atomicAdd(&s_n, 1)] = dq;
  }
  __syncthreads();
  const int n = s_n;
  for (int j = 0; j < n; ++j) {
    u32x4* dp = reinterpret_cast<u32x4*>(pool + (int64_t)s_dst[j] * slot_bytes);
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const int64_t e = base + (int64_t)i * kT;
      if (e < n16) __builtin_nontemporal_store(buf[i], dp + e);
    }
  }
}

}  // namespace

hipError_t launch_copy(const CopyArgs& a, hipStream_t st) {
  if (a.n_pairs == 0) return hipSuccess;
  const int bpp = (int)((a.slot_bytes + kBlockBytes - 1) / kBlockBytes);
  const int64_t blocks = (int64_t)bpp * a.n_pairs;
  hipLaunchKernelGGL(kda_copy_kernel, dim3((unsigned)blocks), dim3(kT), 0, st,
                     static_cast<uint8_t*>(a.pool.base), a.pool.n_slots, a.slot_bytes, bpp,
                     a.src_slot, a.dst_slot, a.n_pairs, a.dev_err);
  return hipGetLastError();
}

}  // namespace kda
