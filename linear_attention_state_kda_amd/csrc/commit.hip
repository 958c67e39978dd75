// RecoverSSM commit for gfx950 (vLLM PR #51855 summary, implementation
// breakdown step 4): rebuild the state after n accepted positions in one
// pass, without re-running the recurrence,
//   S_n = Diag(A) S_0 + sum_{t<n} c_t u_t^T,
//   c_t = k_t * prod_{t<s<n} alpha_s,   A = prod_{s<n} alpha_s,
// where the products are accumulated in reverse order t = n-1 .. 0 with a
// running decay.  Every state element is read once and written once (one
// RNE cast into the pool dtype); an in-place request with n = 0 is skipped.
//
// One workgroup per (request, head).  Thread layout: 32 threads span one
// 512-byte state row (4 consecutive key entries each) and a thread owns 16
// rows, so each wave touches 1 KiB contiguous per load.  The decayed keys
// c_t and the corrections u_t of a block of 32 positions are staged in LDS.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kD = 128;
constexpr int kRows = 16;   // rows per thread
constexpr int kBlk = 32;    // positions staged per pass

template <typename TPool, typename TRec>
__global__ __launch_bounds__(kT) void kda_commit_kernel(
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ ckpt,
    const int32_t* __restrict__ dst_slot, const int32_t* __restrict__ accepted,
    const float* __restrict__ u_rec, const TRec* __restrict__ kg_rec, int n_req, int L, int H,
    int32_t* __restrict__ dev_err) {
  __shared__ float s_c[kBlk][kD];
  __shared__ float s_u[kBlk][kD];
  __shared__ float s_dec[kD];

  const int tid = threadIdx.x;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= n_req) return;
  const int n = accepted[r];
  const int src = ckpt[r];
  const int dst = dst_slot ? dst_slot[r] : src;
  if (n < 0 || n > L) {
    if (tid == 0 && h == 0) set_err(dev_err, 1u << 2);
    return;
  }
  if (src < 0 || (int64_t)src >= n_slots || dst < 0 || (int64_t)dst >= n_slots) {
    if (tid == 0 && h == 0) set_err(dev_err, 1u);
    return;
  }
  if (n == 0 && dst == src) return;  // nothing accepted, checkpoint already right

  const int kq = tid & 31, r0 = tid >> 5;  // rows r0 + 8*j
  const TPool* sp = pool + ((int64_t)src * H + h) * kD * kD;
  floatx4 S0[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) S0[j] = load4(sp + (r0 + 8 * j) * kD + 4 * kq);

  floatx4 acc[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (tid < kD) s_dec[tid] = 1.f;

  const int64_t rec0 = ((int64_t)r * H + h) * L;  // record row of position 0
  // Blocks of positions from the end: [hi - kBlk, hi).
  for (int hi = n; hi > 0; hi -= kBlk) {
    const int lo = hi > kBlk ? hi - kBlk : 0;
    const int cnt = hi - lo;
    __syncthreads();
    if (tid < kD) {
      float dec = s_dec[tid];
      for (int t = hi - 1; t >= lo; --t) {
        const TRec* kg = kg_rec + (rec0 + t) * (2 * kD);
        s_c[t - lo][tid] = dec * to_f32(kg[tid]);
        dec *= __expf(to_f32(kg[kD + tid]));
      }
      s_dec[tid] = dec;
    }
    for (int e = tid; e < cnt * kD; e += kT) {
      const int t = e / kD, vv = e % kD;
      s_u[t][vv] = u_rec[(rec0 + lo + t) * kD + vv];
    }
    __syncthreads();
    for (int t = 0; t < cnt; ++t) {
      const floatx4 c4 = *reinterpret_cast<const floatx4*>(&s_c[t][4 * kq]);
#pragma unroll
      for (int j = 0; j < kRows; ++j) acc[j] += c4 * s_u[t][r0 + 8 * j];
    }
  }
  __syncthreads();
  const floatx4 a4 = *reinterpret_cast<const floatx4*>(&s_dec[4 * kq]);
  TPool* dp = pool + ((int64_t)dst * H + h) * kD * kD;
#pragma unroll
  for (int j = 0; j < kRows; ++j) store4(dp + (r0 + 8 * j) * kD + 4 * kq, a4 * S0[j] + acc[j]);
}

template <typename TPool>
hipError_t by_rec(const CommitArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.n_req * a.H)), block(kT);
#define KDA_COMMIT_LAUNCH(TR)                                                                  \
  hipLaunchKernelGGL((kda_commit_kernel<TPool, TR>), grid, block, 0, st,                       \
                     static_cast<TPool*>(a.pool.base), a.pool.n_slots, a.ckpt_slot, a.dst_slot, \
                     a.accepted_len, a.u_rec, static_cast<const TR*>(a.kg_rec), a.n_req, a.L,   \
                     a.H, a.dev_err)
  switch (a.rec_dtype) {
    case F32: KDA_COMMIT_LAUNCH(float); break;
    case F16: KDA_COMMIT_LAUNCH(f16); break;
    case BF16: KDA_COMMIT_LAUNCH(bf16); break;
    default: return hipErrorInvalidValue;
  }
#undef KDA_COMMIT_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  if (a.d != kD) return hipErrorInvalidValue;
  if (a.n_req == 0) return hipSuccess;
  switch (a.pool.dtype) {
    case F32: return by_rec<float>(a, st);
    case F16: return by_rec<f16>(a, st);
    case BF16: return by_rec<bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
