// RecoverSSM verify for gfx950 (vLLM PR #51855 summary, implementation
// breakdown step 3): read one checkpoint per request (never written), step the
// L speculative positions token by token, and record per position the fp32
// correction u_t plus a lossless copy of the key and raw gate.  The gate
// activations (alpha = exp(g), beta = sigmoid(b)) are applied inside the
// kernel, with the same fp32 code as the prefill path.
//
// One workgroup (4 waves) per (request, head); the d x d fp32 state stays in
// registers.  Lane layout: a half-wave (32 lanes) spans one state row of 128
// key entries, 4 consecutive entries per lane, so every load of the
// checkpoint is a contiguous 1 KiB per wave; each lane holds 16 rows.  Per
// token:
//   pred_v = sum_k S[v][k] alpha_k k_k     -> u_v = beta (v_v - pred_v)
//   oq_v   = sum_k S[v][k] alpha_k q_k     -> o_v = oq_v + u_v (k . q)
//   S[v][k] = alpha_k S[v][k] + k_k u_v
// (o = S_t^T q = (Diag(alpha) S)^T q + u (k . q)).  The two 32-lane dot
// products per row are reduced through LDS.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kD = 128;          // state rows (d_v) and columns (d_k)
constexpr int kRowsPerLane = 16; // 128 rows / (4 waves * 2 half-waves)
constexpr int kRedLd = 33;       // padded row of the reduction scratch

template <typename TIn, typename TPool>
__global__ __launch_bounds__(kT) void kda_verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ bl, TIn* __restrict__ o, int n_req, int L,
    int H, const TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ ckpt,
    float* __restrict__ u_rec, TIn* __restrict__ kg_rec, int32_t* __restrict__ dev_err) {
  __shared__ float s_w[kD], s_x[kD], s_a[kD], s_k[kD], s_v[kD], s_u[kD];
  __shared__ float s_kq[2], s_beta;
  __shared__ float s_red[4][64 * kRedLd];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, kq = lane & 31;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= n_req) return;
  const int slot = ckpt[r];
  if (slot < 0 || (int64_t)slot >= n_slots) {
    if (tid == 0 && h == 0) set_err(dev_err, 1u);
    return;
  }

  // ---- checkpoint rows 32*wave + 2*i + half, key entries 4*kq..4*kq+3
  floatx4 S[kRowsPerLane];
  const TPool* src = pool + ((int64_t)slot * H + h) * kD * kD;
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) S[i] = load4(src + (32 * wave + 2 * i + half) * kD + 4 * kq);

  const int64_t tok_stride = (int64_t)H * kD;
  for (int t = 0; t < L; ++t) {
    const int64_t base = ((int64_t)r * L + t) * tok_stride + (int64_t)h * kD;
    // ---- per-token vectors
    if (tid < kD) {
      const TIn kraw = k[base + tid], graw = g[base + tid];
      const float kk = to_f32(kraw), qq = to_f32(q[base + tid]);
      const float a = __expf(to_f32(graw));
      s_w[tid] = a * kk;
      s_x[tid] = a * qq;
      s_a[tid] = a;
      s_k[tid] = kk;
      TIn* rec = kg_rec + (((int64_t)r * H + h) * L + t) * (2 * kD);
      rec[tid] = kraw;
      rec[kD + tid] = graw;
      float p = kk * qq;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) p += __shfl_xor(p, m);
      if (lane == 0) s_kq[wave] = p;
    } else {
      s_v[tid - kD] = to_f32(v[base + tid - kD]);
      if (tid == kD) s_beta = sigmoidf_(to_f32(bl[((int64_t)r * L + t) * H + h]));
    }
    __syncthreads();

    const floatx4 w4 = *reinterpret_cast<const floatx4*>(&s_w[4 * kq]);
    const floatx4 x4 = *reinterpret_cast<const floatx4*>(&s_x[4 * kq]);
    float* red = s_red[wave];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      const floatx4 s = S[i];
      red[(half * 32 + i) * kRedLd + kq] = s[0] * w4[0] + s[1] * w4[1] + s[2] * w4[2] + s[3] * w4[3];
      red[(half * 32 + 16 + i) * kRedLd + kq] = s[0] * x4[0] + s[1] * x4[1] + s[2] * x4[2] + s[3] * x4[3];
    }
    __syncthreads();
    // lane j of the wave finishes output j: half_j = j / 32, quantity (j/16)&1, row i = j&15
    float acc = 0.f;
    {
      const float* rr = red + lane * kRedLd;
#pragma unroll
      for (int m = 0; m < 32; ++m) acc += rr[m];
    }
    const int hj = lane >> 5, qj = (lane >> 4) & 1, ij = lane & 15;
    const int row = 32 * wave + 2 * ij + hj;
    const float kqv = s_kq[0] + s_kq[1];
    if (qj == 0) {
      const float u = s_beta * (s_v[row] - acc);
      s_u[row] = u;
      u_rec[(((int64_t)r * H + h) * L + t) * kD + row] = u;
    }
    __syncthreads();
    if (qj == 1) {
      o[((int64_t)r * L + t) * tok_stride + (int64_t)h * kD + row] = from_f32<TIn>(acc + s_u[row] * kqv);
    }
    if (t + 1 < L) {
      const floatx4 a4 = *reinterpret_cast<const floatx4*>(&s_a[4 * kq]);
      const floatx4 k4 = *reinterpret_cast<const floatx4*>(&s_k[4 * kq]);
#pragma unroll
      for (int i = 0; i < kRowsPerLane; ++i) S[i] = a4 * S[i] + k4 * s_u[32 * wave + 2 * i + half];
    }
    __syncthreads();
  }
}

template <typename TIn>
hipError_t by_pool(const VerifyArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.n_req * a.H)), block(kT);
#define KDA_VERIFY_LAUNCH(TP)                                                                      \
  hipLaunchKernelGGL((kda_verify_kernel<TIn, TP>), grid, block, 0, st,                             \
                     static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),                   \
                     static_cast<const TIn*>(a.v), static_cast<const TIn*>(a.g),                   \
                     static_cast<const TIn*>(a.b), static_cast<TIn*>(a.o), a.n_req, a.L, a.H,      \
                     static_cast<const TP*>(a.pool.base), a.pool.n_slots, a.ckpt_slot, a.u_rec,    \
                     static_cast<TIn*>(a.kg_rec), a.dev_err)
  switch (a.pool.dtype) {
    case F32: KDA_VERIFY_LAUNCH(float); break;
    case F16: KDA_VERIFY_LAUNCH(f16); break;
    case BF16: KDA_VERIFY_LAUNCH(bf16); break;
    default: return hipErrorInvalidValue;
  }
#undef KDA_VERIFY_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  if (a.d != kD) return hipErrorInvalidValue;
  if (a.n_req == 0) return hipSuccess;
  switch (a.in_dtype) {
    case F32: return by_pool<float>(a, st);
    case F16: return by_pool<f16>(a, st);
    case BF16: return by_pool<bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
