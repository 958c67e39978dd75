// RecoverSSM verify for gfx950 (vLLM PR #51855 summary, implementation
// breakdown step 3): read one checkpoint per request (never written), step the
// L speculative positions token by token, and record per position the fp32
// correction u_t plus a lossless copy of the key and raw gate.  The gate
// activations (alpha = exp(g), beta = sigmoid(b)) are applied inside the
// kernel, with the same fp32 code as the prefill path.
//
// One workgroup (4 waves) per (request, head); the d x d fp32 state stays in
// registers.  An 8-lane group owns 4 state rows (v) and each lane 16 of their
// 128 key entries, k in {4*(lane%8) + 32*j + e}, so each checkpoint load is
// a contiguous 128 bytes per group.  Within a block of kTB positions the
// state is held as S = Diag(D) St, D_t[k] being the product of alpha[k] over
// the block's positions up to and including t.  Then, per position t:
//   S_dec^T k = St^T (D_t k),  S_dec^T q = St^T (D_t q)     (S_dec = Diag(alpha_t) S)
//   u = beta (v - S_dec^T k),  o = S_dec^T q + u (k . q)
//   St += (k / D_t) u^T                                      (one FMA per element)
// and at the end of a block St <- Diag(D) St restarts D at 1.  The two dot
// products reduce across the 8 lanes of a group with DPP, so every lane gets
// its own rows' u with no LDS traffic per position.  The per-position vectors
// (D_t k, D_t q, k / D_t, v, beta, k . q) of a block are built once behind one
// barrier.  D and 1/D stay finite in fp32 while the summed gate over a block
// stays above about -80 (the chunked path's bound over a whole chunk is the
// same, so verify is the less restrictive of the two).
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kD = 128;   // state rows (d_v) and columns (d_k)
constexpr int kTB = 8;    // positions prepared per block

// Sum over the 8 lanes of a group, result in every lane of the group.
__device__ __forceinline__ float group8_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));  // lane ^ 1
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));  // lane ^ 2
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true)); // 7 - lane in 8
  return x;
}

template <typename TIn, typename TPool>
__global__ __launch_bounds__(kT) void kda_verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ bl, TIn* __restrict__ o, int n_req, int L,
    int H, const TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ ckpt,
    float* __restrict__ u_rec, TIn* __restrict__ kg_rec, int32_t* __restrict__ dev_err) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int EP = 16 / (int)sizeof(TIn);   // input elements per 16-byte piece
  constexpr int PPR = kD / EP;                 // pieces per 128-element row
  // per position of the block: D_t k, D_t q (for the dots), k / D_t (update)
  __shared__ __align__(16) float s_wk[kTB][kD];
  __shared__ __align__(16) float s_wq[kTB][kD];
  __shared__ __align__(16) float s_ku[kTB][kD];
  __shared__ __align__(16) float s_dec[kD];      // D at the end of the block
  __shared__ float s_beta[kTB], s_kq[2][kTB];    // k . q as two 64-channel halves
  // the block's inputs as loaded (rows of 128: k, g, q, v), and its outputs
  // u and o, so that every global access moves 16 bytes per lane
  __shared__ __align__(16) TIn s_in[4][kTB][kD];
  __shared__ __align__(16) float s_u[kTB][kD];
  __shared__ __align__(16) TIn s_o[kTB][kD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 3, gl = lane & 7;       // 8 groups of 8 lanes
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= n_req) return;
  const int slot = ckpt[r];
  if (slot < 0 || (int64_t)slot >= n_slots) {
    if (tid == 0 && h == 0) set_err(dev_err, 1u);
    return;
  }

  // ---- checkpoint: rows row0 + i (i < 4), keys 4*gl + 32*j + e
  const int row0 = 32 * wave + 4 * grp;
  floatx4 S[4][4];
  const TPool* src = pool + ((int64_t)slot * H + h) * kD * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) S[i][j] = load4(src + (row0 + i) * kD + 4 * gl + 32 * j);

  const int64_t tok_stride = (int64_t)H * kD;
  const TIn* const arr[4] = {k, g, q, v};
  TIn* const kg_rh = kg_rec + ((int64_t)r * H + h) * L * (2 * kD);   // [L][2 kD] of this (req, head)
  float* const u_rh = u_rec + ((int64_t)r * H + h) * L * kD;        // [L][kD]
  for (int t0 = 0; t0 < L; t0 += kTB) {
    const int nb = min(kTB, L - t0);
    if (t0 > 0) __syncthreads();  // every wave is done with the previous block
    // ---- stage the block's rows: piece p = (array, position, part); rows
    //      past the block end repeat its last position
#pragma unroll
    for (int pp = 0; pp < 4 * kTB * PPR / kT; ++pp) {
      const int pc = tid + kT * pp;
      const int a = pc / (kTB * PPR), jj = (pc / PPR) % kTB, part = pc % PPR;
      const int64_t off = ((int64_t)r * L + t0 + min(jj, nb - 1)) * tok_stride + (int64_t)h * kD + part * EP;
      *reinterpret_cast<u32x4*>(&s_in[a][jj][part * EP]) = *reinterpret_cast<const u32x4*>(arr[a] + off);
    }
    if (tid < kTB) s_beta[tid] = sigmoidf_(to_f32(bl[((int64_t)r * L + t0 + min(tid, nb - 1)) * H + h]));
    __syncthreads();
    // ---- records of k and the raw gate: [position][k | g], contiguous
#pragma unroll
    for (int pp = 0; pp < 2 * kTB * PPR / kT; ++pp) {
      const int pc = tid + kT * pp;
      const int jj = pc / (2 * PPR), a = (pc / PPR) % 2, part = pc % PPR;
      if (jj < nb)
        *reinterpret_cast<u32x4*>(kg_rh + (int64_t)(t0 + jj) * (2 * kD) + a * kD + part * EP) =
            *reinterpret_cast<const u32x4*>(&s_in[a][jj][part * EP]);
    }
    // ---- per-position vectors: threads 0..127 own one key channel each and
    //      run the cumulative decay over the block
    if (tid < kD) {
      float D = 1.f;
#pragma unroll
      for (int jj = 0; jj < kTB; ++jj) {
        const float kk = to_f32(s_in[0][jj][tid]), qq = to_f32(s_in[2][jj][tid]);
        D *= __expf(to_f32(s_in[1][jj][tid]));
        s_wk[jj][tid] = D * kk;
        s_wq[jj][tid] = D * qq;
        s_ku[jj][tid] = kk / D;
        float p = kk * qq;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) p += __shfl_xor(p, m);
        if (lane == 0) s_kq[wave][jj] = p;
      }
      s_dec[tid] = D;  // read only when the block is full (a next block exists)
    }
    __syncthreads();

    for (int jj = 0; jj < nb; ++jj) {
      floatx4 wk[4], wq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wk[j] = *reinterpret_cast<const floatx4*>(&s_wk[jj][4 * gl + 32 * j]);
        wq[j] = *reinterpret_cast<const floatx4*>(&s_wq[jj][4 * gl + 32 * j]);
      }
      float pred[4], oq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = 0.f, b2 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a += S[i][j][e] * wk[j][e];
            b2 += S[i][j][e] * wq[j][e];
          }
        pred[i] = group8_sum(a);
        oq[i] = group8_sum(b2);
      }
      const float beta = s_beta[jj], kqv = s_kq[0][jj] + s_kq[1][jj];
      float u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = beta * (to_f32(s_in[3][jj][row0 + i]) - pred[i]);
      // lanes 0..3 of a group hold u and lanes 4..7 o, one row each
      {
        const int i = gl & 3;
        const float ui = (i == 0) ? u[0] : (i == 1) ? u[1] : (i == 2) ? u[2] : u[3];
        const float oqi = (i == 0) ? oq[0] : (i == 1) ? oq[1] : (i == 2) ? oq[2] : oq[3];
        if (gl < 4) s_u[jj][row0 + i] = ui;
        else s_o[jj][row0 + i] = from_f32<TIn>(oqi + ui * kqv);
      }
      if (t0 + jj + 1 < L) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const floatx4 ku = *reinterpret_cast<const floatx4*>(&s_ku[jj][4 * gl + 32 * j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[i][j] += ku * u[i];
        }
      }
    }
    // ---- rebase: St <- Diag(D_block) St, so the next block starts from D = 1
    if (t0 + kTB < L) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(&s_dec[4 * gl + 32 * j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[i][j] = d4 * S[i][j];
      }
    }
    __syncthreads();
    // ---- the block's u (fp32, contiguous per (req, head)) and o rows
#pragma unroll
    for (int pp = 0; pp < kTB * kD / 4 / kT; ++pp) {
      const int pc = tid + kT * pp;
      const int jj = pc / (kD / 4), part = pc % (kD / 4);
      if (jj < nb)
        *reinterpret_cast<u32x4*>(u_rh + (int64_t)(t0 + jj) * kD + 4 * part) =
            *reinterpret_cast<const u32x4*>(&s_u[jj][4 * part]);
    }
    for (int pc = tid; pc < kTB * PPR; pc += kT) {
      const int jj = pc / PPR, part = pc % PPR;
      if (jj < nb)
        *reinterpret_cast<u32x4*>(o + ((int64_t)r * L + t0 + jj) * tok_stride + (int64_t)h * kD + part * EP) =
            *reinterpret_cast<const u32x4*>(&s_o[jj][part * EP]);
    }
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
