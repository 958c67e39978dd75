// RecoverSSM verify for gfx950 (vLLM PR #51855 summary, implementation
// breakdown step 3): read one checkpoint per request (never written), step the
// L speculative positions, and record per position the fp32 correction u_t
// plus a lossless copy of the key and raw gate.  The gate activations
// (alpha = exp(g), beta = sigmoid(b)) are applied inside the kernel, with the
// same fp32 code as the prefill path.
//
// Two workgroups (4 waves each) per (request, head), one per half of the
// state's value columns: every step below is independent across value
// columns except the per-position vectors and two 8 x 8 matrices, which both
// halves form from the same key/gate/query rows.  The d x (d/2) fp32 state
// half stays in registers as MFMA accumulator tiles.  One workgroup per
// half-item: the hardware starts a new workgroup as soon as one finishes,
// which overlaps one item's stores with the next items' loads better than a
// resident-sized grid stepping through items (132 us against 148 us at 256
// requests x 32 heads x 8 positions).
//
// Positions go in blocks of kTB = 8.  Within a block the state is held as
// S = Diag(D) St, D_t[k] being the product of alpha[k] over the block's
// positions up to and including t; with wk_t = D_t k_t, wq_t = D_t q_t,
// ku_t = k_t / D_t and S_dec,t = Diag(alpha_t) S_{t-1}:
//   S_dec,t^T k_t = St_0^T wk_t + sum_{s<t} u_s (ku_s . wk_t)
//   S_dec,t^T q_t = St_0^T wq_t + sum_{s<t} u_s (ku_s . wq_t)
//   u_t = beta_t (v_t - S_dec,t^T k_t),   o_t = S_dec,t^T q_t + u_t (k_t . q_t)
// so that, column by column of the state, with the Gram matrix
// G[s][n] = ku_s . [wk | wq]_n (n < 8: wk, n >= 8: wq):
//   u = T Diag(beta) (v - St_0^T wk),  T = (I + Diag(beta) Lk)^-1,
//       Lk[t][s] = G[s][t] for s < t  (the token recursion solved per block)
//   o = St_0^T wq + P u,  P[t][s] = G[s][8 + t] for s <= t  (ku_t . wq_t = k_t . q_t)
//   St_0 <- Diag(D_block) (St_0 + sum_t ku_t u_t^T)  (multi-block windows)
// Per block that is one fp32 MFMA product with the state, St_0^T [wk | wq],
// two products of its result with the 8 x 8 matrices T Diag(beta) and
// [P | I] (shared by all value columns), and the rank-8 update.  D and 1/D stay finite
// in fp32 while the summed gate over a block stays above about -80.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kD = 128;   // state rows (d_v) and columns (d_k)
constexpr int kDH = 64;   // value columns per workgroup
constexpr int kTB = 8;    // positions per block
constexpr int kWS = kD + 4;   // padded row stride (floats) of the per-position vectors
constexpr int kXcd = 8;   // consecutive workgroup ids go to the 8 XCDs in turn

// Occupancy the register budget is set for (workgroups per compute unit): 4
// for one-block windows with 16-bit rows, 3 for fp32 rows, 2 for longer
// windows.
constexpr int resident_wgs(size_t in_bytes, bool multi) { return multi ? 2 : in_bytes == 2 ? 4 : 3; }

// fp32 16x16x4 MFMA.  A: lane l holds A[l % 16][l / 16]; B: lane l holds
// B[l / 16][l % 16]; C/D: lane l holds D[4 (l / 16) + i][l % 16].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Copy N bytes (4, 8 or 16; both addresses N-aligned) with one vector
// store.  The outputs (o and the records) are stored non-temporally: the
// next reader is another kernel, and dirty output lines left in the
// memory-side cache slowed the next call's streaming reads (verify in a
// verify / commit / copy loop 146 -> 143 us, commit reading the records
// unchanged).
template <int N, typename TD, typename TS>
__device__ __forceinline__ void store_n(TD* dst, const TS* src) {
  typedef unsigned int vec __attribute__((ext_vector_type(N / 4)));
  __builtin_nontemporal_store(*reinterpret_cast<const vec*>(src), reinterpret_cast<vec*>(dst));
}

// LDS writes of this wave visible to its other lanes
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// kMulti: windows longer than one block (the state is updated between blocks)
template <typename TIn, typename TPool, bool kMulti>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(resident_wgs(sizeof(TIn), kMulti), 8))) void kda_verify_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ bl, TIn* __restrict__ o, int n_req, int L,
    int H, const TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ ckpt,
    float* __restrict__ u_rec, TIn* __restrict__ kg_rec, int32_t* __restrict__ dev_err, int l2norm) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int EP = 16 / (int)sizeof(TIn);   // input elements per 16-byte piece
  constexpr int PPR = kD / EP;                 // pieces per 128-element row
  constexpr int NKGQ = 3 * kTB * PPR;          // pieces of the k, g, q rows
  constexpr int NP = NKGQ + kTB * PPR / 2;     // ... and of this half of the v rows
  constexpr int NR = (NP + kT - 1) / kT;
  // per block: [wk_t | wq_t] by row n (n < 8: wk, n >= 8: wq) and ku_t, rows
  // padded so that 16 lanes reading 16 rows fall in different banks; the
  // Gram matrix as four per-wave partial sums over 32 keys each; T Diag(beta)
  // and [P | I] (rows t, 16 columns s; rows 8..15 and the identity block stay
  // as set at the start); D at the block end; beta (zero past the block end)
  __shared__ __align__(16) float s_w[2 * kTB][kWS];
  __shared__ __align__(16) float s_ku[kTB][kWS];
  __shared__ __align__(16) float s_gp[4][kTB][2 * kTB];
  __shared__ __align__(16) float s_g[kTB][2 * kTB];
  __shared__ __align__(16) float s_tb[16][20];
  __shared__ __align__(16) float s_pi[16][20];
  __shared__ __align__(16) float s_dec[kD];
  __shared__ float s_beta[kTB];
  // the block's inputs as loaded: rows of k, g, q ([3][kTB][kD]) then this
  // half of the v rows ([kTB][kDH]), piece p of 16 bytes at byte 16 p; and
  // the block's outputs u and o, so that every global access moves 16 bytes
  // per lane
  __shared__ __align__(16) TIn s_stage[NP * EP];
  __shared__ __align__(16) float s_u[kTB][kDH];
  __shared__ __align__(16) TIn s_o[kTB][kDH];
  const TIn* const s_v = s_stage + NKGQ * EP;
  auto s_in = [&](int a, int jj, int c) -> float { return to_f32(s_stage[(a * kTB + jj) * kD + c]); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, r = lane & 15;
  const int n_items = n_req * H;
  const int64_t tok_stride = (int64_t)H * kD;

  // Workgroups b and b + kXcd (same XCD) hold the two halves of one
  // (request, head).  A request whose checkpoint slot is out of range is
  // flagged and skipped; its outputs are left untouched.
  const int bid = blockIdx.x, vh = (bid / kXcd) & 1;
  const int item = (bid / (2 * kXcd)) * kXcd + bid % kXcd;
  if (item >= n_items) return;
  {
    const int s = ckpt[item / H];
    if (s < 0 || (int64_t)s >= n_slots) {
      if (tid == 0 && vh == 0) set_err(dev_err, 1u);
      return;
    }
  }

  for (int e = tid; e < 16 * 20; e += kT) {
    const int t = e / 20, c = e % 20;
    (&s_tb[0][0])[e] = 0.f;
    (&s_pi[0][0])[e] = (t < kTB && c == kTB + t) ? 1.f : 0.f;
  }

  // the input rows of block t0 of an item (rows past the block end repeat
  // its last position; pieces past the end reload the last one), and this
  // half of an item's checkpoint as MFMA tiles: wave w owns value columns
  // 64 vh + 16 w + r, and tile kt of lane (g, r) holds St[16 kt + 4g + e][that
  // column], four consecutive keys of one pool row (pool layout [v][k])
  u32x4 buf[NR];
  TIn braw;   // converted where used, so that no wait follows the load
  auto load_rows = [&](int it, int t0) {
    const int rq = it / H, h = it % H, nb = min(kTB, L - t0);
#pragma unroll
    for (int pp = 0; pp < NR; ++pp) {
      const int pc = min(tid + kT * pp, NP - 1);
      const bool is_v = pc >= NKGQ;
      const int a = pc / (kTB * PPR);
      const int jj = is_v ? (pc - NKGQ) / (PPR / 2) : (pc / PPR) % kTB;
      const int col = is_v ? vh * kDH + ((pc - NKGQ) % (PPR / 2)) * EP : (pc % PPR) * EP;
      const TIn* const base = a == 0 ? k : a == 1 ? g : a == 2 ? q : v;
      buf[pp] = *reinterpret_cast<const u32x4*>(
          base + ((int64_t)rq * L + t0 + min(jj, nb - 1)) * tok_stride + (int64_t)h * kD + col);
    }
    braw = bl[((int64_t)rq * L + t0 + min(tid & (kTB - 1), nb - 1)) * H + h];
  };
  // The checkpoint is read with non-temporal loads.  In the decoding loop's
  // order (verify, in-place commit, fork copy, repeated) that took verify
  // from 143 to 125 us and commit from 160 to 164 us per iteration (256
  // requests x 32 heads, fp32 pool): the loop as a whole 14 us faster.
  floatx4 S[8];
  auto load_state = [&](int it) {
    const TPool* const src =
        pool + ((int64_t)ckpt[it / H] * H + it % H) * kD * kD + (int64_t)vh * kDH * kD;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const auto x = __builtin_nontemporal_load(
          reinterpret_cast<const typename Vec4<TPool>::type*>(src + (16 * wave + r) * kD + 16 * kt + 4 * gq));
      S[kt] = floatx4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
    }
  };
  int t0 = 0, rq = 0, h = 0, nb = 0;
  bool last = true;   // the item's last block (always, for one-block windows)
  floatx4 dot;        // St_0^T [wk | wq] of the current block
  auto head = [&]() {
    rq = item / H;
    h = item % H;
    nb = min(kTB, L - t0);
#pragma unroll
    for (int pp = 0; pp < NR; ++pp) {
      const int pc = tid + kT * pp;
      if (pc < NP) *reinterpret_cast<u32x4*>(&s_stage[pc * EP]) = buf[pp];
    }
    if (tid < kTB) s_beta[tid] = tid < nb ? sigmoidf_(to_f32(braw)) : 0.f;
    __syncthreads();
    // ---- optional L2 normalisation of the block's k and q rows in place
    //      (16 threads per row, 8 channels each), rounded once to the input
    //      dtype: the recurrence and the key record both use the result
    if (l2norm) {
      const int rr = tid >> 4, a = rr < kTB ? 0 : 2, c0 = 8 * (tid & 15);
      TIn* const rp = &s_stage[(a * kTB + (rr & (kTB - 1))) * kD + c0];
      float x[8], ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = to_f32(rp[i]);
        ss += x[i] * x[i];
      }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
      const float sc = rsqrtf(ss + 1e-6f);
#pragma unroll
      for (int i = 0; i < 8; ++i) rp[i] = from_f32<TIn>(x[i] * sc);
      __syncthreads();
    }
    // ---- per-position vectors: thread (key channel c, half hh) runs the
    //      cumulative decay over positions 4 hh .. 4 hh + 3 (the second half
    //      first runs it over positions 0..3); 1/D as a product of exp(-g)
    {
      const int c = tid & (kD - 1), hh = tid >> 7;
      float D = 1.f, Di = 1.f;
      if (hh) {
#pragma unroll
        for (int jj = 0; jj < kTB / 2; ++jj) {
          const float gg = s_in(1, jj, c);
          D *= __expf(gg);
          Di *= __expf(-gg);
        }
      }
#pragma unroll
      for (int j4 = 0; j4 < kTB / 2; ++j4) {
        const int jj = (kTB / 2) * hh + j4;
        const float kk = s_in(0, jj, c), qq = s_in(2, jj, c), gg = s_in(1, jj, c);
        D *= __expf(gg);
        Di *= __expf(-gg);
        s_w[jj][c] = D * kk;
        s_w[kTB + jj][c] = D * qq;
        s_ku[jj][c] = kk * Di;
      }
      if (hh) s_dec[c] = D;  // read only when the block is full (a next block exists)
      // 1/D grows with the block's decay: past the fp32 range (a summed gate
      // below about -88 over the block's positions) the gate-range bit is set
      if (!(Di <= 3.40282347e38f)) set_err(dev_err, 1u << 5);
    }
    __syncthreads();
    // ---- Gram partial of wave w over keys 32 w .. 32 w + 31: rows s (8 of
    //      16 used), columns n; MFMA e of key group j contracts over keys
    //      32 w + 16 j + 4g + e
    {
      floatx4 gp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key = 32 * wave + 16 * j + 4 * gq;
        const floatx4 ku4 = *reinterpret_cast<const floatx4*>(&s_ku[r & (kTB - 1)][key]);
        const floatx4 a4 = r < kTB ? ku4 : floatx4{0.f, 0.f, 0.f, 0.f};
        const floatx4 w4 = *reinterpret_cast<const floatx4*>(&s_w[r][key]);
#pragma unroll
        for (int e = 0; e < 4; ++e) gp = mfma4(a4[e], w4[e], gp);   // A[s = r][key], B[key][n = r]
      }
      if (gq < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_gp[wave][4 * gq + i][r] = gp[i];
      }
    }
    __syncthreads();
    // ---- one wave (a different one per item) sums the Gram partials and
    //      forms T Diag(beta) and P; lane j < 8 solves column j of the unit
    //      lower-triangular T by forward substitution
    if (wave == (item & 3)) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int e = lane + 64 * hf, s2 = e >> 4, n = e & 15;
        const float gsum = s_gp[0][s2][n] + s_gp[1][s2][n] + s_gp[2][s2][n] + s_gp[3][s2][n];
        if (n < kTB) s_g[s2][n] = gsum;
        else s_pi[n - kTB][s2] = s2 <= n - kTB ? gsum : 0.f;
      }
      wave_sync();
      if (lane < kTB) {
        const int j = lane;
        float tc[kTB];
#pragma unroll
        for (int t = 0; t < kTB; ++t) {
          float acc = 0.f;
#pragma unroll
          for (int s2 = 0; s2 < t; ++s2) acc += s_g[s2][t] * tc[s2];
          tc[t] = t == j ? 1.f : (t > j ? -s_beta[t] * acc : 0.f);
        }
        const float bj = s_beta[j];
#pragma unroll
        for (int t = 0; t < kTB; ++t) s_tb[t][j] = tc[t] * bj;
      }
    }
    // ---- St_0^T [wk | wq] as [n][v]: A = [wk | wq] rows n, B = the state
    //      tile kt, whose accumulator element e is key 16 kt + 4g + e
    dot = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const floatx4 w4 = *reinterpret_cast<const floatx4*>(&s_w[r][16 * kt + 4 * gq]);  // A[n = r][key]
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = mfma4(w4[e], S[kt][e], dot);
    }
    // lane (g, r) now holds St_0^T wk_{4g+i} (g < 2) or St_0^T wq_{4g+i-8}
    // (g >= 2) for value column 16 w + r
  };
  auto finish = [&]() {
    TIn* const kg_rh = kg_rec + ((int64_t)rq * H + h) * L * (2 * kD);       // [L][2 kD] of this (req, head)
    float* const u_rh = u_rec + ((int64_t)rq * H + h) * L * kD + vh * kDH;  // [L][kD], this half
    __syncthreads();
    const floatx4 tb4 = *reinterpret_cast<const floatx4*>(&s_tb[r][4 * gq]);
    const floatx4 pi4 = *reinterpret_cast<const floatx4*>(&s_pi[r][4 * gq]);
    floatx4 ua = {0.f, 0.f, 0.f, 0.f}, oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float vv = to_f32(s_v[((4 * gq + i) & (kTB - 1)) * kDH + 16 * wave + r]);
      ua = mfma4(tb4[i], gq < 2 ? vv - dot[i] : 0.f, ua);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) oa = mfma4(pi4[i], gq < 2 ? ua[i] : dot[i], oa);
    if (gq < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_u[4 * gq + i][16 * wave + r] = ua[i];
        s_o[4 * gq + i][16 * wave + r] = from_f32<TIn>(oa[i]);
      }
    }
    // ---- St_0 += sum_t ku_t u_t^T (rank-8 MFMA update over this wave's
    //      own columns), then the rebase St <- Diag(D_block) St so the
    //      next block starts from D = 1
    // the record rows are read here, before the barrier after which the
    // next item's rows may overwrite the staging area
    const int jk = min((kTB / 2) * vh + tid / 64, nb - 1), ek = (tid % 64) * 4;
    typedef unsigned int kgvec __attribute__((ext_vector_type(sizeof(TIn))));
    const kgvec kgv = *reinterpret_cast<const kgvec*>(&s_stage[((ek / kD) * kTB + jk) * kD + ek % kD]);
    if (!last) {
      wave_sync();
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const float a0 = s_ku[gq][16 * kt + r], a1 = s_ku[4 + gq][16 * kt + r];  // A[key = r][s = 4j + g]
        S[kt] = mfma4(a0, s_u[gq][16 * wave + r], S[kt]);                        // B[s = 4j + g][v = r]
        S[kt] = mfma4(a1, s_u[4 + gq][16 * wave + r], S[kt]);
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(&s_dec[16 * kt + 4 * gq]);
        S[kt] = d4 * S[kt];
      }
    }
    __syncthreads();
    // ---- the block's outputs, one store per array per thread and no
    //      branches (rows past the block end rewrite the last position with
    //      the same bytes), so the compiler can count them exactly when it
    //      waits for the next block's rows.  Records of k and the raw gate
    //      ([position][k | g], contiguous): half vh writes positions
    //      4 vh .. 4 vh + 3.  u (fp32, contiguous per (req, head)) and o:
    //      this half's 64 columns.
    __builtin_nontemporal_store(kgv, reinterpret_cast<kgvec*>(kg_rh + (int64_t)(t0 + jk) * (2 * kD) + ek));
    {
      const int jj = min(tid / 32, nb - 1), c = (tid % 32) * 2;
      store_n<8>(u_rh + (int64_t)(t0 + jj) * kD + c, &s_u[jj][c]);
      store_n<2 * sizeof(TIn)>(o + ((int64_t)rq * L + t0 + jj) * tok_stride + (int64_t)h * kD + vh * kDH + c,
                               &s_o[jj][c]);
    }
  };

  // Positions in blocks of kTB: each block's rows are requested at its
  // start (the first block's before the checkpoint, as they are needed
  // first); the state is carried in registers from block to block.
  while (true) {
    load_rows(item, t0);
    if (t0 == 0) load_state(item);
    head();
    last = !kMulti || t0 + kTB >= L;
    finish();
    if (last) break;
    t0 += kTB;
  }
}

template <typename TIn>
hipError_t by_pool(const VerifyArgs& a, hipStream_t st) {
  // two workgroups per (request, head), in groups of 2 kXcd ids
  const int64_t items = (int64_t)a.n_req * a.H;
  const dim3 grid((unsigned)((items + kXcd - 1) / kXcd * 2 * kXcd)), block(kT);
#define KDA_VERIFY_LAUNCH(TP)                                                                      \
  hipLaunchKernelGGL((a.L > kTB ? kda_verify_kernel<TIn, TP, true> : kda_verify_kernel<TIn, TP, false>), \
                     grid, block, 0, st,                                                           \
                     static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),                   \
                     static_cast<const TIn*>(a.v), static_cast<const TIn*>(a.g),                   \
                     static_cast<const TIn*>(a.b), static_cast<TIn*>(a.o), a.n_req, a.L, a.H,      \
                     static_cast<const TP*>(a.pool.base), a.pool.n_slots, a.ckpt_slot, a.u_rec,    \
                     static_cast<TIn*>(a.kg_rec), a.dev_err, (a.flags & 1u) ? 1 : 0)
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
