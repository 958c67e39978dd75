// RecoverSSM commit for gfx950 (vLLM PR #51855 summary, implementation
// breakdown step 4): rebuild the state after n accepted positions in one
// pass, without re-running the recurrence,
//   S_n = Diag(A) S_0 + sum_{t<n} c_t u_t^T,
//   c_t = k_t * prod_{t<s<n} alpha_s,   A = prod_{s<n} alpha_s,
// where the products are accumulated in reverse order t = n-1 .. 0 with a
// running decay.  Every state element is read once and written once (one
// RNE cast into the pool dtype); an in-place request with n = 0 is skipped.
//
// One workgroup per (request, head).  The decayed keys c_t and the
// corrections u_t of a block of 32 positions are staged in LDS.  The
// align-mode variant (block-aligned state slots; same summary, steps 4-5,
// and the review's block-size check) rebuilds up to two states per request
// from one checkpoint read.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kT = 256;
constexpr int kD = 128;
constexpr int kRows = 16;   // rows per thread
constexpr int kBlk = 32;    // positions staged per pass

struct CommitSmem {
  float c[kBlk][kD];   // decayed keys of the staged positions
  float u[kBlk][kD];   // their corrections
  float dec[kD];       // running decay
};

// Applies positions [from, to) of one (request, head)'s records to the
// state S held in registers:
//   S <- Diag(prod_{from<=s<to} alpha_s) S + sum_{from<=t<to} c_t u_t^T,
//   c_t = k_t * prod_{t<s<to} alpha_s,
// accumulated in reverse order with a running decay, positions staged in
// LDS kBlk at a time.  Uniform across the workgroup (it holds barriers).
// The records are read once, with non-temporal loads: in the decoding
// loop's order (verify writes them, commit reads them, the next verify
// rewrites them) that took commit from ~162.5 to 158.9 us, and the commit
// right after a verify in the bench step from ~164 to 160 us.
template <typename TRec>
__device__ __forceinline__ void advance(floatx4 (&S)[kRows], int from, int to, const TRec* __restrict__ kg_rec,
                                        const float* __restrict__ u_rec, int64_t rec0, CommitSmem& sm) {
  const int tid = threadIdx.x, kq = tid & 31, r0 = tid >> 5;  // rows r0 + 8*j
  floatx4 acc[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // earlier readers of the staging arrays are done
  if (tid < kD) sm.dec[tid] = 1.f;
  // Blocks of positions from the end: [lo, hi).
  for (int hi = to; hi > from; hi -= kBlk) {
    const int lo = hi - kBlk > from ? hi - kBlk : from;
    const int cnt = hi - lo;
    __syncthreads();
    if (tid < kD) {
      float dec = sm.dec[tid];
      for (int t = hi - 1; t >= lo; --t) {
        const TRec* kg = kg_rec + (rec0 + t) * (2 * kD);
        sm.c[t - lo][tid] = dec * to_f32(__builtin_nontemporal_load(&kg[tid]));
        dec *= __expf(to_f32(__builtin_nontemporal_load(&kg[kD + tid])));
      }
      sm.dec[tid] = dec;
    }
    for (int e = tid; e < cnt * kD; e += kT) {
      const int t = e / kD, vv = e % kD;
      sm.u[t][vv] = __builtin_nontemporal_load(&u_rec[(rec0 + lo + t) * kD + vv]);
    }
    __syncthreads();
    for (int t = 0; t < cnt; ++t) {
      const floatx4 c4 = *reinterpret_cast<const floatx4*>(&sm.c[t][4 * kq]);
#pragma unroll
      for (int j = 0; j < kRows; ++j) acc[j] += c4 * sm.u[t][r0 + 8 * j];
    }
  }
  __syncthreads();
  const floatx4 a4 = *reinterpret_cast<const floatx4*>(&sm.dec[4 * kq]);
#pragma unroll
  for (int j = 0; j < kRows; ++j) S[j] = a4 * S[j] + acc[j];
}

// Thread layout of a state: 32 threads span one 512-byte row (4 consecutive
// key entries each) and a thread owns 16 rows, so each wave moves 1 KiB
// contiguous per access.
template <typename TPool>
__device__ __forceinline__ void load_state(floatx4 (&S)[kRows], const TPool* sp) {
  const int kq = threadIdx.x & 31, r0 = threadIdx.x >> 5;
#pragma unroll
  for (int j = 0; j < kRows; ++j) S[j] = load4(sp + (r0 + 8 * j) * kD + 4 * kq);
}
// The rebuilt state is stored non-temporally: nothing reads it again within
// this call, and ordinary stores of a whole batch of states (about 0.5 GB at
// 256 requests x 32 heads) leave that much dirty data in the memory-side
// cache, which the next kernel then pays to write back while it streams its
// own reads (a verify right after a commit of the same checkpoints took
// 175 us instead of 149 us).
template <typename TPool>
__device__ __forceinline__ void store_state(TPool* dp, const floatx4 (&S)[kRows]) {
  typedef typename Vec4<TPool>::type V;
  const int kq = threadIdx.x & 31, r0 = threadIdx.x >> 5;
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    V x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = from_f32<TPool>(S[j][e]);
    __builtin_nontemporal_store(x, reinterpret_cast<V*>(dp + (r0 + 8 * j) * kD + 4 * kq));
  }
}

template <typename TPool, typename TRec>
__global__ __launch_bounds__(kT) void kda_commit_kernel(
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ ckpt,
    const int32_t* __restrict__ dst_slot, const int32_t* __restrict__ accepted,
    const float* __restrict__ u_rec, const TRec* __restrict__ kg_rec, int n_req, int L, int H,
    int32_t* __restrict__ dev_err) {
  __shared__ CommitSmem sm;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= n_req) return;
  const int n = accepted[r];
  const int src = ckpt[r];
  const int dst = dst_slot ? dst_slot[r] : src;
  if (n < 0 || n > L) {
    if (threadIdx.x == 0 && h == 0) set_err(dev_err, 1u << 2);
    return;
  }
  if (src < 0 || (int64_t)src >= n_slots || dst < 0 || (int64_t)dst >= n_slots) {
    if (threadIdx.x == 0 && h == 0) set_err(dev_err, 1u);
    return;
  }
  if (n == 0 && dst == src) return;  // nothing accepted, checkpoint already right
  floatx4 S[kRows];
  load_state(S, pool + ((int64_t)src * H + h) * kD * kD);
  advance(S, 0, n, kg_rec, u_rec, ((int64_t)r * H + h) * L, sm);
  store_state(pool + ((int64_t)dst * H + h) * kD * kD, S);
}

// Align mode: states kept per block of bs tokens, the state after p tokens
// in the slot of the block of token p.  Request r holds p = num_tokens[r]
// tokens; with n accepted, b0 = block of token p, b1 = block of token p + n
// (bs > L, so b1 <= b0 + 1).  b1 == b0: S_{p+n} into b0's slot, in place.
// b1 == b0 + 1: the state after the m = b1 bs - p accepted tokens that close
// b0 into b0's slot (when m > 0), then S_{p+n} into b1's slot, continuing
// from S_{p+m} in registers.
// Post-processing for the next step (same summary, step 4: the running
// block index moves on, the next step's copy bias goes back to neutral):
// the head-0 workgroup of each request writes p + n, b1, b1's slot and a
// zero bias to the optional next_* arrays (p, -1, -1, 0 for a request that
// is skipped).
struct AlignNext {
  int32_t *tokens, *block, *ckpt, *bias;
};

template <typename TPool, typename TRec>
__global__ __launch_bounds__(kT) void kda_commit_align_kernel(
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ table, int blocks_per_req,
    const int32_t* __restrict__ num_tokens, const int32_t* __restrict__ accepted, int bs,
    const float* __restrict__ u_rec, const TRec* __restrict__ kg_rec, int n_req, int L, int H,
    AlignNext nx, int32_t* __restrict__ dev_err) {
  __shared__ CommitSmem sm;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  if (r >= n_req) return;
  const int n = accepted[r], p = num_tokens[r];
  const bool post = threadIdx.x == 0 && h == 0;
  auto publish = [&](int tokens, int block, int slot) {
    if (!post) return;
    if (nx.tokens) nx.tokens[r] = tokens;
    if (nx.block) nx.block[r] = block;
    if (nx.ckpt) nx.ckpt[r] = slot;
    if (nx.bias) nx.bias[r] = 0;
  };
  if (n < 0 || n > L) {
    if (post) set_err(dev_err, 1u << 2);
    publish(p, -1, -1);
    return;
  }
  const int b0 = p >= 1 ? (p - 1) / bs : 0, b1 = p >= 1 ? (p + n - 1) / bs : 0;
  const int s0 = p >= 1 && b1 < blocks_per_req ? table[(int64_t)r * blocks_per_req + b0] : -1;
  const int s1 = p >= 1 && b1 < blocks_per_req ? table[(int64_t)r * blocks_per_req + b1] : -1;
  if (s0 < 0 || (int64_t)s0 >= n_slots || s1 < 0 || (int64_t)s1 >= n_slots) {
    if (post) set_err(dev_err, 1u);
    publish(p, -1, -1);
    return;
  }
  publish(p + n, b1, s1);
  if (n == 0) return;
  const int64_t rec0 = ((int64_t)r * H + h) * L;
  const int m = b1 != b0 ? b1 * bs - p : 0;   // accepted tokens that close block b0
  floatx4 S[kRows];
  load_state(S, pool + ((int64_t)s0 * H + h) * kD * kD);
  // segment 0: positions [0, m) into b0's slot (only when m > 0);
  // segment 1: positions [m, n) into b1's slot.  One loop body, so one copy
  // of the accumulation holds registers.
#pragma nounroll
  for (int seg = m > 0 ? 0 : 1; seg < 2; ++seg) {
    advance(S, seg == 0 ? 0 : m, seg == 0 ? m : n, kg_rec, u_rec, rec0, sm);
    store_state(pool + ((int64_t)(seg == 0 ? s0 : s1) * H + h) * kD * kD, S);
  }
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

template <typename TPool>
hipError_t align_by_rec(const CommitAlignArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.n_req * a.H)), block(kT);
#define KDA_COMMIT_ALIGN_LAUNCH(TR)                                                                 \
  hipLaunchKernelGGL((kda_commit_align_kernel<TPool, TR>), grid, block, 0, st,                      \
                     static_cast<TPool*>(a.pool.base), a.pool.n_slots, a.block_table, a.blocks_per_req, \
                     a.num_tokens, a.accepted_len, a.block_size, a.u_rec,                           \
                     static_cast<const TR*>(a.kg_rec), a.n_req, a.L, a.H,                           \
                     AlignNext{a.next_tokens, a.next_block, a.next_ckpt, a.next_bias}, a.dev_err)
  switch (a.rec_dtype) {
    case F32: KDA_COMMIT_ALIGN_LAUNCH(float); break;
    case F16: KDA_COMMIT_ALIGN_LAUNCH(f16); break;
    case BF16: KDA_COMMIT_ALIGN_LAUNCH(bf16); break;
    default: return hipErrorInvalidValue;
  }
#undef KDA_COMMIT_ALIGN_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_commit_align(const CommitAlignArgs& a, hipStream_t st) {
  if (a.d != kD) return hipErrorInvalidValue;
  if (a.n_req == 0) return hipSuccess;
  switch (a.pool.dtype) {
    case F32: return align_by_rec<float>(a, st);
    case F16: return align_by_rec<f16>(a, st);
    case BF16: return align_by_rec<bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

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
