// Chunked KDA prefill for gfx950.
//
// Chunk form of the recurrence (for a chunk of n <= C tokens starting from
// state S, with the in-chunk cumulative log decay Gamma_r = sum_{s<=r} g_s):
//   Kt = K e^Gamma, Kh = K e^-Gamma, Qt = Q e^Gamma, Kb = K e^(Gamma_n - Gamma)
//   M  = strict_tril(Kt Kh^T),   P = tril(Qt Kh^T)
//   T  = (I + Diag(beta) M)^-1                       (unit lower triangular)
//   U  = T Diag(beta) (V - Kt S)                     (rows of U are u_t)
//   O  = Qt S + P U
//   S' = Diag(e^Gamma_n) S + Kb^T U
// Serial steps per sequence = ceil(T_i / C) (state-semantics page, sec. 5);
// the state at a requested chunk boundary is taken from the fp32 accumulator
// and cast once into the pool dtype (SGLang PR #34820 summary,
// implementation breakdown item 2 and the kda_prefill.py excerpt).
//
// Three launches on the caller's stream:
//  1. kda_chunk_map: one block turns cu_seqlens into per-sequence chunk offsets
//     (and validates them) without any host synchronisation.
//  2. kda_chunk_prep: one workgroup per (chunk, head), fully parallel.  Computes
//     everything that does not depend on the state -- Kt, Qt, Kb^T, T, P, beta,
//     e^Gamma_n -- and writes it as one record to the workspace, with every
//     matrix stored as MFMA A-operand fragments (1 KiB blocks, 16 bytes per
//     lane) so that the scan reads them with fully coalesced loads straight
//     into registers.  The gate exponentials take one exp per element plus
//     in-chunk cumulative products; M and P run on MFMA; T is a blocked
//     inverse (16x16 diagonal blocks by forward substitution, off-diagonal
//     blocks on fp32 MFMA).  LDS is reused across phases (~73 KiB) so two
//     workgroups share a CU.
//  3. kda_chunk_scan: one workgroup per (sequence, head, BV-column tile of S).
//     The columns of S evolve independently, so tiles never exchange data.  The
//     fp32 state tile lives in MFMA accumulator registers for the whole
//     sequence.  Each wave keeps the next chunk's fragments in flight while it
//     runs the five state-dependent products of this one (buffer loads off a
//     per-chunk descriptor, so almost no address arithmetic); only the
//     small B operands (S, Y, U in bf16) pass through LDS.  Workgroups of one
//     head land on one XCD so that they share the head's records in that
//     XCD's L2.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kThreads = 256;
constexpr int kXcd = 8;     // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kFB = 1024;   // bytes of one fragment block: 64 lanes x 16 bytes

// K-block sizes: 32 for the 16-bit 16x16x32 MFMAs; fp32 uses 16 so that one
// lane's fragment is 16 bytes as well.
template <typename TOp> struct KBOf { static constexpr int v = (sizeof(TOp) == 4) ? 16 : 32; };

// Workspace record for one (chunk, head).  A-operand matrices are stored as
// fragment blocks: block (tile, kb) of an M x K matrix holds, for lane
// l = 16 g + r, row 16 tile + r at K-block positions kb*KB + (KB/4) g + j.
template <int DK, int C, typename TOp>
struct Rec {
  static constexpr int KBK = KBOf<TOp>::v, KBT = KBOf<TOp>::v;
  static constexpr int NBK = (C / 16) * (DK / KBK);   // Kt and Qt blocks   (tile = token tile)
  static constexpr int NBB = (DK / 16) * (C / KBT);   // Kb^T blocks        (tile = key tile)
  static constexpr int NBT = (C / 16) * (C / KBT);    // T and P blocks     (tile = token tile)
  static constexpr int kKt = 0;
  static constexpr int kQt = kKt + NBK * kFB;
  static constexpr int kKbT = kQt + NBK * kFB;
  static constexpr int kT = kKbT + NBB * kFB;
  static constexpr int kP = kT + NBT * kFB;
  static constexpr int kBeta = kP + NBT * kFB;          // [C]  fp32
  static constexpr int kDec = kBeta + C * 4;            // [DK] fp32, e^Gamma_n
  static constexpr int kEnd = kDec + DK * 4;
  static constexpr int kBytes = (kEnd + 255) / 256 * 256;
  static_assert((KBK / 4) * sizeof(TOp) == 16, "16-byte fragments");
  static_assert(DK % KBK == 0 && C % KBT == 0, "tile sizes");
};

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ inline int64_t map_bytes(int n_seqs) { return round_up(4 * (int64_t)(n_seqs + 1), 256); }
__host__ __device__ inline int64_t chunk_upper_bound(int64_t total_tokens, int n_seqs, int C) {
  return total_tokens / C + n_seqs;
}

// Inverse of pos_in_block: index stored at position p of a K-block.
template <int KB>
__device__ __forceinline__ int idx_in_block(int p) {
  if (KB == 16) return p;
  const int g = p >> 3, j = p & 7;
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// A sequence is processed only if its cu_seqlens entries are sane and the
// chunk map gave it exactly ceil(len / C) chunks.
__device__ __forceinline__ bool seq_ok(const int32_t* cu, const int32_t* off, int seq,
                                       int64_t total, int C, int& t_beg, int& len, int& nch) {
  t_beg = cu[seq];
  const int t_end = cu[seq + 1];
  len = t_end - t_beg;
  nch = (len + C - 1) / C;
  return t_beg >= 0 && len >= 0 && (int64_t)t_end <= total && off[seq + 1] - off[seq] == nch;
}

// 16 bytes viewed as a fragment of TOp elements.
template <typename TOp>
union Frag16 {
  uint4 u;
  TOp e[16 / sizeof(TOp)];
};

template <typename F>
__device__ __forceinline__ F as_frag(const uint4& x) {
  static_assert(sizeof(F) == 16, "fragment size");
  F f;
  __builtin_memcpy(&f, &x, 16);
  return f;
}

// ---------------------------------------------------------------- 1. chunk map

__global__ __launch_bounds__(kThreads) void kda_chunk_map(const int32_t* __restrict__ cu, int n_seqs,
                                                          int64_t total, int C, int64_t cap,
                                                          int32_t* __restrict__ off,
                                                          int32_t* __restrict__ dev_err) {
  __shared__ int32_t s_scan[kThreads];
  __shared__ int64_t s_carry;
  if (threadIdx.x == 0) { s_carry = 0; off[0] = 0; }
  __syncthreads();
  for (int base = 0; base < n_seqs; base += kThreads) {
    const int i = base + threadIdx.x;
    int nch = 0;
    bool bad = false;
    if (i < n_seqs) {
      const int a = cu[i], b2 = cu[i + 1];
      bad = a < 0 || b2 < a || (int64_t)b2 > total;
      nch = bad ? 0 : (b2 - a + C - 1) / C;
    }
    s_scan[threadIdx.x] = nch;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {  // inclusive Hillis-Steele scan
      const int x = threadIdx.x >= d ? s_scan[threadIdx.x - d] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += x;
      __syncthreads();
    }
    if (i < n_seqs) {
      int64_t end = s_carry + s_scan[threadIdx.x];
      // Never let the chunk count exceed what the workspace was sized for
      // (only possible with overlapping, non-monotone cu_seqlens): clamping
      // keeps off[] monotone and makes the offending sequences fail seq_ok.
      if (end > cap) { bad = true; end = cap; }
      if (bad) set_err(dev_err, 1u << 3);
      off[i + 1] = (int32_t)end;
    }
    __syncthreads();
    if (threadIdx.x == kThreads - 1) s_carry += s_scan[kThreads - 1];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- 2. prep

template <int DK, int C, typename TOp>
struct PrepSmem {
  static constexpr int PADK = 16 / (int)sizeof(TOp);
  static constexpr int LDK = DK + PADK;  // row length (elements) of [C][DK] images
  static constexpr int LDT = C + PADK;   // row length of [*][C] TOp images
  static constexpr int LDF = C + 4;      // row length of fp32 [C][C] arrays
  static constexpr int NCQ = DK / 4;
  static constexpr int NTG0 = kThreads / NCQ;
  static constexpr int NTG = NTG0 < C ? NTG0 : C;
  static constexpr int TPG = C / NTG;
  struct A {            // phases 1-2: operand images (positions permuted per K-block)
    TOp kt[C * LDK];
    TOp kh[C * LDK];
    TOp qt[C * LDK];
    TOp kbt[DK * LDT];
  };
  struct B {            // phases 3-5: solve
    float n[C * LDF];   // Diag(beta) strict_tril(M)
    float tr[C * LDF];  // T row-major
    float tt[C * LDF];  // T transposed
    TOp p[C * LDT];     // P image (lower tiles only)
  };
  union { A a; B b; } u;
  float beta[C];
  float gp[NTG * DK];   // per-token-group decay products
};

template <int DK, int C, typename TIn, typename TOp>
__global__ __launch_bounds__(kThreads) void kda_chunk_prep(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ g,
    const TIn* __restrict__ bl, const int32_t* __restrict__ cu, int n_seqs, int64_t total,
    int H, int64_t cap, const int32_t* __restrict__ off, uint8_t* __restrict__ recs) {
  typedef PrepSmem<DK, C, TOp> Sm;
  typedef Rec<DK, C, TOp> R;
  constexpr int KBK = R::KBK, KBT = R::KBT;
  constexpr int NT = C / 16;
  constexpr int EPF = 16 / (int)sizeof(TOp);   // elements per 16-byte fragment
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int h = blockIdx.x % H;
  const int j = blockIdx.x / H;  // global chunk slot
  if (j >= off[n_seqs]) return;
  // sequence owning chunk slot j: largest seq with off[seq] <= j
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int seq = lo;
  int t_beg, len, nch;
  if (!seq_ok(cu, off, seq, total, C, t_beg, len, nch)) return;
  const int c = j - off[seq];
  if (c >= nch) return;
  const int t0 = t_beg + c * C;
  const int n = min(C, len - c * C);
  const int64_t rowstride = (int64_t)H * DK;
  // records are head-major: one sequence's chunks of one head are contiguous
  uint8_t* rec = recs + ((int64_t)h * cap + j) * R::kBytes;

  // ---- phase 1: decay products, Kt, Kh, Qt, Kb^T images
  const int cq = tid % Sm::NCQ, tg = tid / Sm::NCQ;
  const bool active = tg < Sm::NTG;
  floatx4 kv[Sm::TPG], qv[Sm::TPG], fw[Sm::TPG], bw[Sm::TPG];
  floatx4 gprod = {1.f, 1.f, 1.f, 1.f};
  if (active) {
    // Branch-free loads (row clamped in bounds) so they are all in flight at
    // once; rows past the chunk's end become k = q = 0, alpha = 1.
    typename Vec4<TIn>::type kr[Sm::TPG], qr[Sm::TPG], gr[Sm::TPG];
#pragma unroll
    for (int jj = 0; jj < Sm::TPG; ++jj) {
      const int t = min(tg * Sm::TPG + jj, n - 1);
      const int64_t base = (int64_t)(t0 + t) * rowstride + (int64_t)h * DK + 4 * cq;
      kr[jj] = *reinterpret_cast<const typename Vec4<TIn>::type*>(k + base);
      qr[jj] = *reinterpret_cast<const typename Vec4<TIn>::type*>(q + base);
      gr[jj] = *reinterpret_cast<const typename Vec4<TIn>::type*>(g + base);
    }
#pragma unroll
    for (int jj = 0; jj < Sm::TPG; ++jj) {
      const bool valid = tg * Sm::TPG + jj < n;
      floatx4 alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[jj][e] = valid ? to_f32(kr[jj][e]) : 0.f;
        qv[jj][e] = valid ? to_f32(qr[jj][e]) : 0.f;
        alpha[e] = valid ? __expf(to_f32(gr[jj][e])) : 1.f;
      }
      gprod = gprod * alpha;
      fw[jj] = gprod;  // prod_{s <= t, s in group} alpha_s
      bw[jj] = alpha;  // temporarily alpha_t
    }
    // in-group suffix products: bw[jj] = prod_{jj < s < TPG} alpha_s
    floatx4 suf = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int jj = Sm::TPG - 1; jj >= 0; --jj) {
      const floatx4 a = bw[jj];
      bw[jj] = suf;
      suf = suf * a;
    }
    *reinterpret_cast<floatx4*>(&sm.gp[tg * DK + 4 * cq]) = gprod;
  }
  if (tid < C) {
    const float braw = to_f32(bl[(int64_t)(t0 + min(tid, n - 1)) * H + h]);
    const float be = tid < n ? sigmoidf_(braw) : 0.f;
    sm.beta[tid] = be;
    reinterpret_cast<float*>(rec + R::kBeta)[tid] = be;
  }
  __syncthreads();
  if (active) {
    floatx4 pre = {1.f, 1.f, 1.f, 1.f}, post = {1.f, 1.f, 1.f, 1.f};
    for (int x = 0; x < Sm::NTG; ++x) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(&sm.gp[x * DK + 4 * cq]);
      if (x < tg) pre = pre * v;
      if (x > tg) post = post * v;
    }
    const floatx4 total_dec = pre * gprod * post;  // e^Gamma_n
    floatx4 inv_total;
#pragma unroll
    for (int e = 0; e < 4; ++e) inv_total[e] = 1.0f / total_dec[e];
    const int kp = pos_of<KBK>(4 * cq);
#pragma unroll
    for (int jj = 0; jj < Sm::TPG; ++jj) {
      const int t = tg * Sm::TPG + jj;
      const floatx4 epos = pre * fw[jj];                 // e^Gamma_t
      const floatx4 erem = bw[jj] * post;                // e^(Gamma_n - Gamma_t)
      const floatx4 eneg = erem * inv_total;             // e^-Gamma_t
      store4(&sm.u.a.kt[t * Sm::LDK + kp], kv[jj] * epos);
      store4(&sm.u.a.kh[t * Sm::LDK + kp], kv[jj] * eneg);
      store4(&sm.u.a.qt[t * Sm::LDK + kp], qv[jj] * epos);
      const floatx4 kb = kv[jj] * erem;
      const int tp = pos_of<KBT>(t);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.a.kbt[(4 * cq + e) * Sm::LDT + tp] = from_f32<TOp>(kb[e]);
    }
    if (tg == 0) *reinterpret_cast<floatx4*>(rec + R::kDec + 16 * cq) = total_dec;
  }
  __syncthreads();

  // ---- phase 2: M and P tiles (lower triangle only) into registers; the
  //      Kt, Qt and Kb^T images go out as fragment blocks.
  typedef Frag<TOp, KBK> FK;
  constexpr int NTRI = NT * (NT + 1) / 2;
  constexpr int TPW = (2 * NTRI + 3) / 4;  // tiles per wave
  floatx4 tacc[TPW];
#pragma unroll
  for (int q2 = 0; q2 < TPW; ++q2) {
    const int ti = wave + 4 * q2;
    tacc[q2] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (ti < 2 * NTRI) {
      const bool isP = ti >= NTRI;
      int idx = isP ? ti - NTRI : ti, m = 0;
      while (idx > m) { idx -= m + 1; ++m; }
      const TOp* arow = (isP ? sm.u.a.qt : sm.u.a.kt) + (16 * m + l16) * Sm::LDK;
      const TOp* brow = sm.u.a.kh + (16 * idx + l16) * Sm::LDK;
#pragma unroll
      for (int kb = 0; kb < DK / KBK; ++kb)
        tacc[q2] = mma(tacc[q2], FK::load(arow, kb, g16), FK::load(brow, kb, g16));
    }
  }
  {
    // image rows -> fragment blocks: item = (block, lane)
    constexpr int NKB = DK / KBK, NTB = C / KBT;
    for (int it = tid; it < (2 * R::NBK + R::NBB) * 64; it += kThreads) {
      const int blk = it >> 6, ln = it & 63, gg = ln >> 4, rr = ln & 15;
      const TOp* src;
      int dst;
      if (blk < 2 * R::NBK) {
        const int b2 = blk % R::NBK, mt = b2 / NKB, kb = b2 % NKB;
        src = (blk < R::NBK ? sm.u.a.kt : sm.u.a.qt) + (16 * mt + rr) * Sm::LDK + kb * KBK + (KBK / 4) * gg;
        dst = (blk < R::NBK ? R::kKt : R::kQt) + b2 * kFB + ln * 16;
      } else {
        const int b2 = blk - 2 * R::NBK, kt = b2 / NTB, tb = b2 % NTB;
        src = sm.u.a.kbt + (16 * kt + rr) * Sm::LDT + tb * KBT + (KBT / 4) * gg;
        dst = R::kKbT + b2 * kFB + ln * 16;
      }
      *reinterpret_cast<uint4*>(rec + dst) = *reinterpret_cast<const uint4*>(src);
    }
  }
  __syncthreads();

  // ---- phase 3: N = Diag(beta) strict_tril(M) (fp32) and the P image
#pragma unroll
  for (int q2 = 0; q2 < TPW; ++q2) {
    const int ti = wave + 4 * q2;
    if (ti < 2 * NTRI) {
      const bool isP = ti >= NTRI;
      int idx = isP ? ti - NTRI : ti, m = 0;
      while (idx > m) { idx -= m + 1; ++m; }
      const int s = 16 * idx + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * m + 4 * g16 + i;
        if (isP) sm.u.b.p[r * Sm::LDT + pos_of<KBT>(s)] = from_f32<TOp>(tacc[q2][i]);
        else sm.u.b.n[r * Sm::LDF + s] = s < r ? sm.beta[r] * tacc[q2][i] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- phase 4: T = (I + N)^-1; diagonal 16x16 blocks by forward substitution
  if (wave == 0) {
    const int bi = lane >> 4, s = l16;
    if (bi < NT) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == s) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        const float* nrow = sm.u.b.n + (16 * bi + r) * Sm::LDF + 16 * bi;
        float acc = 0.f;
#pragma unroll
        for (int jj = 0; jj < r; ++jj) acc += nrow[jj] * x[jj];
        if (r > s) x[r] = -acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.u.b.tr[(16 * bi + r) * Sm::LDF + 16 * bi + s] = x[r];
        sm.u.b.tt[(16 * bi + s) * Sm::LDF + 16 * bi + r] = x[r];
      }
    }
  }
  // off-diagonal blocks, one block row at a time:
  //   T_ij = -T_ii * sum_{m=j}^{i-1} N_im T_mj   (fp32 MFMA, K-blocks of 16)
  for (int bi = 1; bi < NT; ++bi) {
    __syncthreads();
    const int bj = wave;
    if (bj < bi) {
      floatx4 racc = {0.f, 0.f, 0.f, 0.f};
      for (int bm = bj; bm < bi; ++bm) {
        const floatx4 av = *reinterpret_cast<const floatx4*>(sm.u.b.n + (16 * bi + l16) * Sm::LDF + 16 * bm + 4 * g16);
        const floatx4 bv = *reinterpret_cast<const floatx4*>(sm.u.b.tt + (16 * bj + l16) * Sm::LDF + 16 * bm + 4 * g16);
        f32frag<4> fa, fb;
#pragma unroll
        for (int e = 0; e < 4; ++e) { fa.v[e] = av[e]; fb.v[e] = bv[e]; }
        racc = mma(racc, fa, fb);
      }
      const floatx4 tav = *reinterpret_cast<const floatx4*>(sm.u.b.tr + (16 * bi + l16) * Sm::LDF + 16 * bi + 4 * g16);
      f32frag<4> fa, fb;
#pragma unroll
      for (int e = 0; e < 4; ++e) { fa.v[e] = tav[e]; fb.v[e] = racc[e]; }
      floatx4 tij = mma(floatx4{0.f, 0.f, 0.f, 0.f}, fa, fb);
      tij = -tij;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.u.b.tr[(16 * bi + 4 * g16 + i) * Sm::LDF + 16 * bj + l16] = tij[i];
      *reinterpret_cast<floatx4*>(sm.u.b.tt + (16 * bj + l16) * Sm::LDF + 16 * bi + 4 * g16) = tij;
    }
  }
  __syncthreads();

  // ---- phase 5: T and P fragment blocks, zero above the diagonal
  {
    constexpr int NTB = C / KBT;
    for (int it = tid; it < 2 * R::NBT * 64; it += kThreads) {
      const int blk = it >> 6, ln = it & 63, gg = ln >> 4, rr = ln & 15;
      const bool isP = blk >= R::NBT;
      const int b2 = isP ? blk - R::NBT : blk, mt = b2 / NTB, kb = b2 % NTB;
      const int r = 16 * mt + rr;
      Frag16<TOp> f;
      if (isP) f.u = *reinterpret_cast<const uint4*>(sm.u.b.p + r * Sm::LDT + kb * KBT + (KBT / 4) * gg);
#pragma unroll
      for (int e = 0; e < EPF; ++e) {
        const int s = kb * KBT + idx_in_block<KBT>((KBT / 4) * gg + e);
        if (isP) {
          if (s > r) f.e[e] = from_f32<TOp>(0.f);
        } else {
          f.e[e] = from_f32<TOp>(s <= r ? sm.u.b.tr[r * Sm::LDF + s] : 0.f);
        }
      }
      *reinterpret_cast<uint4*>(rec + (isP ? R::kP : R::kT) + b2 * kFB + ln * 16) = f.u;
    }
  }
}

// ---------------------------------------------------------------- 3. scan

template <int DK, int DV, int C, int BV, typename TOp>
struct ScanSmem {
  static constexpr int PADK = 16 / (int)sizeof(TOp);
  static constexpr int LDK = DK + PADK;
  static constexpr int LDT = C + PADK;
  TOp s[BV * LDK];  // state tile as B operand, [v][pos(k)]
  TOp y[BV * LDT];  // Diag(beta)(V - Kt S), [v][pos(t)]
  TOp u[BV * LDT];  // U, [v][pos(t)]
};

// Per-wave operands of one chunk, loaded straight from the record.
template <int DK, int C, int BV, typename TIn, typename TOp>
struct ChunkOps {
  static constexpr int KBK = KBOf<TOp>::v, KBT = KBOf<TOp>::v;
  static constexpr int NK = DK / 16, NKW = (NK + 3) / 4, NVS = BV / 16;
  static constexpr int NFK = DK / KBK, NFT = C / KBT, NFB = NKW * NFT;
  uint4 kt[NFK], qt[NFK], t[NFT], p[NFT], kb[NFB];
  floatx4 beta;
  floatx4 dec[NKW];
  typename std::conditional<sizeof(TIn) == 2, uint16_t, uint32_t>::type v[NVS][4];  // raw bits
};

template <typename T>
__device__ __forceinline__ T bits_to(uint32_t b) {
  if constexpr (sizeof(T) == 2) {
    const uint16_t h = (uint16_t)b;
    T x;
    __builtin_memcpy(&x, &h, 2);
    return x;
  } else {
    T x;
    __builtin_memcpy(&x, &b, 4);
    return x;
  }
}
template <typename T>
__device__ __forceinline__ uint32_t to_bits(T x) {
  if constexpr (sizeof(T) == 2) {
    uint16_t h;
    __builtin_memcpy(&h, &x, 2);
    return h;
  } else {
    uint32_t b;
    __builtin_memcpy(&b, &x, 4);
    return b;
  }
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return uint4{(unsigned)x[0], (unsigned)x[1], (unsigned)x[2], (unsigned)x[3]};
}
__device__ __forceinline__ floatx4 ld16f(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  floatx4 f;
  __builtin_memcpy(&f, &x, 16);
  return f;
}

template <int DK, int DV, int C, int BV, typename TIn, typename TOp, typename TPool>
__global__ __launch_bounds__(kThreads) void kda_chunk_scan(
    const TIn* __restrict__ v, TIn* __restrict__ o, const int32_t* __restrict__ cu, int n_seqs,
    int64_t total, int H, int64_t cap, const int32_t* __restrict__ off, const uint8_t* __restrict__ recs,
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ init_slot,
    const int32_t* __restrict__ final_slot, const int32_t* __restrict__ track_ptr,
    const int32_t* __restrict__ track_chunk, const int32_t* __restrict__ track_slot, int n_track,
    float* __restrict__ track_f32, int32_t* __restrict__ dev_err) {
  typedef ScanSmem<DK, DV, C, BV, TOp> Sm;
  typedef Rec<DK, C, TOp> R;
  typedef ChunkOps<DK, C, BV, TIn, TOp> Ops;
  constexpr int KBK = R::KBK, KBT = R::KBT;
  constexpr int NT = C / 16, NK = DK / 16, NVS = BV / 16, NVT = DV / BV;
  constexpr int NKW = Ops::NKW, NFK = Ops::NFK, NFT = Ops::NFT;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  typedef typename Frag<TOp, KBK>::type FKt;
  typedef typename Frag<TOp, KBT>::type FTt;
  typedef Frag<TOp, KBK> FK;
  typedef Frag<TOp, KBT> FT;

  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  // XCD-aware decode: all NVT tiles of one (seq, head) pair share blockIdx % 8.
  const int xcd = blockIdx.x % kXcd, slot_ = blockIdx.x / kXcd;
  const int vt = slot_ % NVT;
  const int pair = (slot_ / NVT) * kXcd + xcd;
  if (pair >= n_seqs * H) return;
  const int seq = pair / H, h = pair % H;
  int t_beg, len, nch;
  if (!seq_ok(cu, off, seq, total, C, t_beg, len, nch)) return;
  const int v0 = vt * BV;
  const bool lead = (vt == 0 && h == 0);
  const int m = wave;  // token tile of this wave
  // With 4 waves: every wave owns a token tile when C >= 64 and two state
  // tiles when d_k = 128; the guards below fold away in that case.
  constexpr bool kAllTiles = NT >= 4;
  constexpr bool kAllK = NK >= 4 * NKW;

  // ---- tracks of this sequence (CSR)
  int e0 = 0, e1 = 0;
  if (track_ptr != nullptr && n_track > 0) {
    e0 = track_ptr[seq];
    e1 = track_ptr[seq + 1];
    if (e0 < 0 || e1 < e0 || e1 > n_track) {
      if (lead && tid == 0) set_err(dev_err, 1u << 1);
      e0 = e1 = 0;
    }
  }
  if (lead) {
    for (int e = e0 + tid; e < e1; e += kThreads) {
      const int ce = track_chunk[e], se = track_slot[e];
      if (ce < 0 || ce > len / C) set_err(dev_err, 1u << 1);
      if (se < -1 || (int64_t)se >= n_slots) set_err(dev_err, 1u);
    }
  }

  // ---- initial state: S[k][v] = pool[init][h][v][k]
  floatx4 S[NKW][NVS];
  {
    const int is = init_slot[seq];
    const bool ok = is >= 0 && (int64_t)is < n_slots;
    if (!ok && is != -1 && lead && tid == 0) set_err(dev_err, 1u);
#pragma unroll
    for (int a = 0; a < NKW; ++a)
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        S[a][vs] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int kt = wave + 4 * a;
        if (ok && kt < NK) {
          const int vv = v0 + 16 * vs + l16, kk = 16 * kt + 4 * g16;
          S[a][vs] = load4(pool + (((int64_t)is * H + h) * DV + vv) * DK + kk);
        }
      }
  }

  auto snapshot = [&](int c) {
    for (int e = e0; e < e1; ++e) {
      if (track_chunk[e] != c) continue;
      const int se = track_slot[e];
      const bool to_pool = se >= 0 && (int64_t)se < n_slots;
#pragma unroll
      for (int a = 0; a < NKW; ++a)
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs) {
          const int kt = wave + 4 * a;
          if (kt >= NK) continue;
          const int vv = v0 + 16 * vs + l16, kk = 16 * kt + 4 * g16;
          if (track_f32) store4(track_f32 + (((int64_t)e * H + h) * DV + vv) * DK + kk, S[a][vs]);
          if (to_pool) store4(pool + (((int64_t)se * H + h) * DV + vv) * DK + kk, S[a][vs]);
        }
    }
  };

  const int64_t vrow = (int64_t)H * DV;
  const int nkb_m = (16 * m + 15) / KBT + 1;  // K-blocks of T and P rows up to the diagonal

  // ---- issue the loads of chunk c's operands.  Buffer loads: the base is a
  //      per-chunk resource in scalar registers and every per-lane offset is a
  //      constant, so the loads cost almost no vector ALU work, and there are
  //      no branches, so they stay in flight while the previous chunk is
  //      computed.  V reads past the chunk's last row return 0 (range check);
  //      those rows have beta = 0 and zero keys in any case.
  const int mt = m < NT ? m : NT - 1;
  const int lane_off = lane * 16;
  const int beta_off = (16 * mt + 4 * g16) * 4;
  int dec_off[NKW];
#pragma unroll
  for (int a = 0; a < NKW; ++a) dec_off[a] = (16 * min(wave + 4 * a, NK - 1) + 4 * g16) * 4;
  int v_off[NVS][4];  // byte offsets of this lane's V / o elements inside a chunk
#pragma unroll
  for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v_off[vs][i] = (int)(((int64_t)(16 * mt + 4 * g16 + i) * vrow + 16 * vs + l16) * (int)sizeof(TIn));
  const uint8_t* rec_seq = recs + ((int64_t)h * cap + off[seq]) * R::kBytes;

  auto rows_rsrc = [&](const TIn* base, int c) {
    const int n = min(C, len - c * C);
    const TIn* p = base + (int64_t)(t_beg + c * C) * vrow + (int64_t)h * DV + v0;
    return buffer_rsrc(p, (uint32_t)(((int64_t)(n - 1) * vrow + BV) * (int)sizeof(TIn)));
  };

  auto load_ops = [&](Ops& op, int c) {
    const auto rs = buffer_rsrc(rec_seq + (int64_t)c * R::kBytes, R::kBytes);
#pragma unroll
    for (int f = 0; f < NFK; ++f) {
      op.kt[f] = ld16(rs, lane_off, R::kKt + (mt * NFK + f) * kFB);
      op.qt[f] = ld16(rs, lane_off, R::kQt + (mt * NFK + f) * kFB);
    }
#pragma unroll
    for (int f = 0; f < NFT; ++f) {
      op.t[f] = ld16(rs, lane_off, R::kT + (mt * NFT + f) * kFB);
      op.p[f] = ld16(rs, lane_off, R::kP + (mt * NFT + f) * kFB);
    }
    op.beta = ld16f(rs, beta_off, R::kBeta);
#pragma unroll
    for (int a = 0; a < NKW; ++a) {
      const int kt = min(wave + 4 * a, NK - 1);
#pragma unroll
      for (int f = 0; f < NFT; ++f) op.kb[a * NFT + f] = ld16(rs, lane_off, R::kKbT + (kt * NFT + f) * kFB);
      op.dec[a] = ld16f(rs, dec_off[a], R::kDec);
    }
    const auto rv = rows_rsrc(v, c);
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(TIn) == 2) op.v[vs][i] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rv, v_off[vs][i], 0, 0);
        else op.v[vs][i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rv, v_off[vs][i], 0, 0);
      }
  };

  // ---- the state-dependent part of one chunk
  auto step = [&](const Ops& op, int c) {
    // state tile -> LDS as the B operand of Kt S and Qt S
#pragma unroll
    for (int a = 0; a < NKW; ++a) {
      const int kt = wave + 4 * a;
      if (!kAllK && kt >= NK) continue;
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs)
        store4(&sm.s[(16 * vs + l16) * Sm::LDK + pos_of<KBK>(16 * kt + 4 * g16)], S[a][vs]);
    }
    __syncthreads();
    // X = Kt S, O = Qt S, Y = Diag(beta)(V - X)
    floatx4 O[NVS];
    if (kAllTiles || m < NT) {
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        floatx4 X = {0.f, 0.f, 0.f, 0.f};
        O[vs] = X;
        const TOp* srow = sm.s + (16 * vs + l16) * Sm::LDK;
#pragma unroll
        for (int kb = 0; kb < NFK; ++kb) {
          const FKt sf = FK::load(srow, kb, g16);
          X = mma(X, as_frag<FKt>(op.kt[kb]), sf);
          O[vs] = mma(O[vs], as_frag<FKt>(op.qt[kb]), sf);
        }
        floatx4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = op.beta[i] * (to_f32(bits_to<TIn>(op.v[vs][i])) - X[i]);
        store4(&sm.y[(16 * vs + l16) * Sm::LDT + pos_of<KBT>(16 * m + 4 * g16)], Y);
      }
    }
    __syncthreads();
    // U = T Y  (T lower triangular: only K-blocks up to the diagonal)
    if (kAllTiles || m < NT) {
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        floatx4 U = {0.f, 0.f, 0.f, 0.f};
        const TOp* yrow = sm.y + (16 * vs + l16) * Sm::LDT;
#pragma unroll
        for (int kb = 0; kb < NFT; ++kb)
          if (kb < nkb_m) U = mma(U, as_frag<FTt>(op.t[kb]), FT::load(yrow, kb, g16));
        store4(&sm.u[(16 * vs + l16) * Sm::LDT + pos_of<KBT>(16 * m + 4 * g16)], U);
      }
    }
    __syncthreads();
    // O += P U -> o;  S = Diag(e^Gamma_n) S + Kb^T U
    const auto ro = rows_rsrc(o, c);
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) {
      const TOp* urow = sm.u + (16 * vs + l16) * Sm::LDT;
      FTt uf[NFT];
#pragma unroll
      for (int kb = 0; kb < NFT; ++kb) uf[kb] = FT::load(urow, kb, g16);
      if (kAllTiles || m < NT) {
#pragma unroll
        for (int kb = 0; kb < NFT; ++kb)
          if (kb < nkb_m) O[vs] = mma(O[vs], as_frag<FTt>(op.p[kb]), uf[kb]);
        // rows past the chunk's end fall outside the resource and are dropped
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t bits = to_bits(from_f32<TIn>(O[vs][i]));
          if constexpr (sizeof(TIn) == 2) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bits, ro, v_off[vs][i], 0, 0);
          else __builtin_amdgcn_raw_buffer_store_b32(bits, ro, v_off[vs][i], 0, 0);
        }
      }
#pragma unroll
      for (int a = 0; a < NKW; ++a) {
        const int kt = wave + 4 * a;
        if (!kAllK && kt >= NK) continue;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NFT; ++kb) acc = mma(acc, as_frag<FTt>(op.kb[a * NFT + kb]), uf[kb]);
        S[a][vs] = op.dec[a] * S[a][vs] + acc;
      }
    }
    // No trailing barrier: the next chunk's LDS writes come after barriers
    // that a wave passes only once every wave has finished this chunk's reads.
  };

  Ops opA, opB;
  if (nch > 0) load_ops(opA, 0);
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    snapshot(c);
    load_ops(opB, c + 1);
    step(opA, c);
    snapshot(c + 1);
    // unconditional (a redundant reload of the last chunk at the end) so that
    // the waits for opB above stay partial
    load_ops(opA, min(c + 2, nch - 1));
    step(opB, c + 1);
  }
  if (c < nch) {
    snapshot(c);
    step(opA, c);
  }
  if (len % C == 0) snapshot(nch);

  // ---- final state, one cast into the pool dtype
  const int fs = final_slot[seq];
  if (fs >= 0 && (int64_t)fs < n_slots) {
#pragma unroll
    for (int a = 0; a < NKW; ++a)
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        const int kt = wave + 4 * a;
        if (kt >= NK) continue;
        const int vv = v0 + 16 * vs + l16, kk = 16 * kt + 4 * g16;
        store4(pool + (((int64_t)fs * H + h) * DV + vv) * DK + kk, S[a][vs]);
      }
  } else if (fs != -1 && lead && tid == 0) {
    set_err(dev_err, 1u);
  }
}

// ---------------------------------------------------------------- host side

namespace {

template <int DK, int DV, int C, int BV, typename TIn, typename TOp, typename TPool>
hipError_t run(const PrefillArgs& a, hipStream_t st) {
  typedef PrepSmem<DK, C, TOp> SmP;
  typedef ScanSmem<DK, DV, C, BV, TOp> SmS;
  const int64_t cap = chunk_upper_bound(a.total_tokens, a.n_seqs, C);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  int32_t* off = reinterpret_cast<int32_t*>(ws);
  uint8_t* recs = ws + map_bytes(a.n_seqs);

  hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(kThreads), 0, st, a.cu_seqlens, a.n_seqs,
                     a.total_tokens, C, cap, off, a.dev_err);
  if (cap > 0) {
    auto kp = kda_chunk_prep<DK, C, TIn, TOp>;
    const int smp = (int)sizeof(SmP);
    hipError_t e = hipFuncSetAttribute((const void*)kp, hipFuncAttributeMaxDynamicSharedMemorySize, smp);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kp, dim3((unsigned)(cap * a.H)), dim3(kThreads), smp, st,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.g), static_cast<const TIn*>(a.b), a.cu_seqlens,
                       a.n_seqs, a.total_tokens, a.H, cap, off, recs);
  }
  auto ks = kda_chunk_scan<DK, DV, C, BV, TIn, TOp, TPool>;
  const int sms = (int)sizeof(SmS);
  const int64_t pairs = (int64_t)a.n_seqs * a.H;
  const int64_t blocks = (pairs + kXcd - 1) / kXcd * kXcd * (DV / BV);
  hipLaunchKernelGGL(ks, dim3((unsigned)blocks), dim3(kThreads), sms, st,
                     static_cast<const TIn*>(a.v), static_cast<TIn*>(a.o), a.cu_seqlens, a.n_seqs,
                     a.total_tokens, a.H, cap, off, recs, static_cast<TPool*>(a.pool.base),
                     a.pool.n_slots, a.init_slot, a.final_slot, a.track_ptr, a.track_chunk,
                     a.track_slot, a.n_track, a.track_f32, a.dev_err);
  return hipGetLastError();
}

template <int DK, int DV, int C, int BV, typename TIn, typename TOp>
hipError_t by_pool(const PrefillArgs& a, hipStream_t st) {
  switch (a.pool.dtype) {
    case F32: return run<DK, DV, C, BV, TIn, TOp, float>(a, st);
    case F16: return run<DK, DV, C, BV, TIn, TOp, f16>(a, st);
    case BF16: return run<DK, DV, C, BV, TIn, TOp, bf16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int dk, int dv, int chunk, int in_dtype, int pool_dtype) {
  if (pool_dtype != F32 && pool_dtype != F16 && pool_dtype != BF16) return false;
  if (dk == 128 && dv == 128 && chunk == 64) return in_dtype == BF16 || in_dtype == F16;
  if (dk == 16 && dv == 16 && chunk == 16) return in_dtype == F32;
  return false;
}

size_t prefill_workspace_bytes(int n_seqs, int64_t total_tokens, int H, int dk, int dv, int chunk,
                               int in_dtype) {
  (void)dv;
  (void)in_dtype;
  int64_t rec = 0;
  if (dk == 128 && chunk == 64) rec = Rec<128, 64, bf16>::kBytes;
  else if (dk == 16 && chunk == 16) rec = Rec<16, 16, float>::kBytes;
  return (size_t)(map_bytes(n_seqs) + chunk_upper_bound(total_tokens, n_seqs, chunk) * H * rec);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.dk == 128 && a.dv == 128 && a.chunk == 64) {
    if (a.in_dtype == BF16) return by_pool<128, 128, 64, 16, bf16, bf16>(a, st);
    if (a.in_dtype == F16) return by_pool<128, 128, 64, 16, f16, f16>(a, st);
  }
  if (a.dk == 16 && a.dv == 16 && a.chunk == 16 && a.in_dtype == F32)
    return by_pool<16, 16, 16, 16, float, float>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace kda
