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
// Three launches on the caller's stream (two for a single sequence):
//  1. kda_chunk_map: one block turns cu_seqlens into per-sequence chunk offsets
//     (and validates them) and the scan's order of the sequences (longest
//     first), without any host synchronisation.  A single sequence's chunks
//     start at slot 0 and need no map.
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

#include "prefill_common.hpp"

namespace kda {

// ---------------------------------------------------------------- 1. chunk map

__global__ __launch_bounds__(kThreads) void kda_chunk_map(const int32_t* __restrict__ cu, int n_seqs,
                                                          int64_t total, int C, int64_t cap,
                                                          int32_t* __restrict__ off,
                                                          int32_t* __restrict__ dev_err) {
  __shared__ int32_t s_scan[kThreads];
  __shared__ int32_t s_nch[kOrderMax];
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
      if (n_seqs <= kOrderMax) s_nch[i] = nch;
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
  // The scan's order: most chunks first (ties by index), so the longest
  // serial chains start first and the workgroups that start last are
  // short ones (list scheduling, longest first); batch order past
  // kOrderMax sequences, where ranking them here would cost more.
  int32_t* const ord = off + n_seqs + 1;
  for (int i = threadIdx.x; i < n_seqs; i += kThreads) {
    int place = i;
    if (n_seqs <= kOrderMax) {
      const int ni = s_nch[i];
      place = 0;
      for (int j = 0; j < n_seqs; ++j) place += (s_nch[j] > ni || (s_nch[j] == ni && j < i)) ? 1 : 0;
    }
    ord[place] = i;
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
    int H, int64_t cap, const int32_t* __restrict__ off, uint8_t* __restrict__ recs, int l2norm,
    int32_t* __restrict__ dev_err) {
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
  if (off != nullptr && j >= off[n_seqs]) return;
  // sequence owning chunk slot j: largest seq with off[seq] <= j
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  const int seq = lo;
  int t_beg, len, nch;
  if (!seq_ok(cu, off, seq, total, C, t_beg, len, nch)) return;
  const int c = j - chunk_base(off, seq);
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
    // optional L2 normalisation of the k and q rows: the NCQ consecutive
    // lanes cq = 0..NCQ-1 of a token group hold one row, 4 channels each;
    // scaled by 1 / sqrt(sum x^2 + 1e-6) in fp32, rounded once to TIn
    if (l2norm) {
#pragma unroll
      for (int jj = 0; jj < Sm::TPG; ++jj) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sk += kv[jj][e] * kv[jj][e];
          sq += qv[jj][e] * qv[jj][e];
        }
#pragma unroll
        for (int m = 1; m < Sm::NCQ; m <<= 1) {
          sk += __shfl_xor(sk, m);
          sq += __shfl_xor(sq, m);
        }
        const float ks = rsqrtf(sk + 1e-6f), qs = rsqrtf(sq + 1e-6f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[jj][e] = to_f32(from_f32<TIn>(kv[jj][e] * ks));
          qv[jj][e] = to_f32(from_f32<TIn>(qv[jj][e] * qs));
        }
      }
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
    const int kp = 4 * cq;
    // e^-Gamma_t grows with the chunk's decay: an element of K e^-Gamma that
    // is not finite in fp32 (cumulative log decay below about -87 within a
    // chunk) sets the gate-range error bit
    bool range_ok = true;
#pragma unroll
    for (int jj = 0; jj < Sm::TPG; ++jj) {
      const int t = tg * Sm::TPG + jj;
      const floatx4 epos = pre * fw[jj];                 // e^Gamma_t
      const floatx4 erem = bw[jj] * post;                // e^(Gamma_n - Gamma_t)
      const floatx4 eneg = erem * inv_total;             // e^-Gamma_t
      const floatx4 khv = kv[jj] * eneg;
#pragma unroll
      for (int e = 0; e < 4; ++e) range_ok = range_ok && __builtin_fabsf(khv[e]) <= 3.40282347e38f;
      store4(&sm.u.a.kt[t * Sm::LDK + kp], kv[jj] * epos);
      store4(&sm.u.a.kh[t * Sm::LDK + kp], khv);
      store4(&sm.u.a.qt[t * Sm::LDK + kp], qv[jj] * epos);
      const floatx4 kb = kv[jj] * erem;
      const int tp = t;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.a.kbt[(4 * cq + e) * Sm::LDT + tp] = from_f32<TOp>(kb[e]);
    }
    if (tg == 0) *reinterpret_cast<floatx4*>(rec + R::kDec + 16 * cq) = total_dec;
    if (!range_ok) set_err(dev_err, 1u << 5);
  }
  __syncthreads();

  // ---- phase 2: M and P tiles (lower triangle only) into registers; the
  //      Kt, Qt and Kb^T images go out as fragment blocks.
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
        tacc[q2] = mma(tacc[q2], frag_load(arow, kb, g16), frag_load(brow, kb, g16));
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
        if (isP) sm.u.b.p[r * Sm::LDT + s] = from_f32<TOp>(tacc[q2][i]);
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
        const int s = kb * KBT + (KBT / 4) * gg + e;
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

// w*KB/16 ...), so it loads only its own quarter of each record.
template <int DK, int C, typename TOp>
struct ScanGeom {
  static_assert(sizeof(TOp) == 4, "the general chunk form runs on fp32 operands");
  static constexpr int KB = kKB32;
  static constexpr int NT = C / 16, NK = DK / 16, NFK = DK / KB, NFT = C / KB;
  static constexpr int KPW = KB / 16;  // key tiles per S K-block
  __host__ __device__ static constexpr int nkb(int mt) { return scan_nkb<KB>(mt); }
  __host__ __device__ static constexpr int tblk(int mt) { return scan_tblk<KB>(mt); }
  static constexpr int NTB = scan_tblk<KB>(NT);
  static_assert(NT <= 4 && NFK <= 4, "one token tile and one S K-block per wave");
};

template <int DK, int C, typename TIn, typename TOp>
struct ScanRegs {
  typedef ScanGeom<DK, C, TOp> G;
  uint4 kt[G::NFK], qt[G::NFK], p[G::NFT], kb[G::KPW][G::NFT];
  uint4 tb[(G::NTB + 3) / 4];    // the T blocks this wave copies into LDS
  uint4 vv;                      // this wave's 1 KiB share of the chunk's V tile
  uint4 bd;                      // wave 0: beta and e^Gamma_n (16 bytes per lane)
};

template <int DK, int C, typename TIn, typename TOp>
struct ScanLds {
  typedef ScanGeom<DK, C, TOp> G;
  uint4 s[G::NFK][64];           // S as B fragments
  uint4 y[G::NFT][64];           // Y = Diag(beta)(V - Kt S) as B fragments
  uint4 t[G::NTB][64];           // lower T fragment blocks of the current chunk
  float bd[2][C + DK];           // beta, e^Gamma_n; by chunk parity
  TIn vb[C][16];                 // the chunk's V tile, row-major
  TIn ob[C][16];                 // the chunk's output tile, row-major
};

// Four waves per (sequence, head, 16-column tile of S).  Per chunk:
//   S fragments -> LDS, barrier;  X = Kt S and O = Qt S for the wave's token
//   tile; Y and the chunk's T blocks -> LDS, barrier;  U = T Y for all token
//   tiles (every wave, so U never has to be exchanged);  O += P U -> LDS;
//   S = Diag(e^Gamma_n) S + Kb^T U for the wave's key tiles.
// Accumulator tiles (lane l: column l%16, rows 4(l/16)+i) are B fragments of
// the next product as they stand (reg_frag), so S, Y and U go to LDS in
// fragment order and come back with one 16-byte read per lane.  Each wave loads its share of
// every record (its token tile's Kt, Qt, P rows, its key tiles' Kb^T rows,
// a quarter of T) two chunks ahead, into registers.  Every global access
// moves 16 bytes per lane: the address unit costs about the same per
// instruction whatever the width, so the V tile, beta / e^Gamma_n and the
// output tile go through LDS in 1 KiB pieces instead of per-lane scalars.
template <int DK, int DV, int C, typename TIn, typename TOp, typename TPool>
__global__ __launch_bounds__(256) void kda_chunk_scan(
    const TIn* __restrict__ v, TIn* __restrict__ o, const int32_t* __restrict__ cu, int n_seqs,
    int64_t total, int H, int64_t cap, const int32_t* __restrict__ off, const uint8_t* __restrict__ recs,
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ init_slot,
    const int32_t* __restrict__ final_slot, const int32_t* __restrict__ track_ptr,
    const int32_t* __restrict__ track_chunk, const int32_t* __restrict__ track_slot, int n_track,
    float* __restrict__ track_f32, int32_t* __restrict__ dev_err) {
  typedef Rec<DK, C, TOp> R;
  typedef ScanGeom<DK, C, TOp> G;
  typedef ScanRegs<DK, C, TIn, TOp> Regs;
  constexpr int NFK = G::NFK, NFT = G::NFT, KPW = G::KPW, NTB = G::NTB;
  constexpr int BV = 16, NVT = DV / BV;
  // V / o tile: 16-byte pieces, LPR per row, RPI rows per 1 KiB instruction
  constexpr int LPR = BV * (int)sizeof(TIn) / 16, RPI = 64 / LPR, NVQ = C / RPI;
  constexpr int NBD = (C + DK) * 4 / 16;  // lanes holding beta / e^Gamma_n
  static_assert(NVQ >= 1 && NVQ <= 4 && C % RPI == 0 && NBD <= 64, "scan tile shapes");
  static_assert(R::kDec == R::kBeta + C * 4, "beta and e^Gamma_n are contiguous");
  typedef F32Frag FT;
  __shared__ ScanLds<DK, C, TIn, TOp> sm;

  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const bool has_tile = w < G::NT, has_keys = w < NFK, has_vq = w < NVQ;
  const int mt = has_tile ? w : 0, kf = has_keys ? w : 0;
  // XCD-aware decode: all NVT tiles of one (seq, head) pair share blockIdx % 8.
  const int xcd = blockIdx.x % kXcd, slot_ = blockIdx.x / kXcd;
  const int vt = slot_ % NVT;
  const int pair = (slot_ / NVT) * kXcd + xcd;
  if (pair >= n_seqs * H) return;
  const int seq = seq_at(off, n_seqs, pair / H), h = pair % H;
  int t_beg, len, nch;
  if (!seq_ok(cu, off, seq, total, C, t_beg, len, nch)) {
    // with no chunk map (one sequence) nothing else has checked cu_seqlens
    if (off == nullptr && blockIdx.x == 0 && tid == 0) set_err(dev_err, 1u << 3);
    return;
  }
  const int v0 = vt * BV;
  const bool lead = (vt == 0 && h == 0);

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
    for (int e = e0 + tid; e < e1; e += 256) {
      const int ce = track_chunk[e], se = track_slot[e];
      if (ce < 0 || ce > len / C) set_err(dev_err, 1u << 1);
      if (se < -1 || (int64_t)se >= n_slots) set_err(dev_err, 1u);
    }
  }

  // ---- initial state, the wave's key tiles: S[k][v] = pool[init][h][v][k]
  floatx4 S[KPW];
  const int64_t st_off = (int64_t)(v0 + l16) * DK + 16 * KPW * kf + 4 * g16;  // lane's first element
  {
    const int is = init_slot[seq];
    const bool ok = is >= 0 && (int64_t)is < n_slots && has_keys;
    if (is != -1 && !(is >= 0 && (int64_t)is < n_slots) && lead && tid == 0) set_err(dev_err, 1u);
    const TPool* src = pool + ((int64_t)(ok ? is : 0) * H + h) * DV * DK + st_off;
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      S[j] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (ok) S[j] = load4(src + 16 * j);
    }
    // Complete these loads here, so that the waits inside the chunk loop
    // stay partial (the loop head cannot tell the first iteration apart).
#pragma unroll
    for (int j = 0; j < KPW; ++j) asm volatile("" : "+v"(S[j]));
  }

  // Snapshots: `next_snap` is the smallest requested chunk index >= the
  // current one, so the per-chunk test is one scalar compare and the track
  // list is read only when a snapshot is due.
  auto next_track = [&](int c) {
    int best = INT32_MAX;
    for (int e = e0; e < e1; ++e) {
      const int ce = track_chunk[e];
      if (ce >= c && ce < best) best = ce;
    }
    return best;
  };
  int next_snap = next_track(0);
  auto snapshot = [&](int c) {
    if (c != next_snap) return;
    for (int e = e0; e < e1; ++e) {
      if (track_chunk[e] != c) continue;
      const int se = track_slot[e];
      const bool to_pool = se >= 0 && (int64_t)se < n_slots;
      if (has_keys) {
#pragma unroll
        for (int j = 0; j < KPW; ++j) {
          if (track_f32) store4(track_f32 + ((int64_t)e * H + h) * DV * DK + st_off + 16 * j, S[j]);
          if (to_pool) store4(pool + ((int64_t)se * H + h) * DV * DK + st_off + 16 * j, S[j]);
        }
      }
    }
    next_snap = next_track(c + 1);
  };

  const int64_t vrow = (int64_t)H * DV;
  const int lane_off = lane * 16;
  // V / o piece of this lane in wave w's 1 KiB instruction: row, 16-byte part
  const int vq_row = RPI * w + lane / LPR, vq_part = lane % LPR;
  const int vq_off = (int)((int64_t)vq_row * vrow * (int)sizeof(TIn)) + 16 * vq_part;
  const uint8_t* rec_seq = recs + ((int64_t)h * cap + chunk_base(off, seq)) * R::kBytes;

  // Per-chunk buffer resources: the record, and the chunk's rows of V / o
  // (reads past the last row return 0 and stores there are dropped; those
  // rows carry beta = 0 and zero keys in the record as well).
  auto rec_rsrc = [&](int c) { return buffer_rsrc(rec_seq + (int64_t)c * R::kBytes, R::kBytes); };
  auto rows_rsrc = [&](const TIn* base, int c) {
    const int n = min(C, len - c * C);
    const TIn* p = base + (int64_t)(t_beg + c * C) * vrow + (int64_t)h * DV + v0;
    return buffer_rsrc(p, (uint32_t)(((int64_t)(n - 1) * vrow + BV) * (int)sizeof(TIn)));
  };
  // Record offsets of the T blocks this wave copies: lower block j = w + 4 jj
  // (clamped to the last one; only j < NTB is written to LDS).
  int t_src[(NTB + 3) / 4];
#pragma unroll
  for (int jj = 0; jj < (NTB + 3) / 4; ++jj) {
    const int j = min(w + 4 * jj, NTB - 1);
    int m = 0;
    while (m + 1 < G::NT && G::tblk(m + 1) <= j) ++m;
    t_src[jj] = (m * NFT + (j - G::tblk(m))) * kFB;
  }
  // Operand groups, each issued once the current chunk is done with its registers.
  auto ld_front = [&](Regs& r, int c) {  // Kt, Qt rows of the token tile; T, V, beta shares
    const auto rs = rec_rsrc(c);
#pragma unroll
    for (int f = 0; f < NFK; ++f) {
      r.kt[f] = ld16(rs, lane_off, R::kKt + (mt * NFK + f) * kFB);
      r.qt[f] = ld16(rs, lane_off, R::kQt + (mt * NFK + f) * kFB);
    }
#pragma unroll
    for (int jj = 0; jj < (NTB + 3) / 4; ++jj) r.tb[jj] = ld16(rs, lane_off, R::kT + t_src[jj]);
    if (has_vq) r.vv = ld16(rows_rsrc(v, c), vq_off, 0);
    if (w == 0) r.bd = ld16(rs, lane_off, R::kBeta);  // lanes past the record end read 0
  };
  auto ld_p = [&](Regs& r, int c) {
    const auto rs = rec_rsrc(c);
#pragma unroll
    for (int f = 0; f < NFT; ++f)
      if (f < G::nkb(mt)) r.p[f] = ld16(rs, lane_off, R::kP + (mt * NFT + f) * kFB);
  };
  auto ld_back = [&](Regs& r, int c) {  // Kb^T rows of the wave's key tiles
    const auto rs = rec_rsrc(c);
#pragma unroll
    for (int j = 0; j < KPW; ++j) {
      const int kt = KPW * kf + j;
#pragma unroll
      for (int f = 0; f < NFT; ++f) r.kb[j][f] = ld16(rs, lane_off, R::kKbT + (kt * NFT + f) * kFB);
    }
  };
  // Output tile of chunk c (in LDS since the previous barrier) -> o.
  auto store_o = [&](int c) {
    if (has_vq)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                             *reinterpret_cast<const uint4*>(&sm.ob[vq_row][vq_part * (16 / sizeof(TIn))])),
          rows_rsrc(o, c), vq_off, 0, 0);
  };

  // ---- one chunk.  `r` holds chunk c's operands; chunk c + 2's are loaded
  //      into it as its groups fall free (unconditional, clamped: the
  //      waits stay partial).  bp = c % 2.
  auto step = [&](Regs& r, int c, int bp) {
    const int c2 = min(c + 2, nch - 1);
    snapshot(c);
    if (has_keys) sm.s[kf][lane] = __builtin_bit_cast(uint4, reg_frag(S[0]));
    if (has_vq) *reinterpret_cast<uint4*>(&sm.vb[vq_row][vq_part * (16 / sizeof(TIn))]) = r.vv;
    if (w == 0 && lane < NBD) *reinterpret_cast<uint4*>(&sm.bd[bp][4 * lane]) = r.bd;
    __syncthreads();
    if (c > 0) store_o(c - 1);
    // X = Kt S, O = Qt S for the token tile;  Y = Diag(beta)(V - X)
    floatx4 X = {0.f, 0.f, 0.f, 0.f}, O = X;
    if (has_tile) {
#pragma unroll
      for (int f = 0; f < NFK; ++f) {
        const FT sf = __builtin_bit_cast(FT, sm.s[f][lane]);
        X = mma(X, as_frag<FT>(r.kt[f]), sf);
        O = mma(O, as_frag<FT>(r.qt[f]), sf);
      }
      const floatx4 beta = *reinterpret_cast<const floatx4*>(&sm.bd[bp][16 * mt + 4 * g16]);
      floatx4 Y;
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[i] = beta[i] * (to_f32(sm.vb[16 * mt + 4 * g16 + i][l16]) - X[i]);
      sm.y[mt][lane] = __builtin_bit_cast(uint4, reg_frag(Y));   // token tile mt = Y K-block mt
    }
#pragma unroll
    for (int jj = 0; jj < (NTB + 3) / 4; ++jj)
      if (w + 4 * jj < NTB) sm.t[w + 4 * jj][lane] = r.tb[jj];
    __syncthreads();
    ld_front(r, c2);
    // U = T Y for every token tile (T lower triangular: K-blocks up to the diagonal)
    FT yf[NFT];
#pragma unroll
    for (int f = 0; f < NFT; ++f) yf[f] = __builtin_bit_cast(FT, sm.y[f][lane]);
    floatx4 U[G::NT];
#pragma unroll
    for (int m = 0; m < G::NT; ++m) {
      U[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NFT; ++f)
        if (f < G::nkb(m)) U[m] = mma(U[m], __builtin_bit_cast(FT, sm.t[G::tblk(m) + f][lane]), yf[f]);
    }
    FT uf[NFT];
#pragma unroll
    for (int f = 0; f < NFT; ++f) uf[f] = reg_frag(U[f]);
    // O += P U -> output tile in LDS (stored after the next barrier)
    if (has_tile) {
#pragma unroll
      for (int f = 0; f < NFT; ++f)
        if (f < G::nkb(mt)) O = mma(O, as_frag<FT>(r.p[f]), uf[f]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.ob[16 * mt + 4 * g16 + i][l16] = from_f32<TIn>(O[i]);
    }
    ld_p(r, c2);
    // S = Diag(e^Gamma_n) S + Kb^T U for the wave's key tiles
    if (has_keys) {
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NFT; ++f) acc = mma(acc, as_frag<FT>(r.kb[j][f]), uf[f]);
        const floatx4 dec = *reinterpret_cast<const floatx4*>(&sm.bd[bp][C + 16 * (KPW * kf + j) + 4 * g16]);
        S[j] = dec * S[j] + acc;
      }
    }
    ld_back(r, c2);
  };

  Regs rA, rB;
  if (nch > 0) {
    ld_front(rA, 0); ld_p(rA, 0); ld_back(rA, 0);
    const int c1 = min(1, nch - 1);
    ld_front(rB, c1); ld_p(rB, c1); ld_back(rB, c1);
  }
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    step(rA, c, 0);
    step(rB, c + 1, 1);
  }
  if (c < nch) step(rA, c, 0);
  if (nch > 0) {
    __syncthreads();
    store_o(nch - 1);
  }
  if (len % C == 0) snapshot(nch);

  // ---- final state, one cast into the pool dtype
  const int fs = final_slot[seq];
  if (fs >= 0 && (int64_t)fs < n_slots) {
    if (has_keys) {
#pragma unroll
      for (int j = 0; j < KPW; ++j) store4(pool + ((int64_t)fs * H + h) * DV * DK + st_off + 16 * j, S[j]);
    }
  } else if (fs != -1 && lead && tid == 0) {
    set_err(dev_err, 1u);
  }
}

// ---------------------------------------------------------------- host side



namespace {

struct WsView {
  int64_t cap;     // chunk slots per head
  int32_t* off;    // per-sequence chunk offsets (the chunk map)
  uint8_t* recs;   // records, [head][chunk slot]
};

// A single sequence needs no chunk map: the kernels take its chunk slots
// from cu_seqlens alone (and its scan flags a malformed pair), which saves
// a dependent launch.
WsView map_chunks(const PrefillArgs& a, hipStream_t st, int C) {
  WsView w;
  w.cap = chunk_upper_bound(a.total_tokens, a.n_seqs, C);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  w.off = a.n_seqs > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  w.recs = ws + map_bytes(a.n_seqs);
  if (w.off != nullptr)
    hipLaunchKernelGGL(kda_chunk_map, dim3(1), dim3(kThreads), 0, st, a.cu_seqlens, a.n_seqs,
                       a.total_tokens, C, w.cap, w.off, a.dev_err);
  return w;
}

template <int DK, int DV, int C, typename TIn, typename TOp, typename TPool>
hipError_t run(const PrefillArgs& a, hipStream_t st) {
  typedef PrepSmem<DK, C, TOp> SmP;
  const WsView w = map_chunks(a, st, C);
  if (w.cap > 0) {
    auto kp = kda_chunk_prep<DK, C, TIn, TOp>;
    const int smp = (int)sizeof(SmP);
    hipError_t e = hipFuncSetAttribute((const void*)kp, hipFuncAttributeMaxDynamicSharedMemorySize, smp);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kp, dim3((unsigned)(w.cap * a.H)), dim3(kThreads), smp, st,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.g), static_cast<const TIn*>(a.b), a.cu_seqlens,
                       a.n_seqs, a.total_tokens, a.H, w.cap, w.off, w.recs, (a.flags & 1u) ? 1 : 0,
                       a.dev_err);
  }
  auto ks = kda_chunk_scan<DK, DV, C, TIn, TOp, TPool>;
  const int64_t pairs = (int64_t)a.n_seqs * a.H;
  const int64_t blocks = (pairs + kXcd - 1) / kXcd * kXcd * (DV / 16);
  hipLaunchKernelGGL(ks, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const TIn*>(a.v), static_cast<TIn*>(a.o), a.cu_seqlens, a.n_seqs,
                     a.total_tokens, a.H, w.cap, w.off, w.recs, static_cast<TPool*>(a.pool.base),
                     a.pool.n_slots, a.init_slot, a.final_slot, a.track_ptr, a.track_chunk,
                     a.track_slot, a.n_track, a.track_f32, a.dev_err);
  return hipGetLastError();
}

template <int DK, int DV, int C, typename TIn, typename TOp>
hipError_t by_pool(const PrefillArgs& a, hipStream_t st) {
  switch (a.pool.dtype) {
    case F32: return run<DK, DV, C, TIn, TOp, float>(a, st);
    case F16: return run<DK, DV, C, TIn, TOp, f16>(a, st);
    case BF16: return run<DK, DV, C, TIn, TOp, bf16>(a, st);
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
  if (dk == 128 && chunk == 64) rec = rec16_bytes();
  else if (dk == 16 && chunk == 16) rec = Rec<16, 16, float>::kBytes;
  return (size_t)(map_bytes(n_seqs) + chunk_upper_bound(total_tokens, n_seqs, chunk) * H * rec);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.dk == 128 && a.dv == 128 && a.chunk == 64 && (a.in_dtype == BF16 || a.in_dtype == F16)) {
    const WsView w = map_chunks(a, st, 64);
    return launch_prefill16(a, st, w.cap, w.off, w.recs);
  }
  if (a.dk == 16 && a.dv == 16 && a.chunk == 16 && a.in_dtype == F32)
    return by_pool<16, 16, 16, float, float>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace kda