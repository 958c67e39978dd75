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
//     e^Gamma_n -- and writes it as one record to the workspace.  The gate
//     exponentials come from one exp per element plus in-chunk cumulative
//     products; M and P run on MFMA; T is a blocked inverse (16x16 diagonal
//     blocks by forward substitution, off-diagonal blocks on fp32 MFMA).
//  3. kda_chunk_scan: one workgroup per (sequence, head, BV-column tile of S).
//     The columns of S evolve independently, so tiles never exchange data.  The
//     fp32 state tile lives in MFMA accumulator registers for the whole
//     sequence; per chunk it does the five state-dependent products above.
//     Workgroups of one head land on one XCD so that they share the head's
//     records in that XCD's L2.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kThreads = 256;
constexpr int kXcd = 8;  // MI355X: workgroups are dealt round-robin to 8 XCDs

// Workspace record for one (chunk, head).
template <int DK, int C, typename TOp>
struct Rec {
  static constexpr int S = (int)sizeof(TOp);
  static constexpr int kKt = 0;                      // [C][DK]  k positions permuted
  static constexpr int kQt = kKt + C * DK * S;       // [C][DK]
  static constexpr int kKbT = kQt + C * DK * S;      // [DK][C]  token positions permuted
  static constexpr int kT = kKbT + DK * C * S;       // [C][C]   s positions permuted
  static constexpr int kP = kT + C * C * S;          // [C][C]
  static constexpr int kBeta = kP + C * C * S;       // [C]  fp32
  static constexpr int kDec = kBeta + C * 4;         // [DK] fp32, e^Gamma_n
  static constexpr int kEnd = kDec + DK * 4;
  static constexpr int kBytes = (kEnd + 255) / 256 * 256;
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

template <int DK, int C, typename TIn, typename TOp>
struct PrepSmem {
  static constexpr int PADK = 16 / (int)sizeof(TOp);
  static constexpr int LDK = DK + PADK;  // row length (elements) of [C][DK] arrays
  static constexpr int LDT = C + PADK;   // row length of [*][C] TOp arrays
  static constexpr int LDF = C + 4;      // row length of fp32 [C][C] arrays
  static constexpr int NCQ = DK / 4;
  static constexpr int NTG0 = kThreads / NCQ;
  static constexpr int NTG = NTG0 < C ? NTG0 : C;
  static constexpr int TPG = C / NTG;
  TOp kt[C * LDK];
  TOp kh[C * LDK];
  TOp qt[C * LDK];
  TOp kbt[DK * LDT];
  TOp p[C * LDT];
  float n[C * LDF];    // Diag(beta) strict_tril(M)
  float tr[C * LDF];   // T row-major
  float tt[C * LDF];   // T transposed
  float beta[C];
  float gp[NTG * DK];  // per-token-group decay products
};

template <int DK, int C, typename TIn, typename TOp>
__global__ __launch_bounds__(kThreads) void kda_chunk_prep(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ g,
    const TIn* __restrict__ bl, const int32_t* __restrict__ cu, int n_seqs, int64_t total,
    int H, const int32_t* __restrict__ off, uint8_t* __restrict__ recs) {
  typedef PrepSmem<DK, C, TIn, TOp> Sm;
  typedef Rec<DK, C, TOp> R;
  constexpr int KBK = (sizeof(TOp) == 4) ? (DK >= 32 ? 32 : 16) : 32;
  constexpr int KBT = (sizeof(TOp) == 4) ? (C >= 32 ? 32 : 16) : 32;
  constexpr int NT = C / 16;
  static_assert(DK % KBK == 0 && C % KBT == 0, "tile sizes");
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g16 = lane >> 4, l16 = lane & 15;
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

  // ---- elementwise: decay products, Kt, Kh, Qt, Kb^T
  const int cq = tid % Sm::NCQ, tg = tid / Sm::NCQ;
  const bool active = tg < Sm::NTG;
  floatx4 kv[Sm::TPG], qv[Sm::TPG], fw[Sm::TPG], bw[Sm::TPG];
  floatx4 gprod = {1.f, 1.f, 1.f, 1.f};
  if (active) {
#pragma unroll
    for (int jj = 0; jj < Sm::TPG; ++jj) {
      const int t = tg * Sm::TPG + jj;
      floatx4 alpha = {1.f, 1.f, 1.f, 1.f};
      kv[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
      qv[jj] = kv[jj];
      if (t < n) {
        const int64_t base = (int64_t)(t0 + t) * rowstride + (int64_t)h * DK + 4 * cq;
        kv[jj] = load4(k + base);
        qv[jj] = load4(q + base);
        const floatx4 gv = load4(g + base);
#pragma unroll
        for (int e = 0; e < 4; ++e) alpha[e] = __expf(gv[e]);
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
    float be = 0.f;
    if (tid < n) be = sigmoidf_(to_f32(bl[(int64_t)(t0 + tid) * H + h]));
    sm.beta[tid] = be;
  }
  // P is written tile by tile below; tiles above the diagonal stay zero.
  for (int u = tid; u < (int)(sizeof(sm.p) / 16); u += kThreads)
    reinterpret_cast<uint4*>(sm.p)[u] = uint4{0u, 0u, 0u, 0u};
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
      store4(&sm.kt[t * Sm::LDK + kp], kv[jj] * epos);
      store4(&sm.kh[t * Sm::LDK + kp], kv[jj] * eneg);
      store4(&sm.qt[t * Sm::LDK + kp], qv[jj] * epos);
      const floatx4 kb = kv[jj] * erem;
      const int tp = pos_of<KBT>(t);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.kbt[(4 * cq + e) * Sm::LDT + tp] = from_f32<TOp>(kb[e]);
    }
    if (tg == 0) {
      uint8_t* rec = recs + ((int64_t)j * H + h) * R::kBytes;
      *reinterpret_cast<floatx4*>(rec + R::kDec + 16 * cq) = total_dec;
    }
  }
  __syncthreads();

  // ---- M and P tiles (lower triangle only), MFMA
  typedef Frag<TOp, KBK> FK;
  constexpr int NTRI = NT * (NT + 1) / 2;
  for (int ti = wave; ti < 2 * NTRI; ti += 4) {
    const bool isP = ti >= NTRI;
    int idx = isP ? ti - NTRI : ti, m = 0;
    while (idx > m) { idx -= m + 1; ++m; }
    const int nn = idx;
    const TOp* arow = (isP ? sm.qt : sm.kt) + (16 * m + l16) * Sm::LDK;
    const TOp* brow = sm.kh + (16 * nn + l16) * Sm::LDK;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / KBK; ++kb) acc = mma(acc, FK::load(arow, kb, g16), FK::load(brow, kb, g16));
    const int s = 16 * nn + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * g16 + i;
      if (isP) sm.p[r * Sm::LDT + pos_of<KBT>(s)] = from_f32<TOp>(s <= r ? acc[i] : 0.f);
      else sm.n[r * Sm::LDF + s] = s < r ? sm.beta[r] * acc[i] : 0.f;
    }
  }
  __syncthreads();

  // ---- T = (I + N)^-1: diagonal 16x16 blocks by forward substitution
  if (wave == 0) {
    const int bi = lane >> 4, s = l16;
    if (bi < NT) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (r == s) ? 1.f : 0.f;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        const float* nrow = sm.n + (16 * bi + r) * Sm::LDF + 16 * bi;
        float acc = 0.f;
#pragma unroll
        for (int jj = 0; jj < r; ++jj) acc += nrow[jj] * x[jj];
        if (r > s) x[r] = -acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.tr[(16 * bi + r) * Sm::LDF + 16 * bi + s] = x[r];
        sm.tt[(16 * bi + s) * Sm::LDF + 16 * bi + r] = x[r];
      }
    }
  }
  // ---- off-diagonal blocks, one block row at a time:
  //      T_ij = -T_ii * sum_{m=j}^{i-1} N_im T_mj   (fp32 MFMA, K-blocks of 16)
  for (int bi = 1; bi < NT; ++bi) {
    __syncthreads();
    const int bj = wave;
    if (bj < bi) {
      floatx4 racc = {0.f, 0.f, 0.f, 0.f};
      for (int bm = bj; bm < bi; ++bm) {
        const float* na = sm.n + (16 * bi + l16) * Sm::LDF + 16 * bm + 4 * g16;
        const float* tb = sm.tt + (16 * bj + l16) * Sm::LDF + 16 * bm + 4 * g16;
        const floatx4 av = *reinterpret_cast<const floatx4*>(na);
        const floatx4 bv = *reinterpret_cast<const floatx4*>(tb);
        f32frag<4> fa, fb;
#pragma unroll
        for (int e = 0; e < 4; ++e) { fa.v[e] = av[e]; fb.v[e] = bv[e]; }
        racc = mma(racc, fa, fb);
      }
      const floatx4 tav = *reinterpret_cast<const floatx4*>(sm.tr + (16 * bi + l16) * Sm::LDF + 16 * bi + 4 * g16);
      f32frag<4> fa, fb;
#pragma unroll
      for (int e = 0; e < 4; ++e) { fa.v[e] = tav[e]; fb.v[e] = racc[e]; }
      floatx4 tij = mma(floatx4{0.f, 0.f, 0.f, 0.f}, fa, fb);
      tij = -tij;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.tr[(16 * bi + 4 * g16 + i) * Sm::LDF + 16 * bj + l16] = tij[i];
      *reinterpret_cast<floatx4*>(sm.tt + (16 * bj + l16) * Sm::LDF + 16 * bi + 4 * g16) = tij;
    }
  }
  __syncthreads();

  // ---- write the record
  uint8_t* rec = recs + ((int64_t)j * H + h) * R::kBytes;
  {
    // T: [r][pos(s)] with explicit zeros above the diagonal.
    TOp* gt = reinterpret_cast<TOp*>(rec + R::kT);
    for (int u = tid; u < C * C / 4; u += kThreads) {
      const int r = (4 * u) / C, p = (4 * u) % C;
      const int s0 = (p / KBT) * KBT + idx_in_block<KBT>(p % KBT);
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (s0 + e <= r) ? sm.tr[r * Sm::LDF + s0 + e] : 0.f;
      store4(gt + r * C + p, v);
    }
    if (tid < C) reinterpret_cast<float*>(rec + R::kBeta)[tid] = sm.beta[tid];
  }
  // Padded LDS images -> unpadded record, 16 bytes per lane.
  auto copy_out = [&](const TOp* src, int rows, int cols, int ld, int dst_off) {
    constexpr int E = 16 / (int)sizeof(TOp);
    const int upr = cols / E;
    for (int u = tid; u < rows * upr; u += kThreads) {
      const int r = u / upr, cc = (u % upr) * E;
      *reinterpret_cast<uint4*>(rec + dst_off + (r * cols + cc) * (int)sizeof(TOp)) =
          *reinterpret_cast<const uint4*>(src + r * ld + cc);
    }
  };
  copy_out(sm.kt, C, DK, Sm::LDK, R::kKt);
  copy_out(sm.qt, C, DK, Sm::LDK, R::kQt);
  copy_out(sm.kbt, DK, C, Sm::LDT, R::kKbT);
  copy_out(sm.p, C, C, Sm::LDT, R::kP);
}

// ---------------------------------------------------------------- 3. scan

template <int DK, int DV, int C, int BV, typename TOp>
struct ScanSmem {
  static constexpr int PADK = 16 / (int)sizeof(TOp);
  static constexpr int LDK = DK + PADK;
  static constexpr int LDT = C + PADK;
  TOp kt[C * LDK];
  TOp qt[C * LDK];
  TOp kbt[DK * LDT];
  TOp t[C * LDT];
  TOp p[C * LDT];
  float beta[C];
  float dec[DK];
  TOp s[BV * LDK];  // state tile as B operand, [v][pos(k)]
  TOp y[BV * LDT];  // Diag(beta)(V - Kt S), [v][pos(t)]
  TOp u[BV * LDT];  // U, [v][pos(t)]
};

template <int DK, int DV, int C, int BV, typename TIn, typename TOp, typename TPool>
__global__ __launch_bounds__(kThreads) void kda_chunk_scan(
    const TIn* __restrict__ v, TIn* __restrict__ o, const int32_t* __restrict__ cu, int n_seqs,
    int64_t total, int H, const int32_t* __restrict__ off, const uint8_t* __restrict__ recs,
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ init_slot,
    const int32_t* __restrict__ final_slot, const int32_t* __restrict__ track_ptr,
    const int32_t* __restrict__ track_chunk, const int32_t* __restrict__ track_slot, int n_track,
    float* __restrict__ track_f32, int32_t* __restrict__ dev_err) {
  typedef ScanSmem<DK, DV, C, BV, TOp> Sm;
  typedef Rec<DK, C, TOp> R;
  constexpr int KBK = (sizeof(TOp) == 4) ? (DK >= 32 ? 32 : 16) : 32;
  constexpr int KBT = (sizeof(TOp) == 4) ? (C >= 32 ? 32 : 16) : 32;
  constexpr int NT = C / 16, NK = DK / 16, NVS = BV / 16, NVT = DV / BV;
  constexpr int NKW = (NK + 3) / 4;  // k tiles of the state owned per wave
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  typedef Frag<TOp, KBK> FK;
  typedef Frag<TOp, KBT> FT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g16 = lane >> 4, l16 = lane & 15;
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
  for (int c = 0; c < nch; ++c) {
    snapshot(c);
    const int n = min(C, len - c * C);
    const int tc0 = t_beg + c * C;
    // ---- operands of chunk c -> LDS
    const uint8_t* rec = recs + ((int64_t)(off[seq] + c) * H + h) * R::kBytes;
    auto copy_in = [&](TOp* dst, int rows, int cols, int ld, int src_off) {
      constexpr int E = 16 / (int)sizeof(TOp);
      const int upr = cols / E;
      for (int u = tid; u < rows * upr; u += kThreads) {
        const int r = u / upr, cc = (u % upr) * E;
        *reinterpret_cast<uint4*>(dst + r * ld + cc) =
            *reinterpret_cast<const uint4*>(rec + src_off + (r * cols + cc) * (int)sizeof(TOp));
      }
    };
    copy_in(sm.kt, C, DK, Sm::LDK, R::kKt);
    copy_in(sm.qt, C, DK, Sm::LDK, R::kQt);
    copy_in(sm.kbt, DK, C, Sm::LDT, R::kKbT);
    copy_in(sm.t, C, C, Sm::LDT, R::kT);
    copy_in(sm.p, C, C, Sm::LDT, R::kP);
    if (tid < C) sm.beta[tid] = reinterpret_cast<const float*>(rec + R::kBeta)[tid];
    if (tid < DK) sm.dec[tid] = reinterpret_cast<const float*>(rec + R::kDec)[tid];
    // ---- state tile -> LDS as the B operand of Kt S and Qt S
#pragma unroll
    for (int a = 0; a < NKW; ++a) {
      const int kt = wave + 4 * a;
      if (kt >= NK) continue;
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs)
        store4(&sm.s[(16 * vs + l16) * Sm::LDK + pos_of<KBK>(16 * kt + 4 * g16)], S[a][vs]);
    }
    // ---- V tile of this wave's token rows, in accumulator layout
    const int m = wave;
    floatx4 V[NVS];
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) {
      V[vs] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (m < NT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * m + 4 * g16 + i;
          if (t < n) V[vs][i] = to_f32(v[(int64_t)(tc0 + t) * vrow + (int64_t)h * DV + v0 + 16 * vs + l16]);
        }
      }
    }
    __syncthreads();

    // ---- X = Kt S, O = Qt S, Y = Diag(beta)(V - X)
    floatx4 O[NVS];
    if (m < NT) {
      const TOp* krow = sm.kt + (16 * m + l16) * Sm::LDK;
      const TOp* qrow = sm.qt + (16 * m + l16) * Sm::LDK;
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        floatx4 X = {0.f, 0.f, 0.f, 0.f};
        O[vs] = X;
        const TOp* srow = sm.s + (16 * vs + l16) * Sm::LDK;
#pragma unroll
        for (int kb = 0; kb < DK / KBK; ++kb) {
          const auto sf = FK::load(srow, kb, g16);
          X = mma(X, FK::load(krow, kb, g16), sf);
          O[vs] = mma(O[vs], FK::load(qrow, kb, g16), sf);
        }
        floatx4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = sm.beta[16 * m + 4 * g16 + i] * (V[vs][i] - X[i]);
        store4(&sm.y[(16 * vs + l16) * Sm::LDT + pos_of<KBT>(16 * m + 4 * g16)], Y);
      }
    }
    __syncthreads();

    // ---- U = T Y  (T lower triangular: only K-blocks up to the diagonal)
    if (m < NT) {
      const TOp* trow = sm.t + (16 * m + l16) * Sm::LDT;
      const int nkb = (16 * m + 15) / KBT + 1;
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        floatx4 U = {0.f, 0.f, 0.f, 0.f};
        const TOp* yrow = sm.y + (16 * vs + l16) * Sm::LDT;
        for (int kb = 0; kb < nkb; ++kb) U = mma(U, FT::load(trow, kb, g16), FT::load(yrow, kb, g16));
        store4(&sm.u[(16 * vs + l16) * Sm::LDT + pos_of<KBT>(16 * m + 4 * g16)], U);
      }
    }
    __syncthreads();

    // ---- O += P U -> o;  S = Diag(e^Gamma_n) S + Kb^T U
    if (m < NT) {
      const TOp* prow = sm.p + (16 * m + l16) * Sm::LDT;
      const int nkb = (16 * m + 15) / KBT + 1;
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        const TOp* urow = sm.u + (16 * vs + l16) * Sm::LDT;
        for (int kb = 0; kb < nkb; ++kb) O[vs] = mma(O[vs], FT::load(prow, kb, g16), FT::load(urow, kb, g16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * m + 4 * g16 + i;
          if (t < n) o[(int64_t)(tc0 + t) * vrow + (int64_t)h * DV + v0 + 16 * vs + l16] = from_f32<TIn>(O[vs][i]);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < NKW; ++a) {
      const int kt = wave + 4 * a;
      if (kt >= NK) continue;
      const TOp* kbrow = sm.kbt + (16 * kt + l16) * Sm::LDT;
      floatx4 d4;
#pragma unroll
      for (int i = 0; i < 4; ++i) d4[i] = sm.dec[16 * kt + 4 * g16 + i];
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        const TOp* urow = sm.u + (16 * vs + l16) * Sm::LDT;
#pragma unroll
        for (int kb = 0; kb < C / KBT; ++kb) acc = mma(acc, FT::load(kbrow, kb, g16), FT::load(urow, kb, g16));
        S[a][vs] = d4 * S[a][vs] + acc;
      }
    }
    __syncthreads();
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
  typedef PrepSmem<DK, C, TIn, TOp> SmP;
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
                       a.n_seqs, a.total_tokens, a.H, off, recs);
  }
  auto ks = kda_chunk_scan<DK, DV, C, BV, TIn, TOp, TPool>;
  const int sms = (int)sizeof(SmS);
  hipError_t e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, sms);
  if (e != hipSuccess) return e;
  const int64_t pairs = (int64_t)a.n_seqs * a.H;
  const int64_t blocks = (pairs + kXcd - 1) / kXcd * kXcd * (DV / BV);
  hipLaunchKernelGGL(ks, dim3((unsigned)blocks), dim3(kThreads), sms, st,
                     static_cast<const TIn*>(a.v), static_cast<TIn*>(a.o), a.cu_seqlens, a.n_seqs,
                     a.total_tokens, a.H, off, recs, static_cast<TPool*>(a.pool.base),
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
  int64_t rec = 0;
  if (dk == 128 && chunk == 64) rec = (in_dtype == F32) ? Rec<128, 64, float>::kBytes : Rec<128, 64, bf16>::kBytes;
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
