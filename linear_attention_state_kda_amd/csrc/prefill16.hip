// Chunked KDA prefill with 16-bit operands (bf16 or fp16 inputs) on gfx950.
//
// In the chunk form (see prefill.hip for the symbols: Kt, Qt, Kb, Kh, M, P,
// T over a chunk of C tokens with in-chunk cumulative log decay Gamma)
//   U  = T Diag(beta) (V - Kt S),   O = Qt S + P U,   S' = Diag(e^Gamma_n) S + Kb^T U,
// T enters only through the two products that follow it, so it is folded
// into them ahead of the scan:
//   Z  = Kb^T T Diag(beta)   (d_k x C),     Pw = P T Diag(beta)   (C x C, lower),
// and with Y = V - Kt S a chunk is
//   S' = Diag(e^Gamma_n) S + Z Y,           O = Qt S + Pw Y.
// The same arithmetic, regrouped (state-semantics page, sec. 5: the serial
// steps of a sequence are its chunks): the state's serial path per chunk is
// two dependent products (Kt S, then Z Y) instead of four, and a record
// holds Kt, Qt, Z, Pw and e^Gamma_n (54.5 KiB at d_k = 128, C = 64).
//
// Two launches after the chunk map (prefill.hip; a single sequence needs no map):
//  * kda_chunk_prep16: one workgroup per (chunk, head), fully parallel;
//    writes the record as MFMA A-operand fragment blocks.
//  * kda_chunk_scan16: one workgroup per (sequence, head, column tile of S:
//    16, 32 or 64 columns, by how many (sequence, head) pairs there are);
//    four chain waves carry the fp32 state, four output waves compute O,
//    and a ninth wave pulls records into the L2 ahead of them.
#include "prefill_common.hpp"

namespace kda {
namespace {

// Record of one (chunk, head).  Fragment block (1 KiB) of a 16-row tile and
// a 32-wide K-block: lane l = 16 g + r holds row r at K-block positions
// 8g .. 8g+7, which hold the indices 4g .. 4g+3 and 16+4g .. 16+4g+3.
struct Rec16 {
  static constexpr int kKt = 0;               // 16 blocks: (token tile m, channel block f) at 4 m + f
  static constexpr int kQt = kKt + 16 * kFB;  // 16 blocks: (token tile m, channel block f) at 4 m + f
  static constexpr int kZ = kQt + 16 * kFB;   // 16 blocks: (key tile i, token block b) at 2 i + b
  static constexpr int kPw = kZ + 16 * kFB;   //  6 blocks: (token tile m, token block b <= m / 2)
  static constexpr int kDec = kPw + 6 * kFB;  // 128 fp32: e^Gamma_n
  static constexpr int kBytes = kDec + 512;
  static_assert(kBytes % 256 == 0, "records stay 256-byte aligned");
};
// Index of block (m, 0) among the lower-triangular token-block blocks.
__host__ __device__ constexpr int pw_blk(int m) { return m < 2 ? m : 2 * m - 2; }

// ---------------------------------------------------------------- prep
//
// One workgroup per (chunk, head), four waves; wave w owns token tile w
// (tokens 16w .. 16w+15), lane l = 16 g + r holds token 16w + r at the
// channels of its fragment positions (32kb + 4g + e and 32kb + 16 + 4g + e),
// so Kt and Qt are A fragments as computed.
//   * Gamma: prefix sums over the 16 lanes of a row (DPP), tile offsets
//     through LDS; two exponentials per element.
//   * Kb^T: each 16 x 16 tile is transposed by one MFMA against a 0/1
//     selection matrix (exact).
//   * P = Qt Kh^T and M = Kt Kh^T computed transposed, which leaves them in
//     fragment order.
//   * T = (I + Diag(beta) strict_tril(M))^-1 by 16 x 16 blocks: diagonal
//     blocks as (I - N)(I + N^2)(I + N^4)(I + N^8) (N nilpotent), then wave j
//     walks down block column j, T_ij = -T_ii sum_{m=j}^{i-1} N_im T_mj, all
//     on fp32 MFMA.
//   * Wave w then holds block column w of T in the accumulator layout, which
//     is the A fragment of T^T's token tile w: Z^T = Diag(beta) T^T Kb and
//     Pw^T = Diag(beta) T^T P^T come out as halves of Z's and Pw's fragments.
// A 16 x 16 fp32 tile in one of two register forms, for lane l = 16 g + r:
//   row form:    X[r][4g + e]
//   column form: X[4g + e][r]   (also the accumulator layout)
// The row form of X holds the numbers of the column form of X^T.
// Column form of A B from A in row form and B in column form: fp32 16x16x4
// MFMA e contracts over the indices 4g + e, g = 0..3.
__device__ __forceinline__ floatx4 mm16(floatx4 a, floatx4 b) {
  floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ floatx4 plus_eye(floatx4 x, int g, int r) {
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] += (4 * g + e == r) ? 1.f : 0.f;
  return x;
}
__device__ __forceinline__ float row_shr(float x, int s) {
  // value of the lane s places lower in the same 16-lane row, 0 past its start
  int v = __builtin_bit_cast(int, x);
  switch (s) {
    case 1: v = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true); break;
    case 2: v = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true); break;
    case 4: v = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true); break;
    default: v = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true); break;
  }
  return __builtin_bit_cast(float, v);
}
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type cvt4(floatx4 x) {
  typename Vec4<T>::type o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(x[e]);
  return o;
}
// 16-bit fragment from two accumulator tiles: positions 0-3 from `lo`, 4-7 from `hi`
template <typename T>
__device__ __forceinline__ typename OpTraits<T>::frag pack8(floatx4 lo, floatx4 hi) {
  typename OpTraits<T>::frag f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = from_f32<T>(lo[e]); f[4 + e] = from_f32<T>(hi[e]); }
  return f;
}
// Write four 16-bit values into half `hf` of a 16-byte fragment slot.
template <typename T>
__device__ __forceinline__ void put_half(void* slot, int hf, floatx4 x) {
  *reinterpret_cast<typename Vec4<T>::type*>(static_cast<uint8_t*>(slot) + 8 * hf) = cvt4<T>(x);
}

// LDS of the prep, 39.25 KiB: regions reused across phases (the comments
// give the phases that hold each view).
struct Prep16Smem {
  union {
    uint4 kh[4][4][64];        // Kh fragments [token tile][channel block][lane]    (Kh, P/M; then Z assembly)
    struct {
      float nd[4][16][20];     // diagonal N blocks, row-major                        (T solve)
      floatx4 nr[6][64];       // row forms of N_im, m < i, at i (i - 1) / 2 + m
      floatx4 dr[4][64];       // row forms of T_ii
    } t;
  } r1;
  union {
    uint4 stage[4][16][17];    // input rows [wave][row][16-byte piece], padded       (inputs)
    uint4 kbt[8][2][64];       // Kb^T fragments [key tile][token block][lane]        (Kb^T, Z; then Pw assembly)
  } r2;
  union {
    struct {
      float tot[4][128];       // per token tile: sum of g over the tile              (Gamma)
      float off[4][128];       // sum of g over the preceding tiles
      float gn[128], ninv[128];  // Gamma_n, e^-Gamma_n
    } g;
    uint4 p[6][64];            // P fragments, block (m, b) at pw_blk(m) + b          (P, Pw)
  } r3;
  float beta[64];
};

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void kda_chunk_prep16(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ g,
    const T* __restrict__ bl, const int32_t* __restrict__ cu, int n_seqs, int64_t total,
    int H, int64_t cap, const int32_t* __restrict__ off, uint8_t* __restrict__ recs, int l2norm,
    int32_t* __restrict__ dev_err) {
  constexpr int DK = 128, C = 64, NFK = DK / 32;
  typedef Rec16 R;
  typedef typename OpTraits<T>::frag F8;   // 8 x 16-bit fragment
  typedef typename Vec4<T>::type In4;
  __shared__ Prep16Smem sm;

  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // token tile, wave-uniform
  // Chunk slots in descending order: the scan reads records from the first
  // chunk on, and the most recently written ones are the likeliest to still
  // be in the memory-side cache.
  const int h = blockIdx.x % H;
  const int j = (int)(cap - 1) - (int)(blockIdx.x / H);  // global chunk slot
  if (off != nullptr && j >= off[n_seqs]) return;
  int lo = 0, hi = n_seqs - 1;   // sequence owning chunk slot j
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= j) lo = mid; else hi = mid - 1;
  }
  int t_beg, len, nch;
  if (!seq_ok(cu, off, lo, total, C, t_beg, len, nch)) return;
  const int c = j - chunk_base(off, lo);
  if (c >= nch) return;
  const int t0 = t_beg + c * C;
  const int n = min(C, len - c * C);
  uint8_t* rec = recs + ((int64_t)h * cap + j) * R::kBytes;

  // ---- inputs.  Each wave loads its 16 token rows of k, q, g as whole rows
  //      (16 bytes per lane, 1 KiB per load: one L1 request per line), then
  //      regroups them through its own rows of LDS into the fragment layout.
  //      Rows past the chunk's end lie outside the buffer range and read as
  //      zero (zero keys, queries and gates).
  const int t = 16 * w + r;
  const bool valid = t < n;
  const int64_t hd = (int64_t)H * DK;
  const int64_t row = (int64_t)(t0 + min(t, n - 1));
  const T braw = bl[row * H + h];
  const int64_t cbase = (int64_t)t0 * hd + (int64_t)h * DK;
  const uint32_t nbytes = (uint32_t)(((int64_t)(n - 1) * hd + DK) * (int64_t)sizeof(T));
  const auto rk = buffer_rsrc(k + cbase, nbytes), rq = buffer_rsrc(q + cbase, nbytes),
             rg = buffer_rsrc(g + cbase, nbytes);
  uint4 graw[4], kraw[4], qraw[4];
#pragma unroll
  for (int jr = 0; jr < 4; ++jr) {  // rows 16w + 4jr + (lane / 16), bytes 16 (lane % 16) ..
    const int voff = (int)((int64_t)(16 * w + 4 * jr + (lane >> 4)) * hd * (int64_t)sizeof(T)) + 16 * r;
    graw[jr] = ld16(rg, voff, 0);
    kraw[jr] = ld16(rk, voff, 0);
    qraw[jr] = ld16(rq, voff, 0);
  }
  In4 kr[NFK][2], qr[NFK][2], grw[NFK][2];
  auto regroup = [&](const uint4 (&raw)[4], In4 (&out)[NFK][2]) {
#pragma unroll
    for (int jr = 0; jr < 4; ++jr) sm.r2.stage[w][4 * jr + (lane >> 4)][r] = raw[jr];
    wave_sync();
    const uint8_t* rowp = reinterpret_cast<const uint8_t*>(&sm.r2.stage[w][r][0]);
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        out[kb][hf] = *reinterpret_cast<const In4*>(rowp + 64 * kb + 32 * hf + 8 * gq);
    wave_sync();
  };
  regroup(graw, grw);
  regroup(kraw, kr);
  regroup(qraw, qr);
  // ---- optional L2 normalisation of the k and q rows: the four lanes
  //      16 g + r (g = 0..3) hold token r's 128 channels; each row is scaled
  //      by 1 / sqrt(sum x^2 + 1e-6) in fp32 and rounded once to T, so the
  //      record holds what verify would see for the same token
  if (l2norm) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = to_f32(kr[kb][hf][e]), y = to_f32(qr[kb][hf][e]);
          sk += x * x;
          sq += y * y;
        }
    sk += __shfl_xor(sk, 16);
    sq += __shfl_xor(sq, 16);
    sk += __shfl_xor(sk, 32);
    sq += __shfl_xor(sq, 32);
    const float ks = rsqrtf(sk + 1e-6f), qs = rsqrtf(sq + 1e-6f);
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kr[kb][hf][e] = from_f32<T>(to_f32(kr[kb][hf][e]) * ks);
          qr[kb][hf][e] = from_f32<T>(to_f32(qr[kb][hf][e]) * qs);
        }
  }
  const float beta = valid ? sigmoidf_(to_f32(braw)) : 0.f;
  if (gq == 0) sm.beta[t] = beta;

  // ---- Gamma: prefix sums of g over the tile's 16 tokens (DPP), then the
  //      tile totals go through LDS to give every tile its offset
  float gs[NFK][8];
#pragma unroll
  for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) gs[kb][e] = to_f32(grw[kb][e >> 2][e & 3]);
#pragma unroll
  for (int s = 1; s < 16; s <<= 1)
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) gs[kb][e] += row_shr(gs[kb][e], s);
  if (r == 15) {
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        *reinterpret_cast<floatx4*>(&sm.r3.g.tot[w][32 * kb + 16 * hf + 4 * gq]) =
            floatx4{gs[kb][4 * hf], gs[kb][4 * hf + 1], gs[kb][4 * hf + 2], gs[kb][4 * hf + 3]};
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int ch = lane + 64 * cc;
      const float a0 = sm.r3.g.tot[0][ch], a1 = sm.r3.g.tot[1][ch], a2 = sm.r3.g.tot[2][ch],
                  a3 = sm.r3.g.tot[3][ch];
      sm.r3.g.off[0][ch] = 0.f;
      sm.r3.g.off[1][ch] = a0;
      sm.r3.g.off[2][ch] = a0 + a1;
      sm.r3.g.off[3][ch] = a0 + a1 + a2;
      const float gn = a0 + a1 + a2 + a3;
      sm.r3.g.gn[ch] = gn;
      sm.r3.g.ninv[ch] = __expf(-gn);
      __builtin_nontemporal_store(__expf(gn), reinterpret_cast<float*>(rec + R::kDec) + ch);  // whole lines
    }
  }
  __syncthreads();

  // ---- Kt = K e^Gamma, Qt = Q e^Gamma, Kb = K e^(Gamma_n - Gamma), Kh = Kb e^-Gamma_n.
  //      Every factor but Kh's is at most 1.  Kh = K e^-Gamma grows with the
  //      chunk's decay; an element that would round to infinity in T (a
  //      chunk whose cumulative log decay falls below about -11 for fp16, or
  //      leaves the fp32 range, below about -88, for bf16, at |k| <= 1) is
  //      flagged with the gate-range error bit instead of passing silently.
  F8 ktf[NFK], qtf[NFK], kbf[NFK], khf[NFK];
#pragma unroll
  for (int kb = 0; kb < NFK; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int ch = 32 * kb + 16 * hf + 4 * gq;
      const floatx4 of = *reinterpret_cast<const floatx4*>(&sm.r3.g.off[w][ch]);
      const floatx4 gn = *reinterpret_cast<const floatx4*>(&sm.r3.g.gn[ch]);
      const floatx4 ni = *reinterpret_cast<const floatx4*>(&sm.r3.g.ninv[ch]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float G = gs[kb][4 * hf + e] + of[e];
        const float a = __expf(G), b = __expf(gn[e] - G);
        const float kv = to_f32(kr[kb][hf][e]);
        const float qv = to_f32(qr[kb][hf][e]);
        const float kbv = kv * b;
        ktf[kb][4 * hf + e] = from_f32<T>(kv * a);
        qtf[kb][4 * hf + e] = from_f32<T>(qv * a);
        kbf[kb][4 * hf + e] = from_f32<T>(kbv);
        khf[kb][4 * hf + e] = from_f32<T>(kbv * ni[e]);
      }
    }
  // Records are stored non-temporally, in whole 16-byte fragment pieces
  // (Z and Pw are assembled in LDS first): the scan reads each record once,
  // about a prep's duration later, and dirty records left in the
  // memory-side cache cost the next kernel their write-back (a verify right
  // after the prefill 147 -> 134 us).  Non-temporal 8-byte halves, each
  // line completed by a second wave, made the prefill slower instead.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  // Gate range: a 16-bit element whose exponent field is all ones rounded
  // to infinity (or is NaN).  Adding the field's lowest bit to the masked
  // field carries into the sign position exactly then, for both halves of a
  // word at once.
  constexpr uint32_t kExpMask = std::is_same<T, f16>::value ? 0x7C007C00u : 0x7F807F80u;
  constexpr uint32_t kExpLow = std::is_same<T, f16>::value ? 0x04000400u : 0x00800080u;
  uint32_t kh_bad = 0;
#pragma unroll
  for (int kb = 0; kb < NFK; ++kb) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ktf[kb]),
                                reinterpret_cast<u32x4*>(rec + R::kKt + (w * NFK + kb) * kFB + lane * 16));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, qtf[kb]),
                                reinterpret_cast<u32x4*>(rec + R::kQt + (w * NFK + kb) * kFB + lane * 16));
    const uint4 kh = __builtin_bit_cast(uint4, khf[kb]);
    for (uint32_t wd : {kh.x, kh.y, kh.z, kh.w}) kh_bad |= (wd & kExpMask) + kExpLow;
    sm.r1.kh[w][kb][lane] = kh;
  }
  if (__builtin_amdgcn_ballot_w64((kh_bad & 0x80008000u) != 0) != 0 && lane == 0) set_err(dev_err, 1u << 5);

  // 0/1 selection fragments: sel[hf] picks channel 16 hf + r of a K-block, so
  // the product X sel[hf] is the transpose of X's 16 x 16 tile hf, in the
  // accumulator layout (token rows 4g + e, channel column r): half (w % 2)
  // of the transposed matrix's fragment for token block w / 2.
  F8 sel[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int idx = p < 4 ? 4 * gq + p : 16 + 4 * gq + (p - 4);  // channel at position 8g + p
      sel[hf][p] = from_f32<T>(idx == 16 * hf + r ? 1.f : 0.f);
    }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb)
      put_half<T>(&sm.r2.kbt[2 * kb + hf][w >> 1][lane], w & 1,
                  mma(floatx4{0.f, 0.f, 0.f, 0.f}, kbf[kb], sel[hf]));
  __syncthreads();

  // ---- P^T and M^T tiles (jt, w) for jt <= w: Kh of tile jt is the A
  //      operand, this tile's Qt / Kt fragments the B operand.  Lane (g, r)
  //      then holds P[16w + r][16jt + 4g + e], the row form of P_w,jt.
  floatx4 ptile[4], nrow[4];
  const int rr = 16 * w + r;  // this lane's row of P, M, N, T
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    ptile[jt] = nrow[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (jt > w) continue;
    floatx4 pm = {0.f, 0.f, 0.f, 0.f}, pp = pm;
#pragma unroll
    for (int kb = 0; kb < NFK; ++kb) {
      const F8 a = __builtin_bit_cast(F8, sm.r1.kh[jt][kb][lane]);
      pm = mma(pm, a, ktf[kb]);
      pp = mma(pp, a, qtf[kb]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int s = 16 * jt + 4 * gq + e;
      ptile[jt][e] = s <= rr ? pp[e] : 0.f;
      nrow[jt][e] = s < rr ? beta * pm[e] : 0.f;
    }
  }
  // P fragments: block (w, b) = [P_w,2b | P_w,2b+1] for token blocks b up to the diagonal
#pragma unroll
  for (int b = 0; b < 2; ++b)
    if (b <= w / 2) sm.r3.p[pw_blk(w) + b][lane] = __builtin_bit_cast(uint4, pack8<T>(ptile[2 * b], ptile[2 * b + 1]));
  __syncthreads();  // Kh is dead: its space takes the T solve

  // ---- T_ww = (I + N_ww)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), both forms
  const floatx4 n1r = nrow[w];
  *reinterpret_cast<floatx4*>(&sm.r1.t.nd[w][r][4 * gq]) = n1r;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (m < w) sm.r1.t.nr[w * (w - 1) / 2 + m][lane] = nrow[m];
  wave_sync();
  floatx4 n1c;
#pragma unroll
  for (int e = 0; e < 4; ++e) n1c[e] = sm.r1.t.nd[w][4 * gq + e][r];
  const floatx4 n2c = mm16(n1r, n1c), n2r = mm16(n1c, n1r);
  const floatx4 n4c = mm16(n2r, n2c), n4r = mm16(n2c, n2r);
  const floatx4 n8c = mm16(n4r, n4c), n8r = mm16(n4c, n4r);
  floatx4 dc = plus_eye(n8c, gq, r);
  dc = dc + mm16(n4r, dc);
  dc = dc + mm16(n2r, dc);
  dc = dc - mm16(n1r, dc);        // column form of T_ww
  floatx4 dr = plus_eye(n8r, gq, r);
  dr = dr + mm16(n4c, dr);
  dr = dr + mm16(n2c, dr);
  dr = dr - mm16(n1c, dr);        // row form of T_ww
  sm.r1.t.dr[w][lane] = dr;
  __syncthreads();

  // ---- block column w: T_iw = -T_ii sum_{m=w}^{i-1} N_im T_mw, i > w (column forms)
  floatx4 tc[4];
  tc[0] = tc[1] = tc[2] = tc[3] = floatx4{0.f, 0.f, 0.f, 0.f};
  tc[w] = dc;
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    if (i <= w) continue;
    floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 3; ++m)
      if (m >= w && m < i) z = z + mm16(sm.r1.t.nr[i * (i - 1) / 2 + m][lane], tc[m]);
    tc[i] = -mm16(sm.r1.t.dr[i][lane], z);
  }

  // ---- Z^T and Pw^T rows of token tile w.  The column forms tc[2b],
  //      tc[2b + 1] are the A fragment of T^T's row tile w for token block b
  //      (zero above the diagonal); rows are then scaled by beta, and the
  //      accumulators are halves (w % 2) of Z's and Pw's fragments for token
  //      block w / 2.
  F8 ta[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) ta[b] = pack8<T>(tc[2 * b], tc[2 * b + 1]);
  // Z and Pw halves are assembled in LDS (Z over the T solve's space, Pw over
  // Kb^T's once Z is done), then stored as whole 16-byte pieces
  uint4* const zst = &sm.r1.kh[0][0][0];       // 16 blocks x 64 lanes
  uint4* const pst = &sm.r2.kbt[0][0][0];      //  6 blocks x 64 lanes
  __syncthreads();   // every wave is done with the T solve's LDS
  const floatx4 bw = *reinterpret_cast<const floatx4*>(&sm.beta[16 * w + 4 * gq]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b)
      if (b >= w / 2) acc = mma(acc, ta[b], __builtin_bit_cast(F8, sm.r2.kbt[i][b][lane]));
    put_half<T>(reinterpret_cast<uint8_t*>(zst) + (2 * i + (w >> 1)) * kFB + lane * 16, w & 1, bw * acc);
  }
  floatx4 pw_acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    pw_acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (m / 2 < w / 2) continue;  // block (m, w / 2) lies above the diagonal
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (m >= w) {  // else the upper half of a diagonal block: zero
#pragma unroll
      for (int b = 0; b < 2; ++b)
        if (b >= w / 2 && b <= m / 2) acc = mma(acc, ta[b], __builtin_bit_cast(F8, sm.r3.p[pw_blk(m) + b][lane]));
    }
    pw_acc[m] = bw * acc;
  }
  __syncthreads();   // Z assembled; Kb^T no longer read
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m / 2 < w / 2) continue;
    put_half<T>(reinterpret_cast<uint8_t*>(pst) + (pw_blk(m) + (w >> 1)) * kFB + lane * 16, w & 1, pw_acc[m]);
  }
  typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {   // wave w stores Z blocks 4 w .. 4 w + 3
    const uint4 x = zst[(4 * w + jb) * 64 + lane];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4s, x),
                                reinterpret_cast<u32x4s*>(rec + R::kZ + (4 * w + jb) * kFB + lane * 16));
  }
  __syncthreads();   // Pw assembled
  for (int jb = w; jb < 6; jb += 4) {
    const uint4 x = pst[jb * 64 + lane];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4s, x),
                                reinterpret_cast<u32x4s*>(rec + R::kPw + jb * kFB + lane * 16));
  }
}

// ---------------------------------------------------------------- scan
//
// Nine waves per (sequence, head, column tile of S): eight that compute,
// two per SIMD, and one that only warms the L2.  A tile is NC 16-column
// tiles (NC = 1, 2 or 4): every product below runs once per 16-column tile,
// on the same record fragments.  One sequence's 32 heads give 256 narrow
// tiles, one per CU, which keeps the most CUs on the serial chain; with many
// sequences, wider tiles mean fewer passes over each record.
//  * Chain waves 0-3: wave w holds the fp32 state rows of key tiles 2w and
//    2w + 1 (keys 32w .. 32w+31 in the accumulator layout: lane (g, r) has
//    keys 4g + e of a tile, column r) and token tile w.  Per chunk:
//      [barrier 1]  X = Kt S for token tile w (S as B fragments from LDS);
//                   Y = V - X -> LDS, half of Y's B fragment for block w/2;
//      [barrier 2]  S = e^Gamma_n S + Z Y for its key tiles; S's bf16
//                   fragment for key block w -> LDS.
//    Two key tiles of accumulators are exactly the B fragment of key block
//    w, so each chain wave publishes one fragment per chunk.
//  * Output waves 4-7 (token tile m = w - 4): O = Qt S after barrier 1,
//    O += Pw Y after barrier 2, then the tile goes to o.  They also move the
//    next chunk's V tile and e^Gamma_n into LDS.
//  * Each wave loads its share of a record two chunks ahead into registers.
//  * Prefetch wave 8: the NVT workgroups of a head read every line of every
//    record, and the first of them to ask for a line waits for the memory
//    side while the others queue behind that miss.  Each workgroup's wave 8
//    touches its own eighth of the record (one dword per 128-byte line)
//    kScanPrefetch chunks ahead and waits for those loads itself, so the
//    lines are in the XCD's L2 by the time the other waves ask; no other
//    wave's wait counts include these loads.
constexpr int kScanThreads = 9 * 64;
constexpr int kScanPrefetch = 4;   // chunks ahead of the one being scanned

template <typename TIn, int NC>
struct Scan16Lds {
  uint4 sf[NC][4][64];      // S as B fragments per 16-column tile, key block w from chain wave w
  uint4 y[NC][2][64];       // Y as B fragments per 16-column tile, token block b
  float dec[2][128];        // e^Gamma_n, by chunk parity
  TIn vb[2][64][16 * NC];   // V tiles, row-major, by chunk parity
  TIn ob[4][16][16 * NC];   // one output tile per output wave
};

template <typename TIn, typename TPool, int NC>
__global__ __launch_bounds__(kScanThreads) void kda_chunk_scan16(
    const TIn* __restrict__ v, TIn* __restrict__ o, const int32_t* __restrict__ cu, int n_seqs,
    int64_t total, int H, int64_t cap, const int32_t* __restrict__ off, const uint8_t* __restrict__ recs,
    TPool* __restrict__ pool, int64_t n_slots, const int32_t* __restrict__ init_slot,
    const int32_t* __restrict__ final_slot, const int32_t* __restrict__ track_ptr,
    const int32_t* __restrict__ track_chunk, const int32_t* __restrict__ track_slot, int n_track,
    float* __restrict__ track_f32, int32_t* __restrict__ dev_err) {
  constexpr int DK = 128, DV = 128, C = 64, BV = 16 * NC, NVT = DV / BV;
  typedef Rec16 R;
  typedef typename OpTraits<TIn>::frag F8;
  __shared__ Scan16Lds<TIn, NC> sm;

  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, l16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const bool chain = wv < 4;
  const int w = wv & 3;   // token tile; for a chain wave also its key block
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
    for (int e = e0 + tid; e < e1; e += kScanThreads) {
      const int ce = track_chunk[e], se = track_slot[e];
      if (ce < 0 || ce > len / C) set_err(dev_err, 1u << 1);
      if (se < -1 || (int64_t)se >= n_slots) set_err(dev_err, 1u);
    }
  }

  const int64_t vrow = (int64_t)H * DV;
  const int lane_off = lane * 16;
  const uint8_t* rec_seq = recs + ((int64_t)h * cap + chunk_base(off, seq)) * R::kBytes;
  auto rec_rsrc = [&](int c) { return buffer_rsrc(rec_seq + (int64_t)c * R::kBytes, R::kBytes); };
  // Rows of chunk c of V / o in this tile (reads past the last row return 0,
  // stores there are dropped).
  auto rows_rsrc = [&](const TIn* base, int c) {
    const int n = min(C, len - c * C);
    const TIn* p = base + (int64_t)(t_beg + c * C) * vrow + (int64_t)h * DV + v0;
    return buffer_rsrc(p, (uint32_t)(((int64_t)(n - 1) * vrow + BV) * (int)sizeof(TIn)));
  };
  const int last = nch - 1;

  if (chain) {
    // ---- initial state of key tiles 2w, 2w + 1: S[k][v] = pool[init][h][v][k]
    floatx4 S[NC][2];
    const int64_t st_off = (int64_t)(v0 + l16) * DK + 32 * w + 4 * g16;  // lane's first element (tile 0)
    {
      const int is = init_slot[seq];
      const bool ok = is >= 0 && (int64_t)is < n_slots;
      if (is != -1 && !ok && lead && tid == 0) set_err(dev_err, 1u);
      const TPool* src = pool + ((int64_t)(ok ? is : 0) * H + h) * DV * DK + st_off;
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          S[ct][jj] = floatx4{0.f, 0.f, 0.f, 0.f};
          if (ok) S[ct][jj] = load4(src + 16 * ct * DK + 16 * jj);
        }
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) asm volatile("" : "+v"(S[ct][jj]));
    }
    // Snapshots: `next_snap` is the smallest requested chunk index >= the
    // current one, so the per-chunk test is one scalar compare.
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
#pragma unroll
        for (int ct = 0; ct < NC; ++ct)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int64_t el = st_off + 16 * ct * DK + 16 * jj;
            // An opaque copy: with a pool of the operand type the cast below
            // equals the one that built S's LDS fragment at the end of the
            // previous step, and the compiler would otherwise keep those
            // converted values live across the loop for this rare store (a
            // register spill in the 64-column fp16 build).
            floatx4 sv = S[ct][jj];
            asm volatile("" : "+v"(sv));
            if (track_f32) store4(track_f32 + ((int64_t)e * H + h) * DV * DK + el, sv);
            if (to_pool) store4(pool + ((int64_t)se * H + h) * DV * DK + el, sv);
          }
      }
      next_snap = next_track(c + 1);
    };
    struct Ops { uint4 kt[4], z[2][2]; };  // Kt rows of token tile w; Z rows of key tiles 2w, 2w + 1
    auto ld_ops = [&](Ops& r, int c) {
      const auto rs = rec_rsrc(c);
#pragma unroll
      for (int f = 0; f < 4; ++f) r.kt[f] = ld16(rs, lane_off, R::kKt + (4 * w + f) * kFB);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int b = 0; b < 2; ++b) r.z[jj][b] = ld16(rs, lane_off, R::kZ + (2 * (2 * w + jj) + b) * kFB);
    };
    auto step = [&](Ops& r, int c, int bp) {
      snapshot(c);
      __syncthreads();
      // X = Kt S for token tile w;  Y = V - X
      floatx4 X[NC];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        X[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 4; ++f) X[ct] = mma(X[ct], as_frag<F8>(r.kt[f]), __builtin_bit_cast(F8, sm.sf[ct][f][lane]));
      }
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        floatx4 Y;
#pragma unroll
        for (int e = 0; e < 4; ++e) Y[e] = to_f32(sm.vb[bp][16 * w + 4 * g16 + e][16 * ct + l16]) - X[ct][e];
        put_half<TIn>(&sm.y[ct][w >> 1][lane], w & 1, Y);
      }
      __syncthreads();
      // S = e^Gamma_n S + Z Y
      floatx4 dec[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) dec[jj] = *reinterpret_cast<const floatx4*>(&sm.dec[bp][32 * w + 16 * jj + 4 * g16]);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        const F8 y0 = __builtin_bit_cast(F8, sm.y[ct][0][lane]), y1 = __builtin_bit_cast(F8, sm.y[ct][1][lane]);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          floatx4 acc = mma(floatx4{0.f, 0.f, 0.f, 0.f}, as_frag<F8>(r.z[jj][0]), y0);
          acc = mma(acc, as_frag<F8>(r.z[jj][1]), y1);
          S[ct][jj] = dec[jj] * S[ct][jj] + acc;
        }
        sm.sf[ct][w][lane] = __builtin_bit_cast(uint4, pack8<TIn>(S[ct][0], S[ct][1]));
      }
      ld_ops(r, min(c + 2, last));
    };

    if (nch > 0) {
      Ops rA, rB;
      ld_ops(rA, 0);
      ld_ops(rB, min(1, last));
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) sm.sf[ct][w][lane] = __builtin_bit_cast(uint4, pack8<TIn>(S[ct][0], S[ct][1]));
      int c = 0;
      for (; c + 1 < nch; c += 2) {
        step(rA, c, 0);
        step(rB, c + 1, 1);
      }
      if (c < nch) step(rA, c, 0);
    }
    if (len % C == 0) snapshot(nch);

    // ---- final state, one cast into the pool dtype
    const int fs = final_slot[seq];
    if (fs >= 0 && (int64_t)fs < n_slots) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          store4(pool + ((int64_t)fs * H + h) * DV * DK + st_off + 16 * ct * DK + 16 * jj, S[ct][jj]);
    } else if (fs != -1 && lead && tid == 0) {
      set_err(dev_err, 1u);
    }
  } else if (wv == 8 && nch > 0) {   // an empty sequence has no record to touch
    // ---- prefetch wave: lane l touches line l of share vt (one of NVT) of
    //      a record (lanes past the share or the record read nothing), and
    //      consumes each step's load two steps later.  With 64-column
    //      tiles (two per head: half of the record's lines each, four loads
    //      a step) the touches cost the CU's memory pipeline more than they
    //      save (four sequences of 8229 tokens 0.76 -> 0.73 ms without them,
    //      the varlen batch unchanged); there the wave only keeps the
    //      barrier count.
    constexpr bool kTouch = NC <= 2;
    constexpr int kLines = (R::kBytes / 128 + NVT - 1) / NVT;
    constexpr int NPL = (kLines + kWave - 1) / kWave;   // loads per step
    int poff[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int li = kWave * i + lane, line = vt * kLines + li;
      poff[i] = li < kLines && line * 128 < R::kBytes ? line * 128 : 0x7fffff00;  // out of range: no access
    }
    auto touch = [&](uint32_t (&x)[NPL], int c) {
      const auto rs = rec_rsrc(min(c, last));
#pragma unroll
      for (int i = 0; i < NPL; ++i) x[i] = kTouch ? __builtin_amdgcn_raw_buffer_load_b32(rs, poff[i], 0, 0) : 0u;
    };
    uint32_t pa[NPL], pb[NPL];
    touch(pa, kScanPrefetch - 2);
    touch(pb, kScanPrefetch - 1);
    for (int c = 0; c < nch; ++c) {   // two barriers per chunk, as in the other waves
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NPL; ++i) asm volatile("" ::"v"(pa[i]));   // the loads of two steps ago have returned
      touch(pa, c + kScanPrefetch);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const uint32_t t = pa[i];
        pa[i] = pb[i];
        pb[i] = t;
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) asm volatile("" ::"v"(pa[i]), "v"(pb[i]));
  } else if (nch > 0) {
    // ---- output waves, token tile m = w
    const int m = w;
    // V tile of a chunk: 16-byte pieces, 2 NC per row; piece q = 64 m + lane
    // + 256 i of the output waves (NVP loads each)
    constexpr int PPR = 2 * NC, NVP = (64 * PPR + 255) / 256;
    const bool has_dec = w == 2;
    int vq_off[NVP], vq_lds[NVP];
    bool has_v[NVP];
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int q = 64 * w + lane + 256 * i, row = q / PPR, part = q % PPR;
      has_v[i] = q < 64 * PPR;
      vq_off[i] = has_v[i] ? (int)((int64_t)row * vrow * (int)sizeof(TIn)) + 16 * part : 0x7fffff00;
      vq_lds[i] = has_v[i] ? row * 16 * NC + 8 * part : 0;
    }
    auto ld_v = [&](uint4 (&x)[NVP], int c) {
      const auto rs = rows_rsrc(v, c);
#pragma unroll
      for (int i = 0; i < NVP; ++i) x[i] = ld16(rs, vq_off[i], 0);
    };
    auto put_v = [&](int bp, const uint4 (&x)[NVP]) {
#pragma unroll
      for (int i = 0; i < NVP; ++i)
        if (has_v[i]) *reinterpret_cast<uint4*>(&sm.vb[bp][0][0] + vq_lds[i]) = x[i];
    };
    auto ld_dec = [&](int c) { return ld16(rec_rsrc(c), lane_off, R::kDec); };  // lanes >= 32 read 0
    auto put_dec = [&](int bp, uint4 x) {
      if (has_dec && lane < 32) *reinterpret_cast<uint4*>(&sm.dec[bp][4 * lane]) = x;
    };
    struct Ops { uint4 qt[4], pw[2]; };  // Qt rows of token tile m; Pw blocks (m, b), b <= m / 2
    auto ld_ops = [&](Ops& r, int c) {
      const auto rs = rec_rsrc(c);
#pragma unroll
      for (int f = 0; f < 4; ++f) r.qt[f] = ld16(rs, lane_off, R::kQt + (4 * m + f) * kFB);
      r.pw[0] = ld16(rs, lane_off, R::kPw + pw_blk(m) * kFB);
      if (m >= 2) r.pw[1] = ld16(rs, lane_off, R::kPw + (pw_blk(m) + 1) * kFB);
    };
    // the output tile goes out in 16-byte pieces, 2 NC per row
    constexpr int NSO = (32 * NC + 63) / 64;
    auto store_out = [&](const floatx4 (&O)[NC], int c) {
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.ob[m][4 * g16 + e][16 * ct + l16] = from_f32<TIn>(O[ct][e]);
      wave_sync();
      const auto rs = rows_rsrc(o, c);
#pragma unroll
      for (int i = 0; i < NSO; ++i) {
        const int q = lane + 64 * i;
        if (q < 32 * NC) {
          const int orow = q / PPR, opart = q % PPR;
          const uint4 x = *reinterpret_cast<const uint4*>(&sm.ob[m][orow][8 * opart]);
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, x), rs,
              (int)((int64_t)(16 * m + orow) * vrow * (int)sizeof(TIn)) + 16 * opart, 0, 0);
        }
      }
    };
    // step c: r = chunk c's operands; vr = V_{c+1}, dr = e^Gamma_n of chunk c + 1
    auto step = [&](Ops& r, uint4 (&vr)[NVP], uint4& dr, int c, int bp) {
      __syncthreads();
      floatx4 O[NC];
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        O[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 4; ++f) O[ct] = mma(O[ct], as_frag<F8>(r.qt[f]), __builtin_bit_cast(F8, sm.sf[ct][f][lane]));
      }
      put_v(bp ^ 1, vr);
      ld_v(vr, min(c + 3, last));
      put_dec(bp ^ 1, dr);
      dr = ld_dec(min(c + 3, last));
      __syncthreads();
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        O[ct] = mma(O[ct], as_frag<F8>(r.pw[0]), __builtin_bit_cast(F8, sm.y[ct][0][lane]));
        if (m >= 2) O[ct] = mma(O[ct], as_frag<F8>(r.pw[1]), __builtin_bit_cast(F8, sm.y[ct][1][lane]));
      }
      ld_ops(r, min(c + 2, last));
      store_out(O, c);
    };

    Ops rA, rB;
    uint4 vA[NVP], vB[NVP], dA, dB;
    // prologue: V_0 and e^Gamma_n of chunk 0 into LDS; V_1, V_2, dec_1, dec_2
    // in registers, issued in the order the loop issues them so that its
    // wait counts stay partial
    {
      uint4 v0r[NVP];
      ld_v(v0r, 0);
      put_v(0, v0r);
    }
    put_dec(0, ld_dec(0));
    ld_v(vA, min(1, last));
    dA = ld_dec(min(1, last));
    ld_ops(rA, 0);
    ld_v(vB, min(2, last));
    dB = ld_dec(min(2, last));
    ld_ops(rB, min(1, last));
    int c = 0;
    for (; c + 1 < nch; c += 2) {
      step(rA, vA, dA, c, 0);
      step(rB, vB, dB, c + 1, 1);
    }
    if (c < nch) step(rA, vA, dA, c, 0);
    // Nothing of this branch stays in flight: the compiler's wait counts for
    // the chain branch would otherwise assume these loads and stores could
    // still be outstanding there and wait for everything.
    __builtin_amdgcn_s_waitcnt(0);
  }
}

template <typename TIn, typename TPool>
hipError_t run16(const PrefillArgs& a, hipStream_t st, int64_t cap, const int32_t* off, uint8_t* recs) {
  if (cap > 0)
    hipLaunchKernelGGL(kda_chunk_prep16<TIn>, dim3((unsigned)(cap * a.H)), dim3(kThreads), 0, st,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.g), static_cast<const TIn*>(a.b), a.cu_seqlens,
                       a.n_seqs, a.total_tokens, a.H, cap, off, recs, (a.flags & 1u) ? 1 : 0, a.dev_err);
  const int64_t pairs = (int64_t)a.n_seqs * a.H;
  const int64_t pairs8 = (pairs + kXcd - 1) / kXcd * kXcd;
  // Each workgroup streams its head's whole record per chunk through its
  // CU's vector memory path, so the column tile width trades parallelism on
  // the serial chain against record passes: the narrowest tiles (16, 32 or
  // 64 columns) whose workgroups all fit on the CUs at once, else 64.
  const int nc = pairs8 * 8 <= kNumCU ? 1 : pairs8 * 4 <= kNumCU ? 2 : 4;
  auto ks = nc == 1 ? kda_chunk_scan16<TIn, TPool, 1>
                    : nc == 2 ? kda_chunk_scan16<TIn, TPool, 2> : kda_chunk_scan16<TIn, TPool, 4>;
  const int64_t blocks = pairs8 * (8 / nc);
  // With 16-column tiles, reserve enough LDS (unused) that no two
  // workgroups share a CU (the wider tiles' registers already ensure it).
  int lds_pad = 0;
  if (nc == 1) {
    lds_pad = kSpreadLds;
    hipError_t e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, lds_pad);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ks, dim3((unsigned)blocks), dim3(kScanThreads), lds_pad, st,
                     static_cast<const TIn*>(a.v), static_cast<TIn*>(a.o), a.cu_seqlens, a.n_seqs,
                     a.total_tokens, a.H, cap, off, recs, static_cast<TPool*>(a.pool.base),
                     a.pool.n_slots, a.init_slot, a.final_slot, a.track_ptr, a.track_chunk,
                     a.track_slot, a.n_track, a.track_f32, a.dev_err);
  return hipGetLastError();
}

template <typename TIn>
hipError_t by_pool16(const PrefillArgs& a, hipStream_t st, int64_t cap, const int32_t* off, uint8_t* recs) {
  switch (a.pool.dtype) {
    case F32: return run16<TIn, float>(a, st, cap, off, recs);
    case F16: return run16<TIn, f16>(a, st, cap, off, recs);
    case BF16: return run16<TIn, bf16>(a, st, cap, off, recs);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int64_t rec16_bytes() { return Rec16::kBytes; }

hipError_t launch_prefill16(const PrefillArgs& a, hipStream_t st, int64_t cap, const int32_t* off,
                            uint8_t* recs) {
  if (a.dk != 128 || a.dv != 128 || a.chunk != 64) return hipErrorInvalidValue;
  if (a.in_dtype == BF16) return by_pool16<bf16>(a, st, cap, off, recs);
  if (a.in_dtype == F16) return by_pool16<f16>(a, st, cap, off, recs);
  return hipErrorInvalidValue;
}

}  // namespace kda
