// Pieces shared by the two chunked-prefill paths (prefill.hip: the general
// chunk form, for fp32 operands; prefill16.hip: the chunk transition form
// for 16-bit operands): launch constants, the chunk map, record sizes and
// raw buffer loads.
#pragma once

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kThreads = 256;
constexpr int kXcd = 8;     // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kFB = 1024;   // bytes of one fragment block: 64 lanes x 16 bytes
constexpr int kNumCU = 256; // MI355X compute units
constexpr int kSpreadLds = 72 * 1024;  // with the static part, > half of a CU's 160 KiB LDS

// K-block size of the general chunk form's fp32 fragments (16x16x4 MFMAs,
// one 16-byte fragment per lane).
constexpr int kKB32 = 16;

// Workspace record of the general chunk form for one (chunk, head), fp32.
// A-operand matrices are stored as fragment blocks: block (tile, kb) of an
// M x K matrix holds, for lane l = 16 g + r, row 16 tile + r at K-block
// positions kb*16 + 4 g + j.
template <int DK, int C, typename TOp>
struct Rec {
  static_assert(sizeof(TOp) == 4, "the general chunk form runs on fp32 operands");
  static constexpr int KBK = kKB32, KBT = kKB32;
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
// The chunk map in the workspace: off[n_seqs + 1], then the scan's order of
// the sequences, ord[n_seqs].
__host__ __device__ inline int64_t map_bytes(int n_seqs) { return round_up(4 * (2 * (int64_t)n_seqs + 1), 256); }
// Batches up to this many sequences are scanned longest first (the map
// ranks them); larger ones in batch order.
constexpr int kOrderMax = 128;
__host__ __device__ inline int64_t chunk_upper_bound(int64_t total_tokens, int n_seqs, int C) {
  return total_tokens / C + n_seqs;
}

// Chunk map: sequence i owns chunk slots off[i] .. off[i + 1] - 1.  A
// single sequence needs no map (off == nullptr): its chunks take slots
// 0 .. ceil(len / C) - 1, and ceil(len / C) <= total / C + 1 slots exist.
__device__ __forceinline__ int chunk_base(const int32_t* off, int seq) { return off ? off[seq] : 0; }
// The sequence at place i of the scan's order (ord, written by the chunk
// map after off); without a map, i itself.
__device__ __forceinline__ int seq_at(const int32_t* off, int n_seqs, int i) {
  return off ? off[n_seqs + 1 + i] : i;
}

// A sequence is processed only if its cu_seqlens entries are sane and the
// chunk map (if any) gave it exactly ceil(len / C) chunks.
__device__ __forceinline__ bool seq_ok(const int32_t* cu, const int32_t* off, int seq,
                                       int64_t total, int C, int& t_beg, int& len, int& nch) {
  t_beg = cu[seq];
  const int t_end = cu[seq + 1];
  len = t_end - t_beg;
  nch = (len + C - 1) / C;
  return t_beg >= 0 && len >= 0 && (int64_t)t_end <= total &&
         (off == nullptr || off[seq + 1] - off[seq] == nch);
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

// K-blocks of T and P rows of token tile mt up to the diagonal, and the
// index of block (mt, 0) among the lower (incl. diagonal) T blocks.
template <int KB>
__host__ __device__ constexpr int scan_nkb(int mt) { return (16 * mt + 15) / KB + 1; }
template <int KB>
__host__ __device__ constexpr int scan_tblk(int mt) {
  int j = 0;
  for (int m = 0; m < mt; ++m) j += scan_nkb<KB>(m);
  return j;
}

// 16-bit path (prefill16.hip): record bytes per (chunk, head), and the prep
// and scan launches once the chunk map is in the workspace.
int64_t rec16_bytes();
hipError_t launch_prefill16(const PrefillArgs& a, hipStream_t st, int64_t cap, const int32_t* off,
                            uint8_t* recs);

}  // namespace kda
