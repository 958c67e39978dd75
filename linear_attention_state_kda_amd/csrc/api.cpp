// C ABI of libkda.so: host-side validation, then one asynchronous launch
// sequence on the caller's stream.  Everything checkable on the host is
// rejected here, before any device memory is touched (vLLM PR #51855 summary,
// risks item 1: a configuration the kernel cannot serve must fail at call
// time, not inside the first step that hits it).
#include <algorithm>
#include <cstring>
#include <hip/hip_runtime.h>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

// A dispatch carries its size in work-items in a 32-bit field, so a launch
// of `blocks` workgroups of `threads` work-items must keep the product
// within 2^32 - 1.  The work-items per unit of each call, from its kernels:
// the prefill's prep 256 per (chunk slot, head), its scan at most 2,048 per
// (sequence, head) pair, the pairs rounded up to a multiple of 8 (the
// general form: d_v / 16 <= 8 tiles of 256; the 16-bit form: 1,152 once
// more than 64 pairs, fewer pairs giving a grid far below the limit);
// verify 512 per
// (request, head), the items rounded up to a multiple of 8; commit and
// align commit 256 per (request, head); copy 256 per 16 KiB of a slot per
// pair; the conv update 256 per (op, tensor).
bool grid_fits(int64_t blocks, int64_t threads) { return blocks <= (int64_t)UINT32_MAX / threads; }
int64_t up8(int64_t x) { return (x + 7) / 8 * 8; }
bool prefill_grids_fit(int64_t total_tokens, int32_t n_seqs, int32_t H, int32_t chunk) {
  return grid_fits((total_tokens / chunk + n_seqs) * (int64_t)H, 256) &&
         grid_fits(up8((int64_t)n_seqs * H), 2048);
}

bool dtype_ok(int32_t dt) { return dt == KDA_F32 || dt == KDA_F16 || dt == KDA_BF16; }

size_t dtype_size(int32_t dt) { return dt == KDA_F32 ? 4 : 2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

kda::PoolDesc pool_desc(const kda_pool& p) { return kda::PoolDesc{p.base, p.n_slots, p.dtype}; }

kda_status check_pool(const kda_pool& p, int32_t H, int32_t dk, int32_t dv) {
  if (p.base == nullptr || p.n_slots <= 0) return KDA_ERR_INVALID_ARG;
  if (!dtype_ok(p.dtype)) return KDA_ERR_UNSUPPORTED;
  if (!aligned(p.base, 16)) return KDA_ERR_INVALID_ARG;
  if (p.H != H || p.d_k != dk || p.d_v != dv) return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

kda_status launched(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* kda_status_string(kda_status status) {
  // Callers may pass any integer (a C enum is an int); read it as one, since
  // loading an out-of-range value through the C++ enum type is undefined.
  int32_t s;
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
  }
  return "KDA_ERR_UNKNOWN";
}

kda_status kda_chunk_prefill_workspace(int32_t n_seqs, int64_t total_tokens, int32_t H,
                                       int32_t d_k, int32_t d_v, int32_t chunk, int32_t in_dtype,
                                       size_t* bytes) {
  if (bytes == nullptr || n_seqs < 0 || total_tokens < 0 || H <= 0) return KDA_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype)) return KDA_ERR_UNSUPPORTED;
  if (!kda::prefill_supported(d_k, d_v, chunk, in_dtype, KDA_F32)) return KDA_ERR_UNSUPPORTED;
  if (total_tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (!prefill_grids_fit(total_tokens, n_seqs, H, chunk)) return KDA_ERR_UNSUPPORTED;
  *bytes = kda::prefill_workspace_bytes(n_seqs, total_tokens, H, d_k, d_v, chunk, in_dtype);
  return KDA_OK;
}

}  // extern "C"

namespace {

// Every host-side check of a prefill call except the workspace's; *need
// receives the workspace bytes the call takes.  KDA_OK with n_seqs == 0
// means there is nothing to do.
kda_status prefill_check(const void* q, const void* k, const void* v, const void* g, const void* b,
                         int32_t in_dtype, const void* o, const int32_t* cu_seqlens, int32_t n_seqs,
                         int64_t total_tokens, int32_t H, int32_t d_k, int32_t d_v, int32_t chunk,
                         const kda_pool& pool, const int32_t* init_slot, const int32_t* final_slot,
                         const int32_t* track_ptr, const int32_t* track_chunk, const int32_t* track_slot,
                         int32_t n_track, const float* track_f32, uint32_t flags, size_t* need) {
  if (n_seqs < 0 || total_tokens < 0 || H <= 0 || n_track < 0) return KDA_ERR_INVALID_ARG;
  if ((flags & ~KDA_QK_L2NORM) != 0) return KDA_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype)) return KDA_ERR_UNSUPPORTED;
  if (!kda::prefill_supported(d_k, d_v, chunk, in_dtype, pool.dtype)) return KDA_ERR_UNSUPPORTED;
  if (total_tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (!prefill_grids_fit(total_tokens, n_seqs, H, chunk)) return KDA_ERR_UNSUPPORTED;
  kda_status ps = check_pool(pool, H, d_k, d_v);
  if (ps != KDA_OK) return ps;
  if (n_seqs == 0) return KDA_OK;
  if (cu_seqlens == nullptr || init_slot == nullptr || final_slot == nullptr) return KDA_ERR_INVALID_ARG;
  if (total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || g == nullptr ||
                           b == nullptr || o == nullptr))
    return KDA_ERR_INVALID_ARG;
  if (n_track > 0 && (track_ptr == nullptr || track_chunk == nullptr || track_slot == nullptr))
    return KDA_ERR_INVALID_ARG;
  // 16-byte vector loads of q, k, g and v, 16-byte stores of o and track_f32
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(g, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(track_f32, 16))
    return KDA_ERR_INVALID_ARG;
  *need = kda::prefill_workspace_bytes(n_seqs, total_tokens, H, d_k, d_v, chunk, in_dtype);
  return KDA_OK;
}

kda_status prefill_launch(const void* q, const void* k, const void* v, const void* g, const void* b,
                          int32_t in_dtype, void* o, const int32_t* cu_seqlens, int32_t n_seqs,
                          int64_t total_tokens, int32_t H, int32_t d_k, int32_t d_v, int32_t chunk,
                          const kda_pool& pool, const int32_t* init_slot, const int32_t* final_slot,
                          const int32_t* track_ptr, const int32_t* track_chunk, const int32_t* track_slot,
                          int32_t n_track, float* track_f32, uint32_t flags, int32_t* dev_err,
                          void* workspace, void* stream) {
  kda::PrefillArgs a{q, k, v, g, b, o, in_dtype, cu_seqlens, n_seqs, total_tokens, H, d_k, d_v,
                     chunk, pool_desc(pool), init_slot, final_slot,
                     n_track > 0 ? track_ptr : nullptr, track_chunk, track_slot, n_track,
                     track_f32, dev_err, workspace, flags};
  return launched(kda::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, const void* g,
                             const void* b, int32_t in_dtype, void* o,
                             const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t H, int32_t d_k, int32_t d_v, int32_t chunk, kda_pool pool,
                             const int32_t* init_slot, const int32_t* final_slot,
                             const int32_t* track_ptr, const int32_t* track_chunk,
                             const int32_t* track_slot, int32_t n_track, float* track_f32,
                             uint32_t flags, int32_t* dev_err, void* workspace,
                             size_t workspace_bytes, void* stream) {
  size_t need = 0;
  kda_status s = prefill_check(q, k, v, g, b, in_dtype, o, cu_seqlens, n_seqs, total_tokens, H, d_k, d_v,
                               chunk, pool, init_slot, final_slot, track_ptr, track_chunk, track_slot,
                               n_track, track_f32, flags, &need);
  if (s != KDA_OK || n_seqs == 0) return s;
  if (workspace == nullptr || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return KDA_ERR_WORKSPACE;
  return prefill_launch(q, k, v, g, b, in_dtype, o, cu_seqlens, n_seqs, total_tokens, H, d_k, d_v, chunk,
                        pool, init_slot, final_slot, track_ptr, track_chunk, track_slot, n_track, track_f32,
                        flags, dev_err, workspace, stream);
}

kda_status kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                                     const void* b, int32_t in_dtype, void* o,
                                     const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                                     int32_t H, int32_t d_k, int32_t d_v, int32_t chunk, kda_pool pool,
                                     const int32_t* init_slot, const int32_t* final_slot,
                                     const int32_t* track_ptr, const int32_t* track_chunk,
                                     const int32_t* track_slot, int32_t n_track, float* track_f32,
                                     uint32_t flags, int32_t* dev_err, void* stream) {
  size_t need = 0;
  kda_status s = prefill_check(q, k, v, g, b, in_dtype, o, cu_seqlens, n_seqs, total_tokens, H, d_k, d_v,
                               chunk, pool, init_slot, final_slot, track_ptr, track_chunk, track_slot,
                               n_track, track_f32, flags, &need);
  if (s != KDA_OK || n_seqs == 0) return s;
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
  // the library's static scratch on the current device: its address, never the array's name
  void* ws = nullptr;
  if (kda::noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_LAUNCH;
  return prefill_launch(q, k, v, g, b, in_dtype, o, cu_seqlens, n_seqs, total_tokens, H, d_k, d_v, chunk,
                        pool, init_slot, final_slot, track_ptr, track_chunk, track_slot, n_track, track_f32,
                        flags, dev_err, ws, stream);
}

kda_status kda_recurrent_verify(const void* q, const void* k, const void* v, const void* g,
                                const void* b, int32_t in_dtype, void* o, int32_t n_req,
                                int32_t L, int32_t H, int32_t d_k, int32_t d_v, kda_pool pool,
                                const int32_t* ckpt_slot, float* u_rec, void* kg_rec,
                                uint32_t flags, int32_t* dev_err, void* stream) {
  if (n_req < 0 || H <= 0 || L < 1) return KDA_ERR_INVALID_ARG;
  if ((flags & ~KDA_QK_L2NORM) != 0) return KDA_ERR_INVALID_ARG;
  if (L > 256) return KDA_ERR_UNSUPPORTED;
  if (!dtype_ok(in_dtype)) return KDA_ERR_UNSUPPORTED;
  if (d_k != 128 || d_v != 128) return KDA_ERR_UNSUPPORTED;
  kda_status ps = check_pool(pool, H, d_k, d_v);
  if (ps != KDA_OK) return ps;
  if (n_req == 0) return KDA_OK;
  if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || b == nullptr ||
      o == nullptr || ckpt_slot == nullptr || u_rec == nullptr || kg_rec == nullptr)
    return KDA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(o, 16) ||
      !aligned(u_rec, 16) || !aligned(kg_rec, 16))
    return KDA_ERR_INVALID_ARG;
  if (!grid_fits(up8((int64_t)n_req * H), 512)) return KDA_ERR_UNSUPPORTED;
  kda::VerifyArgs a{q, k, v, g, b, o, in_dtype, n_req, L, H, d_k, pool_desc(pool), ckpt_slot,
                    u_rec, kg_rec, dev_err, flags};
  return launched(kda::launch_verify(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_commit(kda_pool pool, const int32_t* ckpt_slot, const int32_t* dst_slot,
                      const int32_t* accepted_len, const float* u_rec, const void* kg_rec,
                      int32_t rec_dtype, int32_t n_req, int32_t L, int32_t H, int32_t d_k,
                      int32_t d_v, int32_t* dev_err, void* stream) {
  if (n_req < 0 || H <= 0 || L < 1) return KDA_ERR_INVALID_ARG;
  if (L > 256) return KDA_ERR_UNSUPPORTED;
  if (!dtype_ok(rec_dtype)) return KDA_ERR_UNSUPPORTED;
  if (d_k != 128 || d_v != 128) return KDA_ERR_UNSUPPORTED;
  kda_status ps = check_pool(pool, H, d_k, d_v);
  if (ps != KDA_OK) return ps;
  if (n_req == 0) return KDA_OK;
  if (ckpt_slot == nullptr || accepted_len == nullptr || u_rec == nullptr || kg_rec == nullptr)
    return KDA_ERR_INVALID_ARG;
  if (!grid_fits((int64_t)n_req * H, 256)) return KDA_ERR_UNSUPPORTED;
  kda::CommitArgs a{pool_desc(pool), ckpt_slot, dst_slot, accepted_len, u_rec, kg_rec, rec_dtype,
                    n_req, L, H, d_k, dev_err};
  return launched(kda::launch_commit(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_commit_align(kda_pool pool, const int32_t* block_table, int32_t blocks_per_req,
                            const int32_t* num_tokens, const int32_t* accepted_len,
                            int32_t block_size, const float* u_rec, const void* kg_rec,
                            int32_t rec_dtype, int32_t n_req, int32_t L, int32_t H, int32_t d_k,
                            int32_t d_v, kda_align_next next, int32_t* dev_err, void* stream) {
  if (n_req < 0 || H <= 0 || L < 1 || blocks_per_req < 1) return KDA_ERR_INVALID_ARG;
  if (L > 256) return KDA_ERR_UNSUPPORTED;
  if (block_size <= L) return KDA_ERR_INVALID_ARG;   // a window would close more than one block
  if (!dtype_ok(rec_dtype)) return KDA_ERR_UNSUPPORTED;
  if (d_k != 128 || d_v != 128) return KDA_ERR_UNSUPPORTED;
  kda_status ps = check_pool(pool, H, d_k, d_v);
  if (ps != KDA_OK) return ps;
  if (n_req == 0) return KDA_OK;
  if (block_table == nullptr || num_tokens == nullptr || accepted_len == nullptr || u_rec == nullptr ||
      kg_rec == nullptr)
    return KDA_ERR_INVALID_ARG;
  if (!grid_fits((int64_t)n_req * H, 256)) return KDA_ERR_UNSUPPORTED;
  kda::CommitAlignArgs a{pool_desc(pool), block_table, blocks_per_req, num_tokens, accepted_len, block_size,
                         u_rec, kg_rec, rec_dtype, n_req, L, H, d_k, next.num_tokens, next.block,
                         next.ckpt_slot, next.copy_bias, dev_err};
  return launched(kda::launch_commit_align(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_state_copy(kda_pool pool, const int32_t* src_slot, const int32_t* dst_slot,
                          int32_t n_pairs, int32_t* dev_err, void* stream) {
  if (n_pairs < 0) return KDA_ERR_INVALID_ARG;
  if (pool.base == nullptr || pool.n_slots <= 0 || pool.H <= 0 || pool.d_k <= 0 || pool.d_v <= 0)
    return KDA_ERR_INVALID_ARG;
  if (!dtype_ok(pool.dtype)) return KDA_ERR_UNSUPPORTED;
  const int64_t slot_bytes = (int64_t)pool.H * pool.d_k * pool.d_v * (int64_t)dtype_size(pool.dtype);
  if (slot_bytes % 16 != 0) return KDA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(pool.base) & 15u) != 0) return KDA_ERR_INVALID_ARG;
  if (n_pairs == 0) return KDA_OK;
  if (src_slot == nullptr || dst_slot == nullptr) return KDA_ERR_INVALID_ARG;
  const int64_t bpp = (slot_bytes + 16383) / 16384;
  if (!grid_fits(bpp * n_pairs, 256)) return KDA_ERR_UNSUPPORTED;
  kda::CopyArgs a{pool_desc(pool), src_slot, dst_slot, n_pairs, slot_bytes, dev_err};
  return launched(kda::launch_copy(a, static_cast<hipStream_t>(stream)));
}

static_assert(KDA_MAX_CONV_TENSORS == kda::kMaxConvTensors, "conv tensor limit");
static_assert(KDA_NOALLOC_SCRATCH_BYTES == kda::kNoallocScratchBytes, "static scratch size");

kda_status kda_conv_state_update(const kda_conv_tensor* tensors, int32_t n_tensors,
                                 const int32_t* dst_slot, const int32_t* src_slot,
                                 const int32_t* shift, int32_t n_ops, int32_t* dev_err,
                                 void* stream) {
  if (n_ops < 0 || tensors == nullptr || n_tensors < 1 || n_tensors > KDA_MAX_CONV_TENSORS)
    return KDA_ERR_INVALID_ARG;
  kda::ConvArgs a{};
  a.set.n = n_tensors;
  a.set.min_slots = INT64_MAX;
  a.set.max_shift = INT32_MAX;
  for (int i = 0; i < n_tensors; ++i) {
    const kda_conv_tensor& t = tensors[i];
    if (t.base == nullptr || (reinterpret_cast<uintptr_t>(t.base) & 15u) != 0 || t.n_slots <= 0 ||
        t.rows < 1 || t.keep < 1 || t.keep > t.rows || t.dim < 1)
      return KDA_ERR_INVALID_ARG;
    if (t.elem_bytes != 2 && t.elem_bytes != 4) return KDA_ERR_UNSUPPORTED;
    const int64_t row_bytes = (int64_t)t.dim * t.elem_bytes;
    if (row_bytes % 16 != 0 || row_bytes * t.rows > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (t.slot_stride % 16 != 0 || t.slot_stride < row_bytes * t.rows) return KDA_ERR_INVALID_ARG;
    a.set.t[i] = kda::ConvDesc{static_cast<uint8_t*>(t.base), t.slot_stride, t.n_slots, t.rows, t.keep,
                               t.dim, t.elem_bytes};
    a.set.min_slots = std::min<int64_t>(a.set.min_slots, t.n_slots);
    a.set.max_shift = std::min(a.set.max_shift, t.rows - t.keep);
  }
  if (n_ops == 0) return KDA_OK;
  if (dst_slot == nullptr || src_slot == nullptr || shift == nullptr) return KDA_ERR_INVALID_ARG;
  if (!grid_fits((int64_t)n_ops * n_tensors, 256)) return KDA_ERR_UNSUPPORTED;
  a.dst_slot = dst_slot;
  a.src_slot = src_slot;
  a.shift = shift;
  a.n_ops = n_ops;
  a.dev_err = dev_err;
  return launched(kda::launch_conv_update(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
