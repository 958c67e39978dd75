// Internal launch interface between the C ABI layer (api.cpp) and the
// kernels.  Every launcher assumes its arguments were validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum Dt { F32 = 0, F16 = 1, BF16 = 2 };

struct PoolDesc {
  void* base;
  int64_t n_slots;
  int dtype;
};

struct PrefillArgs {
  const void *q, *k, *v, *g, *b;
  void* o;
  int in_dtype;
  const int32_t* cu_seqlens;
  int n_seqs;
  int64_t total_tokens;
  int H, dk, dv, chunk;
  PoolDesc pool;
  const int32_t *init_slot, *final_slot;
  const int32_t *track_ptr, *track_chunk, *track_slot;
  int n_track;
  float* track_f32;
  int32_t* dev_err;
  void* workspace;
  uint32_t flags;   // KDA_QK_L2NORM
};

struct VerifyArgs {
  const void *q, *k, *v, *g, *b;
  void* o;
  int in_dtype;
  int n_req, L, H, d;
  PoolDesc pool;
  const int32_t* ckpt_slot;
  float* u_rec;
  void* kg_rec;
  int32_t* dev_err;
  uint32_t flags;   // KDA_QK_L2NORM
};

struct CommitArgs {
  PoolDesc pool;
  const int32_t *ckpt_slot, *dst_slot, *accepted_len;
  const float* u_rec;
  const void* kg_rec;
  int rec_dtype;
  int n_req, L, H, d;
  int32_t* dev_err;
};

struct CopyArgs {
  PoolDesc pool;
  const int32_t *src_slot, *dst_slot;
  int n_pairs;
  int64_t slot_bytes;
  int32_t* dev_err;
};

struct CommitAlignArgs {
  PoolDesc pool;
  const int32_t* block_table;
  int blocks_per_req;
  const int32_t *num_tokens, *accepted_len;
  int block_size;
  const float* u_rec;
  const void* kg_rec;
  int rec_dtype;
  int n_req, L, H, d;
  int32_t *next_tokens, *next_block, *next_ckpt, *next_bias;   // optional outputs [n_req]
  int32_t* dev_err;
};

// One conv tensor of a fused conv-state update: per slot `rows` positions of
// `dim` channels (position-major), the first `keep` rows the carried history.
constexpr int kMaxConvTensors = 8;
struct ConvDesc {
  uint8_t* base;
  int64_t slot_stride;   // bytes
  int64_t n_slots;
  int rows, keep, dim, elem_bytes;
};
struct ConvSet {
  ConvDesc t[kMaxConvTensors];
  int n;
  int64_t min_slots;   // smallest n_slots over the tensors
  int max_shift;       // smallest rows - keep over the tensors
};
struct ConvArgs {
  ConvSet set;
  const int32_t *dst_slot, *src_slot, *shift;
  int n_ops;
  int32_t* dev_err;
};

// Static scratch of the allocation-free prefill entry point (noalloc.hip):
// its size, and its device address on the current device (resolved once per
// device, then cached).
constexpr size_t kNoallocScratchBytes = (size_t)256 << 20;
hipError_t noalloc_scratch(void** out);

// Shape support and sizes.
bool prefill_supported(int dk, int dv, int chunk, int in_dtype, int pool_dtype);
size_t prefill_workspace_bytes(int n_seqs, int64_t total_tokens, int H, int dk, int dv,
                               int chunk, int in_dtype);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, hipStream_t s);
hipError_t launch_commit_align(const CommitAlignArgs& a, hipStream_t s);
hipError_t launch_conv_update(const ConvArgs& a, hipStream_t s);

}  // namespace kda
