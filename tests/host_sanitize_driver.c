/* Host-side checks of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure, built and run by
 * tests/test_host_sanitizers.py on the CPU).
 *
 * Every call below is rejected, or has nothing to do, before any launch:
 * the library validates host-checkable arguments first and touches no
 * device memory, so the fake device addresses are never dereferenced.
 * The driver exits non-zero when a status differs from the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;

static void expect(const char* what, kda_status got, kda_status want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, kda_status_string(got), (int)want);
    ++failures;
  }
}

int main(void) {
  void* fake = (void*)(uintptr_t)0x100000;   /* 16-byte aligned, never dereferenced */
  void* fake_ws = (void*)(uintptr_t)0x200000;
  const int32_t* fi = (const int32_t*)fake;
  kda_pool pool = {fake, 8, KDA_F32, 2, 128, 128};
  size_t ws = 0;

  /* workspace query */
  expect("workspace null out", kda_chunk_prefill_workspace(1, 64, 2, 128, 128, 64, KDA_BF16, NULL), KDA_ERR_INVALID_ARG);
  expect("workspace ok", kda_chunk_prefill_workspace(16, 135168, 32, 128, 128, 64, KDA_BF16, &ws), KDA_OK);
  if (ws == 0) { fprintf(stderr, "workspace size 0\n"); ++failures; }
  expect("workspace bad shape", kda_chunk_prefill_workspace(1, 64, 2, 32, 32, 16, KDA_BF16, &ws), KDA_ERR_UNSUPPORTED);
  expect("workspace grid beyond range", kda_chunk_prefill_workspace(1, INT32_MAX, 129, 128, 128, 64, KDA_BF16, &ws),
         KDA_ERR_UNSUPPORTED);
  expect("workspace scan grid beyond range", kda_chunk_prefill_workspace(1 << 20, 64, 256, 128, 128, 64, KDA_BF16, &ws),
         KDA_ERR_UNSUPPORTED);

  /* prefill */
#define PREFILL(q, n_seqs, dk, chunk, in_dt, flags, wsb) \
  kda_chunk_prefill(q, fake, fake, fake, fake, in_dt, fake, fi, n_seqs, 100, 2, dk, dk, chunk, pool, fi, fi, \
                    NULL, NULL, NULL, 0, NULL, flags, NULL, fake_ws, wsb, NULL)
  expect("prefill null q", PREFILL(NULL, 1, 128, 64, KDA_BF16, 0u, (size_t)1 << 40), KDA_ERR_INVALID_ARG);
  expect("prefill n_seqs < 0", PREFILL(fake, -1, 128, 64, KDA_BF16, 0u, (size_t)1 << 40), KDA_ERR_INVALID_ARG);
  expect("prefill unknown flag", PREFILL(fake, 1, 128, 64, KDA_BF16, 6u, (size_t)1 << 40), KDA_ERR_INVALID_ARG);
  expect("prefill chunk 32", PREFILL(fake, 1, 128, 32, KDA_BF16, 0u, (size_t)1 << 40), KDA_ERR_UNSUPPORTED);
  expect("prefill fp32 at d 128", PREFILL(fake, 1, 128, 64, KDA_F32, 0u, (size_t)1 << 40), KDA_ERR_UNSUPPORTED);
  expect("prefill small workspace", PREFILL(fake, 1, 128, 64, KDA_BF16, 0u, 16), KDA_ERR_WORKSPACE);
  {
    void* mis = (void*)(uintptr_t)0x100008;   /* 8-byte aligned only */
    expect("prefill misaligned v", kda_chunk_prefill(fake, fake, mis, fake, fake, KDA_BF16, fake, fi, 1, 100, 2, 128, 128,
                                                     64, pool, fi, fi, NULL, NULL, NULL, 0, NULL, 0u, NULL, fake_ws,
                                                     (size_t)1 << 40, NULL), KDA_ERR_INVALID_ARG);
    expect("prefill misaligned o", kda_chunk_prefill(fake, fake, fake, fake, fake, KDA_BF16, mis, fi, 1, 100, 2, 128, 128,
                                                     64, pool, fi, fi, NULL, NULL, NULL, 0, NULL, 0u, NULL, fake_ws,
                                                     (size_t)1 << 40, NULL), KDA_ERR_INVALID_ARG);
  }
  expect("noalloc pool H", kda_chunk_prefill_noalloc(fake, fake, fake, fake, fake, KDA_BF16, fake, fi, 2, 2 * 8229, 3,
                                                     128, 128, 64, pool, fi, fi, NULL, NULL, NULL, 0, NULL, 0u,
                                                     NULL, NULL), KDA_ERR_INVALID_ARG);   /* pool H = 2, call H = 3 */
  {
    kda_pool p32 = {fake, 8, KDA_F32, 32, 128, 128};
    expect("noalloc over the scratch", kda_chunk_prefill_noalloc(fake, fake, fake, fake, fake, KDA_BF16, fake, fi, 2,
                                                                 2 * 8229, 32, 128, 128, 64, p32, fi, fi, NULL, NULL,
                                                                 NULL, 0, NULL, 0u, NULL, NULL), KDA_ERR_WORKSPACE);
  }
  expect("noalloc nothing to do", kda_chunk_prefill_noalloc(NULL, fake, fake, fake, fake, KDA_BF16, fake, NULL, 0, 0, 2,
                                                            128, 128, 64, pool, NULL, NULL, NULL, NULL, NULL, 0, NULL,
                                                            0u, NULL, NULL), KDA_OK);
  expect("prefill nothing to do", PREFILL(NULL, 0, 128, 64, KDA_BF16, KDA_QK_L2NORM, 0), KDA_OK);
#undef PREFILL

  /* verify */
#define VERIFY(n_req, L, dk, flags, o) \
  kda_recurrent_verify(fake, fake, fake, fake, fake, KDA_BF16, o, n_req, L, 2, dk, dk, pool, fi, (float*)fake, \
                       fake, flags, NULL, NULL)
  expect("verify L 0", VERIFY(4, 0, 128, 0u, fake), KDA_ERR_INVALID_ARG);
  expect("verify L 257", VERIFY(4, 257, 128, 0u, fake), KDA_ERR_UNSUPPORTED);
  expect("verify d 64", VERIFY(4, 8, 64, 0u, fake), KDA_ERR_UNSUPPORTED);
  expect("verify unknown flag", VERIFY(4, 8, 128, 2u, fake), KDA_ERR_INVALID_ARG);
  expect("verify null o", VERIFY(4, 8, 128, 0u, NULL), KDA_ERR_INVALID_ARG);
  expect("verify nothing to do", VERIFY(0, 8, 128, KDA_QK_L2NORM, fake), KDA_OK);
#undef VERIFY

  /* commit and align commit */
  expect("commit null accepted", kda_commit(pool, fi, NULL, NULL, (const float*)fake, fake, KDA_BF16, 4, 8, 2, 128, 128, NULL, NULL), KDA_ERR_INVALID_ARG);
  expect("commit L 300", kda_commit(pool, fi, NULL, fi, (const float*)fake, fake, KDA_BF16, 4, 300, 2, 128, 128, NULL, NULL), KDA_ERR_UNSUPPORTED);
  expect("commit nothing to do", kda_commit(pool, fi, NULL, fi, (const float*)fake, fake, KDA_BF16, 0, 8, 2, 128, 128, NULL, NULL), KDA_OK);
  {
    kda_align_next nx = {(int32_t*)fake, NULL, (int32_t*)fake, NULL};
    expect("align block <= L", kda_commit_align(pool, fi, 4, fi, fi, 8, (const float*)fake, fake, KDA_BF16, 4, 8, 2, 128, 128, nx, NULL, NULL), KDA_ERR_INVALID_ARG);
    expect("align null table", kda_commit_align(pool, NULL, 4, fi, fi, 64, (const float*)fake, fake, KDA_BF16, 4, 8, 2, 128, 128, nx, NULL, NULL), KDA_ERR_INVALID_ARG);
    expect("align nothing to do", kda_commit_align(pool, fi, 4, fi, fi, 64, (const float*)fake, fake, KDA_BF16, 0, 8, 2, 128, 128, nx, NULL, NULL), KDA_OK);
  }

  /* copy */
  expect("copy n < 0", kda_state_copy(pool, fi, fi, -1, NULL, NULL), KDA_ERR_INVALID_ARG);
  expect("copy nothing to do", kda_state_copy(pool, fi, fi, 0, NULL, NULL), KDA_OK);

  /* conv state */
  kda_conv_tensor ts[9];
  for (int i = 0; i < 9; ++i) {
    kda_conv_tensor t = {fake, 11 * 128 * 2, 8, 11, 3, 128, 2};
    ts[i] = t;
  }
  expect("conv n_ops < 0", kda_conv_state_update(ts, 1, fi, fi, fi, -1, NULL, NULL), KDA_ERR_INVALID_ARG);
  expect("conv 9 tensors", kda_conv_state_update(ts, 9, fi, fi, fi, 0, NULL, NULL), KDA_ERR_INVALID_ARG);
  ts[0].keep = 0;
  expect("conv keep 0", kda_conv_state_update(ts, 1, fi, fi, fi, 0, NULL, NULL), KDA_ERR_INVALID_ARG);
  ts[0].keep = 3;
  expect("conv nothing to do", kda_conv_state_update(ts, 2, fi, fi, fi, 0, NULL, NULL), KDA_OK);

  /* status names, including an unknown code */
  for (int s = -1; s <= 5; ++s) {
    const char* name = kda_status_string((kda_status)s);
    if (name == NULL || strlen(name) == 0) { fprintf(stderr, "status %d has no name\n", s); ++failures; }
  }

  printf("host sanitizer driver: %d failure(s)\n", failures);
  return failures != 0;
}
