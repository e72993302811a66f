// Host-side argument validation of every libpsb entry point, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_capi_sanitized.py builds and runs
// it on the CPU).  Every call here must return its error before anything is enqueued: the
// device pointers are fake, aligned addresses that no host code may dereference, and no GPU
// is needed.  Exit status 0 when every status code matches.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "psb.h"

static int failures = 0;

#define EXPECT(call, code)                                                                  \
  do {                                                                                      \
    const psb_status got_ = (call);                                                         \
    if (got_ != (code)) {                                                                   \
      fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (code)); \
      ++failures;                                                                           \
    }                                                                                       \
  } while (0)

int main() {
  void* F = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned, never dereferenced
  void* U = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);  // misaligned
  int32_t* Fi = static_cast<int32_t*>(F);
  float* Ff = static_cast<float*>(F);
  uint8_t* Fb = static_cast<uint8_t*>(F);
  const float nan_ = nanf("");

  // status strings: every code has a message, unknown codes too
  for (int c = -8; c <= 1; ++c) {
    const char* s = psb_status_string(c);
    if (s == nullptr || strlen(s) == 0) ++failures;
  }
  if (psb_version() < 100) ++failures;

  // boundaries
  EXPECT(psb_doc_ids_from_cu_seqlens(nullptr, 3, 10, Fi, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_doc_ids_from_cu_seqlens(Fi, -1, 10, Fi, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_doc_ids_from_cu_seqlens(Fi, 3, -5, Fi, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_doc_ids_from_cu_seqlens(Fi, 3, 10, nullptr, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_segment_cu_seqlens(Fi, 100, Fi, 100, Fi, nullptr), PSB_ERR_CAPACITY);
  EXPECT(psb_segment_cu_seqlens(Fi, -1, Fi, 100, Fi, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_segment_cu_seqlens(Fi, 10, nullptr, 11, Fi, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_segment_cu_seqlens(Fi, 10, Fi, 11, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_validate_doc_ids(Fi, 1, 10, 10, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_validate_doc_ids(Fi, 1, 10, 5, Fi, nullptr), PSB_ERR_SHAPE);
  EXPECT(psb_validate_doc_ids(nullptr, 0, 10, 10, Fi, nullptr), PSB_OK);
  EXPECT(psb_doc_ids_from_seq_lens(Fi, 1, 5000, 10, -1000, Fi, nullptr, nullptr), PSB_ERR_UNSUPPORTED);
  EXPECT(psb_doc_ids_from_seq_lens(Fi, 70000, 5, 10, -1000, Fi, nullptr, nullptr), PSB_ERR_SHAPE);
  EXPECT(psb_doc_ids_from_seq_lens(Fi, -1, 5, 10, -1000, Fi, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_unpack_row_layout(Fi, Fi, 1, 5000, 10, Fb, Fi, nullptr, nullptr), PSB_ERR_UNSUPPORTED);
  EXPECT(psb_unpack_row_layout(Fi, Fi, -1, 5, 10, Fb, Fi, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_validate_document_positions(Fb, Fi, 1, 10, nullptr, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_shard_kv_window_start(Fi, 1, 10, 5, 6, Fi, nullptr), PSB_ERR_SHAPE);
  EXPECT(psb_shard_kv_window_start(Fi, 1, 10, -1, 6, Fi, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_blockdiag_dense_mask(Fi, 1, 10, 0, 10, Fb, 6, nullptr), PSB_ERR_SHAPE);

  // forward: shapes, scale, pointers, strides, workspace
  const size_t ws = psb_blockdiag_attn_fwd_workspace_size(1, 4, 2, 64, 128);
  if (ws == 0 || psb_blockdiag_attn_fwd_workspace_size(0, 0, 0, 0, 64) == 0) ++failures;
  auto fwd = [&](int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D, int64_t s0, float sc,
                 int32_t gqa, void* q, void* out, void* w, size_t wb, const int64_t* qs) {
    return psb_blockdiag_attn_fwd(q, F, F, Fi, B, Hq, Hkv, L, S, D, qs, nullptr, s0, sc, gqa, out, w, wb, nullptr,
                                  nullptr);
  };
  EXPECT(fwd(1, 4, 2, 64, 64, 96, 0, 0.1f, 1, F, F, F, ws, nullptr), PSB_ERR_UNSUPPORTED);
  EXPECT(fwd(1, 6, 4, 64, 64, 128, 0, 0.1f, 1, F, F, F, ws, nullptr), PSB_ERR_SHAPE);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, 0.1f, 0, F, F, F, ws, nullptr), PSB_ERR_SHAPE);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 1, 0.1f, 1, F, F, F, ws, nullptr), PSB_ERR_SHAPE);
  EXPECT(fwd(-1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, F, F, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, nan_, 1, F, F, F, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, INFINITY, 1, F, F, F, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, 0.1f, 1, nullptr, F, F, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, U, F, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, F, nullptr, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, F, F, 16, nullptr), PSB_ERR_CAPACITY);
  const int64_t bad_qs[3] = {64 * 128 * 4, 64 * 128, 100};
  EXPECT(fwd(1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, F, F, ws, bad_qs), PSB_ERR_SHAPE);
  EXPECT(fwd(0, 4, 2, 64, 64, 128, 0, 0.1f, 1, nullptr, nullptr, nullptr, 0, nullptr), PSB_OK);
  EXPECT(psb_blockdiag_attn_plan(Fi, 1, 4, 2, 64, 64, 128, 0, 1, F, 16, nullptr), PSB_ERR_CAPACITY);
  EXPECT(psb_blockdiag_attn_plan(nullptr, 1, 4, 2, 64, 64, 128, 0, 1, F, ws, nullptr), PSB_ERR_INVALID_ARG);
  EXPECT(psb_blockdiag_attn_fwd_planned(F, F, F, Fi, 1, 4, 2, 64, 64, 128, nullptr, nullptr, 0, nan_, 1, F, F, ws,
                                        nullptr, nullptr),
         PSB_ERR_INVALID_ARG);
  EXPECT(psb_blockdiag_attn_fwd_lse_planned(F, F, F, Fi, 1, 4, 2, 64, 64, 128, nullptr, nullptr, 0, 0.1f, 1, F,
                                            nullptr, F, ws, nullptr, nullptr),
         PSB_ERR_INVALID_ARG);
  EXPECT(psb_blockdiag_attn_fwd_window_planned(F, F, F, Fi, 1, 4, 2, 32, 64, 128, nullptr, nullptr, 16, 20, 44, 0.1f,
                                               1, F, nullptr, F, ws, nullptr, nullptr),
         PSB_ERR_SHAPE);  // the window starts after the shard
  EXPECT(psb_blockdiag_prepare(Fi, 4, 3, 1, 4, 2, 64, 64, 128, 0, 1, Fi, Fi, Fi, F, 16, nullptr, nullptr),
         PSB_ERR_CAPACITY);
  EXPECT(psb_blockdiag_prepare(Fi, 4, 3, 70000, 4, 2, 64, 64, 128, 0, 1, Fi, Fi, Fi, F, ws, nullptr, nullptr),
         PSB_ERR_SHAPE);
  EXPECT(psb_masked_attn_fwd(F, F, F, Fb, 0, 6, 1, 4, 2, 8, 10, 128, nullptr, nullptr, 0.1f, 1, F, nullptr, nullptr),
         PSB_ERR_SHAPE);  // mask rows shorter than S rounded up to 4
  EXPECT(psb_masked_attn_fwd(F, F, F, Fb + 2, 0, 12, 1, 4, 2, 8, 10, 128, nullptr, nullptr, 0.1f, 1, F, nullptr,
                             nullptr),
         PSB_ERR_INVALID_ARG);

  // no-allocation forward: a plan larger than the static array is refused before any HIP call
  const size_t cap = psb_blockdiag_attn_fwd_noalloc_max_workspace();
  int64_t B = 64;
  while (psb_blockdiag_attn_fwd_workspace_size(B, 4, 4, 65536, 64) <= cap) B *= 2;
  EXPECT(psb_blockdiag_attn_fwd_noalloc(F, F, F, Fi, B, 4, 4, 65536, 65536, 64, nullptr, nullptr, 0, 0.1f, 0, F,
                                        nullptr, nullptr),
         PSB_ERR_SCRATCH_LIMIT);
  EXPECT(psb_blockdiag_attn_fwd_noalloc(F, F, F, Fi, 1, 4, 2, 64, 64, 96, nullptr, nullptr, 0, 0.1f, 1, F, nullptr,
                                        nullptr),
         PSB_ERR_UNSUPPORTED);

  // backward
  const size_t bws = psb_blockdiag_attn_bwd_workspace_size(1, 4, 2, 64, 64, 128);
  if (bws <= ws) ++failures;
  EXPECT(psb_blockdiag_attn_bwd_planned(F, F, F, F, F, Ff, Fi, 1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, F, F, F, 16,
                                        nullptr, nullptr),
         PSB_ERR_CAPACITY);
  EXPECT(psb_blockdiag_attn_bwd_planned(F, F, F, F, F, Ff, Fi, 1, 4, 2, 64, 64, 96, 0, 0.1f, 1, F, F, F, F, bws,
                                        nullptr, nullptr),
         PSB_ERR_UNSUPPORTED);
  EXPECT(psb_blockdiag_attn_bwd_planned(F, F, F, F, F, nullptr, Fi, 1, 4, 2, 64, 64, 128, 0, 0.1f, 1, F, F, F, F,
                                        bws, nullptr, nullptr),
         PSB_ERR_INVALID_ARG);
  EXPECT(psb_blockdiag_attn_bwd_window_planned(F, F, F, F, F, Ff, Fi, 1, 4, 2, 32, 64, 128, 16, 20, 44, 0.1f, 1, F,
                                               F, F, F, bws, nullptr, nullptr),
         PSB_ERR_SHAPE);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
