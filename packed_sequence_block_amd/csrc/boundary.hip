// Document-id and segment-boundary kernels.
//
// glm5_next.cp page, API entries doc_ids_from_cu_seqlens (cumulative document
// boundaries -> ids [1, sequence]) and segment_cu_seqlens (boundaries of the
// runs of equal ids that cover the whole row).  Both are O(S) integer passes
// bound by launch latency at the sizes packed training uses (S <= 64K): the
// designs below aim at few launches and coalesced int4 traffic, not at FLOPs.
#include "psb_internal.h"

namespace psb {
namespace {

// ---- doc_ids_from_cu_seqlens ---------------------------------------------------
// One thread per position: the position's document is the last boundary
// cu[i] <= p (binary search over the n_docs + 1 boundaries), provided p < cu[n_docs].
// Each workgroup first copies the boundaries into LDS (when they fit), so the
// search costs one global load latency instead of one per search step.
// Threads below n_docs also check that the boundaries are non-decreasing.
constexpr int kCuLds = 4096;

__global__ void __launch_bounds__(256) doc_ids_kernel(const int32_t* __restrict__ cu, int32_t n_docs,
                                                      int32_t seq_len, int32_t* __restrict__ ids,
                                                      int32_t* __restrict__ status) {
  __shared__ int32_t scu[kCuLds];
  const int32_t p = blockIdx.x * blockDim.x + threadIdx.x;
  if (status != nullptr) {
    int32_t bits = 0;
    if (p < n_docs && cu[p + 1] < cu[p]) bits |= PSB_DATA_CU_NOT_MONOTONE;
    if (p == 0 && (cu[0] < 0 || cu[n_docs] > seq_len)) bits |= PSB_DATA_CU_OUT_OF_RANGE;
    if (bits) atomicOr(status, bits);
  }
  int32_t i;
  if (n_docs + 1 <= kCuLds) {  // uniform over the grid
    for (int32_t j = threadIdx.x; j <= n_docs; j += blockDim.x) scu[j] = cu[j];
    __syncthreads();
    if (p >= seq_len) return;
    i = last_le(scu, n_docs + 1, p);
  } else {
    if (p >= seq_len) return;
    i = last_le(cu, n_docs + 1, p);
  }
  ids[p] = (i >= 0 && i < n_docs) ? i + 1 : PSB_PAD_DOC_ID;
}

// ---- segment_cu_seqlens -----------------------------------------------------------
// A single workgroup walks the row in chunks of kSegThreads * kSegItems positions.
// Each thread flags the run starts among its kSegItems consecutive positions,
// a workgroup-wide exclusive scan of the per-thread counts gives each thread its
// output slot, and the running total carries across chunks.
constexpr int kSegThreads = 1024;
constexpr int kSegItems = 16;

__global__ void __launch_bounds__(kSegThreads) segment_kernel(const int32_t* __restrict__ ids,
                                                              int32_t seq_len,
                                                              int32_t* __restrict__ cu_out,
                                                              int32_t* __restrict__ n_out) {
  __shared__ int32_t wave_tot[kSegThreads / kWave];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid % kWave, wid = tid / kWave;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < seq_len; base += (int64_t)kSegThreads * kSegItems) {
    const int64_t p0 = base + (int64_t)tid * kSegItems;
    int32_t v[kSegItems];
    if (p0 + kSegItems <= seq_len && (reinterpret_cast<uintptr_t>(ids + p0) % 16) == 0) {
      const int4* src = reinterpret_cast<const int4*>(ids + p0);
#pragma unroll
      for (int j = 0; j < kSegItems / 4; ++j) {
        const int4 t = src[j];
        v[4 * j] = t.x; v[4 * j + 1] = t.y; v[4 * j + 2] = t.z; v[4 * j + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSegItems; ++j) v[j] = (p0 + j < seq_len) ? ids[p0 + j] : 0;
    }
    const int32_t prev = (p0 > 0 && p0 < seq_len) ? ids[p0 - 1] : 0;
    uint32_t flags = 0;
#pragma unroll
    for (int j = 0; j < kSegItems; ++j) {
      const int64_t p = p0 + j;
      const int32_t before = (j == 0) ? prev : v[j - 1];
      if (p > 0 && p < seq_len && v[j] != before) flags |= 1u << j;
    }
    const int32_t cnt = __popc(flags);
    // inclusive scan of cnt across the wave
    int32_t inc = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t t = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += t;
    }
    if (lane == kWave - 1) wave_tot[wid] = inc;
    __syncthreads();
    int32_t wave_off = 0, chunk_tot = 0;
    for (int w = 0; w < kSegThreads / kWave; ++w) {
      const int32_t t = wave_tot[w];
      wave_off += (w < wid) ? t : 0;
      chunk_tot += t;
    }
    int32_t slot = carry + wave_off + inc - cnt + 1;  // +1: cu_out[0] is the leading 0
    while (flags) {
      const int j = __ffs(flags) - 1;
      flags &= flags - 1;
      cu_out[slot++] = (int32_t)(p0 + j);
    }
    __syncthreads();  // everyone has read carry and wave_tot
    if (tid == 0) carry += chunk_tot;
    __syncthreads();
  }
  if (tid == 0) {
    cu_out[0] = 0;
    if (seq_len > 0) {
      cu_out[carry + 1] = seq_len;
      *n_out = carry + 1;
    } else {
      *n_out = 0;
    }
  }
}

// ---- contiguity check ------------------------------------------------------------
// One wave per (row, position).  A wave whose position starts a non-padding run
// scans every earlier position of the row for the same id; finding one means the
// id occurs in two separate runs.  Cost is (number of runs) x S / 64 wave steps.
__global__ void __launch_bounds__(256) contiguity_kernel(const int32_t* __restrict__ ids, int64_t B,
                                                         int32_t S, int64_t row_stride,
                                                         int32_t* __restrict__ status) {
  const int64_t wave_global = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (wave_global >= B * S) return;  // tail waves of the last workgroup
  const int64_t b = wave_global / S;
  const int32_t p = (int32_t)(wave_global % S);
  const int32_t* row = ids + b * row_stride;
  const int32_t x = row[p];
  if (x == PSB_PAD_DOC_ID || (p > 0 && row[p - 1] == x)) return;
  bool dup = false;
  for (int32_t base = 0; base < p; base += kWave) {
    const int32_t j = base + lane;
    if (j < p && row[j] == x) dup = true;
  }
  if (__any(dup) && lane == 0) atomicOr(status, PSB_DATA_DOC_NOT_CONTIGUOUS);
}

// ---- doc_ids_from_seq_lens / unpack_row_layout -------------------------------------
// Grid (position chunks, rows).  Each workgroup copies its row's length table into
// LDS (at most kCuLds entries), turns it into boundaries with a workgroup scan (a
// negative entry ends the list), then maps its positions like doc_ids_kernel.
constexpr int kLensThreads = 256;

// Boundaries of one row's length table: scu[0..n] = 0, l0, l0 + l1, ... (capped at
// INT32_MAX), where n is the index of the first negative entry (n_docs if none).
// Every thread of the workgroup must call it; returns n.
__device__ int32_t lens_to_bounds(const int32_t* __restrict__ row, int32_t n_docs, int32_t* scu,
                                  int32_t* wtot, int32_t* s_n) {
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  if (tid == 0) *s_n = n_docs;
  __syncthreads();
  constexpr int kPer = kCuLds / kLensThreads;
  int32_t v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int32_t i = tid * kPer + j;
    v[j] = (i < n_docs) ? row[i] : -1;
    if (i < n_docs && v[j] < 0) atomicMin(s_n, i);
  }
  __syncthreads();
  const int32_t n = *s_n;
  int64_t loc = 0;  // sums of up to 4096 int32 lengths fit in int64; capped below
#pragma unroll
  for (int j = 0; j < kPer; ++j) loc += (tid * kPer + j < n) ? v[j] : 0;
  int64_t inc = loc;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t t = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += t;
  }
  if (lane == kWave - 1) wtot[wv] = (int32_t)min(inc, (int64_t)INT32_MAX);
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < wv; ++w) base += wtot[w];
  int64_t run = base + inc - loc;  // exclusive prefix of this thread's first entry
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int32_t i = tid * kPer + j;
    if (i < n) {
      scu[i] = (int32_t)min(run, (int64_t)INT32_MAX);
      run += v[j];
    }
    if (i == n - 1) scu[n] = (int32_t)min(run, (int64_t)INT32_MAX);
  }
  if (tid == 0 && n == 0) scu[0] = 0;
  __syncthreads();
  return n;
}

__global__ void __launch_bounds__(kLensThreads) doc_ids_lens_kernel(const int32_t* __restrict__ lens,
                                                                     int32_t n_docs, int32_t seq_len,
                                                                     int32_t pad_value, int32_t* __restrict__ ids,
                                                                     int32_t* __restrict__ status) {
  __shared__ int32_t scu[kCuLds + 1];
  __shared__ int32_t wtot[kLensThreads / kWave];
  __shared__ int32_t s_n;
  const int32_t b = blockIdx.y;
  const int32_t n = lens_to_bounds(lens + (int64_t)b * n_docs, n_docs, scu, wtot, &s_n);
  if (blockIdx.x == 0 && threadIdx.x == 0 && status != nullptr && scu[n] > seq_len)
    atomicOr(status, PSB_DATA_LENS_EXCEED_SEQ);
  const int32_t p = blockIdx.x * kLensThreads + threadIdx.x;
  if (p >= seq_len) return;
  const int32_t i = last_le(scu, n + 1, p);
  ids[(int64_t)b * seq_len + p] = (i >= 0 && i < n) ? i + 1 : pad_value;
}

// unpack_row_layout: the padded lengths place the documents (boundaries as above);
// inside document i the first real[i] positions are tokens at positions 0, 1, ...,
// the rest of its block and everything past the last block are padding (mask 1,
// position 0).  Workgroup (0, b) also checks 0 <= real[i] <= padded[i].
__global__ void __launch_bounds__(kLensThreads) unpack_kernel(const int32_t* __restrict__ real,
                                                               const int32_t* __restrict__ padded, int32_t n_docs,
                                                               int32_t seq_len, uint8_t* __restrict__ mask,
                                                               int32_t* __restrict__ pos,
                                                               int32_t* __restrict__ status) {
  __shared__ int32_t scu[kCuLds + 1];
  __shared__ int32_t sreal[kCuLds];
  __shared__ int32_t wtot[kLensThreads / kWave];
  __shared__ int32_t s_n;
  const int32_t b = blockIdx.y;
  const int32_t* rrow = real + (int64_t)b * n_docs;
  const int32_t n = lens_to_bounds(padded + (int64_t)b * n_docs, n_docs, scu, wtot, &s_n);
  bool bad = false;
  for (int32_t i = threadIdx.x; i < n; i += kLensThreads) {
    const int32_t r = rrow[i];
    sreal[i] = r;
    bad |= r < 0 || r > scu[i + 1] - scu[i];
  }
  __syncthreads();
  if (status != nullptr && blockIdx.x == 0) {
    if (__any(bad) && (threadIdx.x % kWave) == 0) atomicOr(status, PSB_DATA_BAD_LENGTHS);
    if (threadIdx.x == 0 && scu[n] > seq_len) atomicOr(status, PSB_DATA_LENS_EXCEED_SEQ);
  }
  const int32_t p = blockIdx.x * kLensThreads + threadIdx.x;
  if (p >= seq_len) return;
  const int32_t i = last_le(scu, n + 1, p);
  const int32_t off = p - (i >= 0 ? scu[i] : 0);
  const bool tok = i >= 0 && i < n && off < sreal[i];
  mask[(int64_t)b * seq_len + p] = tok ? 0 : 1;
  pos[(int64_t)b * seq_len + p] = tok ? off : 0;
}

// ---- document positions ------------------------------------------------------------
// One workgroup per row.  Pass 1 finds the first kept token; pass 2 checks every kept
// token against its predecessor (the rule of document_positions_valid in the oracle:
// first kept >= 0; after a kept token previous + 1 or 0; after a dropped one 0).
constexpr int kPosThreads = 1024;

__global__ void __launch_bounds__(kPosThreads) positions_kernel(const uint8_t* __restrict__ keep,
                                                                 const int32_t* __restrict__ pos, int32_t S,
                                                                 int32_t* __restrict__ status) {
  __shared__ int32_t s_first;
  const int32_t b = blockIdx.x;
  const uint8_t* krow = keep + (int64_t)b * S;
  const int32_t* prow = pos + (int64_t)b * S;
  if (threadIdx.x == 0) s_first = INT32_MAX;
  __syncthreads();
  for (int32_t p = threadIdx.x; p < S; p += kPosThreads)
    if (krow[p]) { atomicMin(&s_first, p); break; }
  __syncthreads();
  const int32_t first = s_first;
  bool bad = false;
  for (int32_t p = threadIdx.x; p < S; p += kPosThreads) {
    if (!krow[p]) continue;
    const int32_t x = prow[p];
    if (p == first) bad |= x < 0;
    else if (krow[p - 1]) bad |= !(x == 0 || x == prow[p - 1] + 1);
    else bad |= x != 0;
  }
  if (__any(bad) && (threadIdx.x % kWave) == 0) atomicOr(status, PSB_DATA_BAD_POSITIONS);
}

// ---- dense per-document causal mask ----------------------------------------------------
// One thread per 4 mask bytes: row i of the shard (global position seq_start + i) may
// see key k iff doc[k] == doc[q], doc[q] is not padding and k <= q.  Bytes past S in a
// padded row are written 0.
__global__ void __launch_bounds__(256) dense_mask_kernel(const int32_t* __restrict__ doc_ids, int32_t S,
                                                         int32_t seq_start, int32_t L, int64_t words_per_row,
                                                         int64_t total_words, uint32_t* __restrict__ mask) {
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= total_words) return;
  const int64_t row = w / words_per_row;            // b * L + i
  const int32_t c = (int32_t)(w - row * words_per_row);
  const int32_t b = (int32_t)(row / L), i = (int32_t)(row - (int64_t)b * L);
  const int32_t* doc = doc_ids + (int64_t)b * S;
  const int32_t qpos = seq_start + i;
  const int32_t dq = doc[qpos];
  uint32_t x = 0u;
  if (dq != PSB_PAD_DOC_ID) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int32_t key = 4 * c + t;
      if (key < S && key <= qpos && doc[key] == dq) x |= 1u << (8 * t);
    }
  }
  mask[w] = x;
}

}  // namespace
}  // namespace psb

using namespace psb;

PSB_API psb_status psb_doc_ids_from_cu_seqlens(const int32_t* cu_seqlens, int64_t n_docs, int64_t seq_len,
                                               int32_t* doc_ids_out, int32_t* status_word, void* stream) {
  if (cu_seqlens == nullptr || n_docs < 0 || seq_len < 0) return PSB_ERR_INVALID_ARG;
  if (seq_len > 0 && doc_ids_out == nullptr) return PSB_ERR_INVALID_ARG;
  if (n_docs >= INT32_MAX || seq_len >= INT32_MAX) return PSB_ERR_SHAPE;
  const int64_t work = seq_len > n_docs + 1 ? seq_len : n_docs + 1;
  const int threads = 256;
  const int64_t blocks = ceil_div(work, threads);
  doc_ids_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, as_stream(stream)>>>(
      cu_seqlens, (int32_t)n_docs, (int32_t)seq_len, doc_ids_out, status_word);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

PSB_API psb_status psb_segment_cu_seqlens(const int32_t* doc_ids_row, int64_t seq_len, int32_t* cu_out,
                                          int64_t cu_capacity, int32_t* n_segments_out, void* stream) {
  if (seq_len < 0 || cu_out == nullptr || n_segments_out == nullptr) return PSB_ERR_INVALID_ARG;
  if (seq_len > 0 && doc_ids_row == nullptr) return PSB_ERR_INVALID_ARG;
  if (seq_len >= INT32_MAX) return PSB_ERR_SHAPE;
  if (cu_capacity < seq_len + 1) return PSB_ERR_CAPACITY;
  segment_kernel<<<dim3(1), dim3(kSegThreads), 0, as_stream(stream)>>>(doc_ids_row, (int32_t)seq_len,
                                                                         cu_out, n_segments_out);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

namespace psb {

psb_status launch_contiguity_check(const int32_t* doc_ids, int64_t B, int64_t S, int64_t row_stride,
                                   int32_t* status_word, hipStream_t stream) {
  if (B == 0 || S == 0) return PSB_OK;
  if (doc_ids == nullptr || status_word == nullptr) return PSB_ERR_INVALID_ARG;
  if (row_stride < S || S >= INT32_MAX) return PSB_ERR_SHAPE;
  const int64_t waves = B * S;
  const int64_t blocks = ceil_div(waves, 256 / kWave);
  if (blocks >= INT32_MAX) return PSB_ERR_SHAPE;
  contiguity_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(doc_ids, B, (int32_t)S, row_stride,
                                                                      status_word);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

}  // namespace psb

PSB_API psb_status psb_validate_doc_ids(const int32_t* doc_ids, int64_t B, int64_t S, int64_t row_stride,
                                        int32_t* status_word, void* stream) {
  if (B < 0 || S < 0 || status_word == nullptr) return PSB_ERR_INVALID_ARG;
  return launch_contiguity_check(doc_ids, B, S, row_stride, status_word, as_stream(stream));
}

PSB_API psb_status psb_doc_ids_from_seq_lens(const int32_t* seq_lens, int64_t B, int64_t n_docs, int64_t seq_len,
                                             int32_t padding_value, int32_t* doc_ids_out, int32_t* status_word,
                                             void* stream) {
  if (B < 0 || n_docs < 0 || seq_len < 0) return PSB_ERR_INVALID_ARG;
  if (B == 0 || seq_len == 0) return PSB_OK;
  if (doc_ids_out == nullptr || (n_docs > 0 && seq_lens == nullptr)) return PSB_ERR_INVALID_ARG;
  if (seq_len >= INT32_MAX || B > 65535) return PSB_ERR_SHAPE;
  if (n_docs > kCuLds) return PSB_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)ceil_div(seq_len, kLensThreads), (unsigned)B);
  doc_ids_lens_kernel<<<grid, dim3(kLensThreads), 0, as_stream(stream)>>>(
      seq_lens, (int32_t)n_docs, (int32_t)seq_len, padding_value, doc_ids_out, status_word);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

PSB_API psb_status psb_validate_document_positions(const uint8_t* keep, const int32_t* positions, int64_t B,
                                                   int64_t S, int32_t* status_word, void* stream) {
  if (B < 0 || S < 0 || status_word == nullptr) return PSB_ERR_INVALID_ARG;
  if (B == 0 || S == 0) return PSB_OK;
  if (keep == nullptr || positions == nullptr) return PSB_ERR_INVALID_ARG;
  if (S >= INT32_MAX || B >= INT32_MAX) return PSB_ERR_SHAPE;
  positions_kernel<<<dim3((unsigned)B), dim3(kPosThreads), 0, as_stream(stream)>>>(keep, positions, (int32_t)S,
                                                                                 status_word);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

PSB_API psb_status psb_unpack_row_layout(const int32_t* seq_lens, const int32_t* seq_lens_padded, int64_t B,
                                         int64_t n_docs, int64_t seq_len, uint8_t* padding_mask_out,
                                         int32_t* position_ids_out, int32_t* status_word, void* stream) {
  if (B < 0 || n_docs < 0 || seq_len < 0) return PSB_ERR_INVALID_ARG;
  if (B == 0 || seq_len == 0) return PSB_OK;
  if (padding_mask_out == nullptr || position_ids_out == nullptr) return PSB_ERR_INVALID_ARG;
  if (n_docs > 0 && (seq_lens == nullptr || seq_lens_padded == nullptr)) return PSB_ERR_INVALID_ARG;
  if (seq_len >= INT32_MAX || B > 65535) return PSB_ERR_SHAPE;
  if (n_docs > kCuLds) return PSB_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)ceil_div(seq_len, kLensThreads), (unsigned)B);
  unpack_kernel<<<grid, dim3(kLensThreads), 0, as_stream(stream)>>>(seq_lens, seq_lens_padded, (int32_t)n_docs,
                                                                     (int32_t)seq_len, padding_mask_out,
                                                                     position_ids_out, status_word);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

PSB_API psb_status psb_blockdiag_dense_mask(const int32_t* doc_ids, int64_t B, int64_t S, int64_t seq_start,
                                            int64_t L, uint8_t* mask_out, int64_t row_stride, void* stream) {
  if (B < 0 || S < 0 || L < 0 || seq_start < 0) return PSB_ERR_INVALID_ARG;
  if (seq_start + L > S || S >= INT32_MAX || L >= INT32_MAX) return PSB_ERR_SHAPE;
  if (row_stride < S || (row_stride % 4) != 0) return PSB_ERR_SHAPE;
  if (B == 0 || L == 0 || row_stride == 0) return PSB_OK;
  if (doc_ids == nullptr || mask_out == nullptr || (reinterpret_cast<uintptr_t>(mask_out) & 3u) != 0)
    return PSB_ERR_INVALID_ARG;
  const int64_t wpr = row_stride / 4;
  const int64_t total = B * L * wpr;
  const int64_t blocks = ceil_div(total, 256);
  if (blocks >= INT32_MAX) return PSB_ERR_SHAPE;
  dense_mask_kernel<<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(
      doc_ids, (int32_t)S, (int32_t)seq_start, (int32_t)L, wpr, total, reinterpret_cast<uint32_t*>(mask_out));
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}
