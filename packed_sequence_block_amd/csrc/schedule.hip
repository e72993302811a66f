// Tile scheduler for block-diagonal attention: which keys each query block needs.
//
// The mask (blockdiag_cp page, package overview and cp_blockdiag_sdpa) lets the
// query at global position q see keys [start(q), q] where start(q) is the first
// position of q's document — given that each non-padding id is one contiguous
// run of its row.  For a block of 32 consecutive query rows the union of those
// ranges is [start(first valid row), last valid row + 1): every key tile in that
// range holds at least one allowed pair unless the block straddles documents.
//
// Kernel 1 (one wave per 32-row block) computes that range.  The document start
// is found by a 64-way search: "doc[p] == doc[q]" is false before start(q) and
// true from there to q, so each step probes 64 positions and keeps the bracket
// around the first true one (3 dependent steps for S = 64K).
// Kernel 2 (one workgroup) merges NR blocks into a row tile record, and orders
// the records by descending key-range length (counting sort), so the attention
// workgroups take the longest tiles first.  When even the longest record is short next
// to the share of the work each concurrent workgroup slot gets (4 x longest x slots <=
// all tiles x head units), the tail that longest-first avoids cannot arise, and the
// records keep row order instead: consecutive workgroups then read the same documents'
// keys, which stay in L2.
#include "psb_internal.h"
#include "schedule.h"

namespace psb {
namespace {

__global__ void __launch_bounds__(256) block_range_kernel(const int32_t* __restrict__ doc_ids, int32_t S,
                                                          int32_t L, int32_t seq_start, int32_t nblk,
                                                          int32_t total_blocks, int32_t* __restrict__ blk_lo,
                                                          int32_t* __restrict__ blk_hi) {
  const int32_t wid = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (wid >= total_blocks) return;
  const int32_t b = wid / nblk, blk = wid % nblk;
  const int32_t* row = doc_ids + (int64_t)b * S;
  const int32_t r = blk * kRowsPerBlock + (lane % kRowsPerBlock);
  const bool valid = lane < kRowsPerBlock && r < L && row[seq_start + r] != PSB_PAD_DOC_ID;
  const uint64_t m = __ballot(valid);
  if (m == 0) {
    if (lane == 0) { blk_lo[wid] = 0; blk_hi[wid] = 0; }
    return;
  }
  const int32_t first = __ffsll((unsigned long long)m) - 1;
  const int32_t last = 63 - __clzll((long long)m);
  const int32_t qf = seq_start + blk * kRowsPerBlock + first;
  const int32_t x = row[qf];
  int32_t lo = 0, hi = qf;  // the document start lies in [lo, hi]; doc[hi] == x
  while (lo < hi) {
    const int32_t step = (hi - lo + kWave - 1) / kWave;
    int32_t p = lo + lane * step;
    if (p > hi) p = hi;
    const uint64_t t = __ballot(row[p] == x);
    if (t == 0) {
      // every probe lies before the start: it is beyond lane 63's probe
      lo = lo + (kWave - 1) * step + 1;
    } else {
      const int32_t i = __ffsll((unsigned long long)t) - 1;
      const int32_t pi = min(hi, lo + i * step);
      lo = (i == 0) ? lo : lo + (i - 1) * step + 1;
      hi = pi;
    }
  }
  if (lane == 0) {
    blk_lo[wid] = lo;
    blk_hi[wid] = seq_start + blk * kRowsPerBlock + last + 1;
  }
}

constexpr int kSortThreads = 1024;
constexpr int kBuckets = 2048;

__device__ inline int32_t tile_iters(int32_t lo, int32_t hi) {
  return hi > lo ? (hi - lo + kKeysPerTile - 1) / kKeysPerTile : 0;
}

__device__ inline TileRecord make_record(const int32_t* __restrict__ blk_lo, const int32_t* __restrict__ blk_hi,
                                         int32_t t, int32_t nblk, int32_t nr, int32_t ntile_row) {
  TileRecord r;
  r.b = t / ntile_row;
  r.rt = t % ntile_row;
  int32_t lo = 0x7fffffff, hi = 0;
  for (int j = 0; j < 4; ++j) {
    const int32_t blk = r.rt * nr + j;
    int32_t l = 0, h = 0;
    if (j < nr && blk < nblk) {
      l = blk_lo[r.b * nblk + blk];
      h = blk_hi[r.b * nblk + blk];
    }
    r.blk_lo[j] = l;
    r.blk_hi[j] = h;
    if (h > l) { lo = min(lo, l); hi = max(hi, h); }
  }
  r.lo = (hi == 0) ? 0 : lo;
  r.hi = hi;
  r.pad[0] = r.pad[1] = r.pad[2] = r.pad[3] = 0;
  return r;
}

// Turns the bucket counts hist[kBuckets] into exclusive offsets in DESCENDING bucket
// order (offset(bk) = sum of the counts of the buckets above bk), with one workgroup of NT
// threads; ends with a barrier.  wsum: NT / 64 ints of LDS.
template <int NT>
__device__ void bucket_offsets_desc(int32_t* hist, int32_t* wsum) {
  static_assert(kBuckets % NT == 0, "buckets split evenly over the threads");
  constexpr int PER = kBuckets / NT;  // consecutive buckets (in descending order) per thread
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int32_t c[PER];
  int32_t own = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    c[k] = hist[kBuckets - 1 - (PER * tid + k)];
    own += c[k];
  }
  int32_t inc = own;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t v = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += v;
  }
  if (lane == kWave - 1) wsum[wv] = inc;
  __syncthreads();
  int32_t run = inc - own;
  for (int w = 0; w < wv; ++w) run += wsum[w];
  __syncthreads();  // all reads of hist done before it is overwritten with offsets
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    hist[kBuckets - 1 - (PER * tid + k)] = run;
    run += c[k];
  }
  __syncthreads();
}

// Records of all B * ntile_row row tiles into work[], longest key range first: a counting
// sort over the tile count of each record's range (bucket kBuckets - 1 collects the
// rest), done by one workgroup of NT threads; or in row order when the longest record is
// short next to a workgroup slot's share (slots = workgroups the attention kernel runs at
// once, 0 = always longest first; units = head units per row tile).  hist: kBuckets ints
// of LDS, wsum: NT / 64.
template <int NT>
__device__ void order_tiles(const int32_t* blk_lo, const int32_t* blk_hi, int32_t B, int32_t nblk, int32_t nr,
                            int32_t ntile_row, int32_t slots, int32_t units, TileRecord* __restrict__ work,
                            int32_t* hist, int32_t* wsum) {
  __shared__ unsigned long long s_total;
  __shared__ int32_t s_longest;
  const int tid = threadIdx.x;
  const int32_t T = B * ntile_row;
  for (int i = tid; i < kBuckets; i += NT) hist[i] = 0;
  if (tid == 0) { s_total = 0ull; s_longest = 0; }
  __syncthreads();
  unsigned long long total = 0ull;
  int32_t longest = 0;
  for (int32_t t = tid; t < T; t += NT) {
    const TileRecord r = make_record(blk_lo, blk_hi, t, nblk, nr, ntile_row);
    const int32_t n = tile_iters(r.lo, r.hi);
    total += (unsigned long long)n;
    longest = max(longest, n);
    atomicAdd(&hist[min(n, kBuckets - 1)], 1);
  }
  atomicAdd(&s_total, total);
  atomicMax(&s_longest, longest);
  __syncthreads();
  if (slots > 0 && 4ull * (unsigned long long)s_longest * (unsigned long long)slots <=
                       s_total * (unsigned long long)units) {  // uniform
    for (int32_t t = tid; t < T; t += NT) work[t] = make_record(blk_lo, blk_hi, t, nblk, nr, ntile_row);
    return;
  }
  bucket_offsets_desc<NT>(hist, wsum);
  for (int32_t t = tid; t < T; t += NT) {
    const TileRecord r = make_record(blk_lo, blk_hi, t, nblk, nr, ntile_row);
    const int32_t bk = min(tile_iters(r.lo, r.hi), kBuckets - 1);
    work[atomicAdd(&hist[bk], 1)] = r;
  }
}

__global__ void __launch_bounds__(kSortThreads) tile_order_kernel(const int32_t* __restrict__ blk_lo,
                                                                  const int32_t* __restrict__ blk_hi,
                                                                  int32_t B, int32_t nblk, int32_t nr,
                                                                  int32_t ntile_row, int32_t slots,
                                                                  int32_t units,
                                                                  TileRecord* __restrict__ work) {
  __shared__ int32_t hist[kBuckets];
  __shared__ int32_t wsum[kSortThreads / kWave];
  order_tiles<kSortThreads>(blk_lo, blk_hi, B, nblk, nr, ntile_row, slots, units, work, hist, wsum);
}

// ---- key side (backward dK / dV) -----------------------------------------------------
// One wave per tile of kKeyTile keys of the window [kv_start, kv_end) (tile t starts at
// kv_start + t * kKeyTile): the local query rows that see any of its keys,
// [max(first valid key, seq_start), min(end of the last valid key's document,
// seq_start + L)) - seq_start (key k is seen by the rows of its document at or after
// k; the run end is found by a 64-way search).  Empty tiles get (0, 0).
__global__ void __launch_bounds__(256) key_range_kernel(const int32_t* __restrict__ doc_ids, int32_t S, int32_t L,
                                                        int32_t seq_start, int32_t kv_start, int32_t kv_end,
                                                        int32_t nkt, int32_t total, int32_t* __restrict__ klo,
                                                        int32_t* __restrict__ khi) {
  const int32_t wid = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (wid >= total) return;
  const int32_t b = wid / nkt, kt = wid % nkt;
  const int32_t* row = doc_ids + (int64_t)b * S;
  const int32_t k0 = kv_start + kt * kKeyTile;
  static_assert(kKeyTile == 2 * kWave, "two keys per lane");
  const int32_t ka = k0 + lane, kb = k0 + kWave + lane;
  const bool va = ka < kv_end && row[ka] != PSB_PAD_DOC_ID;
  const bool vb = kb < kv_end && row[kb] != PSB_PAD_DOC_ID;
  const uint64_t ma = __ballot(va), mb = __ballot(vb);
  if ((ma | mb) == 0) {
    if (lane == 0) { klo[wid] = 0; khi[wid] = 0; }
    return;
  }
  const int32_t kf = ma ? k0 + __ffsll((unsigned long long)ma) - 1 : k0 + kWave + __ffsll((unsigned long long)mb) - 1;
  const int32_t kl = mb ? k0 + kWave + 63 - __clzll((long long)mb) : k0 + 63 - __clzll((long long)ma);
  // last position of kl's run: in [lo, hi]
  const int32_t x = row[kl];
  int32_t lo = kl, hi = S - 1;
  while (lo < hi) {
    const int32_t step = (hi - lo + kWave - 1) / kWave;
    int32_t p = lo + lane * step + 1;
    if (p > hi) p = hi;
    const uint64_t diff = __ballot(row[p] != x);
    if (diff == 0) {
      lo = min(lo + (kWave - 1) * step + 1, hi);
    } else {
      const int32_t i = __ffsll((unsigned long long)diff) - 1;
      const int32_t pi = min(hi, lo + i * step + 1);
      hi = pi - 1;
      lo = (i == 0) ? lo : lo + (i - 1) * step + 1;
    }
  }
  const int32_t r0 = max(kf, seq_start), r1 = min(lo + 1, seq_start + L);
  if (lane == 0) {
    klo[wid] = (r1 > r0) ? r0 - seq_start : 0;
    khi[wid] = (r1 > r0) ? r1 - seq_start : 0;
  }
}

// Key-side plan (one workgroup): splits key tiles whose row range is far longer than a
// workgroup slot's balanced share into row chunks and orders all records longest first.
//   * W = total rows over all tiles; a record of r rows costs r x group per workgroup and
//     there are B * nkt x Hkv workgroups' worth of records, so the chunk length is
//     Rc = max(kMinChunkRows, W * Hkv / kKeySlots rounded up to 32 rows).  kKeySlots is
//     three quarters of the concurrent slots (two workgroups on each of 256 CUs): chunks
//     somewhat longer than a slot's even share split fewer tiles (less fp32 partial
//     traffic) and leave the short records to fill the slots that finish early; 384 was
//     faster than 256, 320, 448, 512 and 768 on the packed-row and shard workloads;
//   * a tile of len > Rc rows would take n = ceil(len / Rc) chunks (at most kMaxChunks);
//     partial slots go to the tiles with the most chunks first, as long as the slot budget
//     lasts; a tile that gets none stays one record;
//   * records are counting-sorted by ceil(rows / 64), descending.
constexpr int kKeyPlanThreads = 1024;
constexpr int kKeySlots = 384;
constexpr int kMinChunkRows = 256;
constexpr int kMaxChunks = 16;

__device__ inline int32_t chunks_of(int32_t len, int32_t rc) {
  return len > rc ? min((len + rc - 1) / rc, kMaxChunks) : 1;
}

// chunk j of a tile with rows [lo, hi) in n chunks of rc rows (the last one shorter)
__device__ inline TileRecord key_record(int32_t b, int32_t kt, int32_t lo, int32_t hi, int32_t n, int32_t j,
                                        int32_t rc, int32_t slot) {
  TileRecord r;
  r.b = b;
  r.rt = kt;
  r.lo = (n > 1) ? lo + j * rc : lo;
  r.hi = (n > 1) ? min(hi, lo + (j + 1) * rc) : hi;
  r.blk_lo[0] = (slot >= 0) ? slot + j : -1;
  r.blk_lo[1] = j;
  r.blk_lo[2] = n;
  r.blk_lo[3] = 0;
  r.blk_hi[0] = r.blk_hi[1] = r.blk_hi[2] = r.blk_hi[3] = 0;
  r.pad[0] = r.pad[1] = r.pad[2] = r.pad[3] = 0;
  return r;
}

__global__ void __launch_bounds__(kKeyPlanThreads) key_plan_kernel(
    const int32_t* __restrict__ klo, const int32_t* __restrict__ khi, int32_t B, int32_t nkt, int32_t Hkv,
    int32_t max_slots, int32_t nrec, int32_t* __restrict__ tslot, TileRecord* __restrict__ work,
    int32_t* __restrict__ split, int32_t* __restrict__ split_n) {
  constexpr int NT = kKeyPlanThreads;
  __shared__ int32_t hist[kBuckets];
  __shared__ int32_t wsum[NT / kWave];
  __shared__ unsigned long long s_total;
  __shared__ int32_t s_rc, s_nsplit, s_nrec;
  __shared__ int32_t cnt[kMaxChunks + 1], take[kMaxChunks + 1], base[kMaxChunks + 1], ticket[kMaxChunks + 1];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int32_t T = B * nkt;
  if (tid == 0) { s_total = 0ull; s_nsplit = 0; s_nrec = 0; }
  if (tid <= kMaxChunks) { cnt[tid] = 0; take[tid] = 0; base[tid] = 0; ticket[tid] = 0; }
  for (int i = tid; i < kBuckets; i += NT) hist[i] = 0;
  __syncthreads();
  unsigned long long part = 0ull;
  for (int32_t t = tid; t < T; t += NT) part += (unsigned long long)max(0, khi[t] - klo[t]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) part += __shfl_xor(part, off, kWave);
  if (lane == 0) atomicAdd(&s_total, part);
  __syncthreads();
  if (tid == 0) {
    unsigned long long rc = (s_total * (unsigned long long)Hkv + kKeySlots - 1) / kKeySlots;
    rc = (rc + 31ull) / 32ull * 32ull;
    if (rc < (unsigned long long)kMinChunkRows) rc = kMinChunkRows;
    s_rc = (int32_t)min(rc, (unsigned long long)0x40000000);
  }
  __syncthreads();
  const int32_t rc = s_rc;
  for (int32_t t = tid; t < T; t += NT) {
    const int32_t n = chunks_of(max(0, khi[t] - klo[t]), rc);
    if (n >= 2) atomicAdd(&cnt[n], 1);
  }
  __syncthreads();
  if (tid == 0) {  // the slot budget, tiles with the most chunks first
    int32_t used = 0;
    for (int n = kMaxChunks; n >= 2; --n) {
      const int32_t k = min(cnt[n], (max_slots - used) / n);
      take[n] = k;
      base[n] = used;
      used += k * n;
    }
  }
  __syncthreads();
  for (int32_t t = tid; t < T; t += NT) {
    const int32_t n = chunks_of(max(0, khi[t] - klo[t]), rc);
    int32_t sl = -1;
    if (n >= 2) {
      const int32_t tk = atomicAdd(&ticket[n], 1);
      if (tk < take[n]) sl = base[n] + tk * n;
    }
    tslot[t] = sl;
    if (sl >= 0) {
      const int32_t i = atomicAdd(&s_nsplit, 1);
      split[4 * i + 0] = t / nkt;
      split[4 * i + 1] = t % nkt;
      split[4 * i + 2] = sl;
      split[4 * i + 3] = n;
    }
  }
  __syncthreads();  // tslot written by other threads of this workgroup is visible after this
  // records: histogram of lengths, descending offsets, scatter
  for (int32_t t = tid; t < T; t += NT) {
    const int32_t lo = klo[t], hi = khi[t], sl = tslot[t];
    const int32_t n = (sl >= 0) ? chunks_of(hi - lo, rc) : 1;
    for (int32_t j = 0; j < n; ++j) {
      const TileRecord r = key_record(t / nkt, t % nkt, lo, hi, n, j, rc, sl);
      atomicAdd(&hist[min(tile_iters(r.lo, r.hi), kBuckets - 1)], 1);
    }
    atomicAdd(&s_nrec, n);
  }
  __syncthreads();
  bucket_offsets_desc<NT>(hist, wsum);
  for (int32_t t = tid; t < T; t += NT) {
    const int32_t lo = klo[t], hi = khi[t], sl = tslot[t];
    const int32_t n = (sl >= 0) ? chunks_of(hi - lo, rc) : 1;
    for (int32_t j = 0; j < n; ++j) {
      const TileRecord r = key_record(t / nkt, t % nkt, lo, hi, n, j, rc, sl);
      work[atomicAdd(&hist[min(tile_iters(r.lo, r.hi), kBuckets - 1)], 1)] = r;
    }
  }
  for (int32_t i = s_nrec + tid; i < nrec; i += NT) {  // the grid covers nrec records: the rest are empty
    TileRecord r = key_record(-1, 0, 0, 0, 1, 0, 1, -1);
    work[i] = r;
  }
  if (tid == 0) *split_n = s_nsplit;
}

// ---- one-launch preparation from batched boundaries --------------------------------------
// The per-step work before attention, for B rows at once from their boundaries cu
// [B][n_docs + 1] (a row with fewer documents repeats its last boundary: zero-length
// documents change neither ids nor segments nor ranges).  Three kinds of workgroups in
// one grid:
//   * ids:      one thread per position, the doc_ids_from_cu_seqlens rule (boundaries
//               staged in LDS when they fit), plus the boundary checks;
//   * ranges:   one wave per 32-row query block: the first valid row q_f is
//               max(first row, cu[0]) and the last q_l = min(end, cu[n]) - 1; the range is
//               [start of q_f's document, q_l + 1) — what block_range_kernel finds from the
//               ids, computed from the boundaries directly;
//   * segments: one workgroup per row: the run boundaries of the ids the row will hold,
//               from the boundaries (cu[0] when a non-empty document follows leading
//               padding, and the end of every non-empty document short of S).
//   * plan:     when B * nblk <= kPlanBlocks, one more workgroup computes every block's
//               range itself (from the boundaries staged in LDS) and orders the row tiles
//               as tile_order_kernel does, so the whole preparation is one launch.
constexpr int kPrepThreads = 256;
constexpr int kPlanBlocks = 2048;

// key range [lo, hi) of 32-row query block blk from the row's boundaries cu[0..n_docs]
__device__ inline void block_range_from_cu(const int32_t* cu, int32_t n_docs, int32_t blk, int32_t L,
                                           int32_t seq_start, int32_t& lo, int32_t& hi) {
  const int32_t c0 = cu[0], cn = cu[n_docs];
  const int32_t r0 = seq_start + blk * kRowsPerBlock;
  const int32_t r1 = seq_start + min(L, (blk + 1) * kRowsPerBlock);
  const int32_t qf = max(r0, c0), ql = min(r1, cn) - 1;
  lo = 0;
  hi = 0;
  if (qf <= ql) {
    lo = cu[max(last_le(cu, n_docs + 1, qf), 0)];  // >= 0 for valid boundaries
    hi = ql + 1;
  }
}

__global__ void __launch_bounds__(kPrepThreads) prepare_kernel(
    const int32_t* __restrict__ cu_all, int64_t cu_stride, int32_t n_docs, int32_t B, int32_t S, int32_t L,
    int32_t seq_start, int32_t nblk, int32_t id_chunks, int32_t range_groups, int32_t* __restrict__ ids,
    int32_t* __restrict__ seg_cu, int32_t* __restrict__ seg_n, int32_t* __restrict__ blk_lo,
    int32_t* __restrict__ blk_hi, int32_t* __restrict__ status, int32_t nr, int32_t ntile_row, int32_t slots,
    int32_t units, TileRecord* __restrict__ work, int32_t plan_in_grid) {
  constexpr int kCuStage = 4096;
  __shared__ int32_t scu[kCuStage];
  __shared__ int32_t wsum[kPrepThreads / kWave];
  __shared__ int32_t carry;
  __shared__ int32_t hist[kBuckets];
  __shared__ int32_t plo[kPlanBlocks];
  __shared__ int32_t phi[kPlanBlocks];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int64_t id_blocks = (int64_t)B * id_chunks;
  const int64_t bx = blockIdx.x;
  if (bx < id_blocks) {
    const int32_t b = (int32_t)(bx / id_chunks), chunk = (int32_t)(bx % id_chunks);
    const int32_t* cu = cu_all + (int64_t)b * cu_stride;
    if (status != nullptr && chunk == 0) {
      int32_t bits = 0;
      for (int32_t j = tid; j < n_docs; j += kPrepThreads)
        if (cu[j + 1] < cu[j]) bits |= PSB_DATA_CU_NOT_MONOTONE;
      if (tid == 0 && (cu[0] < 0 || cu[n_docs] > S)) bits |= PSB_DATA_CU_OUT_OF_RANGE;
      if (bits) atomicOr(status, bits);
    }
    const int32_t p = chunk * kPrepThreads + tid;
    int32_t i;
    if (n_docs + 1 <= kCuStage) {  // uniform over the grid
      for (int32_t j = tid; j <= n_docs; j += kPrepThreads) scu[j] = cu[j];
      __syncthreads();
      if (p >= S) return;
      i = last_le(scu, n_docs + 1, p);
    } else {
      if (p >= S) return;
      i = last_le(cu, n_docs + 1, p);
    }
    ids[(int64_t)b * S + p] = (i >= 0 && i < n_docs) ? i + 1 : PSB_PAD_DOC_ID;
    return;
  }
  if (bx < id_blocks + range_groups) {
    const int64_t w = (bx - id_blocks) * (kPrepThreads / kWave) + wv;
    if (w >= (int64_t)B * nblk) return;
    const int32_t b = (int32_t)(w / nblk), blk = (int32_t)(w % nblk);
    int32_t lo, hi;
    block_range_from_cu(cu_all + (int64_t)b * cu_stride, n_docs, blk, L, seq_start, lo, hi);
    if (lane == 0) {
      blk_lo[w] = lo;
      blk_hi[w] = hi;
    }
    return;
  }
  if (plan_in_grid && bx == id_blocks + range_groups + B) {
    // the plan: block ranges into LDS (boundaries staged there when they fit), then the
    // longest-first order of the row tiles
    const int32_t ncu = n_docs + 1;
    const bool staged = (int64_t)B * ncu <= kCuStage;  // uniform
    if (staged)
      for (int32_t j = tid; j < B * ncu; j += kPrepThreads) scu[j] = cu_all[(int64_t)(j / ncu) * cu_stride + j % ncu];
    __syncthreads();
    for (int32_t w = tid; w < B * nblk; w += kPrepThreads) {
      const int32_t b = w / nblk;
      const int32_t* cu = staged ? scu + b * ncu : cu_all + (int64_t)b * cu_stride;
      block_range_from_cu(cu, n_docs, w % nblk, L, seq_start, plo[w], phi[w]);
    }
    __syncthreads();
    order_tiles<kPrepThreads>(plo, phi, B, nblk, nr, ntile_row, slots, units, work, hist, wsum);
    return;
  }
  // segments of row b
  const int32_t b = (int32_t)(bx - id_blocks - range_groups);
  if (b >= B) return;
  const int32_t* cu = cu_all + (int64_t)b * cu_stride;
  int32_t* out = seg_cu + (int64_t)b * (S + 1);
  const int32_t c0 = cu[0], cn = cu[n_docs];
  if (tid == 0) {
    carry = 0;
    out[0] = 0;
  }
  __syncthreads();
  for (int32_t j0 = 0; j0 <= n_docs; j0 += kPrepThreads) {
    const int32_t j = j0 + tid;
    bool f = false;
    int32_t val = 0;
    if (j <= n_docs) {
      val = cu[j];
      f = (j == 0) ? (c0 > 0 && cn > c0) : (val > cu[j - 1] && val < S);
    }
    const uint64_t m = __ballot(f);
    const int32_t below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(m);
    __syncthreads();
    int32_t base = carry;
    for (int w = 0; w < wv; ++w) base += wsum[w];
    // valid boundaries flag at most S - 1 strictly increasing values; the bound keeps
    // invalid ones (reported by the ids workgroups) inside the row
    if (f && base + below < S - 1) out[1 + base + below] = val;
    __syncthreads();
    if (tid == 0) carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) {
    if (S > 0) {
      const int32_t r = min(carry, S - 1);
      out[1 + r] = S;
      seg_n[b] = 1 + r;
    } else {
      seg_n[b] = 0;
    }
  }
}

// ---- key window of a query shard ----------------------------------------------------
// One wave per batch row: the first non-padding row of the shard (64 rows per ballot),
// then the start of its document by the same 64-way search as block_range_kernel.
__global__ void __launch_bounds__(256) shard_window_kernel(const int32_t* __restrict__ doc_ids, int32_t B, int32_t S,
                                                           int32_t seq_start, int32_t L,
                                                           int32_t* __restrict__ kv_start_out) {
  const int32_t b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (b >= B) return;
  const int32_t* row = doc_ids + (int64_t)b * S;
  int32_t qf = -1;
  for (int32_t r0 = 0; r0 < L; r0 += kWave) {
    const int32_t r = r0 + lane;
    const uint64_t m = __ballot(r < L && row[seq_start + r] != PSB_PAD_DOC_ID);
    if (m != 0) {
      qf = seq_start + r0 + __ffsll((unsigned long long)m) - 1;
      break;
    }
  }
  int32_t lo = seq_start;
  if (qf >= 0) {
    const int32_t x = row[qf];
    int32_t hi = qf;  // the document start lies in [lo, hi]; doc[hi] == x
    lo = 0;
    while (lo < hi) {
      const int32_t step = (hi - lo + kWave - 1) / kWave;
      int32_t p = lo + lane * step;
      if (p > hi) p = hi;
      const uint64_t t = __ballot(row[p] == x);
      if (t == 0) {
        lo = lo + (kWave - 1) * step + 1;
      } else {
        const int32_t i = __ffsll((unsigned long long)t) - 1;
        const int32_t pi = min(hi, lo + i * step);
        lo = (i == 0) ? lo : lo + (i - 1) * step + 1;
        hi = pi;
      }
    }
    lo = min(lo, seq_start);
  }
  if (lane == 0) kv_start_out[b] = lo;
}

}  // namespace

hipError_t launch_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                           int32_t nr, int32_t slots, int32_t units, const ScheduleBuffers& buf,
                           hipStream_t stream) {
  const int32_t nblk = (L + kRowsPerBlock - 1) / kRowsPerBlock;
  const int32_t total = B * nblk;
  const int waves_per_wg = 256 / kWave;
  const int32_t grid = (total + waves_per_wg - 1) / waves_per_wg;
  block_range_kernel<<<dim3(grid), dim3(256), 0, stream>>>(doc_ids, S, L, seq_start, nblk, total, buf.blk_lo,
                                                           buf.blk_hi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t ntile_row = (nblk + nr - 1) / nr;
  tile_order_kernel<<<dim3(1), dim3(kSortThreads), 0, stream>>>(buf.blk_lo, buf.blk_hi, B, nblk, nr, ntile_row,
                                                                slots, units, buf.work);
  return hipGetLastError();
}

}  // namespace psb

namespace psb {

hipError_t launch_key_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                               int32_t kv_start, int32_t kv_len, int32_t Hkv, const KeySchedule& ks,
                               hipStream_t stream) {
  const int32_t nkt = (kv_len + kKeyTile - 1) / kKeyTile;
  const int32_t total = B * nkt;
  if (total == 0) return hipSuccess;
  const int waves_per_wg = 256 / kWave;
  const int32_t grid = (total + waves_per_wg - 1) / waves_per_wg;
  key_range_kernel<<<dim3(grid), dim3(256), 0, stream>>>(doc_ids, S, L, seq_start, kv_start, kv_start + kv_len, nkt,
                                                         total, ks.klo, ks.khi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  key_plan_kernel<<<dim3(1), dim3(kKeyPlanThreads), 0, stream>>>(ks.klo, ks.khi, B, nkt, Hkv, ks.max_slots, ks.nrec,
                                                                 ks.tslot, ks.work, ks.split, ks.split_n);
  return hipGetLastError();
}

}  // namespace psb

using namespace psb;

PSB_API psb_status psb_shard_kv_window_start(const int32_t* doc_ids, int64_t B, int64_t S, int64_t seq_start,
                                             int64_t L, int32_t* kv_start_out, void* stream) {
  if (B < 0 || S < 0 || L < 0 || seq_start < 0) return PSB_ERR_INVALID_ARG;
  if (seq_start + L > S || S >= INT32_MAX || B >= INT32_MAX) return PSB_ERR_SHAPE;
  if (B == 0) return PSB_OK;
  if (kv_start_out == nullptr || (L > 0 && doc_ids == nullptr)) return PSB_ERR_INVALID_ARG;
  const int64_t grid = (B + 3) / 4;
  shard_window_kernel<<<dim3((unsigned)grid), dim3(256), 0, as_stream(stream)>>>(
      doc_ids, (int32_t)B, (int32_t)S, (int32_t)seq_start, (int32_t)L, kv_start_out);
  PSB_LAUNCH_CHECK();
  return PSB_OK;
}

namespace psb {

hipError_t launch_prepare(const int32_t* cu, int64_t cu_stride, int32_t n_docs, int32_t B, int32_t S, int32_t L,
                          int32_t seq_start, int32_t nr, int32_t slots, int32_t units, int32_t* ids,
                          int32_t* seg_cu, int32_t* seg_n, const ScheduleBuffers& buf, int32_t* status,
                          hipStream_t stream) {
  const int32_t nblk = (L + kRowsPerBlock - 1) / kRowsPerBlock;
  const int32_t id_chunks = (S + kPrepThreads - 1) / kPrepThreads;
  const int64_t waves_per_wg = kPrepThreads / kWave;
  const int32_t range_groups = (int32_t)(((int64_t)B * nblk + waves_per_wg - 1) / waves_per_wg);
  const int32_t ntile_row = (nblk + nr - 1) / nr;
  // small plans are ordered by one extra workgroup of the same grid; larger ones by
  // tile_order_kernel afterwards
  const bool fused = nblk > 0 && (int64_t)B * nblk <= kPlanBlocks;
  const int64_t grid = (int64_t)B * id_chunks + range_groups + B + (fused ? 1 : 0);
  prepare_kernel<<<dim3((unsigned)grid), dim3(kPrepThreads), 0, stream>>>(
      cu, cu_stride, n_docs, B, S, L, seq_start, nblk, id_chunks, range_groups, ids, seg_cu, seg_n, buf.blk_lo,
      buf.blk_hi, status, nr, ntile_row, slots, units, buf.work, fused ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nblk == 0 || fused) return e;
  tile_order_kernel<<<dim3(1), dim3(kSortThreads), 0, stream>>>(buf.blk_lo, buf.blk_hi, B, nblk, nr, ntile_row,
                                                                slots, units, buf.work);
  return hipGetLastError();
}

}  // namespace psb
