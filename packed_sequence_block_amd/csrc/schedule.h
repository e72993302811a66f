// Scheduler tables shared by schedule.hip and attn_fwd.hip (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psb {

constexpr int kRowsPerBlock = 32;  // query rows per wave (one 32-wide MFMA n-block)
constexpr int kKeysPerTile = 64;   // keys staged in LDS per step

// One row tile of the attention grid, as the kernel reads it (64 bytes, so one
// workgroup fetches it with a single scalar load).
struct TileRecord {
  int32_t b, rt;          // batch row, row tile index
  int32_t lo, hi;         // key range of the whole tile (hi <= lo: no valid query row)
  int32_t blk_lo[4];      // key range of each 32-row block of the tile
  int32_t blk_hi[4];
  int32_t pad[4];
};
static_assert(sizeof(TileRecord) == 64, "tile record is 64 bytes");

// Device tables, carved out of the caller's workspace.
//   blk_lo/blk_hi [B * nblk]: key range of each 32-row query block (hi <= lo: no valid row)
//   work [T]:                 tile records, longest key range first (or in row order, see
//                             launch_schedule)
struct ScheduleBuffers {
  int32_t* blk_lo;
  int32_t* blk_hi;
  TileRecord* work;
};

inline int64_t schedule_nblk(int64_t L) { return (L + kRowsPerBlock - 1) / kRowsPerBlock; }
inline int64_t schedule_ntiles(int64_t B, int64_t L, int64_t nr) {
  return B * ((schedule_nblk(L) + nr - 1) / nr);
}
inline int64_t pad256(int64_t bytes) { return (bytes + 255) / 256 * 256; }
inline int64_t schedule_bytes(int64_t B, int64_t L, int64_t nr) {
  return 2 * pad256(4 * B * schedule_nblk(L)) + pad256(64 * schedule_ntiles(B, L, nr));
}
inline ScheduleBuffers schedule_carve(void* ws, int64_t B, int64_t L, int64_t nr) {
  char* p = static_cast<char*>(ws);
  const int64_t nb = pad256(4 * B * schedule_nblk(L));
  ScheduleBuffers s;
  s.blk_lo = reinterpret_cast<int32_t*>(p);
  s.blk_hi = reinterpret_cast<int32_t*>(p + nb);
  s.work = reinterpret_cast<TileRecord*>(p + 2 * nb);
  return s;
}

// slots: workgroups the attention kernel runs at once (0: always longest first); units:
// head units per row tile (the plan picks row order when the longest record is short next
// to a slot's share of all records x units)
hipError_t launch_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                           int32_t nr, int32_t slots, int32_t units, const ScheduleBuffers& buf,
                           hipStream_t stream);

// Document ids, run boundaries and the plan above for B rows at once, from boundaries
// cu [B][n_docs + 1] (row stride cu_stride): one launch when B * ceil(L / 32) <= 2048,
// else two.
hipError_t launch_prepare(const int32_t* cu, int64_t cu_stride, int32_t n_docs, int32_t B, int32_t S, int32_t L,
                          int32_t seq_start, int32_t nr, int32_t slots, int32_t units, int32_t* ids,
                          int32_t* seg_cu, int32_t* seg_n, const ScheduleBuffers& buf, int32_t* status,
                          hipStream_t stream);

// Backward key side: tiles of kKeyTile keys of the window [kv_start, kv_start + kv_len),
// each with the local query rows that see its keys.  A tile whose row range is much longer
// than the balanced share of a workgroup slot is cut into row chunks, each run by its own
// workgroup, which writes fp32 partial dK / dV into a slot of the partial buffer; a reduce
// kernel then sums each split tile's chunks in chunk order.  The records (one per chunk,
// one per unsplit tile) are ordered by row-range length, longest first.  The tables are
// sized for the whole row (kv_len <= S).
//   klo/khi [B * nkt]: row range of each tile (hi <= lo: no row sees the tile)
//   tslot   [B * nkt]: first partial slot of a split tile, or -1
//   work    [B * nkt + max_slots]: records {b, rt = key tile, lo, hi = chunk rows,
//           blk_lo[0] = slot of this chunk or -1, blk_lo[1] = chunk index, blk_lo[2] =
//           chunk count}; unused records have b = -1
//   split   [max_slots / 2] x {b, key tile, first slot, chunks}, count at split_n
//   partial [max_slots][Hkv][2 * kKeyTile * D] fp32 (dK then dV, MFMA accumulator order)
constexpr int kKeyTile = 128;
constexpr int64_t kPartialBudget = int64_t(64) << 20;  // bytes of fp32 partials at most
constexpr int kMaxSlots = 256;                          // partial slots at most
inline int64_t key_ntiles(int64_t B, int64_t S) { return B * ((S + kKeyTile - 1) / kKeyTile); }
inline int64_t key_slot_bytes(int64_t Hkv, int64_t D) { return Hkv * 2 * kKeyTile * D * 4; }
inline int64_t key_max_slots(int64_t B, int64_t S, int64_t Hkv, int64_t D) {
  const int64_t by_budget = kPartialBudget / key_slot_bytes(Hkv, D);
  const int64_t by_tiles = 2 * key_ntiles(B, S);  // never more partials than the outputs' worth twice
  int64_t m = by_budget < by_tiles ? by_budget : by_tiles;
  return m < kMaxSlots ? (m < 0 ? 0 : m) : kMaxSlots;
}
struct KeySchedule {
  int32_t* klo;
  int32_t* khi;
  int32_t* tslot;
  TileRecord* work;
  int32_t* split;    // 4 ints per split tile
  int32_t* split_n;  // number of split tiles
  float* partial;
  int32_t max_slots;
  int32_t nrec;      // records in work (B * nkt + max_slots)
};
inline int64_t key_schedule_bytes(int64_t B, int64_t S, int64_t Hkv, int64_t D) {
  const int64_t T = key_ntiles(B, S), ms = key_max_slots(B, S, Hkv, D);
  return 3 * pad256(4 * T) + pad256(64 * (T + ms)) + pad256(16 * (ms / 2 + 1) + 16) +
         pad256(ms * key_slot_bytes(Hkv, D));
}
inline KeySchedule key_schedule_carve(void* ws, int64_t B, int64_t S, int64_t Hkv, int64_t D, int64_t kv_len) {
  const int64_t T = key_ntiles(B, S), ms = key_max_slots(B, S, Hkv, D);
  char* p = static_cast<char*>(ws);
  KeySchedule k;
  k.klo = reinterpret_cast<int32_t*>(p);
  k.khi = reinterpret_cast<int32_t*>(p + pad256(4 * T));
  k.tslot = reinterpret_cast<int32_t*>(p + 2 * pad256(4 * T));
  p += 3 * pad256(4 * T);
  k.work = reinterpret_cast<TileRecord*>(p);
  p += pad256(64 * (T + ms));
  k.split_n = reinterpret_cast<int32_t*>(p);
  k.split = reinterpret_cast<int32_t*>(p + 16);
  p += pad256(16 * (ms / 2 + 1) + 16);
  k.partial = reinterpret_cast<float*>(p);
  k.max_slots = (int32_t)ms;
  k.nrec = (int32_t)(B * ((kv_len + kKeyTile - 1) / kKeyTile) + ms);
  return k;
}
hipError_t launch_key_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                               int32_t kv_start, int32_t kv_len, int32_t Hkv, const KeySchedule& ks,
                               hipStream_t stream);

}  // namespace psb
