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
//   work [T]:                 tile records, longest key range first
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

hipError_t launch_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                           int32_t nr, const ScheduleBuffers& buf, hipStream_t stream);

// Document ids, run boundaries and the plan above for B rows at once, from boundaries
// cu [B][n_docs + 1] (row stride cu_stride): one launch when B * ceil(L / 32) <= 2048,
// else two.
hipError_t launch_prepare(const int32_t* cu, int64_t cu_stride, int32_t n_docs, int32_t B, int32_t S, int32_t L,
                          int32_t seq_start, int32_t nr, int32_t* ids, int32_t* seg_cu, int32_t* seg_n,
                          const ScheduleBuffers& buf, int32_t* status, hipStream_t stream);

// Backward key side: tiles of kKeyTile keys of the window [kv_start, kv_start + kv_len),
// each with the local query rows that see its keys, ordered by row-range length
// (longest first).  The tables are sized for the whole row (kv_len <= S).
//   klo/khi [B * nkt], work [B * nkt] (records with b = batch row, rt = key tile)
constexpr int kKeyTile = 128;
inline int64_t key_ntiles(int64_t B, int64_t S) { return B * ((S + kKeyTile - 1) / kKeyTile); }
inline int64_t key_schedule_bytes(int64_t B, int64_t S) {
  return 2 * pad256(4 * key_ntiles(B, S)) + pad256(64 * key_ntiles(B, S));
}
hipError_t launch_key_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                               int32_t kv_start, int32_t kv_len, int32_t* klo, int32_t* khi, TileRecord* work,
                               hipStream_t stream);

}  // namespace psb
