// Scheduler tables shared by schedule.hip and attn_fwd.hip (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psb {

constexpr int kRowsPerBlock = 32;  // query rows per wave (one 32-wide MFMA n-block)
constexpr int kKeysPerTile = 64;   // keys staged in LDS per step

// Device tables, carved out of the caller's workspace.
//   blk_lo/blk_hi [B * nblk]: key range of each 32-row query block (hi <= lo: no valid row)
//   tile_lo/tile_hi [T]:      union over the NR blocks of a row tile
//   order [T]:                tile ids, longest key range first
struct ScheduleBuffers {
  int32_t* blk_lo;
  int32_t* blk_hi;
  int32_t* tile_lo;
  int32_t* tile_hi;
  int32_t* order;
};

inline int64_t schedule_nblk(int64_t L) { return (L + kRowsPerBlock - 1) / kRowsPerBlock; }
inline int64_t schedule_ntiles(int64_t B, int64_t L, int64_t nr) {
  return B * ((schedule_nblk(L) + nr - 1) / nr);
}
// bytes of the five tables, each padded to 256 bytes
inline int64_t schedule_bytes(int64_t B, int64_t L, int64_t nr) {
  auto pad = [](int64_t n) { return (n * 4 + 255) / 256 * 256; };
  return 2 * pad(B * schedule_nblk(L)) + 3 * pad(schedule_ntiles(B, L, nr));
}
inline ScheduleBuffers schedule_carve(void* ws, int64_t B, int64_t L, int64_t nr) {
  auto pad = [](int64_t n) { return (n * 4 + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  ScheduleBuffers s;
  const int64_t nb = pad(B * schedule_nblk(L)), nt = pad(schedule_ntiles(B, L, nr));
  s.blk_lo = reinterpret_cast<int32_t*>(p);
  s.blk_hi = reinterpret_cast<int32_t*>(p + nb);
  s.tile_lo = reinterpret_cast<int32_t*>(p + 2 * nb);
  s.tile_hi = reinterpret_cast<int32_t*>(p + 2 * nb + nt);
  s.order = reinterpret_cast<int32_t*>(p + 2 * nb + 2 * nt);
  return s;
}

hipError_t launch_schedule(const int32_t* doc_ids, int32_t B, int32_t S, int32_t L, int32_t seq_start,
                           int32_t nr, const ScheduleBuffers& buf, hipStream_t stream);

}  // namespace psb
