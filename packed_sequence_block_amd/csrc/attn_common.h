// Device helpers shared by the attention forward and backward kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// dword 3 of a raw buffer resource for gfx9-class GPUs (32-bit data format, no
// swizzle); loads at offsets >= num_records return 0
constexpr int kBufferFlags = 0x00020000;

// 16 bytes per lane from a buffer straight into LDS (lane i lands at lds + 16 i).
// A device-only function: inside a lambda the address-space cast would make the
// host compilation drop the kernel's launch stub.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

// two transposing LDS reads (rows r and r + 8) -> the 8 bf16 of one transposed operand
__device__ __forceinline__ bf16x8 vtr_pair(const __bf16* p, int row8) {
  const short4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
  const short4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p + row8));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// the same pair from two byte addresses (swizzled tiles, where the second read's chunk
// differs from the first's)
__device__ __forceinline__ bf16x8 vtr_pair_at(const char* p0, const char* p1) {
  const short4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p0));
  const short4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Swizzled LDS tile for a tile read both row-wise (ds_read_b128: 16 lanes, 16 rows, one
// 16-byte chunk each) and through transposing reads (ds_read_b64_tr_b16: 32 lanes, 4
// aligned rows, 64 bytes = 4 chunks each).  Rows hold D elements with no padding and
// chunk c of row r sits at chunk c ^ tile_swz(r).  Assuming 64 four-byte banks, the
// row-wise read needs tile_swz to be one-to-one over 16 consecutive rows within each
// 256-byte bank window; the transposing read needs the 4 rows' chunk quads (c / 4) ^
// (tile_swz(r) / 4) to differ within a window.  D = 128 (one row per window):
// 4 (r % 4) + (r / 4) % 4; D = 64 (two rows per window, told apart by r % 2):
// 4 ((r / 2) % 2) + (r / 4) % 4.  Rows 8 apart differ only in bit 1 of tile_swz, so
// the second read of a transposing pair is the first's address ^ 32 plus 8 rows.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  static_assert(D == 64 || D == 128, "head dims");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ __forceinline__ bf16x2 cvt_bf16x2(float a, float b) {
  const float2v f = {a, b};
  return __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, round to nearest even
}

__device__ __forceinline__ float partner_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Stores one 32 x 32 fp32 MFMA block as bf16 into this lane's output row: the lane
// (row = lane & 31, h = lane >> 5) holds d = 8 g4 + 4 h + {0..3} (g4 = 0..3) at acc[4 g4 ..].
// One swap with the partner lane (lane ^ 32, same row) per pair of g4 leaves lane h with
// d = 16 pr + 8 h + {0..7} (pr = 0, 1), so each of the two stores writes 16 bytes per lane and
// 32 contiguous bytes per row.  Every lane must call it (the swap is cross-lane); only lanes
// with `in` store.  row points at the block's first element of this lane's row; h = lane >> 5.
__device__ __forceinline__ void store_block_bf16(__bf16* row, const floatx16& acc, float mul, bool in, int h) {
  uint32_t w[4][2];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    w[g4][0] = __builtin_bit_cast(uint32_t, cvt_bf16x2(acc[4 * g4] * mul, acc[4 * g4 + 1] * mul));
    w[g4][1] = __builtin_bit_cast(uint32_t, cvt_bf16x2(acc[4 * g4 + 2] * mul, acc[4 * g4 + 3] * mul));
  }
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
#pragma unroll
    for (int dw = 0; dw < 2; ++dw) {
      const auto r = __builtin_amdgcn_permlane32_swap(w[2 * pr][dw], w[2 * pr + 1][dw], false, false);
      w[2 * pr][dw] = r[0];
      w[2 * pr + 1][dw] = r[1];
    }
  if (in) {
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const u32x4v v4 = {w[2 * pr][0], w[2 * pr][1], w[2 * pr + 1][0], w[2 * pr + 1][1]};
      *(u32x4v*)(row + 16 * pr + 8 * h) = v4;
    }
  }
}

}  // namespace
}  // namespace psb
