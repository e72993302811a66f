// Block-diagonal (per-document causal) attention forward for gfx950.
//
// blockdiag_cp page, package overview (a packed row needs a causal mask per
// document) and cp_blockdiag_sdpa (local query rows at seq_start + i against the
// delivered keys, mask rebuilt from document ids, GQA as in PyTorch sdpa,
// output [B, Hq, L, D]).
//
// Work decomposition
//   * one wave = 32 query rows of one query head;
//   * one workgroup = 4 waves sharing every K/V tile staged in LDS: NH heads of
//     one GQA group x NR = 4 / NH consecutive 32-row blocks (NH = 4 whenever the
//     group size allows, so the K/V bytes staged once feed 4 heads);
//   * grid = row tiles (ordered longest key range first by the scheduler) x
//     head units; unit u uses kv head u % Hkv, so with 8 kv heads the blocks that
//     land on one XCD (blockIdx % 8) all read the same kv head from that XCD's L2.
//
// Per key tile (64 keys) each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T held in registers), so a
// lane owns one query row and 16 keys per 32-key block: the row max and row sum
// are lane-local plus one exchange with the partner lane (lane ^ 32).  The online
// softmax runs in fp32 with exp2 (scale * log2 e folded into one multiply), then
// O^T += V^T P^T with the same MFMA: P comes straight from the lane's own scores
// (the k-slot order of the MFMA is permuted to match the score layout) and V^T is
// read from the row-major LDS tile with ds_read_b64_tr_b16.
//
// Key blocks outside a wave's range [start of first row's document, last valid
// row] are skipped; blocks entirely inside one document's causal triangle take no
// mask; the rest compare each key with the row's [doc start, row] range.
#include <math.h>

#include "psb_internal.h"
#include "schedule.h"

namespace psb {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* doc;
  __bf16* out;
  int64_t q_sb, q_sh, q_ss;
  int64_t kv_sb, kv_sh, kv_ss;
  int32_t B, Hq, Hkv, L, S, seq_start, group;
  int32_t nblk, ntile_row, units;
  float sc;  // softmax scale * log2(e)
  const int32_t* blk_lo;
  const int32_t* blk_hi;
  const int32_t* tile_lo;
  const int32_t* tile_hi;
  const int32_t* order;
};

// XOR swizzle of the 16-byte chunks of an LDS row (row = D bf16).  D = 128: the
// 16 rows read together by one b128 K read, and the 4 rows x 4 chunks of one V
// transpose read, land on distinct banks.  D = 64 (two rows per 256-byte bank
// window): the same for rows of equal parity.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

template <int D>
__device__ __forceinline__ int lds_index(int row, int col) {  // col in bf16 elements
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

__device__ __forceinline__ short4v tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(p));
}

template <int D, int NH>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(AttnParams p) {
  constexpr int NR = kWaves / NH;
  constexpr int NCH = D / 8;                               // 16-byte chunks per row
  constexpr int KS = D / 16;                               // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                               // 32-row blocks of O^T
  constexpr int CPT = kKeysPerTile * NCH / kThreads;       // chunks per thread per tensor
  static_assert(CPT * kThreads == kKeysPerTile * NCH, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) __bf16 sK[kKeysPerTile * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kKeysPerTile * D];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = lane >> 5, lr = lane & 31;
  const int32_t rank = blockIdx.x / p.units, unit = blockIdx.x % p.units;
  const int32_t tile = p.order[rank];
  // the tables come from the caller's workspace: never index with an entry that a
  // plan for this shape cannot have written
  if (tile < 0 || tile >= p.B * p.ntile_row) return;
  const int32_t b = tile / p.ntile_row, rt = tile % p.ntile_row;
  const int32_t g = unit % p.Hkv, sub = unit / p.Hkv;
  const int32_t hq = g * p.group + sub * NH + (wv % NH);
  const int32_t blk = rt * NR + wv / NH;
  const int32_t row_local = blk * kRowsPerBlock + lr;
  const bool row_in = blk < p.nblk && row_local < p.L;
  const int32_t qpos = p.seq_start + row_local;
  const int32_t tlo = max(p.tile_lo[tile], 0), thi = min(p.tile_hi[tile], p.S);
  __bf16* out_row = p.out + (((int64_t)b * p.Hq + hq) * p.L + row_local) * D;

  if (thi <= tlo) {  // no valid query row in the whole tile: outputs are 0
    if (row_in) {
      const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) *(bf16x4*)(out_row + 32 * db + 8 * g4 + 4 * h) = z;
    }
    return;
  }

  // ---- per-wave query block description ------------------------------------------
  int32_t w_lo = 0, w_hi = 0;
  if (blk < p.nblk) {
    w_lo = p.blk_lo[(int64_t)b * p.nblk + blk];
    w_hi = p.blk_hi[(int64_t)b * p.nblk + blk];
  }
  w_lo = __builtin_amdgcn_readfirstlane(w_lo);
  w_hi = __builtin_amdgcn_readfirstlane(w_hi);
  const int32_t* docrow = p.doc + (int64_t)b * p.S;
  const int32_t dq = row_in ? docrow[qpos] : PSB_PAD_DOC_ID;
  const bool valid = dq != PSB_PAD_DOC_ID;
  const int32_t dprev = __shfl_up(dq, 1, kWave);
  const bool flag = (lr == 0) || (dq != dprev);
  const uint64_t fm = __ballot(flag) & 0xffffffffull;
  const uint64_t upto = fm & ((2ull << lr) - 1ull);
  const int rs = 63 - __clzll((long long)upto);            // last run start at or before my row
  const int32_t wq0 = p.seq_start + blk * kRowsPerBlock;    // global position of the block's row 0
  const int32_t start_q = (rs == 0) ? w_lo : wq0 + rs;      // my document's first position
  const int32_t qlim = valid ? qpos : -1;                   // last allowed key (none for padding)
  const bool single = (fm == 1ull) && ((__ballot(valid) & 0xffffffffull) == 0xffffffffull);

  // ---- Q^T operand, resident for the whole tile loop -------------------------------
  bf16x8 qreg[KS];
  {
    const __bf16* qsrc = p.q + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)row_local * p.q_ss;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row_in) {
        qreg[ks] = *(const bf16x8*)(qsrc + 16 * ks + 8 * h);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) qreg[ks][t] = (__bf16)0.f;
      }
    }
  }

  const __bf16* kbase = p.k + (int64_t)b * p.kv_sb + (int64_t)g * p.kv_sh;
  const __bf16* vbase = p.v + (int64_t)b * p.kv_sb + (int64_t)g * p.kv_sh;
  bf16x8 kr[CPT], vr[CPT];
  auto gload = [&](int32_t kt) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ci = tid + j * kThreads;
      const int row = ci / NCH, c = ci % NCH;
      const int32_t kg = kt + row;
      if (kg < thi) {
        kr[j] = *(const bf16x8*)(kbase + (int64_t)kg * p.kv_ss + 8 * c);
        vr[j] = *(const bf16x8*)(vbase + (int64_t)kg * p.kv_ss + 8 * c);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) { kr[j][t] = (__bf16)0.f; vr[j][t] = (__bf16)0.f; }
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ci = tid + j * kThreads;
      const int row = ci / NCH, c = ci % NCH;
      const int idx = lds_index<D>(row, 8 * c);
      *(bf16x8*)(sK + idx) = kr[j];
      *(bf16x8*)(sV + idx) = vr[j];
    }
  };

  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  gload(tlo);
  for (int32_t kt = tlo; kt < thi; kt += kKeysPerTile) {
    __syncthreads();  // previous tile fully consumed
    lstore();
    __syncthreads();
    if (kt + kKeysPerTile < thi) gload(kt + kKeysPerTile);

    float sv[2][16];
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int32_t k0 = kt + 32 * kb;
      act[kb] = (k0 < w_hi) && (k0 + 32 > w_lo);
      if (act[kb]) {
        floatx16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const int krow = 32 * kb + lr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *(const bf16x8*)(sK + lds_index<D>(krow, 16 * ks + 8 * h));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], acc, 0, 0, 0);
        }
        const bool full = single && k0 >= w_lo && (k0 + 31) <= wq0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float t = acc[i] * p.sc;
          if (!full) {
            const int32_t key = k0 + (i >> 2) * 8 + h * 4 + (i & 3);
            if (key < start_q || key > qlim) t = -INFINITY;
          }
          sv[kb][i] = t;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[kb][i] = -INFINITY;
      }
    }
    if (!act[0] && !act[1]) continue;

    // ---- online softmax (fp32, base 2) ---------------------------------------------
    float mx = sv[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m_run = m_new;

    bf16x8 pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float e = __builtin_amdgcn_exp2f(sv[j >> 1][8 * (j & 1) + t] - m_use);
        l_run += e;
        pk[j][t] = (__bf16)e;
      }
    }

    // ---- O^T += V^T P^T -------------------------------------------------------------
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!act[j >> 1]) continue;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int vrow0 = 16 * j + 4 * h + ((lane & 15) >> 2);
        const short4v r0 = tr_read(sV + lds_index<D>(vrow0, col));
        const short4v r1 = tr_read(sV + lds_index<D>(vrow0 + 8, col));
        const short8v s8 = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 a = __builtin_bit_cast(bf16x8, s8);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[j], o[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l, padding rows (l == 0) -> 0 ------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (row_in) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = (__bf16)(o[db][4 * g4 + t] * inv);
        *(bf16x4*)(out_row + 32 * db + 8 * g4 + 4 * h) = w;
      }
  }
}

int heads_per_wg(int64_t group) { return (group % 4 == 0) ? 4 : ((group % 2 == 0) ? 2 : 1); }

template <int D>
hipError_t launch_attn(int nh, const AttnParams& prm, unsigned grid, hipStream_t s) {
  switch (nh) {
    case 4: attn_fwd_kernel<D, 4><<<dim3(grid), dim3(kThreads), 0, s>>>(prm); break;
    case 2: attn_fwd_kernel<D, 2><<<dim3(grid), dim3(kThreads), 0, s>>>(prm); break;
    default: attn_fwd_kernel<D, 1><<<dim3(grid), dim3(kThreads), 0, s>>>(prm); break;
  }
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace
}  // namespace psb

using namespace psb;

namespace psb {
namespace {

// Host-side checks shared by the three attention entry points.  On success fills
// the derived launch geometry.
struct AttnGeometry {
  int64_t group, nh, nr, ntiles, units, grid;
};

psb_status check_attn_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D, int64_t seq_start,
                            int32_t enable_gqa, AttnGeometry* geo) {
  if (B < 0 || Hq < 0 || Hkv < 0 || L < 0 || S < 0 || D < 0 || seq_start < 0) return PSB_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return PSB_ERR_UNSUPPORTED;
  if (Hq > 0 && Hkv == 0) return PSB_ERR_SHAPE;
  if (enable_gqa ? (Hkv > 0 && Hq % Hkv != 0) : (Hq != Hkv)) return PSB_ERR_SHAPE;
  if (seq_start + L > S) return PSB_ERR_SHAPE;
  if (L >= INT32_MAX || S >= INT32_MAX || Hq >= INT32_MAX || B >= INT32_MAX) return PSB_ERR_SHAPE;
  geo->group = Hkv > 0 ? Hq / Hkv : 1;
  geo->nh = heads_per_wg(geo->group);
  geo->nr = kWaves / geo->nh;
  geo->ntiles = (B > 0 && L > 0) ? schedule_ntiles(B, L, geo->nr) : 0;
  geo->units = geo->nh > 0 ? Hq / geo->nh : 0;
  geo->grid = geo->ntiles * geo->units;
  if (geo->grid >= INT32_MAX) return PSB_ERR_SHAPE;
  return PSB_OK;
}

psb_status plan_impl(const int32_t* doc_ids, int64_t B, int64_t L, int64_t S, int64_t seq_start,
                     const AttnGeometry& geo, void* workspace, size_t workspace_bytes, hipStream_t s) {
  if (doc_ids == nullptr || workspace == nullptr || !aligned16(workspace)) return PSB_ERR_INVALID_ARG;
  if (workspace_bytes < (size_t)schedule_bytes(B, L, geo.nr)) return PSB_ERR_CAPACITY;
  const ScheduleBuffers buf = schedule_carve(workspace, B, L, geo.nr);
  if (launch_schedule(doc_ids, (int32_t)B, (int32_t)S, (int32_t)L, (int32_t)seq_start, (int32_t)geo.nr, buf, s) !=
      hipSuccess)
    return PSB_ERR_HIP;
  return PSB_OK;
}

psb_status run_impl(const void* q, const void* k, const void* v, const int32_t* doc_ids, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                    const int64_t* kv_strides, int64_t seq_start, float scale, const AttnGeometry& geo, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t s) {
  if (!isfinite(scale)) return PSB_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || doc_ids == nullptr || out == nullptr || workspace == nullptr)
    return PSB_ERR_INVALID_ARG;
  const int64_t qs_def[3] = {Hq * L * D, L * D, D};
  const int64_t kvs_def[3] = {Hkv * S * D, S * D, D};
  const int64_t* qs = q_strides ? q_strides : qs_def;
  const int64_t* kvs = kv_strides ? kv_strides : kvs_def;
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || kvs[i] < 0 || (qs[i] % 8) != 0 || (kvs[i] % 8) != 0) return PSB_ERR_SHAPE;
  }
  if (qs[2] < D || kvs[2] < D) return PSB_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return PSB_ERR_INVALID_ARG;
  if (workspace_bytes < (size_t)schedule_bytes(B, L, geo.nr)) return PSB_ERR_CAPACITY;
  const ScheduleBuffers buf = schedule_carve(workspace, B, L, geo.nr);
  AttnParams prm;
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(v);
  prm.doc = doc_ids;
  prm.out = static_cast<__bf16*>(out);
  prm.q_sb = qs[0]; prm.q_sh = qs[1]; prm.q_ss = qs[2];
  prm.kv_sb = kvs[0]; prm.kv_sh = kvs[1]; prm.kv_ss = kvs[2];
  prm.B = (int32_t)B; prm.Hq = (int32_t)Hq; prm.Hkv = (int32_t)Hkv; prm.L = (int32_t)L; prm.S = (int32_t)S;
  prm.seq_start = (int32_t)seq_start; prm.group = (int32_t)geo.group;
  prm.nblk = (int32_t)schedule_nblk(L);
  prm.ntile_row = (int32_t)(geo.ntiles / B);
  prm.units = (int32_t)geo.units;
  prm.sc = scale * kLog2e;
  prm.blk_lo = buf.blk_lo; prm.blk_hi = buf.blk_hi;
  prm.tile_lo = buf.tile_lo; prm.tile_hi = buf.tile_hi; prm.order = buf.order;
  const hipError_t e = (D == 128) ? launch_attn<128>((int)geo.nh, prm, (unsigned)geo.grid, s)
                                  : launch_attn<64>((int)geo.nh, prm, (unsigned)geo.grid, s);
  return e == hipSuccess ? PSB_OK : PSB_ERR_HIP;
}

}  // namespace
}  // namespace psb

using namespace psb;

PSB_API size_t psb_blockdiag_attn_fwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t D) {
  (void)D;
  if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0) return 256;
  const int64_t group = (Hq % Hkv == 0) ? Hq / Hkv : 1;
  const int64_t nr = kWaves / heads_per_wg(group);
  return (size_t)schedule_bytes(B, L, nr);
}

PSB_API psb_status psb_blockdiag_attn_plan(const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                           int64_t S, int64_t D, int64_t seq_start, int32_t enable_gqa,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  AttnGeometry geo;
  const psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  return plan_impl(doc_ids, B, L, S, seq_start, geo, workspace, workspace_bytes, as_stream(stream));
}

PSB_API psb_status psb_blockdiag_attn_fwd_planned(const void* q, const void* k, const void* v,
                                                  const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                  int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                                  const int64_t* kv_strides, int64_t seq_start, float scale,
                                                  int32_t enable_gqa, void* out, const void* workspace,
                                                  size_t workspace_bytes, int32_t* status_word, void* stream) {
  (void)status_word;
  AttnGeometry geo;
  const psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  return run_impl(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, scale, geo, out,
                  const_cast<void*>(workspace), workspace_bytes, as_stream(stream));
}

PSB_API psb_status psb_blockdiag_attn_fwd(const void* q, const void* k, const void* v, const int32_t* doc_ids,
                                          int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D,
                                          const int64_t* q_strides, const int64_t* kv_strides, int64_t seq_start,
                                          float scale, int32_t enable_gqa, void* out, void* workspace,
                                          size_t workspace_bytes, int32_t* status_word, void* stream) {
  (void)status_word;
  AttnGeometry geo;
  psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  // argument checks of the run step first, so that nothing is enqueued on failure
  if (!isfinite(scale)) return PSB_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return PSB_ERR_INVALID_ARG;
  const int64_t qs_def[3] = {Hq * L * D, L * D, D};
  const int64_t kvs_def[3] = {Hkv * S * D, S * D, D};
  const int64_t* qs = q_strides ? q_strides : qs_def;
  const int64_t* kvs = kv_strides ? kv_strides : kvs_def;
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || kvs[i] < 0 || (qs[i] % 8) != 0 || (kvs[i] % 8) != 0) return PSB_ERR_SHAPE;
  }
  if (qs[2] < D || kvs[2] < D) return PSB_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PSB_ERR_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  st = plan_impl(doc_ids, B, L, S, seq_start, geo, workspace, workspace_bytes, s);
  if (st != PSB_OK) return st;
  return run_impl(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, scale, geo, out,
                  workspace, workspace_bytes, s);
}
