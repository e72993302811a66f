// Block-diagonal (per-document causal) attention backward for gfx950.
//
// The gradients of the forward in attn_fwd.hip (blockdiag_cp page: the packed
// block-diagonal path stays active while backward recomputes checkpointed
// forwards; glm5_next.cp page: K/V gradients flow back to the rank that owns each
// shard, so a shard's call returns the dK / dV of its own rows).  With the
// forward's log-sum-exp per row, for each (batch, query head):
//   P  = exp(scale Q K^T - lse)  on the allowed pairs, 0 elsewhere
//   dP = dO V^T,  delta = rowsum(dO * O),  dS = P * (dP - delta)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO   (dK, dV summed over a kv
//   head's query heads)
//
// Two kernels:
//   dq_kernel     query-stationary like the forward: a wave owns 32 query rows of one
//                 head, computes their delta = rowsum(dO * O) in fp32 from the rows it
//                 loads anyway (and stores it for dkdv_kernel), walks the key tiles of the
//                 forward's plan, recomputes S^T and dP^T = V dO^T (lane = row), and
//                 accumulates dQ^T += K^T dS^T with the K^T operand gathered from the K
//                 tile by transposing LDS reads;
//   dkdv_kernel   key-stationary: a wave owns 32 keys of one kv head (K held in VGPRs
//                 as an MFMA B operand; V too at D = 64, in LDS at D = 128), a workgroup
//                 128 keys, two waves per SIMD; it walks every query head of the group and
//                 the query rows that can see its keys, 32 (D = 128) or 64 (D = 64) rows
//                 per step, recomputes S and dP (lane = key), and accumulates
//                 dV^T += dO^T P and dK^T += Q^T dS with Q^T / dO^T gathered by
//                 transposing LDS reads.  When a 128-key tile is
//                 seen by many rows, the plan splits those rows into chunks that run as
//                 separate items writing fp32 partial dK / dV, and dkdv_reduce_kernel
//                 adds each tile's chunks in chunk order.
// All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are
// rounded to bf16 for the MFMAs that consume them.
#include <math.h>

#include <type_traits>

#include "attn_common.h"
#include "psb_internal.h"
#include "schedule.h"

namespace psb {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * kWave;
constexpr int kKeysPerWave = 32;                       // dkdv: keys per wave
constexpr int kKeysPerItem = kKeysPerWave * kBwdWaves; // dkdv: keys per workgroup

struct BwdParams {
  const __bf16* q;     // [B, Hq, L, D]
  const __bf16* k;     // [B, Hkv, kv_len, D]: keys at global positions [kv_start, kv_start + kv_len)
  const __bf16* v;
  const __bf16* dout;  // [B, Hq, L, D]
  const __bf16* out;   // [B, Hq, L, D]: the forward's output
  const float* lse;    // [B, Hq, L] natural log
  float* delta;        // [B, Hq, L]: written by dq_kernel, read by dkdv_kernel
  const int32_t* doc;  // [B, S]
  __bf16* dq;          // [B, Hq, L, D]
  __bf16* dk;          // [B, Hkv, kv_len, D]
  __bf16* dv;
  int32_t B, Hq, Hkv, L, S, seq_start, group;
  int32_t nblk, ntile_row, units;
  float scale;         // signed softmax scale
  float sc;            // |scale| * log2(e)
  int64_t items;
  const TileRecord* work;
  const TileRecord* kwork;  // key tiles, longest row range first
  int32_t nkt;              // key tiles per batch row
  int32_t kv_start, kv_len;
  int32_t* status;          // PSB_DATA_KV_WINDOW when a row needs a key before kv_start, or null
  int32_t nrec;             // key-side records (the dK / dV grid covers nrec x Hkv items)
  int32_t max_slots;        // partial slots in `partial`
  float* partial;           // fp32 partial dK / dV of the chunks of split key tiles
  const int32_t* split;     // split key tiles {b, key tile, first slot, chunks}
  const int32_t* split_n;   // their number
};

// fp32 partials of one (slot, kv head): per wave, dK then dV accumulators in MFMA order,
// as float4 [2][DB][4][64 lanes] (each store instruction writes 1 KiB)
template <int D>
__device__ __forceinline__ float4* partial_at(float* base, int32_t slot, int32_t Hkv, int32_t g, int wv) {
  constexpr int64_t per_wave = 2 * (D / 32) * 16 * 64;  // floats
  return reinterpret_cast<float4*>(base + (((int64_t)slot * Hkv + g) * kBwdWaves + wv) * per_wave);
}

// ---- dQ: query-stationary ---------------------------------------------------------
template <int D, int NH>
__global__ void __launch_bounds__(kBwdThreads, 2) dq_kernel(BwdParams p) {
  constexpr int NR = kBwdWaves / NH;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NCH = D / 8;
  // K is read row-wise (S^T = K Q^T) and transposed (dQ^T += K^T dS^T), V row-wise only
  // (dP^T = V dO^T): both are swizzled tiles of unpadded rows (tile_swz), read row-wise at
  // the same addresses.
  constexpr int KROWB = D * 2;                            // K tile row, bytes
  constexpr int KSTAGE = kKeysPerTile * D;
  constexpr int KSEGS = kKeysPerTile * NCH / 64;
  constexpr int KSEG_ITERS = KSEGS / kBwdWaves;
  constexpr int VSTAGE = KSTAGE;
  static_assert(KSEGS % kBwdWaves == 0 && KSTAGE * 2 == KSEGS * 1024, "K / V tile segments");
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[KSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[KSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[VSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[VSTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, lr = lane & 31;
  const int32_t row_bytes = D * 2;  // contiguous k, v
  const bool neg = p.scale < 0.f;
  const float sc = p.sc;  // |scale| * log2(e); Q is sign-flipped for a negative scale
  const floatx16 zero16 = {};

  // slot seg * 64 + lane of a K or V tile holds row slot / NCH, stored chunk slot % NCH,
  // which is global chunk (stored chunk) ^ tile_swz(row)
  int32_t koff[KSEG_ITERS];
#pragma unroll
  for (int j = 0; j < KSEG_ITERS; ++j) {
    const int slot = (j * kBwdWaves + wv) * 64 + lane;
    const int row = slot / NCH, pc = slot % NCH;
    koff[j] = row * row_bytes + 16 * (pc ^ tile_swz<D>(row));
  }
  // A = K rows (and V rows), byte address: k-step ks reads chunk 2 ks + h of row lr, stored
  // at k_rd ^ (32 ks) (the chunk bits and the row bits never overlap)
  const int k_rd = lr * KROWB + 16 * (h ^ tile_swz<D>(lr));
  // transposing read of K^T: key r0 = 4 h + (lane & 15) / 4 (+ 16 j + 32 kb, + 8 for the
  // pair's second read), d bytes 64 db + 32 ((lane >> 4) & 1) + 8 (lane & 3); stored at
  // kt_rd ^ (64 db) (second read: ^ 32, 8 rows on)
  const int kt_r0 = 4 * h + ((lane & 15) >> 2);
  const int kt_rd = kt_r0 * KROWB + 16 * ((2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ tile_swz<D>(kt_r0)) +
                    8 * (lane & 1);

  for (int64_t item = blockIdx.x; item < p.items; item += gridDim.x) {
    const int32_t rank = (int32_t)(item / p.units), unit = (int32_t)(item % p.units);
    const TileRecord& rec = p.work[rank];
    const int32_t b = rec.b, rt = rec.rt;
    if (b < 0 || b >= p.B || rt < 0 || rt >= p.ntile_row) continue;
    const int32_t g = unit % p.Hkv, sub = unit / p.Hkv;
    const int32_t hq = g * p.group + sub * NH + (wv % NH);
    const int32_t blk = rt * NR + wv / NH;
    const int32_t row_local = blk * kRowsPerBlock + lr;
    const bool row_in = blk < p.nblk && row_local < p.L;
    const int32_t qpos = p.seq_start + row_local;
    const int32_t tlo = max(rec.lo, p.kv_start), thi = min(rec.hi, p.kv_start + p.kv_len);
    if (p.status != nullptr && tid == 0 && rec.hi > rec.lo && rec.lo < p.kv_start)
      atomicOr(p.status, PSB_DATA_KV_WINDOW);
    const int64_t qrow = ((int64_t)b * p.Hq + hq) * p.L + row_local;
    __bf16* dq_row = p.dq + qrow * D;
    if (thi <= tlo) {
      if (row_in) {
        // no key for any row of the tile: P is 0 for all of them, any finite delta will do
        if (h == 0) p.delta[qrow] = 0.f;
        const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) *(bf16x4*)(dq_row + 32 * db + 8 * g4 + 4 * h) = z;
      }
      continue;
    }
    const int32_t ntiles = (thi - tlo + kKeysPerTile - 1) / kKeysPerTile;
    const __bf16* kbase = p.k + ((int64_t)b * p.Hkv + g) * p.kv_len * D;
    const __bf16* vbase = p.v + ((int64_t)b * p.Hkv + g) * p.kv_len * D;
    // num_records 0 (on == false) turns every lane of a load into a zero fill with no memory
    // access: the last tile issues such loads into the free stages
    auto rsrc = [&](const __bf16* base, int32_t kt, bool on = true) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)(kt - p.kv_start) * D), (short)0,
                                               on ? min(thi - kt, kKeysPerTile) * row_bytes : 0, kBufferFlags);
    };
    auto issue_k = [&](__bf16* buf, int32_t kt) {
      const __amdgpu_buffer_rsrc_t r = rsrc(kbase, kt);
#pragma unroll
      for (int j = 0; j < KSEG_ITERS; ++j) buffer_load_lds16(r, buf + (j * kBwdWaves + wv) * 512, koff[j]);
    };
    auto issue_v = [&](__bf16* buf, int32_t kt) {
      const __amdgpu_buffer_rsrc_t r = rsrc(vbase, kt);
#pragma unroll
      for (int j = 0; j < KSEG_ITERS; ++j) buffer_load_lds16(r, buf + (j * kBwdWaves + wv) * 512, koff[j]);
    };

    // ---- per-wave rows: document range (as in the forward) --------------------------
    const int32_t w_lo = __builtin_amdgcn_readfirstlane(rec.blk_lo[wv / NH]);
    const int32_t* docrow = p.doc + (int64_t)b * p.S;
    const int32_t dqid = row_in ? docrow[qpos] : PSB_PAD_DOC_ID;
    const bool valid = dqid != PSB_PAD_DOC_ID;
    const int32_t dprev = __shfl_up(dqid, 1, kWave);
    const bool flag = (lr == 0) || (dqid != dprev);
    const uint64_t fm = __ballot(flag) & 0xffffffffull;
    const uint64_t upto = fm & ((2ull << lr) - 1ull);
    const int rs = 63 - __clzll((long long)upto);
    const int32_t wq0 = __builtin_amdgcn_readfirstlane(p.seq_start + blk * kRowsPerBlock);
    const int32_t start_q = (rs == 0) ? w_lo : wq0 + rs;
    const uint32_t span = valid ? (uint32_t)(qpos - start_q) : 0u;
    const int32_t kshift = valid ? start_q : 0x40000000;
    const bool single = __builtin_amdgcn_readfirstlane(
        (fm == 1ull) && ((__ballot(valid) & 0xffffffffull) == 0xffffffffull));

    // ---- stationary operands: Q^T (sign-flipped for a negative scale) and dO^T ----------
    bf16x8 qreg[KS], oreg[KS];
    {
      const __bf16* qsrc = p.q + qrow * D;
      const __bf16* osrc = p.dout + qrow * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (row_in) {
          qreg[ks] = *(const bf16x8*)(qsrc + 16 * ks + 8 * h);
          oreg[ks] = *(const bf16x8*)(osrc + 16 * ks + 8 * h);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) { qreg[ks][t] = (__bf16)0.f; oreg[ks][t] = (__bf16)0.f; }
        }
        if (neg) {
          short8v bits = __builtin_bit_cast(short8v, qreg[ks]);
          bits ^= (short)0x8000;
          qreg[ks] = __builtin_bit_cast(bf16x8, bits);
        }
      }
    }
    // exp2 argument offset of the row (rows without keys never produce a P: any finite value)
    const float lse2 = (valid && row_in) ? p.lse[qrow] * kLog2e : 0.f;
    // delta = rowsum(dO * O): this lane's 64 (D = 128) or 32 d of the row, then the partner
    // lane's half (lane ^ 32 holds the other d)
    float dlt;
    {
      float part = 0.f;
      if (row_in) {
        const __bf16* osrc2 = p.out + qrow * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 o8 = *(const bf16x8*)(osrc2 + 16 * ks + 8 * h);
#pragma unroll
          for (int t = 0; t < 8; ++t) part = __builtin_fmaf((float)o8[t], (float)oreg[ks][t], part);
        }
      }
      dlt = partner_sum(part);
      if (row_in && h == 0) p.delta[qrow] = dlt;
    }

    floatx16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero16;

    // one 32-key half kb of the tile in kbuf / vbuf; half 0 also issues the next tile's
    // loads (K segments, then V), one after each k-step's pair of MFMAs: issued as one burst
    // they queue behind each other
    constexpr int NLOAD = 2 * KSEG_ITERS;
    auto half = [&](const __bf16* kbuf, const __bf16* vbuf, int32_t kt, int kb, __amdgpu_buffer_rsrc_t rkn,
                    __bf16* kn, __amdgpu_buffer_rsrc_t rvn, __bf16* vn) {
      // S^T and dP^T for keys 32 kb .. 32 kb + 31
      floatx16 s = zero16, dp = zero16;
      const char* kp = (const char*)kbuf + 32 * KROWB * kb;
      const char* vp = (const char*)vbuf + 32 * KROWB * kb;
      auto next_load = [&](int n) {
        if (n < KSEG_ITERS)
          buffer_load_lds16(rkn, kn + (n * kBwdWaves + wv) * 512, koff[n]);
        else
          buffer_load_lds16(rvn, vn + ((n - KSEG_ITERS) * kBwdWaves + wv) * 512, koff[n - KSEG_ITERS]);
      };
      // K and V operands read AH k-steps ahead of their MFMAs (pinned below: issued one
      // pair at a time right before its MFMAs, each read would hold its MFMA for the whole
      // LDS latency)
      constexpr int AH = (KS < 2) ? KS : 2;
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 ar[AH], cr[AH];
#pragma unroll
      for (int ks = 0; ks < AH; ++ks) {
        ar[ks] = *(const bf16x8*)(kp + (k_rd ^ (32 * ks)));
        cr[ks] = *(const bf16x8*)(vp + (k_rd ^ (32 * ks)));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = ar[ks % AH], c = cr[ks % AH];
        if (ks + AH < KS) {
          ar[ks % AH] = *(const bf16x8*)(kp + (k_rd ^ (32 * (ks + AH))));
          cr[ks % AH] = *(const bf16x8*)(vp + (k_rd ^ (32 * (ks + AH))));
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c, oreg[ks], dp, 0, 0, 0);
        if (kb == 0 && ks < NLOAD) next_load(ks);
      }
      if (kb == 0) {
#pragma unroll
        for (int n = KS; n < NLOAD; ++n) next_load(n);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (ks + AH < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (kb == 0 && ks < NLOAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the first dQ step's K^T operands, read under the dS VALU work below
      bf16x8 ta[DB];
      {
        const char* tp = (const char*)kbuf + 32 * kb * KROWB;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          ta[db] = vtr_pair_at(tp + (kt_rd ^ (64 * db)), tp + 8 * KROWB + (kt_rd ^ (64 * db + 32)));
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool full = single && kt >= w_lo && (kt + 63) <= wq0;
      const int32_t e = kt + 32 * kb + 4 * h - kshift;
      bf16x8 dsk[2];
      // dS = P * (dP - delta) rounded to bf16; a tile inside one document's causal triangle
      // for every row of the wave takes the copy without the per-key range test (the
      // condition is wave-uniform, so the branch costs nothing and saves three VALU ops
      // per score)
      auto ds_step = [&](auto masked) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int t = 0; t < 8; t += 2) {
            float d2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int i = 8 * j + t + u;
              const float arg = __builtin_fmaf(s[i], sc, -lse2);
              float pr;
              if constexpr (decltype(masked)::value) {
                const uint32_t rel = (uint32_t)(e + (i >> 2) * 8 + (i & 3));
                pr = (rel <= span) ? __builtin_amdgcn_exp2f(arg) : 0.f;
              } else {
                pr = __builtin_amdgcn_exp2f(arg);
              }
              d2[u] = pr * (dp[i] - dlt);
            }
            const bf16x2 pk = cvt_bf16x2(d2[0], d2[1]);
            dsk[j][t] = pk[0];
            dsk[j][t + 1] = pk[1];
          }
        }
      };
      if (full) ds_step(std::false_type{});
      else ds_step(std::true_type{});
      // dQ^T += K^T dS^T over the two 16-key steps of this half, the second step's operands
      // read one step ahead
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[db], dsk[j], acc[db], 0, 0, 0);
          if (j == 0) {
            const char* tp = (const char*)kbuf + (32 * kb + 16) * KROWB;
            ta[db] = vtr_pair_at(tp + (kt_rd ^ (64 * db)), tp + 8 * KROWB + (kt_rd ^ (64 * db + 32)));
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    __syncthreads();  // the previous item no longer reads LDS
    issue_k(sK0, tlo);
    issue_v(sV0, tlo);
    auto step = [&](int32_t t, const __bf16* kc, __bf16* kn, const __bf16* vc, __bf16* vn) {
      const int32_t kt = tlo + t * kKeysPerTile;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const bool more = t + 1 < ntiles;
      const __amdgpu_buffer_rsrc_t rkn = rsrc(kbase, kt + kKeysPerTile, more);
      const __amdgpu_buffer_rsrc_t rvn = rsrc(vbase, kt + kKeysPerTile, more);
      half(kc, vc, kt, 0, rkn, kn, rvn, vn);
      half(kc, vc, kt, 1, rkn, kn, rvn, vn);
    };
    int32_t t = 0;
    for (; t + 1 < ntiles; t += 2) {
      step(t, sK0, sK1, sV0, sV1);
      step(t + 1, sK1, sK0, sV1, sV0);
    }
    if (t < ntiles) step(t, sK0, sK1, sV0, sV1);

    // ---- epilogue: dQ = scale * dQ^T, bf16 ------------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) store_block_bf16(dq_row + 32 * db, acc[db], p.scale, row_in, h);
  }
}

// ---- dK, dV: key-stationary -------------------------------------------------------
// Workgroup item = (b, kv head g, 128 keys [k0, k0 + 128)).  Wave w owns keys
// k0 + 32 w + (lane % 32).  Key k is seen by the rows r of its document with r >= k:
// k <= r < end(k), end(k) = one past the last position of k's document (a padding key
// has no rows).  Rows are local query rows [0, L) at global positions seq_start + r.
template <int D>
__global__ void __launch_bounds__(kBwdThreads, 2) dkdv_kernel(BwdParams p) {
  // Two waves per SIMD.  At D = 128: 32 query rows per step, and a wave's V rows wait in
  // LDS (its own 32 rows, read back as the dP MFMA operand) instead of 32 VGPRs, which
  // keeps the wave within 256 registers next to its 128 dK / dV accumulators.  At D = 64:
  // 64 rows per step (two independent 32-row halves), half the barriers and load waits per
  // flop of 32-row steps.
  constexpr int kRowsPerStep = D == 64 ? 64 : 32;
  constexpr bool VLDS = D == 128;
  constexpr int VROW = D + 8;  // padded V row: the 16 rows of one b128 read on distinct banks
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NCH = D / 8;
  // Q and dO tiles are read row-wise (S = Q K^T, dP = dO V^T) and transposed (dK^T +=
  // Q^T dS, dV^T += dO^T P): swizzled tiles of unpadded rows (tile_swz)
  constexpr int QROWB = D * 2;                                // Q / dO tile row, bytes
  constexpr int QSLOTS = kRowsPerStep * NCH;                  // 16-byte slots of a tile
  constexpr int QSEGS = QSLOTS / 64;                          // 1 KiB wave-wide loads
  constexpr int QSEG_ITERS = (QSEGS + kBwdWaves - 1) / kBwdWaves;
  constexpr int QSTAGE = QSEGS * 512;                         // elements
  static_assert(QSEGS * 64 == QSLOTS, "Q tile segments");
  __shared__ __attribute__((aligned(1024))) __bf16 sQ0[QSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sQ1[QSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sO0[QSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sO1[QSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV[VLDS ? kKeysPerItem * VROW : 8];
  __shared__ __attribute__((aligned(16))) float sL[2][kRowsPerStep];   // per row: lse * log2(e)
  __shared__ __attribute__((aligned(16))) float sDl[2][kRowsPerStep];  // per row: delta
  __shared__ int32_t s_rng[kBwdWaves][2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, lr = lane & 31;
  const int32_t row_bytes = D * 2;
  const float ssc = p.scale * kLog2e;  // signed: exp2(s * ssc - lse2) = exp(scale s - lse)
  const floatx16 zero16 = {};
  const int32_t nkt = p.nkt;
  static_assert(kKeysPerItem == kKeyTile, "key tiles of the plan");

  // slot seg * 64 + lane holds row slot / NCH, stored chunk slot % NCH = global chunk ^
  // tile_swz(row)
  int32_t qoff[QSEG_ITERS];
#pragma unroll
  for (int j = 0; j < QSEG_ITERS; ++j) {
    const int slot = (j * kBwdWaves + wv) * 64 + lane;
    const int row = slot / NCH, pc = slot % NCH;
    qoff[j] = (slot < QSLOTS) ? row * row_bytes + 16 * (pc ^ tile_swz<D>(row)) : 0x7ffffff0;
  }
  // A = Q / dO rows (lane = row), bytes: k-step ks reads chunk 2 ks + h of row lr at a_rd ^ (32 ks)
  const int a_rd = lr * QROWB + 16 * (h ^ tile_swz<D>(lr));
  // transposing read of Q^T / dO^T: row r0 = 4 h + (lane & 15) / 4 (+ 16 j, + 8 for the pair's
  // second read), d bytes 64 db + 32 ((lane >> 4) & 1) + 8 (lane & 3): at t_rd ^ (64 db), the
  // second read at t_rd ^ (64 db + 32) 8 rows on
  const int t_r0 = 4 * h + ((lane & 15) >> 2);
  const int t_rd = t_r0 * QROWB + 16 * ((2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ tile_swz<D>(t_r0)) +
                   8 * (lane & 1);

  // item = key-tile rank x kv head; kv head = item % Hkv keeps (with 8 kv heads) one kv
  // head per XCD
  for (int64_t item = blockIdx.x; item < (int64_t)p.nrec * p.Hkv; item += gridDim.x) {
    const TileRecord& rec = p.kwork[item / p.Hkv];
    const int32_t g = (int32_t)(item % p.Hkv);
    const int32_t b = rec.b, kt_i = rec.rt;
    // empty records, and records a plan for this shape cannot have written
    if (b < 0 || b >= p.B || kt_i < 0 || kt_i >= nkt) continue;
    // a chunk of a split tile: rows [rec.lo, rec.hi) only, into partial slot rec.blk_lo[0]
    const int32_t slot = rec.blk_lo[0], nchunks = rec.blk_lo[2];
    const bool chunked = nchunks > 1 && slot >= 0 && slot < p.max_slots;
    const int32_t key = p.kv_start + kt_i * kKeysPerItem + kKeysPerWave * wv + lr;  // global position
    const bool key_in = key < p.kv_start + p.kv_len;
    const int32_t* docrow = p.doc + (int64_t)b * p.S;

    // ---- this lane's key: the rows that see it -------------------------------------------
    const int32_t dk_id = key_in ? docrow[key] : PSB_PAD_DOC_ID;
    // end of the key's document: the next run start inside the wave's 32 keys, else the
    // end of the run that covers the wave's last key (one 64-way search per wave)
    const int32_t dnext = __shfl_down(dk_id, 1, kWave);
    const bool last_of_run = (lr == 31) || (dnext != dk_id);
    const uint64_t lm = __ballot(last_of_run) & 0xffffffffull;
    int32_t kend;
    {
      const uint64_t from = lm & ~((1ull << lr) - 1ull);       // run ends at or after this key
      const int e = __ffsll((unsigned long long)from) - 1;      // lane of this run's last key
      const int32_t wkey0 =
          __builtin_amdgcn_readfirstlane(p.kv_start + kt_i * kKeysPerItem + kKeysPerWave * wv);
      int32_t tail_end = 0;
      {
        // run end after the wave's last key (lane 31); the search is wave-uniform
        const int32_t q31 = min(wkey0 + 31, p.S - 1);
        const int32_t x = docrow[q31];
        int32_t lo = q31, hi = p.S - 1;  // last position of the run lies in [lo, hi]
        while (lo < hi) {
          const int32_t step = (hi - lo + kWave - 1) / kWave;
          int32_t pp = lo + lane * step + 1;
          if (pp > hi) pp = hi;
          const uint64_t diff = __ballot(docrow[pp] != x);
          if (diff == 0) {
            lo = lo + (kWave - 1) * step + 1;
            if (lo > hi) lo = hi;
          } else {
            const int i = __ffsll((unsigned long long)diff) - 1;
            const int32_t pi = min(hi, lo + i * step + 1);  // first differing probe
            hi = pi - 1;
            lo = (i == 0) ? lo : lo + (i - 1) * step + 1;
          }
        }
        tail_end = lo + 1;
      }
      kend = (e < 31) ? wkey0 + e + 1 : tail_end;
    }
    const bool key_valid = key_in && dk_id != PSB_PAD_DOC_ID;
    // local rows [r_lo, r_hi) that see this key
    int32_t r_lo = key_valid ? max(key, p.seq_start) - p.seq_start : 0;
    int32_t r_hi = key_valid ? min(kend, p.seq_start + p.L) - p.seq_start : 0;
    if (chunked) {  // this chunk's rows only: each row is counted by exactly one chunk
      r_lo = max(r_lo, rec.lo);
      r_hi = min(r_hi, rec.hi);
    }
    if (r_hi < r_lo) r_hi = r_lo;
    // wave range: min / max over its keys (empty keys excluded)
    // and the rows every key of the wave sees: [max r_lo, min r_hi) (empty when some key
    // sees no row), so that a step inside it needs no per-row test
    // (only used at D = 64: at D = 128 the unmasked copy below would push the kernel past
    // its 256 registers)
    int32_t full_lo = 0x7fffffff, full_hi = 0;
    {
      int32_t lo_m = (r_hi > r_lo) ? r_lo : 0x7fffffff, hi_m = (r_hi > r_lo) ? r_hi : 0;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        lo_m = min(lo_m, __shfl_xor(lo_m, off, kWave));
        hi_m = max(hi_m, __shfl_xor(hi_m, off, kWave));
      }
      if (lane == 0) { s_rng[wv][0] = lo_m; s_rng[wv][1] = hi_m; }
      if constexpr (D == 64) {
        int32_t lo_x = (r_hi > r_lo) ? r_lo : 0x7fffffff, hi_n = (r_hi > r_lo) ? r_hi : 0;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          lo_x = max(lo_x, __shfl_xor(lo_x, off, kWave));
          hi_n = min(hi_n, __shfl_xor(hi_n, off, kWave));
        }
        full_lo = __builtin_amdgcn_readfirstlane(lo_x);
        full_hi = __builtin_amdgcn_readfirstlane(hi_n);
      }
    }
    __syncthreads();
    int32_t wg_lo = 0x7fffffff, wg_hi = 0;
#pragma unroll
    for (int w = 0; w < kBwdWaves; ++w) { wg_lo = min(wg_lo, s_rng[w][0]); wg_hi = max(wg_hi, s_rng[w][1]); }
    const int32_t w_lo = s_rng[wv][0], w_hi = s_rng[wv][1];
    // for the mask: row r (local) sees this key iff r - r_lo < r_hi - r_lo (unsigned)
    const uint32_t kspan = (uint32_t)(r_hi - r_lo);

    // ---- stationary K^T and V^T operands (B operands: lane = key) --------------------------
    bf16x8 kreg[KS], vreg[KS];
    // this lane's V row in the wave's own LDS rows (VLDS): written and read by this wave only
    const int v_rd = (kKeysPerWave * wv + lr) * VROW + 8 * h;
    {
      const int64_t kvrow = ((int64_t)b * p.Hkv + g) * p.kv_len + (key - p.kv_start);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (key_in) {
          kreg[ks] = *(const bf16x8*)(p.k + kvrow * D + 16 * ks + 8 * h);
          vreg[ks] = *(const bf16x8*)(p.v + kvrow * D + 16 * ks + 8 * h);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) { kreg[ks][t] = (__bf16)0.f; vreg[ks][t] = (__bf16)0.f; }
        }
        if constexpr (VLDS) *(bf16x8*)(sV + v_rd + 16 * ks) = vreg[ks];
      }
    }
    floatx16 dka[DB], dva[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dka[db] = zero16; dva[db] = zero16; }

    const int32_t nsteps_h = (wg_hi > wg_lo) ? (wg_hi - wg_lo + kRowsPerStep - 1) / kRowsPerStep : 0;
    float pend_l = 0.f, pend_d = 0.f;
    const int32_t nsteps = nsteps_h * p.group;
    // Step st covers query head hh = st / nsteps_h of the group and the kRowsPerStep rows
    // from wg_lo + kRowsPerStep ri, ri = st % nsteps_h.  The steps run in order, so (hh, ri) is carried from step to step
    // instead of divided out (a runtime division is some 40 scalar instructions).
    struct StepPos { int32_t hh, ri; };
    auto advance = [&](StepPos s) {
      if (++s.ri == nsteps_h) { s.ri = 0; ++s.hh; }
      return s;
    };
    // buffer resources of step st's Q and dO rows; a step past the last gets zero records,
    // so its loads become zero fills of the free stage with no memory access
    struct StepRsrc { __amdgpu_buffer_rsrc_t q, o; };
    auto step_rsrc = [&](int32_t st, StepPos sp) {
      const bool on = st < nsteps;
      const int32_t hh = on ? sp.hh : 0, rr = wg_lo + (on ? sp.ri : 0) * kRowsPerStep;
      const int32_t hq = g * p.group + hh;
      const int64_t base = ((int64_t)b * p.Hq + hq) * p.L + rr;
      const int32_t nrows = on ? min(kRowsPerStep, p.L - rr) : 0;
      StepRsrc r;
      r.q = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + base * D), (short)0, nrows * row_bytes, kBufferFlags);
      r.o = __builtin_amdgcn_make_buffer_rsrc((void*)(p.dout + base * D), (short)0, nrows * row_bytes, kBufferFlags);
      return r;
    };
    // segments every wave loads (QFULL rounds) and the rest (waves wv < QSEGS % waves)
    constexpr int QFULL = QSEGS / kBwdWaves;
    // at D = 64 (32-row steps, 8 MFMAs) the loads need the whole step to land: issued at
    // the top as one burst there, spread over the first MFMA loop at D = 128
    constexpr bool SPREAD = D == 128;
    auto issue_seg = [&](const StepRsrc& r, __bf16* qb, __bf16* ob, int j) {
      const int seg = j * kBwdWaves + wv;
      buffer_load_lds16(r.q, qb + seg * 512, qoff[j]);
      buffer_load_lds16(r.o, ob + seg * 512, qoff[j]);
    };
    auto issue_rest = [&](const StepRsrc& r, __bf16* qb, __bf16* ob) {
      if constexpr (QSEGS % kBwdWaves != 0) {
        if (QFULL * kBwdWaves + wv < QSEGS) issue_seg(r, qb, ob, QFULL);
      }
    };
    // the step's row lse / delta go to registers now and to LDS at the step's start,
    // after the wait that the tile loads need anyway
    auto issue_rows = [&](StepPos sp) {
      const int32_t hh = sp.hh, rr = wg_lo + sp.ri * kRowsPerStep;
      const int32_t hq = g * p.group + hh;
      const int64_t base = ((int64_t)b * p.Hq + hq) * p.L + rr;
      const int32_t nrows = min(kRowsPerStep, p.L - rr);
      if (tid < kRowsPerStep) {
        const bool in = tid < nrows;
        const float l = in ? p.lse[base + tid] : 0.f;
        pend_l = (l == -INFINITY) ? 0.f : l * kLog2e;  // rows without keys: P is masked to 0
        pend_d = in ? p.delta[base + tid] : 0.f;
      }
    };
    auto issue = [&](int32_t st, StepPos sp, __bf16* qb, __bf16* ob) {
      const StepRsrc r = step_rsrc(st, sp);
#pragma unroll
      for (int j = 0; j < QFULL; ++j) issue_seg(r, qb, ob, j);
      issue_rest(r, qb, ob);
      issue_rows(sp);
    };

    // one step: kRowsPerStep rows as NHALF independent 32-row halves, so the MFMAs of one
    // half can run while the other's probabilities are computed
    constexpr int NHALF = kRowsPerStep / 32;
    // the next step's full-round segments are issued inside the first MFMA loop, one every
    // KS / QFULL k-steps, alternating Q and dO (a wave with nothing to compute issues them
    // at once)
    auto compute = [&](StepPos sp, const __bf16* qb, const __bf16* ob, int stage, const StepRsrc& rn, __bf16* qn,
                       __bf16* on) {
      const int32_t rr = wg_lo + sp.ri * kRowsPerStep;
      // rows of this step that this wave's keys can see at all
      if (rr >= w_hi || rr + kRowsPerStep <= w_lo) {
        if constexpr (SPREAD) {
#pragma unroll
          for (int j = 0; j < QFULL; ++j) issue_seg(rn, qn, on, j);
        }
        return;
      }
      // S = Q K^T and dP = dO V^T: C[row][key], lane = key, rows {8 a + 4 h + c}
      floatx16 s[NHALF], dp[NHALF];
#pragma unroll
      for (int hf = 0; hf < NHALF; ++hf) { s[hf] = zero16; dp[hf] = zero16; }
      constexpr int EVERY = (KS / QFULL >= 1) ? KS / QFULL : 1;
      auto spread_load = [&](int ks) {
        if (SPREAD && (ks % EVERY) == EVERY - 1 && ks / EVERY < QFULL) {
          const int j = ks / EVERY;
          const int seg = j * kBwdWaves + wv;
          buffer_load_lds16(rn.q, qn + seg * 512, qoff[j]);
          buffer_load_lds16(rn.o, on + seg * 512, qoff[j]);
        }
      };
      if constexpr (D == 64) {
        // Q / dO operands read two k-steps ahead of their MFMAs, pinned below (V is in
        // VGPRs at D = 64; at D = 128 a ring of Q, dO and V operands spills 13 more registers)
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 rq[2][NHALF], ro[2][NHALF];
        auto rd = [&](int ks, int hf, bf16x8& aq, bf16x8& ao) {
          aq = *(const bf16x8*)((const char*)qb + 32 * hf * QROWB + (a_rd ^ (32 * ks)));
          ao = *(const bf16x8*)((const char*)ob + 32 * hf * QROWB + (a_rd ^ (32 * ks)));
        };
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int hf = 0; hf < NHALF; ++hf) rd(ks, hf, rq[ks][hf], ro[ks][hf]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int hf = 0; hf < NHALF; ++hf) {
            const bf16x8 aq = rq[ks & 1][hf], ao = ro[ks & 1][hf];
            if (ks + 2 < KS) rd(ks + 2, hf, rq[ks & 1][hf], ro[ks & 1][hf]);
            s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[ks], s[hf], 0, 0, 0);
            dp[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vreg[ks], dp[hf], 0, 0, 0);
          }
          spread_load(ks);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * NHALF, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int hf = 0; hf < NHALF; ++hf) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          if (SPREAD && (ks % EVERY) == EVERY - 1 && ks / EVERY < QFULL) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int hf = 0; hf < NHALF; ++hf) {
            const bf16x8 aq = *(const bf16x8*)((const char*)qb + 32 * hf * QROWB + (a_rd ^ (32 * ks)));
            const bf16x8 ao = *(const bf16x8*)((const char*)ob + 32 * hf * QROWB + (a_rd ^ (32 * ks)));
            s[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[ks], s[hf], 0, 0, 0);
            const bf16x8 bv = VLDS ? *(const bf16x8*)(sV + v_rd + 16 * ks) : vreg[ks];
            dp[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bv, dp[hf], 0, 0, 0);
          }
          spread_load(ks);
        }
      }
      if constexpr (SPREAD && KS / QFULL < 1) {
#pragma unroll
        for (int j = KS; j < QFULL; ++j) issue_seg(rn, qn, on, j);
      }
      bf16x8 pk[NHALF][2], dsk[NHALF][2];
      // P and dS; a step whose rows all see every key of the wave takes the copy without the
      // per-row test (wave-uniform condition)
      // row r = rr + 32 hf + 8 a + 4 h + c of the step is one of the key's rows iff
      // r - r_lo = rbase + (32 hf + 8 a + c) < kspan (unsigned); rbase is opaque so that each
      // test stays one add of a constant (the compiler otherwise rebuilds r - r_lo per pair)
      uint32_t rbase = (uint32_t)(rr + 4 * h - r_lo);
      asm volatile("" : "+v"(rbase));
      auto p_ds = [&](auto masked) {
#pragma unroll
        for (int hf = 0; hf < NHALF; ++hf) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float4 l4 = *(const float4*)&sL[stage][32 * hf + 8 * a + 4 * h];
            const float4 d4 = *(const float4*)&sDl[stage][32 * hf + 8 * a + 4 * h];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int c = 0; c < 4; c += 2) {
              float pp[2], dd[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int i = 4 * a + c + u;
                const float arg = __builtin_fmaf(s[hf][i], ssc, -lv[c + u]);  // Q is not sign-flipped here
                float pr;
                if constexpr (decltype(masked)::value) {
                  const bool ok = rbase + (uint32_t)(32 * hf + 8 * a + c + u) < kspan;
                  pr = ok ? __builtin_amdgcn_exp2f(arg) : 0.f;
                } else {
                  pr = __builtin_amdgcn_exp2f(arg);
                }
                pp[u] = pr;
                dd[u] = pr * (dp[hf][i] - dv4[c + u]);
              }
              const bf16x2 p2 = cvt_bf16x2(pp[0], pp[1]);
              const bf16x2 d2 = cvt_bf16x2(dd[0], dd[1]);
              const int j = a >> 1, t = 4 * (a & 1) + c;
              pk[hf][j][t] = p2[0]; pk[hf][j][t + 1] = p2[1];
              dsk[hf][j][t] = d2[0]; dsk[hf][j][t + 1] = d2[1];
            }
          }
        }
      };
      if constexpr (D == 64) {
        if (rr >= full_lo && rr + kRowsPerStep <= full_hi) p_ds(std::false_type{});
        else p_ds(std::true_type{});
      } else {
        // the masked loop written out: at D = 128 the same loop through p_ds (one copy only)
        // compiled to 26 spilled registers instead of 10
#pragma unroll
        for (int hf = 0; hf < NHALF; ++hf) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float4 l4 = *(const float4*)&sL[stage][32 * hf + 8 * a + 4 * h];
            const float4 d4 = *(const float4*)&sDl[stage][32 * hf + 8 * a + 4 * h];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int c = 0; c < 4; c += 2) {
              float pp[2], dd[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int i = 4 * a + c + u;
                const bool ok = rbase + (uint32_t)(32 * hf + 8 * a + c + u) < kspan;
                const float arg = __builtin_fmaf(s[hf][i], ssc, -lv[c + u]);  // Q is not sign-flipped here
                const float pr = ok ? __builtin_amdgcn_exp2f(arg) : 0.f;
                pp[u] = pr;
                dd[u] = pr * (dp[hf][i] - dv4[c + u]);
              }
              const bf16x2 p2 = cvt_bf16x2(pp[0], pp[1]);
              const bf16x2 d2 = cvt_bf16x2(dd[0], dd[1]);
              const int j = a >> 1, t = 4 * (a & 1) + c;
              pk[hf][j][t] = p2[0]; pk[hf][j][t + 1] = p2[1];
              dsk[hf][j][t] = d2[0]; dsk[hf][j][t + 1] = d2[1];
            }
          }
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 16-row k-steps
#pragma unroll
      for (int hf = 0; hf < NHALF; ++hf) {
        // operands read two MFMA pairs ahead (pinned below): issued one pair at a time right
        // before their MFMAs, each pair would hold its MFMAs for the whole LDS latency
        auto opnd = [&](const __bf16* base, int i) {
          const char* tp = (const char*)base + (32 * hf + 16 * (i / DB)) * QROWB;
          const int db = i % DB;
          return vtr_pair_at(tp + (t_rd ^ (64 * db)), tp + 8 * QROWB + (t_rd ^ (64 * db + 32)));
        };
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 ro[2], rq[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) { ro[i] = opnd(ob, i); rq[i] = opnd(qb, i); }
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
          const int j = i / DB, db = i % DB;
          const bf16x8 co = ro[i & 1], cq = rq[i & 1];
          if (i + 2 < 2 * DB) { ro[i & 1] = opnd(ob, i + 2); rq[i & 1] = opnd(qb, i + 2); }
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(co, pk[hf][j], dva[db], 0, 0, 0);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cq, dsk[hf][j], dka[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (i + 2 < 2 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    __syncthreads();  // the previous item no longer reads LDS (and s_rng is read)
    StepPos cur = {0, 0};  // position of step st in the loop below
    if (nsteps > 0) issue(0, cur, sQ0, sO0);
    auto step = [&](int32_t st, const __bf16* qc, const __bf16* oc, __bf16* qn, __bf16* on, int stage) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (tid < kRowsPerStep) { sL[stage][tid] = pend_l; sDl[stage][tid] = pend_d; }
      __syncthreads();
      const StepPos nxt = advance(cur);
      const StepRsrc rn = step_rsrc(st + 1, nxt);
      if constexpr (!SPREAD) {
#pragma unroll
        for (int j = 0; j < QFULL; ++j) issue_seg(rn, qn, on, j);
      }
      issue_rest(rn, qn, on);
      if (st + 1 < nsteps) issue_rows(nxt);
      compute(cur, qc, oc, stage, rn, qn, on);
      cur = nxt;
    };
    int32_t st = 0;
    for (; st + 1 < nsteps; st += 2) {
      step(st, sQ0, sO0, sQ1, sO1, 0);
      step(st + 1, sQ1, sO1, sQ0, sO0, 1);
    }
    if (st < nsteps) step(st, sQ0, sO0, sQ1, sO1, 0);

    // ---- epilogue: C[d][key] -> dk, dv rows (lane = key), or the chunk's fp32 partial -------
    if (chunked) {
      float4* pp = partial_at<D>(p.partial, slot, p.Hkv, g, wv);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          pp[((0 * DB + db) * 4 + i4) * 64 + lane] =
              make_float4(dka[db][4 * i4], dka[db][4 * i4 + 1], dka[db][4 * i4 + 2], dka[db][4 * i4 + 3]);
          pp[((1 * DB + db) * 4 + i4) * 64 + lane] =
              make_float4(dva[db][4 * i4], dva[db][4 * i4 + 1], dva[db][4 * i4 + 2], dva[db][4 * i4 + 3]);
        }
    } else {
      const int64_t kvrow = ((int64_t)b * p.Hkv + g) * p.kv_len + (key - p.kv_start);
      __bf16* dkr = p.dk + kvrow * D;
      __bf16* dvr = p.dv + kvrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        store_block_bf16(dkr + 32 * db, dka[db], p.scale, key_in, h);
        store_block_bf16(dvr + 32 * db, dva[db], 1.f, key_in, h);
      }
    }
  }
}

// ---- dK, dV of split key tiles: the chunks' partials summed in chunk order -------------
// Workgroup = (split tile, kv head, 32-wide d block), the dK / dV kernel's lane layout; the
// grid covers the most split tiles a plan can make, the rest exit.  Chunk j + 1's partials
// are loaded before chunk j's are added, so consecutive chunks' loads overlap while the sum
// keeps chunk order.
template <int D>
__global__ void __launch_bounds__(kBwdThreads) dkdv_reduce_kernel(BwdParams p) {
  constexpr int DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, lr = lane & 31;
  const int32_t db = blockIdx.x % DB, tg = blockIdx.x / DB;
  const int32_t i = tg / p.Hkv, g = tg % p.Hkv;
  if (i >= *p.split_n) return;
  const int32_t b = p.split[4 * i], kt_i = p.split[4 * i + 1], slot0 = p.split[4 * i + 2], n = p.split[4 * i + 3];
  if (b < 0 || b >= p.B || kt_i < 0 || slot0 < 0 || n < 2 || n > p.max_slots || slot0 > p.max_slots - n) return;
  floatx16 dka = {}, dva = {};
  float4 a[2][4], c[2][4];
  auto load = [&](int32_t j, float4 (&aa)[4], float4 (&cc)[4]) {
    const float4* pp = partial_at<D>(p.partial, slot0 + j, p.Hkv, g, wv);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      aa[i4] = pp[((0 * DB + db) * 4 + i4) * 64 + lane];
      cc[i4] = pp[((1 * DB + db) * 4 + i4) * 64 + lane];
    }
  };
  auto add = [&](const float4 (&aa)[4], const float4 (&cc)[4]) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      dka[4 * i4] += aa[i4].x; dka[4 * i4 + 1] += aa[i4].y; dka[4 * i4 + 2] += aa[i4].z; dka[4 * i4 + 3] += aa[i4].w;
      dva[4 * i4] += cc[i4].x; dva[4 * i4 + 1] += cc[i4].y; dva[4 * i4 + 2] += cc[i4].z; dva[4 * i4 + 3] += cc[i4].w;
    }
  };
  load(0, a[0], c[0]);  // n >= 2
  int32_t j = 0;
  for (; j + 2 <= n; j += 2) {
    load(j + 1, a[1], c[1]);
    add(a[0], c[0]);
    if (j + 2 < n) load(j + 2, a[0], c[0]);
    add(a[1], c[1]);
  }
  if (j < n) add(a[0], c[0]);
  const int32_t key = p.kv_start + kt_i * kKeysPerItem + kKeysPerWave * wv + lr;
  const bool key_in = key < p.kv_start + p.kv_len;
  const int64_t kvrow = ((int64_t)b * p.Hkv + g) * p.kv_len + (key - p.kv_start);
  store_block_bf16(p.dk + kvrow * D + 32 * db, dka, p.scale, key_in, h);
  store_block_bf16(p.dv + kvrow * D + 32 * db, dva, 1.f, key_in, h);
}

int heads_per_wg_bwd(int64_t group) { return (group % 4 == 0) ? 4 : ((group % 2 == 0) ? 2 : 1); }

bool aligned_to(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

int64_t bwd_plan_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t L) {
  const int64_t group = (Hkv > 0 && Hq % Hkv == 0) ? Hq / Hkv : 1;
  return pad256(schedule_bytes(B, L, kBwdWaves / heads_per_wg_bwd(group)));
}

// workspace: [forward plan][delta: fp32 B*Hq*L][key schedule]
int64_t bwd_delta_bytes(int64_t B, int64_t Hq, int64_t L) { return pad256(4 * B * Hq * L); }

template <int D>
hipError_t launch_bwd(int nh, const BwdParams& prm, int64_t rows, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (rows > 0) {  // L == 0: no query rows, dq is empty and dk / dv are all zero
    const unsigned qgrid = (unsigned)prm.items;
    switch (nh) {
      case 4: dq_kernel<D, 4><<<dim3(qgrid), dim3(kBwdThreads), 0, s>>>(prm); break;
      case 2: dq_kernel<D, 2><<<dim3(qgrid), dim3(kBwdThreads), 0, s>>>(prm); break;
      default: dq_kernel<D, 1><<<dim3(qgrid), dim3(kBwdThreads), 0, s>>>(prm); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t kgrid = (int64_t)prm.nrec * prm.Hkv;
  if (kgrid == 0) return hipSuccess;
  dkdv_kernel<D><<<dim3((unsigned)kgrid), dim3(kBwdThreads), 0, s>>>(prm);
  e = hipGetLastError();
  if (e != hipSuccess || prm.max_slots < 2) return e;
  dkdv_reduce_kernel<D><<<dim3((unsigned)(prm.max_slots / 2 * prm.Hkv * (D / 32))), dim3(kBwdThreads), 0, s>>>(prm);
  return hipGetLastError();
}

}  // namespace
}  // namespace psb

using namespace psb;

PSB_API size_t psb_blockdiag_attn_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S,
                                                     int64_t D) {
  if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || (D != 64 && D != 128)) return 256;
  return (size_t)(bwd_plan_bytes(B, Hq, Hkv, L) + bwd_delta_bytes(B, Hq, L) + key_schedule_bytes(B, S, Hkv, D));
}

namespace {

// The backward with k, v, dk, dv holding the keys [kv_start, kv_start + kv_len) of each row.
psb_status bwd_run(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                   const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D,
                   int64_t seq_start, int64_t kv_start, int64_t kv_len, float scale, int32_t enable_gqa, void* dq,
                   void* dk, void* dv, void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || L < 0 || S < 0 || D < 0 || seq_start < 0) return PSB_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return PSB_ERR_UNSUPPORTED;
  if (Hq > 0 && Hkv == 0) return PSB_ERR_SHAPE;
  if (enable_gqa ? (Hkv > 0 && Hq % Hkv != 0) : (Hq != Hkv)) return PSB_ERR_SHAPE;
  if (seq_start + L > S) return PSB_ERR_SHAPE;
  if (L >= INT32_MAX || S >= INT32_MAX || Hq >= INT32_MAX || B >= INT32_MAX) return PSB_ERR_SHAPE;
  // the window holds the shard's own keys and lies inside the row
  if (kv_start < 0 || kv_len < 0 || kv_start > seq_start || kv_start + kv_len < seq_start + L ||
      kv_start + kv_len > S)
    return PSB_ERR_SHAPE;
  if (B == 0 || Hq == 0 || kv_len == 0) return PSB_OK;
  if (!isfinite(scale)) return PSB_ERR_INVALID_ARG;
  const void* kv_side[] = {k, v, dk, dv, workspace};
  for (const void* ptr : kv_side)
    if (ptr == nullptr || !aligned_to(ptr, 16)) return PSB_ERR_INVALID_ARG;
  if (L > 0) {  // an empty query shard passes empty (possibly null) row tensors
    const void* q_side[] = {q, out, dout, dq};
    for (const void* ptr : q_side)
      if (ptr == nullptr || !aligned_to(ptr, 16)) return PSB_ERR_INVALID_ARG;
    if (lse == nullptr || !aligned_to(lse, 4)) return PSB_ERR_INVALID_ARG;
  }
  if (doc_ids == nullptr) return PSB_ERR_INVALID_ARG;
  if (workspace_bytes < psb_blockdiag_attn_bwd_workspace_size(B, Hq, Hkv, L, S, D)) return PSB_ERR_CAPACITY;
  const int64_t group = Hq / Hkv;
  const int64_t nh = heads_per_wg_bwd(group);
  const int64_t nr = kBwdWaves / nh;
  const int64_t ntiles = (L > 0) ? schedule_ntiles(B, L, nr) : 0;
  const int64_t units = Hq / nh;
  if (ntiles * units >= INT32_MAX ||
      (B * ((kv_len + kKeysPerItem - 1) / kKeysPerItem) + key_max_slots(B, S, Hkv, D)) * Hkv >= INT32_MAX)
    return PSB_ERR_SHAPE;
  const ScheduleBuffers buf = schedule_carve(workspace, B, L, nr);
  char* wsb = static_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(wsb + bwd_plan_bytes(B, Hq, Hkv, L));
  const KeySchedule ks =
      key_schedule_carve(wsb + bwd_plan_bytes(B, Hq, Hkv, L) + bwd_delta_bytes(B, Hq, L), B, S, Hkv, D, kv_len);
  BwdParams prm;
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(v);
  prm.dout = static_cast<const __bf16*>(dout);
  prm.lse = lse;
  prm.delta = delta;
  prm.out = static_cast<const __bf16*>(out);
  prm.doc = doc_ids;
  prm.dq = static_cast<__bf16*>(dq);
  prm.dk = static_cast<__bf16*>(dk);
  prm.dv = static_cast<__bf16*>(dv);
  prm.B = (int32_t)B; prm.Hq = (int32_t)Hq; prm.Hkv = (int32_t)Hkv; prm.L = (int32_t)L; prm.S = (int32_t)S;
  prm.seq_start = (int32_t)seq_start; prm.group = (int32_t)group;
  prm.nblk = (int32_t)schedule_nblk(L);
  prm.ntile_row = (B > 0 && L > 0) ? (int32_t)(ntiles / B) : 0;
  prm.units = (int32_t)units;
  prm.scale = scale;
  prm.sc = fabsf(scale) * kLog2e;
  prm.items = ntiles * units;
  prm.work = buf.work;
  prm.kwork = ks.work;
  prm.nrec = ks.nrec;
  prm.max_slots = ks.max_slots;
  prm.partial = ks.partial;
  prm.split = ks.split;
  prm.split_n = ks.split_n;
  prm.nkt = (int32_t)((kv_len + kKeyTile - 1) / kKeyTile);
  prm.kv_start = (int32_t)kv_start;
  prm.kv_len = (int32_t)kv_len;
  prm.status = status;
  const int64_t rows = B * Hq * L;
  if (launch_key_schedule(doc_ids, (int32_t)B, (int32_t)S, (int32_t)L, (int32_t)seq_start, (int32_t)kv_start,
                          (int32_t)kv_len, (int32_t)Hkv, ks, as_stream(stream)) != hipSuccess)
    return PSB_ERR_HIP;
  const hipError_t e = (D == 128)
      ? launch_bwd<128>((int)nh, prm, rows, as_stream(stream))
      : launch_bwd<64>((int)nh, prm, rows, as_stream(stream));
  if (e != hipSuccess) return PSB_ERR_HIP;
  // with a status word, also the precondition check the plans rely on (one launch)
  return status != nullptr ? launch_contiguity_check(doc_ids, B, S, S, status, as_stream(stream)) : PSB_OK;
}

}  // namespace

PSB_API psb_status psb_blockdiag_attn_bwd_planned(const void* q, const void* k, const void* v, const void* out,
                                                  const void* dout, const float* lse, const int32_t* doc_ids,
                                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S,
                                                  int64_t D, int64_t seq_start, float scale, int32_t enable_gqa,
                                                  void* dq, void* dk, void* dv, void* workspace,
                                                  size_t workspace_bytes, int32_t* status_word, void* stream) {
  return bwd_run(q, k, v, out, dout, lse, doc_ids, B, Hq, Hkv, L, S, D, seq_start, 0, S, scale, enable_gqa, dq, dk,
                 dv, workspace, workspace_bytes, status_word, stream);
}

PSB_API psb_status psb_blockdiag_attn_bwd_window_planned(const void* q, const void* k, const void* v,
                                                         const void* out, const void* dout, const float* lse,
                                                         const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                         int64_t L, int64_t S, int64_t D, int64_t seq_start,
                                                         int64_t kv_start, int64_t kv_len, float scale,
                                                         int32_t enable_gqa, void* dq, void* dk, void* dv,
                                                         void* workspace, size_t workspace_bytes,
                                                         int32_t* status_word, void* stream) {
  return bwd_run(q, k, v, out, dout, lse, doc_ids, B, Hq, Hkv, L, S, D, seq_start, kv_start, kv_len, scale,
                 enable_gqa, dq, dk, dv, workspace, workspace_bytes, status_word, stream);
}
