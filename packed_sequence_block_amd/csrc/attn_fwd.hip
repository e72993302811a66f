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
// read from the row-major LDS tile with ds_read_b64_tr_b16 (the transposing LDS
// read), so both K and V go from HBM straight into LDS with buffer_load ... lds.
//
// A workgroup walks the key tiles of its row tile's range [start of the first valid
// row's document, last valid row]; tiles entirely inside one document's causal
// triangle for all of a wave's rows take no mask, the rest compare each key with
// the row's [doc start, row] range.
#include <float.h>
#include <math.h>

#include <atomic>
#include <mutex>

#include "attn_common.h"
#include "psb_internal.h"
#include "schedule.h"

namespace psb {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

struct AttnParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* doc;
  __bf16* out;
  int64_t q_sb, q_sh, q_ss;
  int64_t kv_sb, kv_sh, kv_ss;
  int32_t kv_start, kv_end;  // k / v hold the keys at global positions [kv_start, kv_end)
  int32_t B, Hq, Hkv, L, S, seq_start, group;
  int32_t nblk, ntile_row, units;
  float sc;  // softmax scale * log2(e)
  int64_t items;  // row tiles x head units
  const TileRecord* work;
  float* lse;     // [B, Hq, L] natural-log sum of exp(scale * q.k) per row, or null
  int32_t* status;  // PSB_DATA_KV_WINDOW when a row needs a key before kv_start, or null
  // explicit-mask variant: mask[b * mask_sb + row * mask_ss + key] != 0 where row may see
  // key; every row readable up to S rounded up to 4 bytes, 4-byte aligned
  const uint8_t* mask;
  int64_t mask_sb, mask_ss;
};

// the exp2 offset is only moved (and O, l rescaled) when the P of a 64-key tile sums to
// more than 2^8 in some lane; until then every p < 2^8, harmless in fp32 / bf16
constexpr float kRetuneSum = 256.0f;

// LDS tiles, 64 keys each, rows of D bf16 with no padding; 16-byte chunk c of row r is
// stored at chunk c ^ f(r), so that every read is free of bank conflicts (64 banks of 4
// bytes) and a load fills whole 1 KiB segments with data:
//   K: f = tile_swz (one-to-one over 16 consecutive rows): the 16 rows that one b128 read
//      serves per pass land on distinct bank groups.  The read of k-step ks sits at the
//      lane's base ^ (32 ks).
//   V: a PV k-step feeds lane (h = lane / 32) the keys 16j + 4h + {0..3} and
//      16j + 8 + 4h + {0..3} of one d: two ds_read_b64_tr_b16, each gathering 4 keys x 4 d
//      from 16 lanes' row addresses and handing every lane its own d.  One half-wave of
//      such a read covers 4 aligned rows x 64 bytes (a chunk quad); f = 4 (r % 4) at
//      D = 128 (one row per 256-byte bank window) or 4 ((r / 2) % 2) at D = 64 (two rows
//      per window) puts the 4 rows' quads on distinct banks.  Rows 8 apart share f, so
//      both reads of a pair use the lane's base ^ (64 db).
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// DENSE: the explicit-mask variant (the dense-mask path next to the varlen kernels in
// the blockdiag_cp package overview).  No plan: every row tile walks all keys [0, S) and
// takes its mask bits from p.mask, prefetched one tile ahead.
template <int D, int NH, bool DENSE>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(AttnParams p) {
  constexpr int NR = kWaves / NH;
  constexpr int KS = D / 16;                              // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;                              // 32-row blocks of O^T
  constexpr int NCH = D / 8;                              // 16-byte chunks per K / V row
  constexpr int ROWB = D * 2;                             // K / V tile row, bytes
  constexpr int KSTAGE = kKeysPerTile * D;                // elements per K stage
  constexpr int VSTAGE = kKeysPerTile * D;                // elements per V stage
  constexpr int VSEGS = kKeysPerTile * NCH / 64;          // 1 KiB wave-wide loads per V tile
  constexpr int VSEG_ITERS = (VSEGS + kWaves - 1) / kWaves;
  static_assert(VSEGS * 64 == kKeysPerTile * NCH && VSTAGE * 2 == VSEGS * 1024, "V tile segments");
  constexpr int KSEGS = kKeysPerTile * NCH / 64;          // 1 KiB wave-wide loads per K tile
  constexpr int KSEG_ITERS = (KSEGS + kWaves - 1) / kWaves;
  static_assert(KSEGS * 64 == kKeysPerTile * NCH && KSTAGE * 2 == KSEGS * 1024, "K tile segments");

  // Two K and two V stages as separate objects, so the compiler can tell a load in
  // flight into one from reads of the other (the tile loop is unrolled by two for that
  // reason) and issues no wait for it.
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[KSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[KSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[VSTAGE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[VSTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: uniform, kept in an SGPR
  const int h = lane >> 5, lr = lane & 31;
  // bytes between consecutive keys; a 64-key tile spans < 2^31 bytes (checked on the host)
  const int32_t row_bytes = (int32_t)(p.kv_ss * 2);
  const bool neg = p.sc < 0.f;
  // |scale| * log2(e), held at least at the smallest normal float.  For scale = +-0 every
  // exp2 argument of an allowed key is then below 2^-26 in magnitude (|q.k| < 2^100), so
  // its weight rounds to exactly 1 as scale 0 means, while a masked score (-inf) still
  // gives exp2(-inf) = 0; with sc = 0 it would give exp2(-inf * 0) = NaN.
  const float sc = fmaxf(neg ? -p.sc : p.sc, FLT_MIN);
  const floatx16 zero16 = {};
  [[maybe_unused]] const bf16x2 ones2 = {(__bf16)1.f, (__bf16)1.f};

  // K and V loads: lane `lane` of segment seg fills 16-byte slot seg*64 + lane of the
  // tile, i.e. row slot / NCH at stored chunk slot % NCH, which holds global chunk
  // (stored chunk) ^ f(row)
  int32_t koff[KSEG_ITERS];
#pragma unroll
  for (int j = 0; j < KSEG_ITERS; ++j) {
    const int slot = (j * kWaves + wv) * 64 + lane;
    const int row = slot / NCH, pc = slot % NCH;
    koff[j] = row * row_bytes + 16 * (pc ^ tile_swz<D>(row));
  }
  int32_t voff[VSEG_ITERS];
#pragma unroll
  for (int j = 0; j < VSEG_ITERS; ++j) {
    const int slot = (j * kWaves + wv) * 64 + lane;
    const int row = slot / NCH, pc = slot % NCH;
    voff[j] = row * row_bytes + 16 * (pc ^ v_swz<D>(row));
  }
  // K operand (rows lr and lr + 32, chunk 2 ks + h), byte address: k_rd ^ (32 ks)
  const int k_rd = lr * ROWB + 16 * (h ^ tile_swz<D>(lr));
  // tr read: lane reads 4 d at row r0 = 4 h + (lane & 15) / 4 (+ 16 j, + 8), d bytes
  // 64 db + 32 ((lane >> 4) & 1) + 8 (lane & 3): byte address vt_rd ^ (64 db)
  const int vt_r0 = 4 * h + ((lane & 15) >> 2);
  const int vt_rd = vt_r0 * ROWB + 16 * ((2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ v_swz<D>(vt_r0)) +
                    8 * (lane & 1);

  // workgroup blockIdx.x takes items blockIdx.x, + gridDim.x, ... (one item when the
  // grid covers them all); with 8 kv heads, unit % Hkv == blockIdx.x % 8 keeps each
  // kv head on one XCD
  for (int64_t item = blockIdx.x; item < p.items; item += gridDim.x) {
    const int32_t rank = (int32_t)(item / p.units), unit = (int32_t)(item % p.units);
    int32_t b, rt, rec_lo, rec_hi;
    const TileRecord* recp = nullptr;
    if constexpr (DENSE) {
      b = rank / p.ntile_row;
      rt = rank % p.ntile_row;
      rec_lo = 0;
      rec_hi = p.S;
    } else {
      recp = &p.work[rank];
      b = recp->b;
      rt = recp->rt;
      rec_lo = recp->lo;
      rec_hi = recp->hi;
    }
    // the records come from the caller's workspace: never index with a value that a
    // plan for this shape cannot have written
    if (b < 0 || b >= p.B || rt < 0 || rt >= p.ntile_row) continue;
    const int32_t g = unit % p.Hkv, sub = unit / p.Hkv;
    const int32_t hq = g * p.group + sub * NH + (wv % NH);
    const int32_t blk = rt * NR + wv / NH;
    const int32_t row_local = blk * kRowsPerBlock + lr;
    const bool row_in = blk < p.nblk && row_local < p.L;
    const int32_t qpos = p.seq_start + row_local;
    // keys outside the delivered window are never loaded; a row that needs one (the
    // window does not reach back to its document start) is reported
    const int32_t tlo = max(rec_lo, p.kv_start), thi = min(rec_hi, p.kv_end);
    if (!DENSE && p.status != nullptr && tid == 0 && rec_hi > rec_lo && rec_lo < p.kv_start)
      atomicOr(p.status, PSB_DATA_KV_WINDOW);
    __bf16* out_row = p.out + (((int64_t)b * p.Hq + hq) * p.L + row_local) * D;

    if (thi <= tlo) {  // no valid query row in the whole tile: outputs are 0, lse -inf
      if (row_in) {
        const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) *(bf16x4*)(out_row + 32 * db + 8 * g4 + 4 * h) = z;
        if (p.lse != nullptr && h == 0) p.lse[((int64_t)b * p.Hq + hq) * p.L + row_local] = -INFINITY;
      }
      continue;
    }
    const int32_t ntiles = (thi - tlo + kKeysPerTile - 1) / kKeysPerTile;

    // ---- tile loads: K and V global -> LDS directly (buffer_load ... lds) -------------------
    // A resource with num_records 0 turns every lane of a load into a zero fill with no
    // memory access; the step after the last tile issues such loads into the free stage.
    const __bf16* kbase = p.k + (int64_t)b * p.kv_sb + (int64_t)g * p.kv_sh;
    const __bf16* vbase = p.v + (int64_t)b * p.kv_sb + (int64_t)g * p.kv_sh;
    auto rsrc_k = [&](int32_t kt, bool on) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)(kt - p.kv_start) * p.kv_ss), (short)0,
                                               on ? min(thi - kt, kKeysPerTile) * row_bytes : 0, kBufferFlags);
    };
    auto rsrc_v = [&](int32_t kt, bool on) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)(kt - p.kv_start) * p.kv_ss), (short)0,
                                               on ? min(thi - kt, kKeysPerTile) * row_bytes : 0, kBufferFlags);
    };
    constexpr int KFULL = KSEGS / kWaves;  // K segments every wave loads
    auto issue_k = [&](__bf16* kbuf, int32_t kt) {
      const __amdgpu_buffer_rsrc_t rk = rsrc_k(kt, true);
#pragma unroll
      for (int j = 0; j < KSEG_ITERS; ++j) {
        const int seg = j * kWaves + wv;
        if (KSEGS % kWaves == 0 || seg < KSEGS) buffer_load_lds16(rk, kbuf + seg * 512, koff[j]);
      }
    };
    auto issue_v = [&](__bf16* vbuf, int32_t kt) {
      const __amdgpu_buffer_rsrc_t rv = rsrc_v(kt, true);
#pragma unroll
      for (int j = 0; j < VSEG_ITERS; ++j) {
        const int seg = j * kWaves + wv;
        if (VSEGS % kWaves == 0 || seg < VSEGS) buffer_load_lds16(rv, vbuf + seg * 512, voff[j]);
      }
    };
    // ---- this item's Q^T operand, document id and block start ---------------------------
    // The loads that depend only on the record go out first, then the tile-0 loads, so all of
    // them are in flight together (the first use of the document id still waits for most of
    // tile 0: vmcnt counts in issue order).
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
    int32_t w_lo = 0, dq = PSB_PAD_DOC_ID;
    const uint8_t* mrow = nullptr;
    if constexpr (DENSE) {
      mrow = p.mask + (int64_t)b * p.mask_sb + (int64_t)row_local * p.mask_ss;
    } else {
      w_lo = recp->blk_lo[wv / NH];
      if (row_in) dq = p.doc[(int64_t)b * p.S + qpos];
    }
    // the previous item of this workgroup no longer reads LDS (its operands were consumed by
    // its MFMAs): a plain barrier, which leaves the loads above in flight; a workgroup's first
    // item has no predecessor and issues its tile-0 loads at once
    if (item != blockIdx.x) __builtin_amdgcn_s_barrier();
    issue_k(sK0, tlo);
    issue_v(sV0, tlo);

    // ---- per-wave query block description ------------------------------------------
    int32_t wq0 = 0, kshift = 0;
    uint32_t span = 0u;
    bool single = false;
    if constexpr (!DENSE) {
      w_lo = __builtin_amdgcn_readfirstlane(w_lo);
      const bool valid = dq != PSB_PAD_DOC_ID;
      const int32_t dprev = __shfl_up(dq, 1, kWave);
      const bool flag = (lr == 0) || (dq != dprev);
      const uint64_t fm = __ballot(flag) & 0xffffffffull;
      const uint64_t upto = fm & ((2ull << lr) - 1ull);
      const int rs = 63 - __clzll((long long)upto);             // last run start at or before my row
      wq0 = __builtin_amdgcn_readfirstlane(p.seq_start + blk * kRowsPerBlock);
      const int32_t start_q = (rs == 0) ? w_lo : wq0 + rs;       // my document's first position
      // key k is allowed iff 0 <= k - start_q <= span (unsigned compare); padding rows: none
      span = valid ? (uint32_t)(qpos - start_q) : 0u;
      kshift = valid ? start_q : 0x40000000;                     // padding: k - kshift < 0 always
      single = __builtin_amdgcn_readfirstlane(
          (fm == 1ull) && ((__ballot(valid) & 0xffffffffull) == 0xffffffffull));
    }
    // a negative scale is folded into Q (sign flip) so the loop can use |scale|
    if (neg) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        short8v bits = __builtin_bit_cast(short8v, qreg[ks]);
        bits ^= (short)0x8000;
        qreg[ks] = __builtin_bit_cast(bf16x8, bits);
      }
    }

    floatx16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = zero16;
    // p = exp2(s sc + nmsc) with the exp2 offset nmsc = -m sc for the row max m last taken,
    // l the running sum of p.  nmsc starts at FLT_MAX: a row's first finite score then gives
    // p = inf and forces the exact max, while masked scores (-inf) still give 0.
    float l_run = 0.f, nmsc = FLT_MAX;

    // S^T of one 64-key tile (both 32-key blocks, chains interleaved) from K stage `st`;
    // operands read two k-steps ahead of their MFMAs
    // Both MFMA phases (qk and softmax_pv) run at raised wave priority: the other wave on
    // the SIMD is then usually in its VALU / memory phases, and the arbiter lets the MFMA
    // issue first instead of leaving the matrix pipe idle.
    static_assert(VSEGS % kWaves == 0, "V segments split evenly over the waves");
    auto qk = [&](const __bf16* kbuf, floatx16 (&s)[2], __amdgpu_buffer_rsrc_t rkn, __bf16* knext,
                  __amdgpu_buffer_rsrc_t rvn, __bf16* vnext) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      const char* kp = (const char*)kbuf;
      constexpr int AH = (KS < 2) ? KS : 2;
      bf16x8 ka[AH][2];
#pragma unroll
      for (int ks = 0; ks < AH; ++ks) {
        ka[ks][0] = *(const bf16x8*)(kp + (k_rd ^ (32 * ks)));
        ka[ks][1] = *(const bf16x8*)(kp + 32 * ROWB + (k_rd ^ (32 * ks)));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a0 = ka[ks % AH][0], a1 = ka[ks % AH][1];
        if (ks + AH < KS) {
          ka[ks % AH][0] = *(const bf16x8*)(kp + (k_rd ^ (32 * (ks + AH))));
          ka[ks % AH][1] = *(const bf16x8*)(kp + 32 * ROWB + (k_rd ^ (32 * (ks + AH))));
        }
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], ks ? s[0] : zero16, 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], ks ? s[1] : zero16, 0, 0, 0);
        // next tile's loads, one segment per k-step: K first, then V
        if (ks < KFULL) {
          buffer_load_lds16(rkn, knext + (ks * kWaves + wv) * 512, koff[ks]);
        } else if (ks - KFULL < VSEG_ITERS) {
          buffer_load_lds16(rvn, vnext + ((ks - KFULL) * kWaves + wv) * 512, voff[ks - KFULL]);
        }
      }
#pragma unroll
      for (int j = KS - KFULL; j < VSEG_ITERS; ++j) buffer_load_lds16(rvn, vnext + (j * kWaves + wv) * 512, voff[j]);
      // keep 2*AH operand reads in flight; one load of the next tile after every k-step
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if ((i & 1) && (i >> 1) < KFULL + VSEG_ITERS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (i + 2 * AH < 2 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    };
    // mask (unless both blocks lie inside one document's causal triangle) and row max
    // explicit mask: the 32 bits this lane needs for one tile, 4 per 32-bit word (keys
    // kt + 32 kb + 4 h + 8 g + {0..3} in word 4 kb + g); keys at or past S read as 0
    auto load_mask = [&](int32_t kt, uint32_t (&mw)[8]) {
      if constexpr (DENSE) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int32_t key0 = kt + 32 * (w >> 2) + 4 * h + 8 * (w & 3);
          uint32_t x = 0u;
          if (row_in && key0 < p.S) {
            x = *(const uint32_t*)(mrow + key0);
            if (p.S - key0 < 4) x &= (1u << (8 * (p.S - key0))) - 1u;
          }
          mw[w] = x;
        }
      }
    };
    auto apply_mask = [&](floatx16 (&s)[2], const uint32_t (&mw)[8]) {
      if constexpr (DENSE) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t byte = (mw[4 * kb + (i >> 2)] >> (8 * (i & 3))) & 0xffu;
            s[kb][i] = byte ? s[kb][i] : -INFINITY;
          }
      }
    };
    // row max of the tile (retune path only): the lane's 32 scores as a tree of
    // three-input maxima (v_max3_f32), then the partner lane's
    auto tile_max = [&](const floatx16 (&s)[2]) {
      float m1[12];
#pragma unroll
      for (int j = 0; j < 10; ++j) {
        const int a = 3 * j, b = 3 * j + 1, c = 3 * j + 2;
        m1[j] = fmaxf(fmaxf(s[a >> 4][a & 15], s[b >> 4][b & 15]), s[c >> 4][c & 15]);
      }
      m1[10] = s[1][14];
      m1[11] = s[1][15];
      float m2[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) m2[j] = fmaxf(fmaxf(m1[3 * j], m1[3 * j + 1]), m1[3 * j + 2]);
      return partner_max(fmaxf(fmaxf(fmaxf(m2[0], m2[1]), m2[2]), m2[3]));
    };
    auto mask_tile = [&](int32_t kt, floatx16 (&s)[2]) {
      const bool full = DENSE || (single && kt >= w_lo && (kt + 63) <= wq0);
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int32_t e = kt + 32 * kb + 4 * h - kshift;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t rel = (uint32_t)(e + (i >> 2) * 8 + (i & 3));
            s[kb][i] = (rel <= span) ? s[kb][i] : -INFINITY;
          }
        }
      }
    };
    // P = exp2(s sc + nmsc) as bf16 for 16-key step j; acc += its sum in this lane.  The
    // plan path sums the fp32 values with plain adds: v_dot2c_f32_bf16 (a sum of the bf16
    // pair) does not issue while another wave's MFMA runs, and stalls this wave's in-order
    // VALU work behind it, where adds co-execute.  The explicit-mask variant, one mask
    // register set fuller, keeps the bf16 sum by v_dot2c, which needs no fp32 value live.
    auto softmax_step = [&](const floatx16 (&s)[2], int j, bf16x8& pj, float& acc) {
      bf16x2 pp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j >> 1][8 * (j & 1) + 2 * t], sc, nmsc));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j >> 1][8 * (j & 1) + 2 * t + 1], sc, nmsc));
        pp[t] = cvt_bf16x2(e0, e1);
        if constexpr (DENSE)
          acc = __builtin_amdgcn_fdot2_f32_bf16(pp[t], ones2, acc, false);
        else
          acc += e0 + e1;
      }
      pj = __builtin_shufflevector(__builtin_shufflevector(pp[0], pp[1], 0, 1, 2, 3),
                                   __builtin_shufflevector(pp[2], pp[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // V^T operand of 16-key step j, d block db: rows 16 j + ... and 8 rows on, same chunks
    auto vtr = [&](const char* vb, int j, int db) {
      const char* a = vb + 16 * j * ROWB + (vt_rd ^ (64 * db));
      return vtr_pair_at(a, a + 8 * ROWB);
    };
    // The offset moves (O and l are rescaled) when some lane's P for the tile sums to
    // more than 2^8: nmsc becomes -m sc for the tile's row max m wherever that lies above
    // the current offset.  A lane whose sum passed 2^8 has some p > 2^3, so there
    // m sc + nmsc > 3 and it moves; alpha = 2^(new - old) < 1, and exactly 0 at a row's first
    // finite key (nmsc starts at FLT_MAX, with O and l still 0).
    auto retune = [&](const floatx16 (&s)[2]) {
      const float mx = tile_max(s);
      const float nm = -mx * sc;
      const bool grow = nm < nmsc;
      const float alpha = grow ? __builtin_amdgcn_exp2f(nm - nmsc) : 1.f;
      nmsc = grow ? nm : nmsc;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    };
    // softmax and P V of one tile: all of the tile's P with the offset in force (V^T operands
    // of the first step read meanwhile), one wave-uniform test of the lane sums, then the
    // P V MFMAs with the next step's V^T operands read one step ahead.  With two or three
    // waves per SIMD the other waves' exp2 work runs under these MFMAs.
    // An item's first tile takes the tile's row max as its offset before any P is made: O
    // and l are still 0 there, so this is what the rescale path would do (alpha = 0 at a
    // row's first finite key) without making that tile's P twice and scaling O by 0.  A row
    // with no key in the tile keeps nmsc = FLT_MAX (its max is -inf).
    auto softmax_pv = [&](const floatx16 (&s)[2], const __bf16* vbuf, bool first) {
      const char* vb = (const char*)vbuf;
      bf16x8 pk[4];
      bf16x8 va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = vtr(vb, 0, db);
      if (first) {
        const float nm = -tile_max(s) * sc;
        nmsc = (nm < nmsc) ? nm : nmsc;
      }
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) softmax_step(s, j, pk[j], ls);
      __builtin_amdgcn_sched_barrier(0);
      if (__builtin_amdgcn_ballot_w64(ls > kRetuneSum) != 0) {  // wave-uniform (scalar) test
        retune(s);
        ls = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) softmax_step(s, j, pk[j], ls);
      }
      l_run += ls;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pk[j], o[db], 0, 0, 0);
          if (j < 3) va[db] = vtr(vb, j + 1, db);
        }
      }
#pragma unroll
      for (int i = 0; i < 4 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 3 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    };
    // ---- tile loop ----------------------------------------------------------------------
    // Step t reads K(t), V(t) from sK0 / sV0 (t even) or sK1 / sV1 (t odd), loaded straight
    // into LDS during step t-1, and starts the loads of K(t+1), V(t+1) into the other pair.
    // Those loads are spread over the K Q^T MFMAs, one 1 KiB segment per k-step: issued as
    // one burst at the top of the step they queued behind each other and held the LDS and
    // the waves longer (5-8% of the kernel time on the D = 128 workloads).
    uint32_t mA[8], mB[8];  // explicit-mask words of the current / next tile (DENSE only)
    load_mask(tlo, mA);
    auto step = [&](int32_t t, const __bf16* kcur, __bf16* knext, const __bf16* vcur, __bf16* vnext,
                    const uint32_t (&mcur)[8], uint32_t (&mnext)[8]) {
      const int32_t kt = tlo + t * kKeysPerTile;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's K(t), V(t) loads landed
      __syncthreads();                                   // K(t), V(t) visible; other stages free
      const bool more = t + 1 < ntiles;
      const __amdgpu_buffer_rsrc_t rkn = rsrc_k(kt + kKeysPerTile, more);
      const __amdgpu_buffer_rsrc_t rvn = rsrc_v(kt + kKeysPerTile, more);
      if constexpr (KSEGS % kWaves != 0) {  // the segments left over after KFULL rounds
        const int seg = KFULL * kWaves + wv;
        if (more && seg < KSEGS) buffer_load_lds16(rkn, knext + seg * 512, koff[KFULL]);
      }
      floatx16 st_s[2];
      qk(kcur, st_s, rkn, knext, rvn, vnext);
      if (more) load_mask(kt + kKeysPerTile, mnext);
      apply_mask(st_s, mcur);
      mask_tile(kt, st_s);
      softmax_pv(st_s, vcur, t == 0);
    };
    int32_t t = 0;
    for (; t + 1 < ntiles; t += 2) {
      step(t, sK0, sK1, sV0, sV1, mA, mB);
      step(t + 1, sK1, sK0, sV1, sV0, mB, mA);
    }
    if (t < ntiles) step(t, sK0, sK1, sV0, sV1, mA, mB);

    // ---- epilogue: O / l, padding rows (l == 0) -> 0 ----------------------------------
    const float l_tot = partner_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (p.lse != nullptr && row_in && h == 0) {
      // sum_k exp(scale s_k) = 2^(-nmsc) * l in the exp2 domain of the loop (nmsc is the
      // same in both partner lanes, and finite once the row has a key); a row without keys
      // gets -inf
      const float lse2 = (l_tot > 0.f) ? __log2f(l_tot) - nmsc : -INFINITY;
      p.lse[((int64_t)b * p.Hq + hq) * p.L + row_local] = lse2 * 0.69314718055994531f;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) store_block_bf16(out_row + 32 * db, o[db], inv, row_in, h);
  }  // item loop
}

int heads_per_wg(int64_t group) { return (group % 4 == 0) ? 4 : ((group % 2 == 0) ? 2 : 1); }

template <int D, bool DENSE>
hipError_t launch_attn(int nh, const AttnParams& prm, unsigned grid, hipStream_t s) {
  switch (nh) {
    case 4: attn_fwd_kernel<D, 4, DENSE><<<dim3(grid), dim3(kThreads), 0, s>>>(prm); break;
    case 2: attn_fwd_kernel<D, 2, DENSE><<<dim3(grid), dim3(kThreads), 0, s>>>(prm); break;
    default: attn_fwd_kernel<D, 1, DENSE><<<dim3(grid), dim3(kThreads), 0, s>>>(prm); break;
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

// Workgroups of the attention kernel that run at once on the current device: compute units
// x its workgroups per CU (two at D = 128, three at D = 64, set by its registers); 0 when
// the device cannot be queried (the plan then always orders longest first).
int32_t concurrent_slots(int64_t D) {
  static std::atomic<int32_t> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int32_t n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
    n = v;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n * (D == 64 ? 3 : 2);
}

psb_status plan_impl(const int32_t* doc_ids, int64_t B, int64_t L, int64_t S, int64_t D, int64_t seq_start,
                     const AttnGeometry& geo, void* workspace, size_t workspace_bytes, hipStream_t s) {
  if (doc_ids == nullptr || workspace == nullptr || !aligned16(workspace)) return PSB_ERR_INVALID_ARG;
  if (workspace_bytes < (size_t)schedule_bytes(B, L, geo.nr)) return PSB_ERR_CAPACITY;
  const ScheduleBuffers buf = schedule_carve(workspace, B, L, geo.nr);
  if (launch_schedule(doc_ids, (int32_t)B, (int32_t)S, (int32_t)L, (int32_t)seq_start, (int32_t)geo.nr,
                      concurrent_slots(D), (int32_t)geo.units, buf, s) != hipSuccess)
    return PSB_ERR_HIP;
  return PSB_OK;
}

psb_status run_impl(const void* q, const void* k, const void* v, const int32_t* doc_ids, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                    const int64_t* kv_strides, int64_t seq_start, int64_t kv_start, int64_t kv_len, float scale,
                    const AttnGeometry& geo, void* out, float* lse, void* workspace, size_t workspace_bytes,
                    int32_t* status, hipStream_t s) {
  if (!isfinite(scale)) return PSB_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || doc_ids == nullptr || out == nullptr || workspace == nullptr)
    return PSB_ERR_INVALID_ARG;
  const int64_t qs_def[3] = {Hq * L * D, L * D, D};
  const int64_t kvs_def[3] = {Hkv * kv_len * D, kv_len * D, D};
  const int64_t* qs = q_strides ? q_strides : qs_def;
  const int64_t* kvs = kv_strides ? kv_strides : kvs_def;
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || kvs[i] < 0 || (qs[i] % 8) != 0 || (kvs[i] % 8) != 0) return PSB_ERR_SHAPE;
  }
  if (qs[2] < D || kvs[2] < D) return PSB_ERR_SHAPE;
  if (kvs[2] * 2 * kKeysPerTile >= INT32_MAX) return PSB_ERR_SHAPE;  // tile offsets are 32-bit
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace))
    return PSB_ERR_INVALID_ARG;
  (void)S;
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
  prm.kv_start = (int32_t)kv_start; prm.kv_end = (int32_t)(kv_start + kv_len);
  prm.B = (int32_t)B; prm.Hq = (int32_t)Hq; prm.Hkv = (int32_t)Hkv; prm.L = (int32_t)L; prm.S = (int32_t)S;
  prm.seq_start = (int32_t)seq_start; prm.group = (int32_t)geo.group;
  prm.nblk = (int32_t)schedule_nblk(L);
  prm.ntile_row = (int32_t)(geo.ntiles / B);
  prm.units = (int32_t)geo.units;
  prm.sc = scale * kLog2e;
  prm.items = geo.grid;
  prm.work = buf.work;
  prm.lse = lse;
  prm.status = status;
  prm.mask = nullptr;
  prm.mask_sb = prm.mask_ss = 0;
  // one workgroup per item: the dispatcher starts a new one whenever a slot frees,
  // which balances the longest-first order better than a fixed persistent split
  const int64_t grid = geo.grid;
  const hipError_t e = (D == 128) ? launch_attn<128, false>((int)geo.nh, prm, (unsigned)grid, s)
                                  : launch_attn<64, false>((int)geo.nh, prm, (unsigned)grid, s);
  return e == hipSuccess ? PSB_OK : PSB_ERR_HIP;
}

// After an attention launch that returned `st`: when the caller passed a status word,
// also enqueue the check of the precondition the plan and the range mask rely on (each
// non-padding id one contiguous run of its row); a split id sets
// PSB_DATA_DOC_NOT_CONTIGUOUS.
psb_status data_check(psb_status st, const int32_t* doc_ids, int64_t B, int64_t S, int32_t* status_word,
                      hipStream_t s) {
  if (st != PSB_OK || status_word == nullptr) return st;
  return launch_contiguity_check(doc_ids, B, S, S, status_word, s);
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

PSB_API psb_status psb_blockdiag_prepare(const int32_t* cu_seqlens, int64_t cu_row_stride, int64_t n_docs,
                                         int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D,
                                         int64_t seq_start, int32_t enable_gqa, int32_t* doc_ids_out,
                                         int32_t* seg_cu_out, int32_t* seg_n_out, void* workspace,
                                         size_t workspace_bytes, int32_t* status_word, void* stream) {
  AttnGeometry geo;
  const psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (n_docs < 0 || cu_row_stride < n_docs + 1) return PSB_ERR_SHAPE;
  if (B == 0) return PSB_OK;
  if (B > 65535 || n_docs >= INT32_MAX) return PSB_ERR_SHAPE;
  if (cu_seqlens == nullptr || seg_cu_out == nullptr || seg_n_out == nullptr || (S > 0 && doc_ids_out == nullptr))
    return PSB_ERR_INVALID_ARG;
  const bool plan = Hq > 0 && L > 0;
  if (plan) {
    if (workspace == nullptr || !aligned16(workspace)) return PSB_ERR_INVALID_ARG;
    if (workspace_bytes < (size_t)schedule_bytes(B, L, geo.nr)) return PSB_ERR_CAPACITY;
  }
  const int64_t id_chunks = (S + 255) / 256;
  if (B * id_chunks + B * schedule_nblk(L) + B >= INT32_MAX) return PSB_ERR_SHAPE;
  ScheduleBuffers buf = {nullptr, nullptr, nullptr};
  if (plan) buf = schedule_carve(workspace, B, L, geo.nr);
  const hipError_t e = launch_prepare(cu_seqlens, cu_row_stride, (int32_t)n_docs, (int32_t)B, (int32_t)S,
                                      plan ? (int32_t)L : 0, (int32_t)seq_start, (int32_t)geo.nr,
                                      concurrent_slots(D), (int32_t)geo.units, doc_ids_out, seg_cu_out,
                                      seg_n_out, buf, status_word, as_stream(stream));
  return e == hipSuccess ? PSB_OK : PSB_ERR_HIP;
}

PSB_API psb_status psb_blockdiag_attn_plan(const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv, int64_t L,
                                           int64_t S, int64_t D, int64_t seq_start, int32_t enable_gqa,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  AttnGeometry geo;
  const psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  return plan_impl(doc_ids, B, L, S, D, seq_start, geo, workspace, workspace_bytes, as_stream(stream));
}

PSB_API psb_status psb_blockdiag_attn_fwd_planned(const void* q, const void* k, const void* v,
                                                  const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                  int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                                  const int64_t* kv_strides, int64_t seq_start, float scale,
                                                  int32_t enable_gqa, void* out, const void* workspace,
                                                  size_t workspace_bytes, int32_t* status_word, void* stream) {
  AttnGeometry geo;
  psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  st = run_impl(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, 0, S, scale, geo, out,
                nullptr, const_cast<void*>(workspace), workspace_bytes, nullptr, as_stream(stream));
  return data_check(st, doc_ids, B, S, status_word, as_stream(stream));
}

PSB_API psb_status psb_blockdiag_attn_fwd_lse_planned(const void* q, const void* k, const void* v,
                                                      const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                      int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                                      const int64_t* kv_strides, int64_t seq_start, float scale,
                                                      int32_t enable_gqa, void* out, float* lse,
                                                      const void* workspace, size_t workspace_bytes,
                                                      int32_t* status_word, void* stream) {
  AttnGeometry geo;
  psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  if (lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return PSB_ERR_INVALID_ARG;
  st = run_impl(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, 0, S, scale, geo, out,
                lse, const_cast<void*>(workspace), workspace_bytes, nullptr, as_stream(stream));
  return data_check(st, doc_ids, B, S, status_word, as_stream(stream));
}

namespace psb {
namespace {

// Plan + attention (+ the precondition check with a status word) into `workspace`; every
// argument is checked before anything is enqueued.
psb_status fwd_whole(const void* q, const void* k, const void* v, const int32_t* doc_ids, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                     const int64_t* kv_strides, int64_t seq_start, float scale, int32_t enable_gqa, void* out,
                     void* workspace, size_t workspace_bytes, int32_t* status_word, hipStream_t s) {
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
  if (kvs[2] * 2 * kKeysPerTile >= INT32_MAX) return PSB_ERR_SHAPE;  // tile offsets are 32-bit
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PSB_ERR_INVALID_ARG;
  st = plan_impl(doc_ids, B, L, S, D, seq_start, geo, workspace, workspace_bytes, s);
  if (st != PSB_OK) return st;
  st = run_impl(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, 0, S, scale, geo, out,
                nullptr, workspace, workspace_bytes, nullptr, s);
  return data_check(st, doc_ids, B, S, status_word, s);
}

}  // namespace
}  // namespace psb

PSB_API psb_status psb_blockdiag_attn_fwd(const void* q, const void* k, const void* v, const int32_t* doc_ids,
                                          int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S, int64_t D,
                                          const int64_t* q_strides, const int64_t* kv_strides, int64_t seq_start,
                                          float scale, int32_t enable_gqa, void* out, void* workspace,
                                          size_t workspace_bytes, int32_t* status_word, void* stream) {
  return fwd_whole(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, scale, enable_gqa, out,
                   workspace, workspace_bytes, status_word, as_stream(stream));
}

// ---- no-allocation variant ---------------------------------------------------------------
// The scheduler tables of psb_blockdiag_attn_fwd_noalloc live in this static device array:
// every GPU the library runs on holds one copy (kScratchBytes) until the process ends.  In
// host code `scratch` names a host-side stand-in, never device memory: the host uses only the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace psb {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
psb_status scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PSB_ERR_HIP;
  if (dev >= kMaxDevices) return PSB_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PSB_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PSB_OK;
}

}  // namespace
}  // namespace psb

PSB_API size_t psb_blockdiag_attn_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

PSB_API psb_status psb_blockdiag_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                                  const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                  int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                                  const int64_t* kv_strides, int64_t seq_start, float scale,
                                                  int32_t enable_gqa, void* out, int32_t* status_word,
                                                  void* stream) {
  AttnGeometry geo;
  const psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  // the plan tables must fit the static array: larger problems are refused, never truncated
  if ((size_t)schedule_bytes(B, L, geo.nr) > kScratchBytes) return PSB_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const psb_status sa = scratch_address(&ws);
  if (sa != PSB_OK) return sa;
  return fwd_whole(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, scale, enable_gqa, out,
                   ws, kScratchBytes, status_word, as_stream(stream));
}

PSB_API psb_status psb_blockdiag_attn_fwd_window_planned(const void* q, const void* k, const void* v,
                                                         const int32_t* doc_ids, int64_t B, int64_t Hq, int64_t Hkv,
                                                         int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                                         const int64_t* kv_strides, int64_t seq_start,
                                                         int64_t kv_start, int64_t kv_len, float scale,
                                                         int32_t enable_gqa, void* out, float* lse,
                                                         const void* workspace, size_t workspace_bytes,
                                                         int32_t* status_word, void* stream) {
  AttnGeometry geo;
  const psb_status st = check_attn_shape(B, Hq, Hkv, L, S, D, seq_start, enable_gqa, &geo);
  if (st != PSB_OK) return st;
  // the window holds the shard's own keys and reaches back no further than position 0
  if (kv_start < 0 || kv_len < 0 || kv_start > seq_start || kv_start + kv_len < seq_start + L ||
      kv_start + kv_len > S)
    return PSB_ERR_SHAPE;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return PSB_ERR_INVALID_ARG;
  const psb_status rs = run_impl(q, k, v, doc_ids, B, Hq, Hkv, L, S, D, q_strides, kv_strides, seq_start, kv_start,
                                 kv_len, scale, geo, out, lse, const_cast<void*>(workspace), workspace_bytes,
                                 status_word, as_stream(stream));
  return data_check(rs, doc_ids, B, S, status_word, as_stream(stream));
}

PSB_API psb_status psb_masked_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* mask,
                                       int64_t mask_batch_stride, int64_t mask_row_stride, int64_t B, int64_t Hq,
                                       int64_t Hkv, int64_t L, int64_t S, int64_t D, const int64_t* q_strides,
                                       const int64_t* kv_strides, float scale, int32_t enable_gqa, void* out,
                                       float* lse, void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 0 || L < 0 || S < 0 || D < 0) return PSB_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return PSB_ERR_UNSUPPORTED;
  if (Hq > 0 && Hkv == 0) return PSB_ERR_SHAPE;
  if (enable_gqa ? (Hkv > 0 && Hq % Hkv != 0) : (Hq != Hkv)) return PSB_ERR_SHAPE;
  if (L >= INT32_MAX || S >= INT32_MAX - 64 || Hq >= INT32_MAX || B >= INT32_MAX) return PSB_ERR_SHAPE;
  if (B == 0 || Hq == 0 || L == 0) return PSB_OK;
  if (!isfinite(scale)) return PSB_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || mask == nullptr) return PSB_ERR_INVALID_ARG;
  // the mask is read 4 bytes at a time: aligned rows, each readable up to S rounded up to 4
  if ((reinterpret_cast<uintptr_t>(mask) & 3u) != 0) return PSB_ERR_INVALID_ARG;
  if (mask_batch_stride < 0 || (mask_batch_stride % 4) != 0 || (mask_row_stride % 4) != 0 ||
      mask_row_stride < (S + 3) / 4 * 4)
    return PSB_ERR_SHAPE;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return PSB_ERR_INVALID_ARG;
  const int64_t qs_def[3] = {Hq * L * D, L * D, D};
  const int64_t kvs_def[3] = {Hkv * S * D, S * D, D};
  const int64_t* qs = q_strides ? q_strides : qs_def;
  const int64_t* kvs = kv_strides ? kv_strides : kvs_def;
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || kvs[i] < 0 || (qs[i] % 8) != 0 || (kvs[i] % 8) != 0) return PSB_ERR_SHAPE;
  }
  if (qs[2] < D || kvs[2] < D) return PSB_ERR_SHAPE;
  if (kvs[2] * 2 * kKeysPerTile >= INT32_MAX) return PSB_ERR_SHAPE;  // tile offsets are 32-bit
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PSB_ERR_INVALID_ARG;
  AttnGeometry geo;
  geo.group = Hq / Hkv;
  geo.nh = heads_per_wg(geo.group);
  geo.nr = kWaves / geo.nh;
  geo.ntiles = schedule_ntiles(B, L, geo.nr);
  geo.units = Hq / geo.nh;
  geo.grid = geo.ntiles * geo.units;
  if (geo.grid >= INT32_MAX) return PSB_ERR_SHAPE;
  AttnParams prm;
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(v);
  prm.doc = nullptr;
  prm.out = static_cast<__bf16*>(out);
  prm.q_sb = qs[0]; prm.q_sh = qs[1]; prm.q_ss = qs[2];
  prm.kv_sb = kvs[0]; prm.kv_sh = kvs[1]; prm.kv_ss = kvs[2];
  prm.kv_start = 0; prm.kv_end = (int32_t)S;
  prm.B = (int32_t)B; prm.Hq = (int32_t)Hq; prm.Hkv = (int32_t)Hkv; prm.L = (int32_t)L; prm.S = (int32_t)S;
  prm.seq_start = 0; prm.group = (int32_t)geo.group;
  prm.nblk = (int32_t)schedule_nblk(L);
  prm.ntile_row = (int32_t)(geo.ntiles / B);
  prm.units = (int32_t)geo.units;
  prm.sc = scale * kLog2e;
  prm.items = geo.grid;
  prm.work = nullptr;
  prm.lse = lse;
  prm.status = nullptr;
  prm.mask = mask;
  prm.mask_sb = mask_batch_stride;
  prm.mask_ss = mask_row_stride;
  hipStream_t s = as_stream(stream);
  const hipError_t e = (D == 128) ? launch_attn<128, true>((int)geo.nh, prm, (unsigned)geo.grid, s)
                                  : launch_attn<64, true>((int)geo.nh, prm, (unsigned)geo.grid, s);
  return e == hipSuccess ? PSB_OK : PSB_ERR_HIP;
}
