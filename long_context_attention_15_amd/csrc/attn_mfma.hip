// Gathered-entry attention on bf16 MFMA (gfx950): head dim 512 stored as
// FP8 bulk + BF16 RoPE dims, bf16 queries, 64 heads per workgroup.
//
// Work item: one query row, 64 heads, one split of its entry list (the
// top-k / visible compressed entries followed by the window rows).  Four
// wavefronts; wavefront w owns heads [16 w, 16 w + 16) over all 512 dims,
// so it needs no partial sums from the others, and two workgroups share a
// CU.  Per tile of 32 entries:
//   * the raw 576-byte rows are DMA'd into LDS one tile ahead
//     (global_load_lds), each 16-byte unit placed with a per-row rotation
//     so that both access patterns below are free of bank conflicts;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: each lane reads 8 FP8 bytes
//     (or 8 BF16 RoPE values) of its entry row and converts FP8 * row scale
//     -> BF16 in registers with the exact hardware conversion;
//   * online softmax in base 2 per head (a head is one lane column of the
//     16x16 accumulators);
//   * O^T += V^T P^T: V^T comes straight from the raw rows with the 8-bit
//     (FP8 dims) and 16-bit (RoPE dims) transposing LDS reads; the FP8 codes
//     convert unscaled and the row scale multiplies P instead; P stays in
//     registers as the B operand (its entry order is the one the S^T
//     accumulators already hold, the V^T reads follow it).
#include "common.h"
#include "launch.h"

namespace csa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kMD = 512;                 // head dim
constexpr int kMT = 32;                  // entries per tile
constexpr int kMThreads = 256;           // four wavefronts
constexpr int kMHeads = 16;              // heads per wavefront
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct MfmaArgs {
  const uint16_t* q; int B, Tq, H;
  Store ckv; int64_t n_entries; int mode; const int32_t* sel; int k; int m;
  Store win; int W; int ring; const int64_t* q_pos;
  const float* sink; float tau;
  void* out; int out_f32; float* lse; int partial;
  int nsplit; int split_len; float* ws;
};

__device__ __forceinline__ int64_t m_visible(int64_t t, int m, int64_t n) {
  int64_t v = t < 0 ? 0 : (t + 1) / m;
  return v < n ? v : n;
}

// Index of list slot i that has to come from memory (the sel entry of a
// top-k slot); other slots need no load.
__device__ __forceinline__ int m_slot_sel(const MfmaArgs& a, int64_t bq, int64_t Lc, int64_t i, int64_t i1) {
  return (a.mode == kModeSel && i < Lc && i < i1) ? a.sel[bq * a.k + i] : 0;
}

// Row of list slot i (jsel = its sel entry for top-k slots); src 0 = empty,
// 1 = compressed store, 2 = window store.
__device__ __forceinline__ int m_slot_row(const MfmaArgs& a, int b, int64_t t, int64_t Lc, int64_t i, int64_t i1,
                                          int jsel, int64_t& row) {
  row = 0;
  if (i >= i1) return 0;
  if (i < Lc) {
    const int64_t j = a.mode == kModeSel ? (int64_t)jsel : i;
    if (j < 0 || j >= a.n_entries) return 0;
    row = (int64_t)b * a.ckv.cap + j;
    return 1;
  }
  const int64_t p = t - a.W + 1 + (i - Lc);
  if (p < 0 || (!a.ring && p >= a.win.cap)) return 0;
  row = (int64_t)b * a.win.cap + (a.ring ? p % a.W : p);
  return 2;
}

// 8 FP8 codes -> 8 BF16 values times s (exact for a power-of-two s).
__device__ __forceinline__ u32x4 cvt8_fp8(u32x2 w, float s) {
  u32x4 r;
  r.x = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, s, false));
  r.y = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, s, true));
  r.z = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, s, false));
  r.w = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, s, true));
  return r;
}

// A row of zeros that empty slots gather from (device globals start zeroed).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[1024];

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRawRow = 576;                      // 448 FP8 + 64 BF16
constexpr int kUnits = kRawRow / 16;              // 16-byte units per row
constexpr int kRawTile = kMT * kRawRow;           // 18432 B = 18 wave-wide 1 KiB loads
constexpr int kRawLoads = kRawTile / 1024;

// LDS placement of 16-byte unit c of tile row r: rows follow each other,
// units rotate by unit_rot(r) within a row.  Sixteen consecutive rows
// reading the same unit then hit sixteen different 16-byte bank groups, and
// so do the row sets {0-7, 16-23} and {8-15, 24-31} that the transposing
// reads gather.
__device__ __forceinline__ int unit_rot(int r) { return ((r >> 2) ^ ((r >> 4) << 1)) & 3; }
__device__ __forceinline__ int unit_pos(int r, int c) {
  const int cc = c + unit_rot(r);
  return kUnits * r + (cc >= kUnits ? cc - kUnits : cc);
}

// Entry behind K slot 8 G + i of the PV product (G = lane >> 4): the order
// in which the S^T accumulators hold a lane's entries (16 (i >> 2) + 4 G + (i & 3)).
__device__ __forceinline__ int pv_entry(int G, int i) { return 16 * (i >> 2) + 4 * G + (i & 3); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define CSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define CSA_WAIT_VMCNT0() CSA_WAIT_VMCNT(0)

// Gathered rows come from HBM with microsecond latency: kStages tile buffers
// keep kStages - 1 tiles of row loads in flight per workgroup.
constexpr int kStages = 4;
constexpr int kSlots = 8;                         // slot tables (>= kStages + 2, power of two)
constexpr int kDmaPerWave = 5;                    // DMA loads per wave per tile (18 spread over 4 waves, padded)

__global__ __launch_bounds__(kMThreads, 1) void attn_mfma_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Raw[kStages][kRawTile];
  __shared__ const uint8_t* Tptr[kSlots][kMT];    // per tile slot: row address (zero row if empty)
  __shared__ __attribute__((aligned(16))) float Tscl[kSlots][kMT];   // row scale, 0 if empty
  __shared__ int s_over;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 4, l16 = lane & 15;           // 16-lane group and position in it
  const int64_t bq = xcd_remap(blockIdx.x, gridDim.x);   // query row (b * Tq + q)
  const int b = (int)(bq / a.Tq);
  const int h = blockIdx.y * 64 + wave * kMHeads + l16;   // this lane's head
  const int64_t t = a.q_pos ? a.q_pos[bq] : (int64_t)(bq % a.Tq);
  const int64_t Lc = a.mode == kModeSel ? a.k : (a.mode == kModeRange ? m_visible(t, a.m, a.n_entries) : 0);
  const int64_t L = Lc + a.W;
  const int64_t i0 = (int64_t)blockIdx.z * a.split_len;
  const int64_t i1 = a.nsplit == 1 ? L : (i0 + a.split_len < L ? i0 + a.split_len : L);
  const int ntiles = i1 > i0 ? (int)((i1 - i0 + kMT - 1) / kMT) : 0;

  // slot table of tile `tile` (threads < 32 own one slot each): the row
  // address is stored now, the row scale is loaded now and returned, to be
  // stored one iteration later so its latency never sits on the tile loop.
  auto table_ptr = [&](int tile, int jsel) -> float {
    int64_t row;
    const int64_t slot = i0 + (int64_t)tile * kMT + tid;
    const int src = m_slot_row(a, b, t, Lc, slot, i1, jsel, row);
    const Store& stv = src == 2 ? a.win : a.ckv;
    Tptr[tile & (kSlots - 1)][tid] = src ? stv.rows + row * stv.row_bytes : g_zero_row;
    return src ? ((const float*)stv.scales)[row] : 0.0f;
  };
  auto sel_of = [&](int tile) -> int {
    return m_slot_sel(a, bq, Lc, i0 + (int64_t)tile * kMT + tid, i1);
  };
  // DMA the raw rows of `tile` into Raw[tile % kStages]: 18 wave-wide loads
  // of 1 KiB; lane l of load qd fills LDS unit 64 qd + l, i.e. the (row,
  // unit) that unit_pos places there.  Every wave issues kDmaPerWave loads
  // (waves 2 and 3 repeat one load of theirs, writing the same bytes again)
  // so that all waves can wait on the same vmcnt.
  auto dma_tile = [&](int tile) {
    uint8_t* dst = Raw[tile % kStages];
    const uint8_t* const* tp = Tptr[tile & (kSlots - 1)];
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      int qd = wave + 4 * j;
      qd = qd < kRawLoads ? qd : qd - 4;
      const int u = qd * 64 + lane;
      const int r = u / kUnits, cc = u - r * kUnits;
      int c = cc - unit_rot(r);
      c = c < 0 ? c + kUnits : c;
      __builtin_amdgcn_global_load_lds((const void*)(tp[r] + 16 * c), (lds_void*)(dst + 1024 * qd), 16, 0, 0);
    }
  };

  // Q^T operands: K-step ks covers dims [32 ks, 32 ks + 32); lane group G
  // takes dims 32 ks + 8 G .. +8.  Steps 0..13 are the FP8 dims, 14 and 15
  // the BF16 RoPE dims.
  bf16x8 qf[16];
  {
    const uint16_t* qp = a.q + (bq * a.H + h) * (int64_t)kMD + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 32 * ks));
  }
  // LDS byte offsets (within a tile) of this lane's reads.
  // S^T A operand, row block eb: entry 16 eb + l16; FP8 K-step ks reads bytes
  // 32 ks + 8 G .. +8 = unit 2 ks + (G >> 1), half G & 1; RoPE step 14 + j
  // reads BF16 dims 32 j + 8 G = unit 28 + 4 j + G.
  int s_fp8[2], s_rope[2][2];
#pragma unroll
  for (int eb = 0; eb < 2; ++eb) {
    const int e = 16 * eb + l16;
    s_fp8[eb] = 16 * (kUnits * e + unit_rot(e) + (G >> 1)) + 8 * (G & 1);   // + 32 ks
#pragma unroll
    for (int j = 0; j < 2; ++j) s_rope[eb][j] = 16 * unit_pos(e, 28 + 4 * j + G);
  }
  // V^T A operand, FP8 dim block db (dims 16 db .. +16, unit db): lane
  // (16 G + l16) points at entry pv_entry(G, l16 >> 1), half l16 & 1.
  const int ve = pv_entry(G, l16 >> 1);
  const int v_fp8 = 16 * (kUnits * ve + unit_rot(ve)) + 8 * (l16 & 1);            // + 16 db
  // V^T A operand, RoPE dim block 28 + j, j < 4 (bf16 dims 16 j .. +16), read hh:
  // entry pv_entry(G, 4 hh + (l16 >> 2)), bf16 dims 16 j + 4 (l16 & 3).
  int v_rope[4][2];                                                                 // [j][hh]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int e = pv_entry(G, 4 * hh + (l16 >> 2));
      const int dbyte = 448 + 2 * (16 * j + 4 * (l16 & 3));
      v_rope[j][hh] = 16 * unit_pos(e, dbyte >> 4) + (dbyte & 15);
    }

  f32x4 acc[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) acc[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const float sc2 = a.tau * kLog2e;
  // Softmax reference (log2 units, per head = per lane column): fixed at the
  // head's first non-empty tile and never moved, so no VALU code ever touches
  // the O^T accumulators.  Probabilities relative to it stay below
  // 2^kMaxLift; if some logit climbs further (not seen with normalised
  // inputs) the whole query is recomputed once with the exact maximum, which
  // the first pass tracks in mmax.
  constexpr float kMaxLift = 64.0f;
  float mref = -INFINITY, mmax = -INFINITY, lrun = 0.0f;
  if (tid == 0) s_over = 0;

#pragma nounroll
  for (int attempt = 0; attempt < 2; ++attempt) {
    // ---- prologue: tables of tiles 0 .. kStages-1, rows of tiles 0 .. kStages-2
    // (iteration it stores the scale of tile it + kStages - 1, computes the
    // table of tile it + kStages and loads the sel of tile it + kStages + 1)
    int selreg = 0;
    float scl_pending = 0.0f;
    if (tid < kMT) {
      int jn = sel_of(0);
#pragma unroll
      for (int tl = 0; tl < kStages; ++tl) {
        const int jcur = jn;
        jn = sel_of(tl + 1);
        const float sv = table_ptr(tl, jcur);
        if (tl < kStages - 1) Tscl[tl][tid] = sv;
        else scl_pending = sv;
      }
      selreg = jn;
    }
    __syncthreads();
#pragma unroll
    for (int tl = 0; tl < kStages - 1; ++tl)
      if (tl < ntiles) dma_tile(tl);
    CSA_WAIT_VMCNT0();
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
      if (tid < kMT) {
        Tscl[(it + kStages - 1) & (kSlots - 1)][tid] = scl_pending;
        if (it + kStages < ntiles) scl_pending = table_ptr(it + kStages, selreg);
        if (it + kStages + 1 < ntiles) selreg = sel_of(it + kStages + 1);
      }
      // rows of tile it + kStages - 1 (its table was written one iteration ago)
      if (it + kStages - 1 < ntiles) dma_tile(it + kStages - 1);
      const uint8_t* raw = Raw[it % kStages];
      const float* tsc = Tscl[it & (kSlots - 1)];

      // ---- S^T = K Q^T: two row blocks of 16 entries, this wave's 16 heads.
      // All fragment reads are issued first so that their LDS latency
      // overlaps the conversions and MFMAs.
      u32x2 kf[2][14];
      u32x4 kr[2][2];
#pragma unroll
      for (int ks = 0; ks < 14; ++ks)
#pragma unroll
        for (int eb = 0; eb < 2; ++eb) kf[eb][ks] = *(const u32x2*)(raw + s_fp8[eb] + 32 * ks);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int eb = 0; eb < 2; ++eb) kr[eb][j] = *(const u32x4*)(raw + s_rope[eb][j]);
      __builtin_amdgcn_sched_barrier(0);            // keep the reads ahead of their uses
      f32x4 sa[2], sb[2];                           // even / odd K-step chains
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) { sa[eb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f}; sb[eb] = sa[eb]; }
      const float srow0 = tsc[l16], srow1 = tsc[16 + l16];
#pragma unroll
      for (int ks = 0; ks < 14; ++ks) {
#pragma unroll
        for (int eb = 0; eb < 2; ++eb) {
          const u32x4 k = cvt8_fp8(kf[eb][ks], eb ? srow1 : srow0);
          if (ks & 1) sb[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), qf[ks], sb[eb], 0, 0, 0);
          else sa[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), qf[ks], sa[eb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int eb = 0; eb < 2; ++eb) {
          if (j) sb[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[eb][j]), qf[14 + j], sb[eb], 0, 0, 0);
          else sa[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[eb][j]), qf[14 + j], sa[eb], 0, 0, 0);
        }
      // V^T fragments for the PV product, read now so that the softmax below
      // covers their latency
      v2i32 vf[28];
#pragma unroll
      for (int db = 0; db < 28; ++db) vf[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(raw + v_fp8 + 16 * db));
      v4i16 vr[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) vr[j][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(raw + v_rope[j][hh]));

      // ---- softmax; lane holds entries 16 (i >> 2) + 4 G + (i & 3), i = 0..7, of head h
      const unsigned int vmask = (unsigned int)__ballot(lane < 32 && tsc[lane & 31] > 0.0f);
      float p[8];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = pv_entry(G, i);
        const float tot = sa[i >> 2][i & 3] + sb[i >> 2][i & 3];
        p[i] = ((vmask >> e) & 1u) ? tot * sc2 : -INFINITY;
        mt = fmaxf(mt, p[i]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      mmax = fmaxf(mmax, mt);
      if (mref == -INFINITY) mref = mt;     // the head's first non-empty tile
      if (__ballot(mt > mref + kMaxLift) != 0ull && lane == 0) s_over = 1;
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = mref > -INFINITY ? exp2f(p[i] - mref) : 0.0f;
        psum += p[i];
      }
      psum += __shfl_xor(psum, 16);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
        psum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      lrun += psum;
      // P^T operands: raw for the RoPE dims, times the row scale for the FP8 dims
      bf16x8 pr, ps;
      {
        const float4 e0 = *(const float4*)(tsc + 4 * G), e1 = *(const float4*)(tsc + 16 + 4 * G);
        const float es[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pr[i] = (__bf16)p[i];
          ps[i] = (__bf16)(p[i] * es[i]);
        }
      }

      // ---- O^T += V^T P^T over 32 dim blocks of 16
#pragma unroll
      for (int db = 0; db < 28; ++db) {
        const u32x4 v = cvt8_fp8(u32x2{(unsigned)vf[db].x, (unsigned)vf[db].y}, 1.0f);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), ps, acc[db], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 ux0 = __builtin_bit_cast(u32x2, vr[j][0]), ux1 = __builtin_bit_cast(u32x2, vr[j][1]);
        const u32x4 v = u32x4{ux0.x, ux0.y, ux1.x, ux1.y};
        acc[28 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pr, acc[28 + j], 0, 0, 0);
      }
      // the rows of tile it+1 are in: loads complete in order, and after
      // them this wave issued the DMA of the next kStages - 2 tiles (plus,
      // on wave 0, some table loads), so allowing that many DMA loads to be
      // outstanding is safe; near the end of the list fewer were issued, so
      // wait for everything there
      if (it + kStages - 1 < ntiles) CSA_WAIT_VMCNT((kStages - 2) * kDmaPerWave);
      else CSA_WAIT_VMCNT0();
      __syncthreads();
    }
    __syncthreads();
    if (!s_over) break;                     // uniform
    // recompute with the exact per-head maximum (mref >= every logit now)
#pragma unroll
    for (int db = 0; db < 32; ++db) acc[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lrun = 0.0f;
    mref = mmax;
    __syncthreads();
    if (tid == 0) s_over = 0;
  }
  const float mrun = mref;

  // ---- epilogue: lane holds O^T rows (dims) 16 db + 4 G + (0..3) of head h
  const int64_t qoff = (bq * a.H + h) * (int64_t)kMD;
  if (a.nsplit > 1) {
    // partial: m (natural log units), l, unnormalised o
    float* wo = a.ws + ((bq * a.H + h) * a.nsplit + blockIdx.z) * (int64_t)kMD;
    float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * a.nsplit * kMD + ((bq * a.H + h) * a.nsplit + blockIdx.z) * 2;
#pragma unroll
    for (int db = 0; db < 32; ++db)
      *(float4*)(wo + 16 * db + 4 * G) = make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
    if (G == 0) {
      wml[0] = mrun > -INFINITY ? mrun * kLn2 : -INFINITY;
      wml[1] = lrun;
    }
    return;
  }
  const float sig2 = (a.partial || !a.sink) ? -INFINITY : a.sink[h] * kLog2e;
  const float M = fmaxf(mrun, sig2);
  float scale = 0.0f, lse = -INFINITY;
  if (M > -INFINITY) {
    const float fm = mrun > -INFINITY ? exp2f(mrun - M) : 0.0f;
    const float Z = lrun * fm + (sig2 > -INFINITY ? exp2f(sig2 - M) : 0.0f);
    scale = fm / Z;
    lse = (M + log2f(Z)) * kLn2;
  }
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    const int d = 16 * db + 4 * G;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[db][i] * scale;
    if (a.out_f32) {
      *(float4*)((float*)a.out + qoff + d) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      u32x2 w;
      w.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      w.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      *(u32x2*)((uint16_t*)a.out + qoff + d) = w;
    }
  }
  if (a.lse && G == 0) a.lse[bq * a.H + h] = lse;
}

bool attn_mfma_eligible(int q_fmt, int H, int D, const csa_store& kv, bool has_prior) {
  return !has_prior && q_fmt == CSA_BF16 && D == kMD && H % 64 == 0 && kv.fmt == CSA_FP8_E4M3 &&
         kv.row_bytes == kRawRow;
}

hipError_t launch_attn_mfma(const AttnCall& c, int nsplit, int split_len, hipStream_t st) {
  MfmaArgs a;
  a.q = (const uint16_t*)c.q; a.B = c.B; a.Tq = c.Tq; a.H = c.H;
  a.ckv = c.ckv.rows ? view(c.ckv) : view(c.win);
  a.n_entries = c.n_entries; a.mode = c.mode; a.sel = c.sel; a.k = c.k; a.m = c.m;
  a.win = c.win.rows ? view(c.win) : a.ckv;
  a.W = c.W; a.ring = c.ring; a.q_pos = c.q_pos;
  a.sink = c.sink; a.tau = c.tau;
  a.out = c.out; a.out_f32 = c.partial; a.lse = c.lse; a.partial = c.partial;
  a.nsplit = nsplit; a.split_len = split_len; a.ws = (float*)c.ws;
  const dim3 grid((unsigned)((int64_t)c.B * c.Tq), c.H / 64, nsplit);
  hipLaunchKernelGGL(attn_mfma_kernel, grid, dim3(kMThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
