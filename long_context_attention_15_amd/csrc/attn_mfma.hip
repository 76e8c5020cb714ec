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
constexpr float kEmpty = -1.0e30f;          // logit of an empty slot
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

// Converted tile: 32 rows of 512 BF16 (FP8 dims times the row scale, exact
// since row scales are powers of two; RoPE dims as stored), 1 KiB per row.
// 16-byte unit u of row r sits at unit u ^ (r & 15): the sixteen rows that a
// 128-bit S^T operand read gathers then hit sixteen different 16-byte bank
// groups (measured on gfx950: 180 B/clk/CU, against 128 B/clk for a
// stride-2 pattern and 199 B/clk for a plain contiguous read).
__device__ __forceinline__ int kb_swz(int r) { return r & 15; }

// Gathered rows come from HBM with microsecond latency.  Pipeline per
// iteration it: products on converted tile it, conversion of raw tile it+1,
// row DMA of tile it+4 into the raw buffer that tile it's conversion freed
// (kStages buffers, three tiles of row loads in flight behind the one being
// waited for), slot table of tile it+5.
constexpr int kStages = 4;
constexpr int kLead = kStages;                    // DMA distance in tiles
constexpr int kSlots = 16;                        // slot tables (two build batches of 8 tiles)
constexpr int kBatch = 8;                         // tiles per table build (2 per wavefront)
constexpr int kDmaWaves = 3;                      // waves 0-2 issue the row DMA, wave 3 builds the slot tables
constexpr int kDmaPerWave = kRawLoads / kDmaWaves; // 6 wave-wide loads each

// 16-byte-per-lane LDS DMA (global_load_lds_dwordx4: lane l's 16 bytes land
// at LDS dst + 16 l), written as inline asm.  The compiler's own LDS-DMA
// bookkeeping would otherwise put full LDS and vector-memory waits on the
// next LDS accesses; completion is tracked here by explicit vmcnt waits
// (the asm has no register result, only the address input).
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ void dma4(const void* src, void* dst) {
  const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__global__ __launch_bounds__(kMThreads, 1) void attn_mfma_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Raw[kStages][kRawTile];
  __shared__ __attribute__((aligned(16))) uint8_t Kb[2][kMT * 1024];   // converted tiles (bf16, scaled)
  __shared__ const uint8_t* Tptr[kSlots][kMT];    // per tile slot: row address (zero row if empty)
  __shared__ __attribute__((aligned(16))) float Tscl[kSlots][kMT];   // row scale, 0 if empty
  __shared__ __attribute__((aligned(16))) float Tbias[kSlots][kMT];  // 0 for a filled slot, kEmpty for an empty one
  __shared__ __attribute__((aligned(16))) int32_t Tsel[kSlots][kMT];  // sel entries (top-k lists)
  __shared__ __attribute__((aligned(16))) uint8_t DmaSink[1024];   // target of wave 3's stand-in loads
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

  // Slot tables of tiles `tile` and tile + 1 (tile even), built by one
  // wavefront (lane tl owns slot i0 + 32 tile + tl of the entry list: the
  // W window rows first, whose addresses need no sel entry, then the Lc
  // top-k / visible compressed entries; lanes 32-63 fill slot row ts + 1 of
  // the tables).  All four wavefronts build
  // together, 8 tiles every 8 iterations, so the work never leaves one
  // wavefront behind at the tile barrier.  The row address and
  // the softmax bias are stored now; the row scale goes to Tscl by LDS DMA,
  // as the sel entries go to Tsel one batch earlier, so no load result ever
  // sits in a register of the tile loop.  Slot arithmetic is 32-bit (lists
  // stay far below 2^31 entries); empty slots read the zero row and a zero
  // scale.
  const int tl = lane;
  const int i0i = (int)i0, i1i = (int)i1;
  const int win_p0 = (int)(t - a.W + 1);             // window position of slot x < W
  const bool sel_mode = a.mode == kModeSel;
  const int n_ent = (int)a.n_entries, win_cap = (int)a.win.cap;
  const uint8_t* const ckv_base = a.ckv.rows + (size_t)b * a.ckv.cap * a.ckv.row_bytes;
  const float* const ckv_sc = (const float*)a.ckv.scales + (size_t)b * a.ckv.cap;
  const uint8_t* const win_base = a.win.rows + (size_t)b * a.win.cap * a.win.row_bytes;
  const float* const win_sc = (const float*)a.win.scales + (size_t)b * a.win.cap;
  const int32_t* const sel_row = sel_mode ? a.sel + bq * a.k : nullptr;
  auto table2 = [&](int tile, int jsel) {
    const int ts = tile & (kSlots - 1);            // even
    const int slot = i0i + tile * kMT + tl;        // tl < 64 spans both tiles
    int p = win_p0 + slot;                         // window position (slots < W)
    const bool p_ok = p >= 0 && (a.ring || p < win_cap);
    if (a.ring) p = p >= 0 ? p % a.W : 0;          // uniform branch
    const bool in_list = slot < i1i, is_c = slot >= a.W;
    const int j = sel_mode ? jsel : slot - a.W;
    const bool ok = in_list && (is_c ? (unsigned)j < (unsigned)n_ent : p_ok);
    const int idx = is_c ? j : p;
    const uint8_t* ptr = (is_c ? ckv_base : win_base) + (size_t)idx * (is_c ? a.ckv.row_bytes : a.win.row_bytes);
    const float* sp = (is_c ? ckv_sc : win_sc) + idx;
    (&Tptr[0][0])[ts * kMT + tl] = ok ? ptr : g_zero_row;
    (&Tbias[0][0])[ts * kMT + tl] = ok ? 0.0f : kEmpty;
    dma4(ok ? (const void*)sp : (const void*)g_zero_row, &Tscl[ts][0]);
  };
  // sel entries of tiles `tile` and tile + 1 (tile even), DMA'd into Tsel
  // (top-k slots only; others read a zero)
  auto sel_dma2 = [&](int tile) {
    const int slot = i0i + tile * kMT + tl;
    dma4(sel_mode && slot >= a.W && slot < i1i ? (const void*)(sel_row + (slot - a.W)) : (const void*)g_zero_row,
         &Tsel[tile & (kSlots - 1)][0]);
  };
  // DMA of the raw rows of `tile` into Raw[tile % kStages]: 18 wave-wide
  // loads of 1 KiB, kDmaPerWave on each of waves 0-2; lane l of load qd
  // fills LDS unit 64 qd + l, i.e. the (row, unit) that unit_pos places
  // there.  dma_src reads the slot table (early, so that its LDS latency is
  // hidden); the loads go out in the tile loop and the prologue.
  // Per load j: the slot-table row and the byte offset within the row of
  // this lane's 16 bytes (fixed per lane); wave 3 mirrors wave 0's rows.
  int dma_row[kDmaPerWave], dma_off[kDmaPerWave];
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int qd = (wave < kDmaWaves ? wave : 0) + kDmaWaves * j;
    const int u = qd * 64 + lane;
    const int r = u / kUnits, cc = u - r * kUnits;
    int c = cc - unit_rot(r);
    c = c < 0 ? c + kUnits : c;
    dma_row[j] = r;
    dma_off[j] = 16 * c;
  }
  const bool dma_sink = __builtin_amdgcn_readfirstlane(wave) >= kDmaWaves;
  struct DmaSrc { const uint8_t* p[kDmaPerWave]; };
  auto dma_src = [&](int tile) {
    DmaSrc d;
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) d.p[j] = Tptr[tile & (kSlots - 1)][dma_row[j]];
    return d;
  };


  // the head's sink logit (log2 units), loaded now so that the epilogue
  // does not wait a memory round trip for it
  const float sig2 = (a.nsplit > 1 || a.partial || !a.sink) ? -INFINITY : a.sink[h] * kLog2e;
  // Q^T operands: K-step ks covers dims [32 ks, 32 ks + 32); lane group G
  // takes dims 32 ks + 8 G .. +8.  Steps 0..13 are the FP8 dims, 14 and 15
  // the BF16 RoPE dims.
  bf16x8 qf[16];
  {
    const uint16_t* qp = a.q + (bq * a.H + h) * (int64_t)kMD + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 32 * ks));
  }
  // LDS byte offsets (within a converted tile) of this lane's reads.
  // S^T A operand, row block eb, K-step ks: entry 16 eb + l16, unit 4 ks + G,
  // i.e. byte 16384 eb + 256 (ks >> 2) + s_off[ks & 3].
  int s_off[4];
  {
    const int x = 16 * (G ^ kb_swz(l16));
#pragma unroll
    for (int j = 0; j < 4; ++j) s_off[j] = l16 * 1024 + ((64 * j) ^ x);
  }
  // V^T A operand, dim block db (dims 16 db .. +16), read hh: entry
  // pv_entry(G, 4 hh + (l16 >> 2)) = 16 hh + 4 G + (l16 >> 2), dims
  // 16 db + 4 (l16 & 3) .. +4, i.e. byte 16384 hh + 256 (db >> 3) + v_off[db & 7].
  int v_off[8];
  {
    const int r = 4 * G + (l16 >> 2);
    const int y = 16 * (((l16 >> 1) & 1) ^ kb_swz(r));
#pragma unroll
    for (int j = 0; j < 8; ++j) v_off[j] = r * 1024 + ((32 * j) ^ y) + 8 * (l16 & 1);
  }
  // conversion of a raw tile into Kb: thread -> row tid >> 3; FP8 chunks
  // 7 (tid & 7) + j, j < 7 (8 dims each, one 16-byte BF16 unit), and RoPE
  // unit 56 + (tid & 7)
  const int cv_row = tid >> 3, cv_sub = tid & 7, cv_swz = kb_swz(cv_row);
  auto convert_tile = [&](int tile) {
    const uint8_t* raw = Raw[tile % kStages];
    uint8_t* dst = Kb[tile & 1] + cv_row * 1024;
    const float sc = Tscl[tile & (kSlots - 1)][cv_row];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int c = 7 * cv_sub + j;
      const u32x2 w = *(const u32x2*)(raw + 16 * unit_pos(cv_row, c >> 1) + 8 * (c & 1));
      *(u32x4*)(dst + 16 * (c ^ cv_swz)) = cvt8_fp8(w, sc);
    }
    *(u32x4*)(dst + 16 * ((56 + cv_sub) ^ cv_swz)) = *(const u32x4*)(raw + 16 * unit_pos(cv_row, 28 + cv_sub));
  };

  f32x4 acc[32];
#pragma unroll
  for (int db = 0; db < 32; ++db) acc[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const float sc2 = a.tau * kLog2e;
  // Softmax reference (log2 units, per head = per lane column): fixed at the
  // head's first non-empty tile and never moved, so no VALU code ever touches
  // the O^T accumulators.  Probabilities relative to it stay below
  // 2^kMaxLift; if some logit climbs further (not seen with normalised
  // inputs) the whole query is recomputed once with the exact maximum, which
  // the first pass tracks as xmax.
  constexpr float kMaxLift = 64.0f;
  // mref: reference (log2 units) once mset; xmax: largest logit relative
  // to it; lrun: this lane's share of the denominator (both reduced over the
  // head's 4 lanes after the tile loop).
  float mref = 0.0f, xmax = -INFINITY, lrun = 0.0f;
  bool mset = false;
  if (tid == 0) s_over = 0;

#pragma nounroll
  for (int attempt = 0; attempt < 2; ++attempt) {
    // ---- prologue: sel entries of tiles 0 .. 15, tables of tiles 0 .. 7,
    // rows of tiles 0 .. kLead-1, tile 0 converted.  Iterations it = 0 mod 8
    // build the tables of tiles it + 8 .. it + 15 (wave w: it + 8 + 2 w and
    // the next) and DMA the sel entries of tiles it + 16 .. it + 23.
    // The first kLead tiles hold window rows when the split starts the list
    // and the window spans them (or the list has no sel entries): their row
    // loads then go out before the sel entries of the top-k tiles arrive,
    // which waves 2 and 3 wait for to build tiles 4 .. 7.  Otherwise every
    // wave waits for its sel entries first.  Scale and sel loads issued
    // before a wave's row loads complete before them; barriers without the
    // release fence of __syncthreads (which would wait for every load in
    // flight).
    const bool early = !sel_mode || (i0i == 0 && a.W >= kLead * kMT);
    const bool need_sel = sel_mode && i0i + (2 * wave + 2) * kMT > a.W;   // wave-uniform
    sel_dma2(2 * wave);
    sel_dma2(kBatch + 2 * wave);
    if (early) {
      if (!need_sel) table2(2 * wave, 0);      // window rows / lists without sel entries
    } else {
      CSA_WAIT_VMCNT0();
      asm volatile("" ::: "memory");
      table2(2 * wave, (&Tsel[0][0])[2 * wave * kMT + tl]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // rows of tiles 0 .. kLead-1, branch-free like the loop's (zero rows
    // past the end of the list, wave 3 into the sink)
#pragma unroll
    for (int pt = 0; pt < kLead; ++pt) {
      const DmaSrc d = dma_src(pt);
#pragma unroll
      for (int j = 0; j < kDmaPerWave; ++j) {
        const uint8_t* src = dma_sink ? g_zero_row + 16 * lane : d.p[j] + dma_off[j];
        uint8_t* dst = dma_sink ? DmaSink : Raw[pt] + 1024 * (wave + kDmaWaves * j);
        dma16(src, dst);
      }
    }
    if (early && need_sel) {
      // sel entries of tiles 2 w, 2 w + 1 in (only the second sel load and
      // the kLead kDmaPerWave row loads may still be in flight), then the
      // tables and tiles 0, 1 (their scale load may stay in flight)
      CSA_WAIT_VMCNT(kLead * kDmaPerWave + 1);
      asm volatile("" ::: "memory");
      table2(2 * wave, (&Tsel[0][0])[2 * wave * kMT + tl]);
      CSA_WAIT_VMCNT(2 * kDmaPerWave + 1);
    } else {
      CSA_WAIT_VMCNT(2 * kDmaPerWave);         // tiles 0 and 1 in (loads complete in order)
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    convert_tile(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    for (int it = 0; it < ntiles; ++it) {
      // slot-table reads of this iteration go out first
      const DmaSrc dsrc = dma_src(it + kLead);
      const float* tbs = Tbias[it & (kSlots - 1)];
      const float4 eb0 = *(const float4*)(tbs + 4 * G), eb1 = *(const float4*)(tbs + 16 + 4 * G);
      if ((it & (kBatch - 1)) == 0) {
        // past the end of the list the tables hold empty slots (zero rows).
        // Tile X's tables are built at iteration X-15 .. X-8 and last read at
        // iteration X; its sel entries arrive at X-23 .. X-16 and are read at
        // the build: 16 slot rows cover both.  Table DMAs (2 per wave) go out
        // before the row loads of the iteration, so the wait at its end
        // leaves them in flight and the next iteration's wait lands them,
        // long before their first use.
        table2(it + kBatch + 2 * wave, (&Tsel[0][0])[((it + kBatch + 2 * wave) & (kSlots - 1)) * kMT + tl]);
        sel_dma2(it + 2 * kBatch + 2 * wave);
      }
      const uint8_t* kb = Kb[it & 1];

      // The phases below are issued in a fixed order (scheduling barriers
      // between groups): with one wavefront per SIMD the LDS reads must run
      // ahead of their MFMAs.

      // raw rows of the next tile for this thread's conversion share (tile
      // it+1 < ntiles; past the end the stale buffer converts into a tile
      // that is never read)
      const uint8_t* craw = Raw[(it + 1) % kStages];
      uint8_t* cdst = Kb[(it + 1) & 1] + cv_row * 1024;
      const float csc = Tscl[(it + 1) & (kSlots - 1)][cv_row];
      u32x2 cw[7];
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        const int c = 7 * cv_sub + j;
        cw[j] = *(const u32x2*)(craw + 16 * unit_pos(cv_row, c >> 1) + 8 * (c & 1));
      }
      const u32x4 crope = *(const u32x4*)(craw + 16 * unit_pos(cv_row, 28 + cv_sub));

      // ---- S^T = K Q^T: two row blocks of 16 entries, this wave's 16 heads.
      // The even chain starts at 0 for a filled slot and at kEmpty for an
      // empty one, so empty slots drop out of the softmax by themselves.
      constexpr int kSD = 3;                        // K-step read distance (measured best)
      f32x4 sa[2], sb[2];                           // even / odd K-step chains
      sa[0] = f32x4{eb0.x, eb0.y, eb0.z, eb0.w};
      sa[1] = f32x4{eb1.x, eb1.y, eb1.z, eb1.w};
      sb[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      sb[1] = sb[0];
      u32x4 kq[16][2];
#pragma unroll
      for (int ks = 0; ks < kSD; ++ks) {
        kq[ks][0] = *(const u32x4*)(kb + 256 * (ks >> 2) + s_off[ks & 3]);
        kq[ks][1] = *(const u32x4*)(kb + 16384 + 256 * (ks >> 2) + s_off[ks & 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        if (ks + kSD < 16) {
          const int kn = ks + kSD;
          kq[kn][0] = *(const u32x4*)(kb + 256 * (kn >> 2) + s_off[kn & 3]);
          kq[kn][1] = *(const u32x4*)(kb + 16384 + 256 * (kn >> 2) + s_off[kn & 3]);
        }
        if (ks & 1) {
          sb[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kq[ks][0]), qf[ks], sb[0], 0, 0, 0);
          sb[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kq[ks][1]), qf[ks], sb[1], 0, 0, 0);
        } else {
          sa[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kq[ks][0]), qf[ks], sa[0], 0, 0, 0);
          sa[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kq[ks][1]), qf[ks], sa[1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- V^T reads for the first kVD dim blocks go out before the softmax
      constexpr int kVD = 6;                        // dim-block read distance
      u32x4 vq[32];
#pragma unroll
      for (int db = 0; db < kVD; ++db) {
        const uint8_t* vp = kb + 256 * (db >> 3) + v_off[db & 7];
        const u32x2 x0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)vp));
        const u32x2 x1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 16384)));
        vq[db] = u32x4{x0.x, x0.y, x1.x, x1.y};
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- conversion of the next tile, interleaved with the softmax below
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        const int c = 7 * cv_sub + j;
        *(u32x4*)(cdst + 16 * (c ^ cv_swz)) = cvt8_fp8(cw[j], csc);
      }
      *(u32x4*)(cdst + 16 * ((56 + cv_sub) ^ cv_swz)) = crope;

      // ---- softmax; lane holds entries 16 (i >> 2) + 4 G + (i & 3), i = 0..7, of head h
      float tot[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) tot[i] = sa[i >> 2][i & 3] + sb[i >> 2][i & 3];
      if (!mset && __ballot(eb0.x == 0.0f || eb0.y == 0.0f || eb0.z == 0.0f || eb0.w == 0.0f ||
                            eb1.x == 0.0f || eb1.y == 0.0f || eb1.z == 0.0f || eb1.w == 0.0f) != 0ull) {
        // first tile with a filled slot (slots are shared by all heads, so
        // this is wave-uniform): each head's reference is its maximum over
        // the tile, reduced over the head's 4 lanes
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) mt = fmaxf(mt, tot[i] * sc2);
        {
          const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
          mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
          mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        mref = mt;
        mset = true;
      }
      float psum = 0.0f;
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = fmaf(tot[i], sc2, -mref);
        xmax = fmaxf(xmax, x);
        const float pv = __builtin_amdgcn_exp2f(x);
        psum += pv;
        pb[i] = (__bf16)pv;
      }
      lrun += psum;
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T += V^T P^T over 32 dim blocks of 16
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        if (db + kVD < 32) {
          const int dn = db + kVD;
          const uint8_t* vp = kb + 256 * (dn >> 3) + v_off[dn & 7];
          const u32x2 x0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)vp));
          const u32x2 x1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 16384)));
          vq[dn] = u32x4{x0.x, x0.y, x1.x, x1.y};
        }
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vq[db]), pb, acc[db], 0, 0, 0);
        // rows of tile it + kLead, one load every four dim blocks (its table
        // was written one iteration ago, its raw buffer was last read by the
        // conversion of tile it; issued after this iteration's conversion
        // stores, since LDS stores behind an LDS DMA make the compiler wait
        // for the DMA)
        // Branch-free so that the LDS-read bookkeeping of the compiler stays
        // exact: past the end of the list the rows are zero rows, and wave 3
        // loads a zero row into a sink buffer.
        if ((db & 3) == 1 && (db >> 2) < kDmaPerWave) {
          const int j = db >> 2;
          const uint8_t* src = dma_sink ? g_zero_row + 16 * lane : dsrc.p[j] + dma_off[j];
          uint8_t* dst = dma_sink ? DmaSink : Raw[(it + kLead) % kStages] + 1024 * (wave + kDmaWaves * j);
          dma16(src, dst);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the rows of tile it+2 are in before the barrier: loads complete in
      // order, and after them every wave issued the kDmaPerWave loads of
      // tiles it+3 and it+4 (wave 3 also its table loads, which only makes
      // the wait stricter there)
      CSA_WAIT_VMCNT(2 * kDmaPerWave);
      // Workgroup barrier without the release fence of __syncthreads: the
      // fence would also wait for every LDS DMA in flight (vmcnt(0)) and so
      // drain the row pipeline each iteration.  LDS stores are completed by
      // the lgkmcnt wait, the rows of tile it+2 by the vmcnt wait above; the
      // memory clobber keeps the compiler from moving LDS accesses across.
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // every LDS DMA of this pass has landed (the compiler does not see the
    // asm ones): nothing may write LDS behind the next pass or after exit
    CSA_WAIT_VMCNT0();
    // head-wide maximum (relative to the reference) and sum over the 4 lanes of a head
    {
      auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(xmax), __float_as_uint(xmax), false, false);
      xmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(xmax), __float_as_uint(xmax), false, false);
      xmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(lrun), __float_as_uint(lrun), false, false);
      lrun = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lrun), __float_as_uint(lrun), false, false);
      lrun = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (__ballot(mset && xmax > kMaxLift) != 0ull && lane == 0) s_over = 1;
    __syncthreads();
    if (!s_over) break;                     // uniform
    // recompute with the exact per-head maximum as the reference
#pragma unroll
    for (int db = 0; db < 32; ++db) acc[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    lrun = 0.0f;
    if (mset) mref += xmax;
    xmax = -INFINITY;
    __syncthreads();
    if (tid == 0) s_over = 0;
  }
  const float mrun = mset ? mref : -INFINITY;

  // ---- epilogue: lane holds O^T rows (dims) 16 db + 4 G + (0..3) of head h.
  // The output rows go out through LDS (the raw row buffers are free: every
  // load has landed and every wave is past the tile loop), so that each
  // store instruction writes one contiguous 1 KiB piece of a head's row;
  // stored straight from the accumulators, every instruction would scatter
  // 32-byte pieces over 16 rows, which the memory system absorbs far more
  // slowly under the gather traffic of the other CUs.  Wave w stages its 16
  // heads in 16 rows of kStageRow bytes (1 KiB of data, padded so that the
  // row starts fall in different banks); FP32 rows go in two halves.
  const bool split = a.nsplit > 1;
  float scale = 1.0f, lse = -INFINITY;
  if (!split) {
    const float M = fmaxf(mrun, sig2);
    scale = 0.0f;
    if (M > -INFINITY) {
      const float fm = mrun > -INFINITY ? exp2f(mrun - M) : 0.0f;
      const float Z = lrun * fm + (sig2 > -INFINITY ? exp2f(sig2 - M) : 0.0f);
      scale = fm / Z;
      lse = (M + log2f(Z)) * kLn2;
    }
  }
  const bool f32 = split || a.out_f32;
  constexpr int kStageRow = 1024 + 16;
  uint8_t* const stg = &Raw[0][0] + wave * kMHeads * kStageRow;
  const int64_t hrow0 = bq * a.H + blockIdx.y * 64 + wave * kMHeads;   // this wave's first head row
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c == 1 && !f32) break;                   // uniform
    if (f32) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const f32x4 v = acc[16 * c + k] * scale;
        *(f32x4*)(stg + l16 * kStageRow + 64 * k + 16 * G) = v;
      }
    } else {
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        u32x2 w;
        w.x = f32_to_bf16(acc[db][0] * scale) | (f32_to_bf16(acc[db][1] * scale) << 16);
        w.y = f32_to_bf16(acc[db][2] * scale) | (f32_to_bf16(acc[db][3] * scale) << 16);
        *(u32x2*)(stg + l16 * kStageRow + 32 * db + 8 * G) = w;
      }
    }
    // (one wave writes and reads its own rows: its LDS accesses stay in order)
#pragma unroll
    for (int r = 0; r < kMHeads; ++r) {
      const u32x4 x = *(const u32x4*)(stg + r * kStageRow + 16 * lane);
      const int64_t hr = hrow0 + r;
      uint8_t* dst = split ? (uint8_t*)(a.ws + (hr * a.nsplit + blockIdx.z) * (int64_t)kMD)
                           : (f32 ? (uint8_t*)((float*)a.out + hr * kMD) : (uint8_t*)((uint16_t*)a.out + hr * kMD));
      *(u32x4*)(dst + 1024 * c + 16 * lane) = x;
    }
  }
  if (split) {
    // partial: m (natural log units), l, unnormalised o
    if (G == 0) {
      float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * a.nsplit * kMD + ((bq * a.H + h) * a.nsplit + blockIdx.z) * 2;
      wml[0] = mrun > -INFINITY ? mrun * kLn2 : -INFINITY;
      wml[1] = lrun;
    }
  } else if (a.lse && G == 0) {
    a.lse[bq * a.H + h] = lse;
  }
}

// The MFMA kernel masks empty slots through a -1e30 logit: the scaled logit
// of an empty slot (about -1e30 tau log2 e in base 2) must lie far below
// anything exp2 can resolve, so the kernel takes scales above 1e4 / (1e30
// log2 e) only; other scales (tiny, zero or negative) take the general kernel.
bool attn_mfma_eligible(int q_fmt, int H, int D, const csa_store& kv, bool has_prior, float tau) {
  return !has_prior && tau * kLog2e * 1.0e30f >= 1.0e4f && q_fmt == CSA_BF16 && D == kMD && H % 64 == 0 &&
         kv.fmt == CSA_FP8_E4M3 && kv.row_bytes == kRawRow;
}

hipError_t launch_attn_mfma(const AttnCall& c, int nsplit, int split_len, hipStream_t st) {
  // slot arithmetic in the kernel is 32-bit
  if (c.n_entries + c.W + kMT > INT32_MAX || c.ckv.cap > INT32_MAX || c.win.cap > INT32_MAX) return hipErrorInvalidValue;
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
