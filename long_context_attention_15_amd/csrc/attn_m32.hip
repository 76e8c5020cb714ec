// Gathered-entry attention on bf16 MFMA (gfx950), 32 heads per wavefront:
// head dim 512 stored as FP8 bulk (448 dims, one power-of-two scale per row)
// + BF16 RoPE dims (64), bf16 queries.
//
// Work item: one query row, 64 heads, one split of its entry list (the
// window rows, then the top-k / visible compressed entries).  Two
// wavefronts; wavefront w owns heads [32 w, 32 w + 32) over all 512 dims, so
// every product runs on v_mfma_f32_32x32x16_bf16 with the 32 heads as the N
// side: each operand read from LDS feeds twice the flops of a 16-head
// layout.  Two workgroups share a CU (LDS 77 KiB each, one wavefront per
// SIMD), so one workgroup's barriers and epilogue overlap the other's
// products.  Per tile of 32 entries:
//   * the raw 576-byte rows go HBM -> LDS by LDS DMA three tiles ahead, unit
//     major: 16-byte unit u of row r at position 32 u + (r ^ 4 (u & 1)) of
//     the tile, so a wave-wide load covers units 2 j, 2 j + 1 of all 32 rows
//     (a lane always loads from the same row) and every 16-lane group of the
//     reads below, and both halves of each 32-lane pass of the transposing
//     reads, fall on distinct banks;
//   * S^T = K Q^T (32 entries x 32 heads, K = 16 dims per step): each lane
//     reads 16 FP8 bytes of its entry row (two K-steps) and converts them
//     with the row scale to BF16 exactly (power-of-two scales); RoPE dims
//     are read as BF16;
//   * softmax in base 2 against a per-head reference fixed at the first
//     filled tile (a head is one lane column of the accumulators, split over
//     lanes l and l + 32);
//   * O^T += V^T P^T (32 dims x 32 heads, K = 16 entries per step): V^T comes
//     from 8-bit transposing LDS reads of the FP8 codes, converted unscaled,
//     with the row scale folded into P; RoPE dims from 16-bit transposing
//     reads.  P stays in registers: its K order is the order in which the
//     S^T accumulators hold a lane's entries.
// K = V = the stored entry (shared KV).
#include "common.h"
#include "launch.h"

namespace csa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

constexpr int kD = 512;                    // head dim
constexpr int kT = 32;                     // entries per tile
constexpr int kThreads = 128;              // two wavefronts
constexpr int kRow = 576;                  // 448 FP8 + 64 BF16
constexpr int kUnits = kRow / 16;          // 16-byte units per row
constexpr int kTileBytes = kT * kRow;      // 18432 = 18 wave-wide 1 KiB loads
constexpr int kLoadsW = kTileBytes / 1024 / 2;   // 9 loads per wavefront per tile
constexpr int kStages = 4;                 // raw tile buffers
constexpr int kLead = 3;                   // DMA distance in tiles
constexpr int kSlots = 8;                  // slot tables (two build batches)
constexpr int kBatch = 4;                  // tiles per table build (2 per wavefront)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kEmpty = -1.0e30f;         // logit of an empty slot

struct Args {
  const uint16_t* q; int B, Tq, H;
  Store ckv; int64_t n_entries; int mode; const int32_t* sel; int k; int m;
  Store win; int W; int ring; const int64_t* q_pos;
  const float* sink; float tau;
  void* out; int out_f32; float* lse; int partial;
  int nsplit; int split_len; float* ws;
  NormRope qn;
  const float* prior_o; const float* prior_lse;   // kPrior: partial (o, lse) merged in the epilogue
};

// Zero row that empty slots gather from (device globals start zeroed).
__device__ __attribute__((aligned(16))) uint8_t zero_row[1024];

// byte offset in a raw tile of 16-byte unit u of row r
__device__ __forceinline__ int unit_off(int r, int u) { return 16 * (kT * u + (r ^ (8 * (u & 1)))); }
// entry behind K index 8 h + e of PV step c: the order in which lane
// (head, h) holds its S^T accumulator rows 8 c .. 8 c + 7
__device__ __forceinline__ int pv_entry(int c, int h, int e) { return 16 * c + 8 * h + e; }

__device__ __forceinline__ int64_t visible(int64_t t, int m, int64_t n) {
  int64_t v = t < 0 ? 0 : (t + 1) / m;
  return v < n ? v : n;
}

// 8 FP8 codes -> 8 BF16 values times s (exact for a power-of-two s).
__device__ __forceinline__ u32x4 cvt8(u32x2 w, float s) {
  u32x4 r;
  r.x = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, s, false));
  r.y = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, s, true));
  r.z = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, s, false));
  r.w = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, s, true));
  return r;
}

#define M32_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// 16-byte LDS DMA (lane l's bytes land at dst + 16 l) and 4-byte LDS DMA
// (lane l's word at dst + 4 l), as inline asm with no register result:
// completion is tracked by explicit vmcnt waits.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, void* dst) {
  const unsigned lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ float swap32_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <bool kQPost, bool kPrior>
__global__ __launch_bounds__(kThreads, 1) void attn_m32_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t Raw[kStages][kTileBytes];
  __shared__ const uint8_t* Tptr[kSlots][kT];                     // row address (zero row if empty)
  __shared__ __attribute__((aligned(16))) float Tscl[kSlots][kT];  // row scale (0 if empty)
  __shared__ __attribute__((aligned(16))) float Tbias[kSlots][kT]; // 0 filled, kEmpty empty
  __shared__ __attribute__((aligned(16))) int32_t Tsel[kSlots][kT];
  __shared__ int s_over;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // uniform: scalar registers
  const int hcol = lane & 31, hh = lane >> 5;        // head column, lane half
  const int64_t bq = xcd_remap(blockIdx.x, gridDim.x);   // query row (b * Tq + q)
  const int b = (int)(bq / a.Tq);
  const int h = blockIdx.y * 64 + wave * 32 + hcol;           // this lane's head
  const int64_t t = a.q_pos ? a.q_pos[bq] : (int64_t)(bq % a.Tq);
  const int64_t Lc = a.mode == kModeSel ? a.k : (a.mode == kModeRange ? visible(t, a.m, a.n_entries) : 0);
  const int64_t L = Lc + a.W;
  const int64_t i0 = (int64_t)blockIdx.z * a.split_len;
  const int64_t i1 = a.nsplit == 1 ? L : (i0 + a.split_len < L ? i0 + a.split_len : L);
  const int ntiles = i1 > i0 ? (int)((i1 - i0 + kT - 1) / kT) : 0;

  // ---- slot tables.  Lane tl of a building wavefront owns slot i0 + 32
  // tile + tl of the entry list (lanes 32-63 the next tile): the W window
  // rows first, then the Lc compressed entries.  Row address and bias are
  // stored now; the row scale and the sel entries arrive by LDS DMA, so no
  // load result is carried in registers across tiles.  Slot arithmetic is
  // 32-bit (lists stay far below 2^31 entries).
  const int i0i = (int)i0, i1i = (int)i1;
  const int win_p0 = (int)(t - a.W + 1);
  const bool sel_mode = a.mode == kModeSel;
  const int n_ent = (int)a.n_entries, win_cap = (int)a.win.cap;
  const uint8_t* const ckv_base = a.ckv.rows + (size_t)b * a.ckv.cap * a.ckv.row_bytes;
  const float* const ckv_sc = (const float*)a.ckv.scales + (size_t)b * a.ckv.cap;
  const uint8_t* const win_base = a.win.rows + (size_t)b * a.win.cap * a.win.row_bytes;
  const float* const win_sc = (const float*)a.win.scales + (size_t)b * a.win.cap;
  const int32_t* const sel_row = sel_mode ? a.sel + bq * a.k : nullptr;
  auto table2 = [&](int tile, int jsel) {          // tiles `tile`, tile + 1 (tile even)
    const int ts = tile & (kSlots - 1);
    const int slot = i0i + tile * kT + lane;
    int p = win_p0 + slot;
    const bool p_ok = p >= 0 && (a.ring || p < win_cap);
    if (a.ring) p = p >= 0 ? p % a.W : 0;
    const bool in_list = slot < i1i, is_c = slot >= a.W;
    const int j = sel_mode ? jsel : slot - a.W;
    const bool ok = in_list && (is_c ? (unsigned)j < (unsigned)n_ent : p_ok);
    const int idx = is_c ? j : p;
    const uint8_t* ptr = (is_c ? ckv_base : win_base) + (size_t)idx * kRow;
    const float* sp = (is_c ? ckv_sc : win_sc) + idx;
    (&Tptr[0][0])[ts * kT + lane] = ok ? ptr : zero_row;
    (&Tbias[0][0])[ts * kT + lane] = ok ? 0.0f : kEmpty;
    dma4(ok ? (const void*)sp : (const void*)zero_row, &Tscl[ts][0]);
  };
  auto sel_dma2 = [&](int tile) {                  // sel entries of tiles `tile`, tile + 1
    const int slot = i0i + tile * kT + lane;
    dma4(sel_mode && slot >= a.W && slot < i1i ? (const void*)(sel_row + (slot - a.W)) : (const void*)zero_row,
         &Tsel[tile & (kSlots - 1)][0]);
  };
  // Row DMA of `tile` into Raw[tile % kStages]: wave-wide load j = wave +
  // 2 jj fills positions 64 j .. 64 j + 63, i.e. units 2 j + hh of row
  // hcol ^ (4 hh) for lane (hh, hcol): a lane reads one row of the tile.
  const int dma_row = hcol ^ (8 * hh);
  auto dma_src = [&](int tile) { return Tptr[tile & (kSlots - 1)][dma_row] + 16 * hh; };
  auto dma_rows = [&](const uint8_t* src, int tile, int jj) {
    const int j = wave + 2 * jj;
    dma16(src + 32 * j, Raw[tile % kStages] + 1024 * j);
  };

  const float sig2 = (a.nsplit > 1 || a.partial || !a.sink) ? -INFINITY : a.sink[h] * kLog2e;

  // ---- Q^T operands.  K-step pair s < 14 (FP8 dims 32 s .. 32 s + 31): step
  // 2 s + i, K index 8 hh + e <-> dim 32 s + 16 hh + 8 i + e; RoPE step j < 4:
  // K index 8 hh + e <-> dim 448 + 16 j + 8 hh + e.
  // (S^T runs on 16x16x32 products: head half hq = heads 16 hq .. +16 of the
  // wave, K-step ks = dims 32 ks .. +32; lane l holds head 16 hq + l % 16,
  // dims 32 ks + 8 (l / 16) .. +8.)
  const int g = lane >> 4, i16 = lane & 15;
  // Lane (g, i16) holds head 16 hq + i16, dims 32 ks + 8 g .. +8: 16 bytes at
  // q_src + hq * 16 kD + 32 ks.
  const uint16_t* const q_src = a.q + (bq * a.H + blockIdx.y * 64 + wave * 32 + i16) * (int64_t)kD + 8 * g;
  // RMSNorm / partial RoPE of the query rows (kQPost).  The rows are loaded
  // as in the plain path and processed in registers; the cos / sin of rotation
  // pair p come from a per-wavefront table (lane l forms pairs l, l + 64, ...),
  // so no sincos is replicated in the unrolled code.  The processed BF16
  // operands go through the wavefront's half of the raw tile buffers (free
  // until the first row DMA below), chunk (ks, hq) of lane l at byte
  // 16 (64 (2 ks + hq) + l), and are read back from there: the operand
  // registers have a single source, and the processing temporaries are dead
  // before they are loaded, so the tile loop keeps the plain path's register
  // allocation (operands merged from two sources, a replicated sincos, or
  // processing in place inside the prologue push some of them to scratch
  // inside the loop).
  bf16x8 qf[16][2];
  if constexpr (kQPost) {
    uint8_t* const q_stage = &Raw[0][0] + wave * (32 * kD * 2);
    // after the staging (64 KiB): per wavefront, 2 KiB of cos / sin, then 2 KiB of gain
    float2* const rot_tab = (float2*)(&Raw[0][0] + 2 * (32 * kD * 2)) + wave * 256;
    float* const gain_tab = (float*)(&Raw[0][0] + 2 * (32 * kD * 2) + 4096) + wave * kD;
    for (int pp = lane; pp < (a.qn.rope_dims >> 1); pp += 64) {   // before the rows: few values live
      float sn, cs;
      sincos_angle(__fmul_rn((float)t, a.qn.theta[pp]), &sn, &cs);
      rot_tab[pp] = make_float2(cs, sn);
    }
    bf16x8 qx[16][2];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qx[ks][hq] = __builtin_bit_cast(bf16x8, *(const u32x4*)(q_src + hq * 16 * kD + 32 * ks));
    float4 gl0 = make_float4(1.0f, 1.0f, 1.0f, 1.0f), gl1 = gl0;
    if (a.qn.gain) {
      gl0 = *(const float4*)(a.qn.gain + 8 * lane);
      gl1 = *(const float4*)(a.qn.gain + 8 * lane + 4);
    }
    const int d0 = kD - a.qn.rope_dims, npair = a.qn.rope_dims >> 1;
    *(float4*)(gain_tab + 8 * lane) = gl0;
    *(float4*)(gain_tab + 8 * lane + 4) = gl1;
    float rr[2] = {1.0f, 1.0f};
    if (a.qn.gain) {                              // a head's 512 dims: 4 lanes (i16 + 16 g) x 128
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf((float)qx[ks][hq][e], (float)qx[ks][hq][e], ss);
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        rr[hq] = 1.0f / sqrtf(ss / (float)kD + a.qn.eps);
      }
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));    // lgkmcnt(0): the tables are written
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int dd = 32 * ks + 8 * g;             // this lane's 8 dims of K-step ks
      const float4 g0 = *(const float4*)(gain_tab + dd), g1 = *(const float4*)(gain_tab + dd + 4);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      float2 cs[4];                               // pair (dd + 2 e2, dd + 2 e2 + 1), both head halves
      bool on[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        on[e2] = npair > 0 && dd + 2 * e2 >= d0;
        cs[e2] = make_float2(1.0f, 0.0f);
        if (npair > 0 && 32 * ks + 32 > d0) {     // uniform: K-step ks holds rotated dims
          const float2 tv = rot_tab[on[e2] ? (dd + 2 * e2 - d0) >> 1 : 0];
          if (on[e2]) cs[e2] = tv;
        }
      }
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)qx[ks][hq][e] * rr[hq] * gv[e];
        bf16x8 y;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float c = cs[e2].x, sv = cs[e2].y, x0 = v[2 * e2], x1 = v[2 * e2 + 1];
          y[2 * e2] = (__bf16)(on[e2] ? x0 * c - x1 * sv : x0);   // BF16 queries stay BF16
          y[2 * e2 + 1] = (__bf16)(on[e2] ? x0 * sv + x1 * c : x1);
        }
        *(u32x4*)(q_stage + 16 * (64 * (2 * ks + hq) + lane)) = __builtin_bit_cast(u32x4, y);
      }
    }
#pragma unroll
    for (int hq = 0; hq < 2; ++hq)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qf[ks][hq] = __builtin_bit_cast(bf16x8, *(const u32x4*)(q_stage + 16 * (64 * (2 * ks + hq) + lane)));
    // operands in registers before any row DMA may overwrite the staging
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));    // lgkmcnt(0)
  } else {
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const uint16_t* qp = a.q + (bq * a.H + blockIdx.y * 64 + wave * 32 + 16 * hq + i16) * (int64_t)kD + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks][hq] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 32 * ks));
    }
  }
  // LDS byte offsets of this lane's reads within a raw tile.  The XOR in
  // unit_off touches bit 3 of the row only, so 16 rows (entry half, PV step)
  // are +256 bytes, 4 rows +64 and 4 units +2048 for every lane: one base
  // register per operand, the rest in the read's immediate offset.
  // K (S^T A operand of entry half eh, K-step ks): row 16 eh + i16, FP8
  // bytes 32 ks + 8 g .. +8 (unit 2 ks + g / 2, half g & 1):
  // k_fp8 + 256 eh + 1024 ks; RoPE step ks = 14 + j: BF16 dims 448 + 32 j +
  // 8 g (unit 28 + 4 j + g): k_rope + 256 eh + 2048 j.
  const int k_fp8 = unit_off(i16, g >> 1) + 8 * (g & 1);
  const int k_rope = unit_off(i16, 28 + g);
  // V^T FP8 (8-bit transposing reads): 16-lane group g = lane >> 4 covers
  // dims 16 (g & 1) .. +16 of a 32-dim block (unit 2 db + (g & 1)), entries
  // of half hh = g >> 1; source lane i16 reads 8 bytes of row
  // pv_entry(c, hh, i16 >> 1), half i16 & 1: v_fp8 + 256 c + 1024 db.
  const int v_fp8 = unit_off(pv_entry(0, hh, i16 >> 1), g & 1) + 8 * (i16 & 1);
  // V^T RoPE (16-bit transposing reads): row pv_entry(c, hh, 4 rd + (i16 >> 2)),
  // bf16 dims 448 + 32 bb + 16 (g & 1) + 4 (i16 & 3) .. +4, i.e. unit
  // 28 + 4 bb + 2 (g & 1) + (i16 & 3) / 2, half i16 & 1:
  // v_rope + 256 c + 64 rd + 2048 bb.
  const int v_rope = unit_off(pv_entry(0, hh, i16 >> 2), 28 + 2 * (g & 1) + ((i16 & 3) >> 1)) + 8 * (i16 & 1);

  f32x16 acc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  const float sc2 = a.tau * kLog2e;
  // Softmax reference per head (log2 units): fixed at the first tile with a
  // filled slot; probabilities relative to it stay below 2^kMaxLift, else
  // the query is recomputed once with the exact maximum (tracked as xmax).
  constexpr float kMaxLift = 64.0f;
  float mref = 0.0f, xmax = -INFINITY, lrun = 0.0f;
  bool mset = false;
  if (tid == 0) s_over = 0;

  // One pass over the entry list: prologue and tile loop.  It runs a second
  // time only when some logit exceeded the reference by 2^kMaxLift, as a
  // second trip through the same code, so that both passes share one
  // register assignment (two inlined copies left the accumulators to be
  // reshuffled, partly through scratch memory, between them).
  auto pass = [&]() {
    // ---- prologue: sel entries of tiles 0 .. 7, tables of tiles 0 .. 3,
    // rows of tiles 0 .. kLead-1.  With the window first in the list, the
    // first tiles' tables need no sel entry when the split starts the list
    // and the window covers them (or there are no sel entries): their row
    // loads go out without waiting for the sel loads.
    const bool early = !sel_mode || (i0i == 0 && a.W >= kBatch * kT);
    sel_dma2(2 * wave);
    sel_dma2(kBatch + 2 * wave);
    if (!early) {
      M32_WAIT_VMCNT(0);
      asm volatile("" ::: "memory");
    }
    table2(2 * wave, (&Tsel[0][0])[2 * wave * kT + lane]);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // row loads go out for every tile, past the list's end too (the tables
    // of slots beyond it hold the zero row), so each wait has one form: it
    // counts the row loads issued after the tile it waits for (loads
    // complete in order; the sel-entry loads in between only make a wait
    // stricter)
#pragma unroll
    for (int pt = 0; pt < kLead; ++pt) {
      const uint8_t* src = dma_src(pt);
#pragma unroll
      for (int jj = 0; jj < kLoadsW; ++jj) dma_rows(src, pt, jj);
    }
    static_assert(kLead == 3, "the waits count kLead - 1 tiles of loads");
    M32_WAIT_VMCNT((kLead - 1) * kLoadsW);      // tile 0 in
    // the first tiles' rows, issued back to back, follow within a few
    // hundred cycles; waiting for them here tells the compiler that the
    // query operand loads (issued before any row) have landed, so it puts no
    // waits for them into the tile loop, where they would count row loads
    M32_WAIT_VMCNT(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    for (int it = 0; it < ntiles; ++it) {
      const uint8_t* raw = Raw[it % kStages];
      const int ts = it & (kSlots - 1);
      const uint8_t* dsrc = dma_src(it + kLead);
      if ((it & (kBatch - 1)) == 0) {
        // tables of tiles it+4 .. it+7 (sel entries landed at least one
        // iteration ago) and sel entries of tiles it+8 .. it+11
        const int tb = it + kBatch + 2 * wave;
        table2(tb, (&Tsel[0][0])[(tb & (kSlots - 1)) * kT + lane]);
        sel_dma2(it + 2 * kBatch + 2 * wave);
      }

      // ---- S^T = K Q^T as four 16 x 16 blocks (entry half eh x head half
      // hq), four independent accumulator chains; each starts at the slot
      // bias, so empty slots drop out of the softmax.
      f32x4 sblk[2][2];
      float bmax = kEmpty;                       // 0 if some slot of the tile holds an entry
#pragma unroll
      for (int eh = 0; eh < 2; ++eh) {
        const float4 bv = *(const float4*)(Tbias[ts] + 16 * eh + 4 * g);
        sblk[eh][0] = f32x4{bv.x, bv.y, bv.z, bv.w};
        sblk[eh][1] = sblk[eh][0];
        bmax = fmaxf(bmax, fmaxf(fmaxf(bv.x, bv.y), fmaxf(bv.z, bv.w)));
      }
      const bool tile_filled = __ballot(bmax == 0.0f) != 0ull;
      const float ksc[2] = {Tscl[ts][i16], Tscl[ts][16 + i16]};
      // K operand reads in order r = 2 ks + eh: FP8 (8 bytes) for ks < 14,
      // BF16 (16 bytes) for the RoPE steps
      constexpr int kSD = 3;                     // K read distance (reads)
      u32x2 kf[28];
      u32x4 kb[4];
      auto kread = [&](int r) {
        const int ks = r >> 1, eh = r & 1;
        if (ks < 14) kf[r] = *(const u32x2*)(raw + k_fp8 + 256 * eh + 1024 * ks);
        else kb[r - 28] = *(const u32x4*)(raw + k_rope + 256 * eh + 2048 * (ks - 14));
      };
      // The operand of read r is converted during step r - 1, into the
      // other of two register sets, so that a conversion never writes the
      // registers a product in flight is still reading.
      u32x4 kop[2];
      auto kconv = [&](int r) {
        const int ks = r >> 1, eh = r & 1;
        kop[r & 1] = ks < 14 ? cvt8(kf[r], ksc[eh]) : kb[r - 28];
      };
      // the same conversion in two parts (the first word, then the other
      // three), placed around the first product of a step
      auto kconv_a = [&](int r) {
        const int ks = r >> 1, eh = r & 1;
        if (ks < 14) kop[r & 1].x = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kf[r].x, ksc[eh], false));
        else kop[r & 1] = kb[r - 28];
      };
      auto kconv_b = [&](int r) {
        const int ks = r >> 1, eh = r & 1;
        if (ks < 14) {
          kop[r & 1].y = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kf[r].x, ksc[eh], true));
          kop[r & 1].z = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kf[r].y, ksc[eh], false));
          kop[r & 1].w = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kf[r].y, ksc[eh], true));
        }
      };
#pragma unroll
      for (int r = 0; r < kSD; ++r) kread(r);
      kconv(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        // issue order: read, one conversion word, product, three words,
        // product (eight issue slots in the two products' 32 cycles)
        const int ks = r >> 1, eh = r & 1;
        if (r + kSD < 32) kread(r + kSD);
        if (r + 1 < 32) kconv_a(r + 1);
        __builtin_amdgcn_sched_barrier(0);
        sblk[eh][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[r & 1]), qf[ks][0],
                                                            sblk[eh][0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (r + 1 < 32) kconv_b(r + 1);
        __builtin_amdgcn_sched_barrier(0);
        sblk[eh][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[r & 1]), qf[ks][1],
                                                            sblk[eh][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- V^T reads of the first dim blocks go out before the softmax
      constexpr int kVD = 4;
      v2i32 vf[2][14];
#pragma unroll
      for (int db = 0; db < kVD; ++db)
        vf[0][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(raw + v_fp8 + 1024 * db));
      __builtin_amdgcn_sched_barrier(0);

      // ---- softmax: lane holds entries 8 (r >> 2) + 4 hh + (r & 3) of head h
      // Lane 16 g + c holds, in block (eh, hq), entries 16 eh + 4 g + i of
      // head 16 hq + c.  One 16-lane row swap per value gives lane 32 h' + hc
      // the 16 entries 16 eh + 8 h' + e (e < 8) of head hc: x[8 eh + e].
      float x[16];
#pragma unroll
      for (int eh = 0; eh < 2; ++eh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(sblk[eh][0][i]),
                                                           __float_as_uint(sblk[eh][1][i]), false, false);
          x[8 * eh + i] = __uint_as_float(sw[0]);
          x[8 * eh + 4 + i] = __uint_as_float(sw[1]);
        }
      {
        if (!mset && tile_filled) {
          // first tile with a filled slot (slots are shared by all heads, so
          // this is wave-uniform): the head's maximum over the tile
          float mt = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, x[r] * sc2);
          mref = swap32_max(mt);
          mset = true;
        }
      }
      float p[16];
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = fmaf(x[r], sc2, -mref);
        xmax = fmaxf(xmax, y);
        p[r] = __builtin_amdgcn_exp2f(y);
        psum += p[r];
      }
      lrun += psum;
      // P^T operands of PV step c: unscaled (RoPE dims) and times the row
      // scale of each entry (FP8 dims, whose codes convert unscaled)
      bf16x8 pr[2], ps[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float4 s0 = *(const float4*)(Tscl[ts] + pv_entry(c, hh, 0));
        const float4 s1 = *(const float4*)(Tscl[ts] + pv_entry(c, hh, 4));
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pr[c][e] = (__bf16)p[8 * c + e];
          ps[c][e] = (__bf16)(p[8 * c + e] * sv[e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T += V^T P^T: step c over entries, 14 FP8 dim blocks + 2 RoPE
      // blocks; rows of tile it + kLead go out between the products (their
      // table was written at least one iteration ago, their buffer was
      // freed by the barrier that ended iteration it - 1)
      // Product f = 16 c + db (PV step c, dim block db: 14 FP8 blocks, then
      // 2 RoPE blocks); its operand is read kVD FP8 blocks ahead and
      // converted during product f - 1 into the other of two register sets.
      u32x4 vop[2];
      auto vread = [&](int n) {                  // FP8 block n of the 28 (step n / 14, block n % 14)
        vf[n / 14][n % 14] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(raw + v_fp8 + 256 * (n / 14) + 1024 * (n % 14)));
      };
      auto vconv = [&](int f) {
        const int c = f >> 4, db = f & 15;
        if (db < 14) {
          vop[f & 1] = cvt8(u32x2{(unsigned)vf[c][db].x, (unsigned)vf[c][db].y}, 1.0f);
        } else {
          const int bb = db - 14;
          const u32x2 r0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(raw + v_rope + 256 * c + 2048 * bb)));
          const u32x2 r1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(raw + v_rope + 256 * c + 64 + 2048 * bb)));
          vop[f & 1] = u32x4{r0.x, r0.y, r1.x, r1.y};
        }
      };
      vconv(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < 32; ++f) {
        const int c = f >> 4, db = f & 15;
        const int nf = 14 * c + (db < 14 ? db : 13) + kVD;      // FP8 read kVD blocks ahead
        if (db < 14 && nf < 28) vread(nf);
        if (f + 1 < 32) vconv(f + 1);
        __builtin_amdgcn_sched_barrier(0);       // the next operand's conversion before this product
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vop[f & 1]), db < 14 ? ps[c] : pr[c],
                                                          acc[db], 0, 0, 0);
        if (f % 3 == 1 && f / 3 < kLoadsW)       // 9 row loads, every third product (no branch)
          dma_rows(dsrc, it + kLead, f / 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      // rows of tile it+1 are in before the barrier: after its loads every
      // wave issued those of tiles it+2 and it+3 (and the table loads, which
      // only make the wait stricter)
      M32_WAIT_VMCNT(2 * kLoadsW);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // every LDS DMA of this pass has landed before anything reuses LDS
    M32_WAIT_VMCNT(0);
    xmax = swap32_max(xmax);
    lrun = swap32_sum(lrun);
  };
  // the recompute pass runs the same code: a second trip of this loop
#pragma nounroll
  for (int round = 0; round < 2; ++round) {
    if (round == 1) {
      if (!s_over) break;                        // uniform
#pragma unroll
      for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
      lrun = 0.0f;
      if (mset) mref += xmax;
      xmax = -INFINITY;
    }
    pass();
    if (round == 0) {
      if (__ballot(mset && xmax > kMaxLift) != 0ull && lane == 0) s_over = 1;
      __syncthreads();
    }
  }
  __syncthreads();
  const float mrun = mset ? mref : -INFINITY;

  // ---- epilogue: lane holds O^T dims 32 db + 8 q + 4 hh + (0..3) of head h
  // (acc[db][4 q + 0..3]).  Rows go out through LDS so that each store
  // instruction writes one contiguous piece of a head row.
  const bool split = a.nsplit > 1;
  float scale = 1.0f, lse = -INFINITY;
  float pscale = 0.0f;                           // kPrior: weight of the prior partial's output
  if (!split) {
    // kPrior: the partial enters as one more term with logit lse_p and value
    // o_p (a merge of softmax sums over disjoint entry sets)
    const float lp2 = kPrior ? a.prior_lse[bq * a.H + h] * kLog2e : -INFINITY;
    const float M = fmaxf(fmaxf(mrun, sig2), lp2);
    scale = 0.0f;
    if (M > -INFINITY) {
      const float fm = mrun > -INFINITY ? exp2f(mrun - M) : 0.0f;
      const float fp = lp2 > -INFINITY ? exp2f(lp2 - M) : 0.0f;
      const float Z = lrun * fm + fp + (sig2 > -INFINITY ? exp2f(sig2 - M) : 0.0f);
      scale = fm / Z;
      pscale = fp / Z;
      lse = (M + log2f(Z)) * kLn2;
    }
  }
  const float* const po = kPrior ? a.prior_o + (bq * a.H + h) * (int64_t)kD + 4 * hh : nullptr;
  auto prior4 = [&](int d) {                     // o_p of dims d .. d + 3 (this lane's), or 0
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (kPrior && pscale != 0.0f) v = *(const float4*)(po + d);
    return v;
  };
  const bool f32 = split || a.out_f32;
  constexpr int kStageRow = 1024 + 16;
  uint8_t* const stg = &Raw[0][0] + wave * 32 * kStageRow;
  const int64_t hrow0 = bq * a.H + blockIdx.y * 64 + wave * 32;   // this wave's first head row
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half == 1 && !f32) break;                // uniform
    if (f32) {
      // dims 256 half .. +256: blocks 8 half .. 8 half + 7
#pragma unroll
      for (int k8 = 0; k8 < 8; ++k8) {
        const int db = 8 * half + k8;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 pv = prior4(32 * db + 8 * q4);
          float4 v;
          v.x = acc[db][4 * q4 + 0] * scale + pv.x * pscale; v.y = acc[db][4 * q4 + 1] * scale + pv.y * pscale;
          v.z = acc[db][4 * q4 + 2] * scale + pv.z * pscale; v.w = acc[db][4 * q4 + 3] * scale + pv.w * pscale;
          *(float4*)(stg + hcol * kStageRow + 4 * (32 * k8 + 8 * q4 + 4 * hh)) = v;
        }
      }
    } else {
#pragma unroll
      for (int db = 0; db < 16; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 pv = prior4(32 * db + 8 * q4);
          const float pe[4] = {pv.x, pv.y, pv.z, pv.w};
          bf16x4 w;                              // packed hardware conversion, round to nearest even
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * q4 + e] * scale + pe[e] * pscale);
          *(u32x2*)(stg + hcol * kStageRow + 2 * (32 * db + 8 * q4 + 4 * hh)) = __builtin_bit_cast(u32x2, w);
        }
    }
    // (each wave writes and reads only its own rows: its LDS accesses stay in order)
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      const u32x4 v = *(const u32x4*)(stg + r * kStageRow + 16 * lane);
      const int64_t hr = hrow0 + r;
      uint8_t* dst = split ? (uint8_t*)(a.ws + (hr * a.nsplit + blockIdx.z) * (int64_t)kD)
                           : (f32 ? (uint8_t*)((float*)a.out + hr * kD) : (uint8_t*)((uint16_t*)a.out + hr * kD));
      *(u32x4*)(dst + 1024 * half + 16 * lane) = v;
    }
  }
  if (split) {
    if (hh == 0) {
      float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * a.nsplit * kD + ((bq * a.H + h) * a.nsplit + blockIdx.z) * 2;
      wml[0] = mrun > -INFINITY ? mrun * kLn2 : -INFINITY;
      wml[1] = lrun;
    }
  } else if (a.lse && hh == 0) {
    a.lse[bq * a.H + h] = lse;
  }
}

}  // namespace

// The kernel masks empty slots through a -1e30 logit: the scaled logit of an
// empty slot (about -1e30 tau log2 e in base 2) must lie far below anything
// exp2 can resolve, so it takes scales above 1e4 / (1e30 log2 e) only; other
// scales (tiny, zero or negative) take the general kernel.
bool attn_mfma_eligible(int q_fmt, int H, int D, const csa_store& kv, bool has_prior, float tau) {
  (void)has_prior;                               // a prior partial is merged in the epilogue
  return tau * kLog2e * 1.0e30f >= 1.0e4f && q_fmt == CSA_BF16 && D == kD && H % 64 == 0 &&
         kv.fmt == CSA_FP8_E4M3 && kv.row_bytes == kRow;
}

hipError_t launch_attn_m32(const AttnCall& c, int nsplit, int split_len, hipStream_t st) {
  if (c.n_entries + c.W + kT > INT32_MAX || c.ckv.cap > INT32_MAX || c.win.cap > INT32_MAX) return hipErrorInvalidValue;
  Args a;
  a.q = (const uint16_t*)c.q; a.B = c.B; a.Tq = c.Tq; a.H = c.H;
  a.ckv = c.ckv.rows ? view(c.ckv) : view(c.win);
  a.n_entries = c.n_entries; a.mode = c.mode; a.sel = c.sel; a.k = c.k; a.m = c.m;
  a.win = c.win.rows ? view(c.win) : a.ckv;
  a.W = c.W; a.ring = c.ring; a.q_pos = c.q_pos;
  a.sink = c.sink; a.tau = c.tau;
  a.out = c.out; a.out_f32 = c.partial; a.lse = c.lse; a.partial = c.partial;
  a.nsplit = nsplit; a.split_len = split_len; a.ws = (float*)c.ws;
  a.qn = c.qn;
  a.prior_o = c.prior_o; a.prior_lse = c.prior_lse;
  const dim3 grid((unsigned)((int64_t)c.B * c.Tq), c.H / 64, nsplit);
  const bool post = c.qn.gain || c.qn.rope_dims > 0, prior = c.prior_o != nullptr;
  if (prior && nsplit != 1) return hipErrorInvalidValue;        // a prior merges into the final output only
  if (post && prior) hipLaunchKernelGGL((attn_m32_kernel<true, true>), grid, dim3(kThreads), 0, st, a);
  else if (post) hipLaunchKernelGGL((attn_m32_kernel<true, false>), grid, dim3(kThreads), 0, st, a);
  else if (prior) hipLaunchKernelGGL((attn_m32_kernel<false, true>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((attn_m32_kernel<false, false>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
