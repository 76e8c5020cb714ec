// Gathered-entry attention on bf16 MFMA (gfx950): head dim 512 stored as
// FP8 bulk + BF16 RoPE dims, bf16 queries, 64 heads per workgroup.
//
// Work item: one query row, 64 heads, one split of its entry list (the
// top-k / visible compressed entries followed by the window rows).
// Four waves: wave w owns heads [32*(w>>1), +32) and dims [256*(w&1), +256).
// Per tile of 32 entries:
//   * all threads gather the 32 rows, convert FP8*scale -> BF16 with the
//     hardware scaled conversion (exact), and stage them in LDS twice:
//     Ks[entry][dim] (A operand of S^T) and Vt[dim][entry] (A operand of O^T);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 over the wave's 256 dims, the
//     two dim-halves exchange partial sums through LDS;
//   * online softmax in base 2 per head (a head is one lane column of the
//     32x32 accumulator, so max/sum need one cross-half exchange);
//   * O^T += V^T P^T: P stays in registers as the B operand (the entry order
//     inside a 16-entry K-step is permuted identically on both operands).
// HBM traffic per query: the gathered rows plus q and out; the rows are
// decoded once per workgroup.
#include "common.h"
#include "launch.h"

namespace csa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int kMD = 512;                 // head dim
constexpr int kMT = 32;                  // entries per tile
constexpr int kKsPitch = kMD + 16;       // bf16 elements per Ks row: 264 words, 8 mod 64 banks
constexpr int kVtPitch = kMT + 4;        // bf16 elements per Vt row (+8 B pad)
constexpr int kMThreads = 256;
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
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRawRow = 576;                      // 448 FP8 + 64 BF16
constexpr int kRawTile = kMT * kRawRow;           // 18432 B = 18 wave-wide 1 KiB loads
constexpr int kRawLoads = kRawTile / 1024;
constexpr int kKsTile = kMT * kKsPitch;           // bf16 elements per converted tile

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define CSA_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))

__global__ __launch_bounds__(kMThreads, 1) void attn_mfma_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKsTile];
  __shared__ __attribute__((aligned(16))) uint8_t Raw[2][kRawTile];
  __shared__ __attribute__((aligned(16))) float Sx[4][16][64];
  __shared__ const uint8_t* Tptr[4][kMT];         // per tile slot: row address (zero row if empty)
  __shared__ float Tscl[4][kMT];                  // row scale, 0 if empty

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int rh = wave >> 1, dh = wave & 1;
  const int g32 = lane >> 5, l32 = lane & 31;
  const int64_t bq = xcd_remap(blockIdx.x, gridDim.x);   // query row (b * Tq + q)
  const int b = (int)(bq / a.Tq);
  const int h = blockIdx.y * 64 + rh * 32 + l32;          // this lane's head
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
    Tptr[tile & 3][tid] = src ? stv.rows + row * stv.row_bytes : g_zero_row;
    return src ? ((const float*)stv.scales)[row] : 0.0f;
  };
  auto sel_of = [&](int tile) -> int {
    return m_slot_sel(a, bq, Lc, i0 + (int64_t)tile * kMT + tid, i1);
  };
  // DMA the raw rows of `tile` into Raw[tile & 1]: 18 wave-wide loads of
  // 1 KiB, load q covering raw bytes [1024 q, 1024 q + 1024).
  auto dma_tile = [&](int tile) {
    uint8_t* dst = Raw[tile & 1];
    for (int qd = wave; qd < kRawLoads; qd += 4) {
      const int ci = qd * 64 + lane;                   // 16-byte chunk of the tile
      const int slot = ci / 36, ch = ci - slot * 36;
      const uint8_t* src = Tptr[tile & 3][slot] + 16 * ch;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + 1024 * qd), 16, 0, 0);
    }
  };
  // Raw[tile & 1] -> Ks[tile & 1]: FP8 * row scale -> BF16 (exact), RoPE dims copied.
  auto convert_tile = [&](int tile) {
    const uint8_t* raw = Raw[tile & 1];
    uint16_t* ks = Ks[tile & 1];
    const int row = tid >> 3, sub = tid & 7;
    const float sc = Tscl[tile & 3][row];
    const uint8_t* rr = raw + row * kRawRow;
    uint16_t* kr = ks + row * kKsPitch;
#pragma unroll
    for (int mm = 0; mm < 7; ++mm) {
      const int u = sub + 8 * mm;                       // 8-byte unit of the 448 FP8 bytes
      const u32x2 w = *(const u32x2*)(rr + 8 * u);
      *(u32x4*)(kr + 8 * u) = cvt8_fp8(w, sc);
    }
    *(u32x4*)(kr + 448 + 8 * sub) = *(const u32x4*)(rr + 448 + 16 * sub);
  };

  bf16x8 qf[16];
  {
    const uint16_t* qp = a.q + (bq * a.H + h) * (int64_t)kMD + dh * 256 + g32 * 8;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 16 * s));
  }
  f32x16 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
  const float sc2 = a.tau * kLog2e;
  // Softmax reference (log2 units, per head = per lane column): fixed at the
  // head's first non-empty tile and never moved, so no VALU code ever touches
  // the O^T accumulators.  Probabilities relative to it stay below
  // 2^kMaxLift; if some logit climbs further (not seen with normalised
  // inputs) the whole query is recomputed once with the exact maximum, which
  // the first pass tracks in mmax.
  constexpr float kMaxLift = 64.0f;
  float mref = -INFINITY, mmax = -INFINITY, lrun = 0.0f;
  __shared__ int s_over;
  if (tid == 0) s_over = 0;

  // transposed-read addressing of V^T (see the ds_read_b64_tr_b16 lane map):
  // lane j of a 16-lane group points at entry row 4*g + (j>>2) (+8 for the
  // second half of a K-step), dims D0 + 16*half + 4*(j&3).
  const int trj = lane & 15, trhalf = (lane >> 4) & 1;
  const int tr_row = 4 * g32 + (trj >> 2);
  const int tr_col = dh * 256 + 16 * trhalf + 4 * (trj & 3);

#pragma nounroll
  for (int attempt = 0; attempt < 2; ++attempt) {
    // ---- prologue: tables of tiles 0..2, rows of tiles 0 and 1, tile 0 converted
    int selreg = 0;
    float scl_pending = 0.0f;                       // scale of table tile it+2, stored at iteration it
    if (tid < kMT) {
      const int j0 = sel_of(0), j1 = sel_of(1), j2 = sel_of(2);
      selreg = sel_of(3);
      const float s0v = table_ptr(0, j0), s1v = table_ptr(1, j1);
      scl_pending = table_ptr(2, j2);
      Tscl[0][tid] = s0v;
      Tscl[1][tid] = s1v;
    }
    __syncthreads();
    if (ntiles > 0) dma_tile(0);
    if (ntiles > 1) dma_tile(1);
    CSA_WAIT_VMCNT0();
    __syncthreads();
    if (ntiles > 0) convert_tile(0);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
      const uint16_t* ks = Ks[it & 1];
      // S^T partial over this wave's dims: two accumulators for independent chains
      f32x16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
      const uint16_t* kp = ks + l32 * kKsPitch + dh * 256 + g32 * 8;
#pragma unroll
      for (int s = 0; s < 16; s += 2) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const u32x4*)(kp + 16 * s));
        const bf16x8 kb = __builtin_bit_cast(bf16x8, *(const u32x4*)(kp + 16 * (s + 1)));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[s + 1], s1, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] += s1[r];
        Sx[wave][r][lane] = s0[r];
      }
      CSA_WAIT_VMCNT0();                    // raw rows of tile it+1, the next sel and scale are in
      if (tid < kMT) {
        Tscl[(it + 2) & 3][tid] = scl_pending;
        if (it + 3 < ntiles) scl_pending = table_ptr(it + 3, selreg);
      }
      __syncthreads();                      // B1
      if (it + 2 < ntiles) dma_tile(it + 2);  // into Raw[it & 1], converted last iteration
      if (tid < kMT && it + 4 < ntiles) selreg = sel_of(it + 4);

      // softmax on this tile's logits
      const unsigned int vmask = (unsigned int)__ballot(lane < 32 && Tscl[it & 3][l32] > 0.0f);
      float p[16];
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = (r >> 2) * 8 + g32 * 4 + (r & 3);
        const float tot = s0[r] + Sx[wave ^ 1][r][lane];
        p[r] = ((vmask >> e) & 1u) ? tot * sc2 : -INFINITY;
        mt = fmaxf(mt, p[r]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      mmax = fmaxf(mmax, mt);
      if (mref == -INFINITY) mref = mt;     // the head's first non-empty tile
      if (__ballot(mt > mref + kMaxLift) != 0ull && lane == 0) s_over = 1;
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = mref > -INFINITY ? exp2f(p[r] - mref) : 0.0f;
        psum += p[r];
      }
      psum += __shfl_xor(psum, 32);
      lrun += psum;
      bf16x8 pb0, pb1;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        pb0[r] = (__bf16)p[r];
        pb1[r] = (__bf16)p[r + 8];
      }
      if (it + 1 < ntiles) convert_tile(it + 1);   // Ks[(it+1)&1] was released at the last B2

      // O^T += V^T P^T, V^T read transposed from Ks; K-step major so that
      // consecutive MFMAs write different accumulators
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const bf16x8 pb = ks2 ? pb1 : pb0;
#pragma unroll
        for (int mt8 = 0; mt8 < 8; ++mt8) {
          const uint16_t* vb = ks + (tr_row + 16 * ks2) * kKsPitch + tr_col + 32 * mt8;
          const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb));
          const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + 8 * kKsPitch));
          const u32x2 ux0 = __builtin_bit_cast(u32x2, x0), ux1 = __builtin_bit_cast(u32x2, x1);
          const u32x4 v0 = u32x4{ux0.x, ux0.y, ux1.x, ux1.y};
          acc[mt8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v0), pb, acc[mt8], 0, 0, 0);
        }
      }
      __syncthreads();                      // B2
    }
    CSA_WAIT_VMCNT0();                      // no DMA may still target Raw
    __syncthreads();
    if (!s_over) break;                     // uniform
    // recompute with the exact per-head maximum (mref >= every logit now)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
    lrun = 0.0f;
    mref = mmax;
    __syncthreads();
    if (tid == 0) s_over = 0;
  }
  const float mrun = mref;

  // ---- epilogue
  const int64_t qoff = (bq * a.H + h) * (int64_t)kMD;
  if (a.nsplit > 1) {
    // partial: m (natural log units), l, unnormalised o
    float* wo = a.ws + ((bq * a.H + h) * a.nsplit + blockIdx.z) * (int64_t)kMD;
    float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * a.nsplit * kMD + ((bq * a.H + h) * a.nsplit + blockIdx.z) * 2;
#pragma unroll
    for (int mt8 = 0; mt8 < 8; ++mt8)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = dh * 256 + mt8 * 32 + r4 * 8 + g32 * 4;
        *(float4*)(wo + d) = make_float4(acc[mt8][r4 * 4], acc[mt8][r4 * 4 + 1], acc[mt8][r4 * 4 + 2],
                                         acc[mt8][r4 * 4 + 3]);
      }
    if (dh == 0 && g32 == 0) {
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
  for (int mt8 = 0; mt8 < 8; ++mt8)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = dh * 256 + mt8 * 32 + r4 * 8 + g32 * 4;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = acc[mt8][r4 * 4 + i] * scale;
      if (a.out_f32) {
        *(float4*)((float*)a.out + qoff + d) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        u32x2 w;
        w.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
        w.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
        *(u32x2*)((uint16_t*)a.out + qoff + d) = w;
      }
    }
  if (a.lse && dh == 0 && g32 == 0) a.lse[bq * a.H + h] = lse;
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
