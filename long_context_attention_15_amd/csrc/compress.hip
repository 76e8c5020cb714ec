// Block compression + quantisation (csa_compress_kv, csa_decode_append).
//
// One wavefront per output entry.  Lane l owns VPL contiguous dims
// [l*VPL, l*VPL + VPL), so a row of 512 bf16 is one 16-byte load per lane.
// Pass 1 computes the m logits <x_i, gate> + bias_i (wave reductions), the
// softmax weights are formed in LDS, pass 2 accumulates sum_i alpha_i x_i in
// fixed order (the rows of pass 1 are still in L2), then the row is quantised
// and written; both passes load the block's rows kRowBatch at a time.  HBM
// traffic: the tokens once plus the stored rows.  The same entry code
// (compress_entry, store_entry) serves decode-time appends, so their bytes
// equal prefill's; m = 1 takes the packed quantiser quant_rows_kernel.
#include "common.h"
#include "launch.h"

namespace csa {

constexpr int kCompressWaves = 4;
constexpr int kMaxM = 1024;
constexpr int kRowBatch = 8;   // token rows whose loads are in flight together

template <typename TIn, int VPL>
__device__ __forceinline__ void load_vals(const TIn* p, float (&v)[VPL]);

// one element as float (BF16 widened exactly, as load_vals does)
__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const uint16_t* p) { return bf16_to_f32(*p); }

template <>
__device__ __forceinline__ void load_vals<float, 1>(const float* p, float (&v)[1]) { v[0] = *p; }
template <>
__device__ __forceinline__ void load_vals<float, 2>(const float* p, float (&v)[2]) {
  float2 t = *(const float2*)p; v[0] = t.x; v[1] = t.y;
}
template <>
__device__ __forceinline__ void load_vals<float, 4>(const float* p, float (&v)[4]) {
  float4 t = *(const float4*)p; v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
template <>
__device__ __forceinline__ void load_vals<float, 8>(const float* p, float (&v)[8]) {
  float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <>
__device__ __forceinline__ void load_vals<uint16_t, 1>(const uint16_t* p, float (&v)[1]) {
  v[0] = bf16_to_f32(*p);
}
template <>
__device__ __forceinline__ void load_vals<uint16_t, 2>(const uint16_t* p, float (&v)[2]) {
  uint32_t t = *(const uint32_t*)p; v[0] = bf16_to_f32(t & 0xffffu); v[1] = bf16_to_f32(t >> 16);
}
template <>
__device__ __forceinline__ void load_vals<uint16_t, 4>(const uint16_t* p, float (&v)[4]) {
  uint2 t = *(const uint2*)p;
  v[0] = bf16_to_f32(t.x & 0xffffu); v[1] = bf16_to_f32(t.x >> 16);
  v[2] = bf16_to_f32(t.y & 0xffffu); v[3] = bf16_to_f32(t.y >> 16);
}
template <>
__device__ __forceinline__ void load_vals<uint16_t, 8>(const uint16_t* p, float (&v)[8]) {
  uint4 t = *(const uint4*)p;
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_to_f32(w[i] & 0xffffu); v[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
}

// Quantise one entry (lane l holds dims [l*VPL, l*VPL + VPL) in acc; lanes
// with active == false hold none) into row `row_out` of `out`.  Called by
// the whole wavefront (row maxima are wavefront reductions).
template <int VPL>
__device__ __forceinline__ void store_entry(const float (&acc)[VPL], bool active, StoreW out, int64_t row_out) {
  const int lane = threadIdx.x % kWave;
  const int D = out.dim;
  uint8_t* dst = out.rows + row_out * out.row_bytes;
  if (out.fmt == CSA_F32) {
    if (active) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) ((float*)dst)[lane * VPL + v] = acc[v];
    }
  } else if (out.fmt == CSA_FP8_E4M3) {
    const int nb = D - out.rope;          // bulk dims
    const bool bulk = active && lane * VPL < nb;
    float am = 0.0f;
    if (bulk) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) am = fmaxf(am, fabsf(acc[v]));
    }
    am = wave_max(am);
    const float s = fp8_row_scale(am);
    const int es = ilogbf(s);
    if (bulk) {
      uint8_t c[VPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) c[v] = (uint8_t)f32_to_e4m3(ldexpf(acc[v], -es));
#pragma unroll
      for (int v = 0; v < VPL; ++v) dst[lane * VPL + v] = c[v];
    } else if (active) {
      uint16_t* r = (uint16_t*)(dst + nb);
#pragma unroll
      for (int v = 0; v < VPL; ++v) r[lane * VPL + v - nb] = (uint16_t)f32_to_bf16(acc[v]);
    }
    if (lane == 0) ((float*)out.scales)[row_out] = s;
  } else {  // CSA_MXFP4, VPL == 1, D in {32, 64}
    float am = active ? fabsf(acc[0]) : 0.0f;
    am = wave_max<32>(am);                // lanes 0-31 = block 0, 32-63 = block 1
    const int E = mx_block_exp(am);
    uint32_t c = active ? f32_to_e2m1(ldexpf(acc[0], -E)) : 0u;
    uint32_t hi = __shfl_xor(c, 1);
    if (active && (lane & 1) == 0) dst[lane >> 1] = (uint8_t)(c | (hi << 4));
    if (active && (lane & 31) == 0)
      ((uint8_t*)out.scales)[row_out * (D / 32) + (lane >> 5)] = (uint8_t)(E + 127);
  }
}

// RMSNorm and partial RoPE of one row held VPL dims per lane (lane l: dims
// [l*VPL, l*VPL + VPL); lanes with active == false hold none) at `position`.
// Called by the whole wavefront (the sum of squares is a wavefront
// reduction; with one dim per lane a pair's partner is the neighbour lane).
template <int VPL>
__device__ __forceinline__ void post_row(float (&acc)[VPL], bool active, int D, const NormRope& nr,
                                         int64_t position) {
  const int lane = threadIdx.x % kWave;
  if (nr.gain) {
    float ss = 0.0f;
    if (active) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) ss = fmaf(acc[v], acc[v], ss);
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + nr.eps);
    if (active) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) acc[v] = acc[v] * r * nr.gain[lane * VPL + v];
    }
  }
  if (nr.rope_dims > 0) {
    const int d0 = D - nr.rope_dims;
    const float pf = (float)position;
    if constexpr (VPL >= 2) {
      if (active) {
#pragma unroll
        for (int v = 0; v < VPL; v += 2) {
          const int d = lane * VPL + v;
          if (d >= d0) rope_pair(acc[v], acc[v + 1], pf, nr.theta[(d - d0) >> 1]);
        }
      }
    } else {
      float other = __shfl_xor(acc[0], 1);
      const int d = lane;
      if (active && d >= d0) {
        float x = (d & 1) ? other : acc[0], y = (d & 1) ? acc[0] : other;
        rope_pair(x, y, pf, nr.theta[(d - d0) >> 1]);
        acc[0] = (d & 1) ? y : x;
      }
    }
  }
}

// One output entry per wavefront: the m token rows are row(0) .. row(m-1)
// (lane l owns dims [l*VPL, l*VPL + VPL)); the entry goes to row `row_out`
// of `out`.  Called by every wavefront of the workgroup (the block
// barriers); a wavefront with valid == false computes on row(0) = some
// readable row and stores nothing.
template <typename TIn, int VPL, typename RowFn>
__device__ __forceinline__ void compress_entry(RowFn row, int m, const float* __restrict__ gate,
                                               const float* __restrict__ bias, StoreW out, int64_t row_out,
                                               bool valid, float* alpha, const NormRope& nr, int64_t position) {
  const int lane = threadIdx.x % kWave;
  const int D = out.dim;
  const bool active = valid && lane * VPL < D;

  float g[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) g[v] = active ? gate[lane * VPL + v] : 0.0f;

  // pass 1: logits, the rows loaded kRowBatch at a time, all in flight
  // together: the loads are unconditional (past the block's end they re-read
  // its last row, lanes past the row's dims re-read dims 0 .., all ignored),
  // so nothing waits between them.  Each row's dot product keeps its order.
  const int lo = lane * VPL < D ? lane * VPL : 0;
  for (int i0 = 0; i0 < m; i0 += kRowBatch) {
    float x[kRowBatch][VPL];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) load_vals<TIn, VPL>(row(i0 + u < m ? i0 + u : m - 1) + lo, x[u]);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      if (i0 + u >= m) break;                    // uniform
      float p = 0.0f;
      if (active) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) p = fmaf(x[u][v], g[v], p);
      }
      p = wave_sum(p);
      if (lane == 0) alpha[i0 + u] = p + bias[i0 + u];
    }
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int i = lane; i < m; i += kWave) mx = fmaxf(mx, alpha[i]);
  mx = wave_max(mx);
  float sum = 0.0f;
  for (int i = lane; i < m; i += kWave) {
    float ev = expf(alpha[i] - mx);
    alpha[i] = ev;
    sum += ev;
  }
  sum = wave_sum(sum);
  __syncthreads();
  for (int i = lane; i < m; i += kWave) alpha[i] = alpha[i] / sum;
  __syncthreads();

  // pass 2: weighted sum, fixed order over the block
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.0f;
  if (active) {
    // the sum starts from the first term (not from +0), so m = 1 stores x
    // itself, signed zeros included
    float x0[VPL];
    load_vals<TIn, VPL>(row(0) + lane * VPL, x0);
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] = alpha[0] * x0[v];
    for (int i0 = 1; i0 < m; i0 += kRowBatch) {
      float x[kRowBatch][VPL];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) load_vals<TIn, VPL>(row(i0 + u < m ? i0 + u : m - 1) + lo, x[u]);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        if (i0 + u >= m) break;
        const float a = alpha[i0 + u];
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[v] = fmaf(a, x[u][v], acc[v]);
      }
    }
  }

  if (!valid) return;
  post_row<VPL>(acc, active, D, nr, position);
  store_entry<VPL>(acc, active, out, row_out);
}

template <typename TIn, int VPL>
__global__ __launch_bounds__(kWave * kCompressWaves) void compress_kernel(
    const TIn* __restrict__ tok, int B, int64_t T, int64_t bstride, int m,
    const float* __restrict__ gate, const float* __restrict__ bias, StoreW out, int64_t row0,
    int64_t N, NormRope nr) {
  __shared__ float s_alpha[kCompressWaves][kMaxM];
  const int wave = threadIdx.x / kWave;
  int64_t e = (int64_t)blockIdx.x * kCompressWaves + wave;
  // waves past the end idle through the block barriers
  const bool valid = e < (int64_t)B * N;
  if (!valid) e = 0;
  const int b = (int)(e / N);
  const int64_t j = e % N;
  const int D = out.dim;
  const TIn* base = tok + (int64_t)b * bstride + j * m * (int64_t)D;
  compress_entry<TIn, VPL>([&](int i) { return base + (int64_t)i * D; }, m, gate, bias, out,
                           (int64_t)b * out.cap + row0 + j, valid, s_alpha[wave], nr, nr.pos0 + (j + 1) * m - 1);
}

// Decode-time cache maintenance, one wavefront per sequence b at position
// p = pos[b] (p < 0: nothing): the raw token goes to slot p mod R of the
// sequence's tail ring, its quantised row to window slot p mod W (when a
// window store is given), and when p closes a block ((p + 1) mod m == 0)
// the block's m raw tokens, read back from the tail ring in position order,
// are compressed into entry (p + 1) / m - 1 by the same code as
// compress_kernel (entries at or past out.cap are not written).  Each lane
// writes and reads back only its own dims of the tail row.
template <typename TIn, int VPL>
__global__ __launch_bounds__(kWave * kCompressWaves) void decode_append_kernel(
    const TIn* __restrict__ tok, int B, const int64_t* __restrict__ pos, TIn* tail, int R, int m,
    const float* __restrict__ gate, const float* __restrict__ bias, StoreW out, StoreW win, int W, NormRope nr) {
  __shared__ float s_alpha[kCompressWaves][kMaxM];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int b = (int)blockIdx.x * kCompressWaves + wave;
  const bool in_batch = b < B;
  if (!in_batch) b = 0;
  const int64_t p = pos[b];
  const bool live = in_batch && p >= 0;
  const int D = out.dim;
  const TIn* x = tok + (int64_t)b * D;
  TIn* tb = tail + (int64_t)b * R * D;
  if (live && lane * VPL < D) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) tb[(p % R) * D + lane * VPL + v] = x[lane * VPL + v];
  }
  if (win.rows && live) {                              // the window row: the token quantised
    float xv[VPL];
    const bool act = lane * VPL < D;
    if (act) load_vals<TIn, VPL>(x + lane * VPL, xv);
    else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) xv[v] = 0.0f;
    }
    post_row<VPL>(xv, act, D, nr, p);
    store_entry<VPL>(xv, act, win, (int64_t)b * win.cap + p % W);
  }
  const bool close = live && (p + 1) % m == 0 && (p + 1) / m - 1 < out.cap;
  if (!__syncthreads_or(close)) return;               // no block closes in this workgroup
  const int64_t j = close ? (p + 1) / m - 1 : 0;
  const int r0 = close ? (int)((p + 1 - m) % R) : 0;   // first row of the block in the ring
  compress_entry<TIn, VPL>(
      [&](int i) { return (const TIn*)tb + (int64_t)(r0 + i >= R ? r0 + i - R : r0 + i) * D; }, m, gate, bias, out,
      (int64_t)b * out.cap + j, close, s_alpha[wave], nr, p);
}

// Rebuild of a sequence's decode state from raw tokens: rows 0 .. nb-1 of
// sequence b (nb = min(n, n_valid[b]), or n) are the tokens at positions
// p0[b] .. p0[b] + nb - 1 (p0[b] a multiple of m; otherwise, or p0[b] < 0,
// the sequence is skipped).  One
// wavefront per (sequence, row), with the arithmetic of decode_append_kernel,
// so the stores end byte for byte as n decode appends at those positions
// leave them: the row goes to tail slot q mod R if it is among the last R
// rows, its processed row to window slot q mod W if among the last W, and a
// block that ends at the row is compressed from the rows themselves (they
// hold the same values the appends read back from the tail ring).
template <typename TIn, int VPL>
__global__ __launch_bounds__(kWave * kCompressWaves) void decode_rebuild_kernel(
    const TIn* __restrict__ tok, int B, int n, int64_t bstride, const int64_t* __restrict__ p0,
    const int32_t* __restrict__ n_valid, TIn* tail, int R, int m, const float* __restrict__ gate,
    const float* __restrict__ bias, StoreW out, StoreW win, int W, NormRope nr) {
  __shared__ float s_alpha[kCompressWaves][kMaxM];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t item = (int64_t)blockIdx.x * kCompressWaves + wave;
  const bool in_range = item < (int64_t)B * n;
  const int b = in_range ? (int)(item / n) : 0;
  const int i = in_range ? (int)(item % n) : 0;
  const int64_t q0 = in_range ? p0[b] : -1;
  const int nb = in_range && n_valid ? (n_valid[b] < n ? n_valid[b] : n) : n;
  const bool live = in_range && q0 >= 0 && q0 % m == 0 && i < nb;
  const int64_t q = q0 + i;
  const int D = out.dim;
  const TIn* x = tok + (int64_t)b * bstride + (int64_t)i * D;
  if (live && i >= nb - R && lane * VPL < D) {
    TIn* tb = tail + (int64_t)b * R * D;
#pragma unroll
    for (int v = 0; v < VPL; ++v) tb[(q % R) * D + lane * VPL + v] = x[lane * VPL + v];
  }
  if (win.rows && live && i >= nb - W) {                // uniform per wavefront
    float xv[VPL];
    const bool act = lane * VPL < D;
    if (act) load_vals<TIn, VPL>(x + lane * VPL, xv);
    else {
#pragma unroll
      for (int v = 0; v < VPL; ++v) xv[v] = 0.0f;
    }
    post_row<VPL>(xv, act, D, nr, q);
    store_entry<VPL>(xv, act, win, (int64_t)b * win.cap + q % W);
  }
  const bool close = live && (q + 1) % m == 0 && (q + 1) / m - 1 < out.cap;   // then i >= m - 1
  if (!__syncthreads_or(close)) return;                // no block closes in this workgroup
  const int64_t j = close ? (q + 1) / m - 1 : 0;
  const TIn* first = close ? x - (int64_t)(m - 1) * D : x;
  compress_entry<TIn, VPL>([&](int k) { return first + (int64_t)k * D; }, m, gate, bias, out,
                           (int64_t)b * out.cap + j, close, s_alpha[wave], nr, q);
}

template <typename TIn, int VPL>
static hipError_t launch_rebuild_t(const void* tok, int B, int n, int64_t bstride, const int64_t* p0,
                                   const int32_t* n_valid, void* tail, int R, int m, const float* gate, const float* bias, const csa_store& out,
                                   const csa_store& win, int W, const NormRope& nr, hipStream_t st) {
  const int64_t items = (int64_t)B * n;
  if (items == 0) return hipSuccess;
  const StoreW w = win.rows ? wview(win) : StoreW{nullptr, nullptr, 0, out.dim, 0, out.fmt, 0};
  hipLaunchKernelGGL((decode_rebuild_kernel<TIn, VPL>), dim3((unsigned)((items + kCompressWaves - 1) / kCompressWaves)),
                     dim3(kWave * kCompressWaves), 0, st, (const TIn*)tok, B, n, bstride, p0, n_valid, (TIn*)tail, R, m,
                     gate, bias, wview(out), w, W, nr);
  return hipGetLastError();
}

hipError_t launch_decode_rebuild(const void* tok, int tok_fmt, int B, int n, int64_t bstride, const int64_t* p0,
                                 const int32_t* n_valid, void* tail, int R, int m, const float* gate, const float* bias,
                                 const csa_store& out, const csa_store& win, int W, const NormRope& nr,
                                 hipStream_t st) {
  const int vpl = out.dim >= 64 ? out.dim / 64 : 1;
#define CSA_RB(TT, V) \
  return launch_rebuild_t<TT, V>(tok, B, n, bstride, p0, n_valid, tail, R, m, gate, bias, out, win, W, nr, st)
  if (tok_fmt == CSA_F32) {
    switch (vpl) { case 1: CSA_RB(float, 1); case 2: CSA_RB(float, 2); case 4: CSA_RB(float, 4); default: CSA_RB(float, 8); }
  } else {
    switch (vpl) { case 1: CSA_RB(uint16_t, 1); case 2: CSA_RB(uint16_t, 2); case 4: CSA_RB(uint16_t, 4); default: CSA_RB(uint16_t, 8); }
  }
#undef CSA_RB
}

// Decode-time maintenance for long blocks (m >= kWideMinM, the HCA cache):
// one workgroup of kWideWaves wavefronts per sequence, so a block close does
// not walk all m rows twice in one wavefront.  Wavefront 0 does the tail and
// window rows as decode_append_kernel does.  A close stays byte-identical to
// compress_entry: the wavefronts share the logits row by row with its per-row
// code (lane layout, FMA chain and reduction of one row do not depend on
// which wavefront runs them), wavefront 0 runs its softmax code, each thread
// forms one dim's weighted sum in its order over the rows, and wavefront 0
// takes the sums back into its lane layout for post_row and store_entry.
// The block's last row is the token itself (read from tok, so no thread reads
// another thread's fresh tail write).
constexpr int kWideWaves = 8;
constexpr int kWideMinM = 32;

template <typename TIn, int VPL>
__global__ __launch_bounds__(kWave * kWideWaves) void decode_append_wide_kernel(
    const TIn* __restrict__ tok, int B, const int64_t* __restrict__ pos, TIn* tail, int R, int m,
    const float* __restrict__ gate, const float* __restrict__ bias, StoreW out, StoreW win, int W, NormRope nr) {
  __shared__ float s_alpha[kMaxM];
  __shared__ float s_acc[512];
  // BF16 blocks of up to 128 rows x 512 dims stay in LDS between the logits
  // and the weighted sum (one round trip to memory instead of three)
  constexpr int kLdsRows = 128, kLdsDim = 512;
  __shared__ __attribute__((aligned(16))) uint16_t s_rows[sizeof(TIn) == 2 ? kLdsRows * kLdsDim : 8];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int b = blockIdx.x;
  const int64_t p = pos[b];
  const bool live = p >= 0;
  const int D = out.dim;
  const TIn* x = tok + (int64_t)b * D;
  TIn* tb = tail + (int64_t)b * R * D;
  const bool active = lane * VPL < D;
  if (wave == 0) {
    if (live && active) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) tb[(p % R) * D + lane * VPL + v] = x[lane * VPL + v];
    }
    if (win.rows && live) {
      float xv[VPL];
      if (active) load_vals<TIn, VPL>(x + lane * VPL, xv);
      else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) xv[v] = 0.0f;
      }
      post_row<VPL>(xv, active, D, nr, p);
      store_entry<VPL>(xv, active, win, (int64_t)b * win.cap + p % W);
    }
  }
  const bool close = live && (p + 1) % m == 0 && (p + 1) / m - 1 < out.cap;   // uniform in the workgroup
  if (!close) return;
  const int r0 = (int)((p + 1 - m) % R);              // ring row of the block's first token
  auto row = [&](int i) {                             // r0 + i < 2R: one conditional subtraction
    const int ri = r0 + i >= R ? r0 + i - R : r0 + i;
    return i == m - 1 ? x : (const TIn*)tb + (int64_t)ri * D;
  };
  // logits: rows wave * kWideRows .. +kWideRows, then every kWideWaves * kWideRows
  // on, all of a wavefront's rows in flight together
  constexpr int kWideRows = 16;
  float g[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) g[v] = active ? gate[lane * VPL + v] : 0.0f;
  const int lo = active ? lane * VPL : 0;
  const bool in_lds = sizeof(TIn) == 2 && m <= kLdsRows && D <= kLdsDim;   // uniform
  for (int i0 = wave * kWideRows; i0 < m; i0 += kWideWaves * kWideRows) {
    float xr[kWideRows][VPL];
#pragma unroll
    for (int u = 0; u < kWideRows; ++u) load_vals<TIn, VPL>(row(i0 + u < m ? i0 + u : m - 1) + lo, xr[u]);
#pragma unroll
    for (int u = 0; u < kWideRows; ++u) {
      if (i0 + u >= m) break;                    // uniform
      if (in_lds && active) {                    // the row's BF16 values (exact: they were BF16)
        uint32_t w[(VPL + 1) / 2];
#pragma unroll
        for (int v = 0; v < VPL; v += 2)
          w[v / 2] = (__float_as_uint(xr[u][v]) >> 16) | (VPL > 1 ? (__float_as_uint(xr[u][v + 1 < VPL ? v + 1 : v]) & 0xffff0000u) : 0u);
        if constexpr (VPL == 8) *(uint4*)(s_rows + (i0 + u) * kLdsDim + lo) = make_uint4(w[0], w[1], w[2], w[3]);
        else
#pragma unroll
          for (int v = 0; v < VPL; ++v) s_rows[(i0 + u) * kLdsDim + lo + v] = (uint16_t)(__float_as_uint(xr[u][v]) >> 16);
      }
      float pr = 0.0f;
      if (active) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) pr = fmaf(xr[u][v], g[v], pr);
      }
      pr = wave_sum(pr);
      if (lane == 0) s_alpha[i0 + u] = pr + bias[i0 + u];
    }
  }
  __syncthreads();
  if (wave == 0) {                                // the softmax weights, as compress_entry forms them
    float mx = -INFINITY;
    for (int i = lane; i < m; i += kWave) mx = fmaxf(mx, s_alpha[i]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int i = lane; i < m; i += kWave) {
      const float ev = expf(s_alpha[i] - mx);
      s_alpha[i] = ev;
      sum += ev;
    }
    sum = wave_sum(sum);
    for (int i = lane; i < m; i += kWave) s_alpha[i] = s_alpha[i] / sum;
  }
  __syncthreads();
  // weighted sum: thread t owns dim t, the terms in block order
  if (in_lds) {
    for (int d = threadIdx.x; d < D; d += kWave * kWideWaves) {
      float acc = s_alpha[0] * bf16_to_f32(s_rows[d]);
      for (int i = 1; i < m; ++i) acc = fmaf(s_alpha[i], bf16_to_f32(s_rows[i * kLdsDim + d]), acc);
      s_acc[d] = acc;
    }
  } else
  for (int d = threadIdx.x; d < D; d += kWave * kWideWaves) {
    float acc = s_alpha[0] * ldf(row(0) + d);
    for (int i0 = 1; i0 < m; i0 += 64) {        // 64 rows' loads in flight
      float xv[64];
#pragma unroll
      for (int u = 0; u < 64; ++u) xv[u] = ldf(row(i0 + u < m ? i0 + u : m - 1) + d);
#pragma unroll
      for (int u = 0; u < 64; ++u)
        if (i0 + u < m) acc = fmaf(s_alpha[i0 + u], xv[u], acc);
    }
    s_acc[d] = acc;
  }
  __syncthreads();
  if (wave == 0) {
    float acc[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] = active ? s_acc[lane * VPL + v] : 0.0f;
    post_row<VPL>(acc, active, D, nr, p);
    store_entry<VPL>(acc, active, out, (int64_t)b * out.cap + (p + 1) / m - 1);
  }
}

template <typename TIn, int VPL>
static hipError_t launch_append_wide_t(const void* tok, int B, const int64_t* pos, void* tail, int R, int m,
                                       const float* gate, const float* bias, const csa_store& out,
                                       const csa_store& win, int W, const NormRope& nr, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const StoreW w = win.rows ? wview(win) : StoreW{nullptr, nullptr, 0, out.dim, 0, out.fmt, 0};
  hipLaunchKernelGGL((decode_append_wide_kernel<TIn, VPL>), dim3((unsigned)B), dim3(kWave * kWideWaves), 0, st,
                     (const TIn*)tok, B, pos, (TIn*)tail, R, m, gate, bias, wview(out), w, W, nr);
  return hipGetLastError();
}

template <typename TIn, int VPL>
static hipError_t launch_append_t(const void* tok, int B, const int64_t* pos, void* tail, int R, int m,
                                  const float* gate, const float* bias, const csa_store& out, const csa_store& win,
                                  int W, const NormRope& nr, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const StoreW w = win.rows ? wview(win) : StoreW{nullptr, nullptr, 0, out.dim, 0, out.fmt, 0};
  hipLaunchKernelGGL((decode_append_kernel<TIn, VPL>), dim3((unsigned)((B + kCompressWaves - 1) / kCompressWaves)),
                     dim3(kWave * kCompressWaves), 0, st, (const TIn*)tok, B, pos, (TIn*)tail, R, m, gate, bias,
                     wview(out), w, W, nr);
  return hipGetLastError();
}

hipError_t launch_decode_append(const void* tok, int tok_fmt, int B, const int64_t* pos, void* tail, int R, int m,
                                const float* gate, const float* bias, const csa_store& out, const csa_store& win,
                                int W, const NormRope& nr, hipStream_t st) {
  const int vpl = out.dim >= 64 ? out.dim / 64 : 1;
#define CSA_APP(TT, V)                                                                          \
  return m >= kWideMinM ? launch_append_wide_t<TT, V>(tok, B, pos, tail, R, m, gate, bias, out, win, W, nr, st) \
                        : launch_append_t<TT, V>(tok, B, pos, tail, R, m, gate, bias, out, win, W, nr, st)
  if (tok_fmt == CSA_F32) {
    switch (vpl) { case 1: CSA_APP(float, 1); case 2: CSA_APP(float, 2); case 4: CSA_APP(float, 4); default: CSA_APP(float, 8); }
  } else {
    switch (vpl) { case 1: CSA_APP(uint16_t, 1); case 2: CSA_APP(uint16_t, 2); case 4: CSA_APP(uint16_t, 4); default: CSA_APP(uint16_t, 8); }
  }
#undef CSA_APP
}

// Blocks of one token (m = 1): the softmax weight of a single logit is
// exactly 1, so the entry is the token row itself and only the quantisation
// remains.  Rows are packed LPR lanes to a row, 8 contiguous values per lane
// (one 16-byte load of BF16), 64 / LPR rows per wavefront; the row maxima are
// reductions over the row's lane group.  Codes and scales are the ones the
// general kernel stores for m = 1.
template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) { load_vals<uint16_t, 8>(p, v); }
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) { load_vals<float, 8>(p, v); }

template <typename TIn, int LPR>
__global__ __launch_bounds__(kWave * kCompressWaves) void quant_rows_kernel(
    const TIn* __restrict__ tok, int B, int64_t bstride, StoreW out, int64_t row0, int64_t N, NormRope nr) {
  constexpr int RPW = kWave / LPR;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int li = lane % LPR;
  int64_t e = ((int64_t)blockIdx.x * kCompressWaves + wave) * RPW + lane / LPR;
  // lanes of rows past the end compute on row 0 (they take part in the
  // group reductions) and store nothing
  const bool valid = e < (int64_t)B * N;
  if (!valid) e = 0;
  const int b = (int)(e / N);
  const int64_t j = e % N;
  constexpr int D = LPR * 8;
  const int d0 = li * 8;
  float x[8];
  load8<TIn>(tok + (int64_t)b * bstride + j * D + d0, x);
  if (nr.gain) {                                // RMSNorm over the row's lane group
    float ss = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) ss = fmaf(x[v], x[v], ss);
    ss = wave_sum<LPR>(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + nr.eps);
#pragma unroll
    for (int v = 0; v < 8; ++v) x[v] = x[v] * r * nr.gain[d0 + v];
  }
  if (nr.rope_dims > 0) {                       // pairs start at even dims: within the lane
    const int dr = D - nr.rope_dims;
    const float pf = (float)(nr.pos0 + j);
#pragma unroll
    for (int v = 0; v < 8; v += 2)
      if (d0 + v >= dr) rope_pair(x[v], x[v + 1], pf, nr.theta[(d0 + v - dr) >> 1]);
  }
  const int64_t row = (int64_t)b * out.cap + row0 + j;
  uint8_t* dst = out.rows + row * out.row_bytes;
  if (out.fmt == CSA_F32) {
    if (valid) {
      float4* o = (float4*)((float*)dst + d0);
      o[0] = make_float4(x[0], x[1], x[2], x[3]);
      o[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
  } else if (out.fmt == CSA_FP8_E4M3) {
    const int nb = D - out.rope;                // bulk dims; the rest is the BF16 tail
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v)
      if (d0 + v < nb) am = fmaxf(am, fabsf(x[v]));
    am = wave_max<LPR>(am);
    const float s = fp8_row_scale(am);
    const int es = ilogbf(s);
    if (valid) {
      if (d0 + 8 <= nb) {
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          lo |= f32_to_e4m3(ldexpf(x[v], -es)) << (8 * v);
          hi |= f32_to_e4m3(ldexpf(x[v + 4], -es)) << (8 * v);
        }
        *(uint2*)(dst + d0) = make_uint2(lo, hi);
      } else if (d0 >= nb) {
        uint32_t w[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) w[v] = f32_to_bf16(x[2 * v]) | (f32_to_bf16(x[2 * v + 1]) << 16);
        *(uint4*)(dst + nb + 2 * (d0 - nb)) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int d = d0 + v;
          if (d < nb) dst[d] = (uint8_t)f32_to_e4m3(ldexpf(x[v], -es));
          else ((uint16_t*)(dst + nb))[d - nb] = (uint16_t)f32_to_bf16(x[v]);
        }
      }
      if (li == 0) ((float*)out.scales)[row] = s;
    }
  } else {  // CSA_MXFP4, D in {32, 64}: blocks of 32 values = 4 lanes
    float am = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) am = fmaxf(am, fabsf(x[v]));
    am = wave_max<4>(am);
    const int E = mx_block_exp(am);
    uint32_t pk = 0u;
#pragma unroll
    for (int v = 0; v < 8; ++v) pk |= f32_to_e2m1(ldexpf(x[v], -E)) << (4 * v);
    if (valid) {
      *(uint32_t*)(dst + d0 / 2) = pk;
      if ((li & 3) == 0) ((uint8_t*)out.scales)[row * (D / 32) + li / 4] = (uint8_t)(E + 127);
    }
  }
}

template <typename TIn, int LPR>
static hipError_t launch_quant_t(const void* tok, int B, int64_t T, int64_t bstride, const csa_store& out,
                                 int64_t row0, const NormRope& nr, hipStream_t st) {
  const int64_t items = (int64_t)B * T;
  if (items == 0) return hipSuccess;
  constexpr int rows_per_block = kCompressWaves * (kWave / LPR);
  const int64_t blocks = (items + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((quant_rows_kernel<TIn, LPR>), dim3((unsigned)blocks), dim3(kWave * kCompressWaves), 0, st,
                     (const TIn*)tok, B, bstride, wview(out), row0, T, nr);
  return hipGetLastError();
}

template <typename TIn>
static hipError_t launch_quant(const void* tok, int B, int64_t T, int64_t bstride, const csa_store& out,
                               int64_t row0, const NormRope& nr, hipStream_t st) {
  switch (out.dim / 8) {
    case 4: return launch_quant_t<TIn, 4>(tok, B, T, bstride, out, row0, nr, st);
    case 8: return launch_quant_t<TIn, 8>(tok, B, T, bstride, out, row0, nr, st);
    case 16: return launch_quant_t<TIn, 16>(tok, B, T, bstride, out, row0, nr, st);
    case 32: return launch_quant_t<TIn, 32>(tok, B, T, bstride, out, row0, nr, st);
    default: return launch_quant_t<TIn, 64>(tok, B, T, bstride, out, row0, nr, st);
  }
}

// What the m = 1 path assumes: 8 | dim with a power-of-two lane group of 4
// to 64 lanes, 16-byte aligned token rows and batch stride, 16-byte aligned
// store rows, an FP8 bulk that ends on a 16-byte boundary, MXFP4 rows of 32
// or 64 values.  Every store the entry point accepts meets it (dims 32 to
// 512); the check keeps the kernel's assumptions next to it.
static bool quant_rows_ok(const void* tok, int tok_fmt, int64_t bstride, const csa_store& out) {
  const int D = out.dim, lpr = D / 8;
  if (D % 8 != 0 || lpr < 4 || lpr > 64 || (lpr & (lpr - 1)) != 0) return false;
  if (out.fmt == CSA_MXFP4 && (D > 64 || out.rope_dim != 0)) return false;
  const int esz = tok_fmt == CSA_F32 ? 4 : 2;
  if ((uintptr_t)tok % 16 != 0 || (bstride * esz) % 16 != 0) return false;
  if ((uintptr_t)out.rows % 16 != 0) return false;
  if (out.fmt != CSA_MXFP4 && out.row_bytes % 16 != 0) return false;
  if (out.fmt == CSA_FP8_E4M3 && (D - out.rope_dim) % 16 != 0) return false;
  return true;
}

template <typename TIn, int VPL>
static hipError_t launch_compress_t(const void* tok, int B, int64_t T, int64_t bstride, int m,
                                    const float* gate, const float* bias, const csa_store& out,
                                    int64_t row0, const NormRope& nr, hipStream_t st) {
  const int64_t N = T / m;
  const int64_t items = (int64_t)B * N;
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + kCompressWaves - 1) / kCompressWaves;
  hipLaunchKernelGGL((compress_kernel<TIn, VPL>), dim3((unsigned)blocks), dim3(kWave * kCompressWaves),
                     0, st, (const TIn*)tok, B, T, bstride, m, gate, bias, wview(out), row0, N, nr);
  return hipGetLastError();
}

hipError_t launch_compress(const void* tok, int tok_fmt, int B, int64_t T, int64_t bstride, int m,
                           const float* gate, const float* bias, const csa_store& out, int64_t row0,
                           const NormRope& nr, hipStream_t st) {
  if (m == 1 && quant_rows_ok(tok, tok_fmt, bstride, out))
    return tok_fmt == CSA_F32 ? launch_quant<float>(tok, B, T, bstride, out, row0, nr, st)
                              : launch_quant<uint16_t>(tok, B, T, bstride, out, row0, nr, st);
  const int vpl = out.dim >= 64 ? out.dim / 64 : 1;
#define CSA_CMP(TT, V) return launch_compress_t<TT, V>(tok, B, T, bstride, m, gate, bias, out, row0, nr, st)
  if (tok_fmt == CSA_F32) {
    switch (vpl) { case 1: CSA_CMP(float, 1); case 2: CSA_CMP(float, 2); case 4: CSA_CMP(float, 4); default: CSA_CMP(float, 8); }
  } else {
    switch (vpl) { case 1: CSA_CMP(uint16_t, 1); case 2: CSA_CMP(uint16_t, 2); case 4: CSA_CMP(uint16_t, 4); default: CSA_CMP(uint16_t, 8); }
  }
#undef CSA_CMP
}

int compress_max_m() { return kMaxM; }

}  // namespace csa
