// Lightning Indexer scoring + top-k selection (csa_indexer_topk).
//
// A workgroup scores one chunk of entries for one query into LDS as
// order-preserving uint32 keys, finds the exact k-th largest key with a 4-pass
// 8-bit radix select (LDS histograms, a wavefront suffix scan), and emits the
// selected entries in ascending index order with ballot/prefix counts, ties
// going to the smaller index.  When a query's entries span several chunks,
// each chunk emits its local top-k as candidates and a merge kernel selects
// the final top-k from the candidates (the candidate list is in ascending
// index order, so position order is index order for the tie rule).
#include "common.h"
#include "launch.h"

namespace csa {

constexpr int kIdxThreads = 512;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kMaxChunk = 32768;     // 128 KiB of keys in LDS
constexpr int kMaxCand = 32768;      // merge: candidates per query
constexpr int kMaxHI = 16;
constexpr int kMaxDI = 64;

struct SelShared {
  uint32_t hist[2048];
  uint32_t misc[4];
  uint32_t wtot[2][kIdxWaves];
};

// Exact radix select on keys[0, n): returns the kk-th largest key `thr` and
// how many keys equal to thr are to be taken (the first ones by position).
// Three passes over 11/11/10-bit digits, most significant first; each pass
// histograms the keys that match the digits found so far and one wavefront
// locates the digit holding the kk-th key with a suffix scan.
// Needs 1 <= kk <= #nonzero keys.  Called by all kIdxThreads threads.
__device__ void radix_select(const uint32_t* keys, int n, int kk, SelShared& sh, uint32_t& thr,
                             int& need_eq) {
  const int tid = threadIdx.x, lane = tid % kWave;
  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += kIdxThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kIdxThreads) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      const int per = nb / kWave;            // 32 or 16 bins per lane
      uint32_t local = 0;
      for (int i = 0; i < per; ++i) local += sh.hist[per * lane + i];
      uint32_t suf = local;                  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_down(suf, o);
        if (lane + o < kWave) suf += t;
      }
      uint32_t above = suf - local;          // keys in bins of higher lanes
      if (above < (uint32_t)remaining && suf >= (uint32_t)remaining) {
        for (int i = per - 1; i >= 0; --i) {
          const uint32_t c = sh.hist[per * lane + i];
          if (above + c >= (uint32_t)remaining) {
            sh.misc[0] = per * lane + i;
            sh.misc[1] = above;
            break;
          }
          above += c;
        }
      }
    }
    __syncthreads();
    const uint32_t d = sh.misc[0];
    remaining -= (int)sh.misc[1];
    prefix |= d << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  thr = prefix;
  need_eq = remaining;
}

// Call emit(pos, rank) for each selected position, rank = its index in the
// ascending output.  Wave w walks its own contiguous range of positions in
// 64-wide rounds; a first pass counts keys above / equal to thr per wave,
// one barrier publishes the counts, the second pass emits with ballot
// prefixes (no further barriers).
template <typename Emit>
__device__ void emit_selected(const uint32_t* keys, int n, uint32_t thr, int need_eq, SelShared& sh,
                              Emit emit) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int per = ((n + kIdxWaves * kWave - 1) / (kIdxWaves * kWave)) * kWave;
  const int p0 = wave * per;
  const int p1 = p0 + per < n ? p0 + per : n;
  uint32_t ngt = 0, neq = 0;
  for (int r0 = p0; r0 < p1; r0 += kWave) {
    const int pos = r0 + lane;
    const uint32_t key = pos < p1 ? keys[pos] : 0u;
    ngt += (uint32_t)__popcll(__ballot(key != 0u && key > thr));
    neq += (uint32_t)__popcll(__ballot(key != 0u && key == thr));
  }
  if (lane == 0) { sh.wtot[0][wave] = ngt; sh.wtot[1][wave] = neq; }
  __syncthreads();
  int eq_base = 0, sel_base = 0;
  for (int w = 0; w < wave; ++w) {
    const int gt = (int)sh.wtot[0][w], eq = (int)sh.wtot[1][w];
    int take_eq = need_eq - eq_base;
    take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    sel_base += gt + take_eq;
    eq_base += eq;
  }
  for (int r0 = p0; r0 < p1; r0 += kWave) {
    const int pos = r0 + lane;
    const uint32_t key = pos < p1 ? keys[pos] : 0u;
    const bool eq = key != 0u && key == thr;
    const uint64_t beq = __ballot(eq);
    const bool take = (key != 0u && key > thr) || (eq && eq_base + __popcll(beq & lt) < need_eq);
    const uint64_t bs = __ballot(take);
    if (take) emit(pos, sel_base + __popcll(bs & lt));
    eq_base += __popcll(beq);
    sel_base += __popcll(bs);
  }
}

// ------------------------------------------------------------ row decoding
template <int FMT>
__device__ __forceinline__ void decode_row(const Store& s, int64_t row, int d, float* out);

template <>
__device__ __forceinline__ void decode_row<CSA_F32>(const Store& s, int64_t row, int d, float* out) {
  const float* p = (const float*)(s.rows + row * s.row_bytes);
  for (int i = 0; i < d; i += 4) {
    float4 v = *(const float4*)(p + i);
    out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
  }
}

template <>
__device__ __forceinline__ void decode_row<CSA_FP8_E4M3>(const Store& s, int64_t row, int d, float* out) {
  const uint8_t* p = s.rows + row * s.row_bytes;
  const float sc = ((const float*)s.scales)[row];
  for (int i = 0; i < d; i += 16) {
    uint4 v = *(const uint4*)(p + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) out[i + 4 * q + bb] = e4m3_to_f32((w[q] >> (8 * bb)) & 255u) * sc;
  }
}

template <>
__device__ __forceinline__ void decode_row<CSA_MXFP4>(const Store& s, int64_t row, int d, float* out) {
  const uint8_t* p = s.rows + row * s.row_bytes;
  const uint8_t* e8 = (const uint8_t*)s.scales + row * (d / 32);
  for (int blk = 0; blk < d / 32; ++blk) {
    const float sc = ldexpf(1.0f, (int)e8[blk] - 127);
    uint4 v = *(const uint4*)(p + 16 * blk);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) out[32 * blk + 8 * q + nb] = e2m1_to_f32((w[q] >> (4 * nb)) & 15u) * sc;
  }
}

struct IdxArgs {
  Store qidx, keys;
  const float* head_w;
  int64_t n_entries;
  const int64_t* q_pos;
  int B, Tq, H_I, m, k, chunk, nchunk;
  int32_t* sel;
  uint32_t* ws_key;
  int32_t* ws_idx;
};

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

// Scores of entries [c0, c0 + cn) for one query on MFMA, written to s_keys.
// Heads are the 16 rows of the A operand (H_I <= 16, the rest zero), 16
// entries are the columns; the head-weighted ReLU sum is a lane-local sum
// over 4 heads plus two cross-lane adds.
//   FP8  : v_mfma_f32_16x16x32_fp8_fp8; the row scales of q fold into the
//          head weights, the key scale multiplies the sum (powers of two).
//   MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands and the
//          per-32-element E8M0 scales applied by the instruction; k-blocks
//          beyond d_I are zero.
template <int FMT, int DI>
__device__ __forceinline__ void score_chunk_mfma(const IdxArgs& a, int b, int q, int64_t bq, int64_t c0, int cn,
                                                 uint32_t* s_keys, float* s_w) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, g = lane >> 4;
  const int64_t qrow0 = (int64_t)b * a.qidx.cap + (int64_t)q * a.H_I;
  // head weights for the 4 heads of this lane's accumulator rows
  for (int h = tid; h < 16; h += kIdxThreads) {
    float w = 0.0f;
    if (h < a.H_I) {
      w = a.head_w[bq * a.H_I + h];
      if (FMT == CSA_FP8_E4M3) w *= ((const float*)a.qidx.scales)[qrow0 + h];
    }
    s_w[h] = w;
  }
  __syncthreads();
  float wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wl[i] = s_w[4 * g + i];
  const int64_t krow0 = (int64_t)b * a.keys.cap + c0;
  const int ngroups = (cn + 15) / 16;
  if constexpr (FMT == CSA_FP8_E4M3) {
    // A operand: q row `col`, K-step 0 = bytes [16g, 16g+8), K-step 1 = [16g+8, 16g+16)
    // (DI = 32: one K-step of bytes [8g, 8g+8))
    long long qa0 = 0, qa1 = 0;
    if (col < a.H_I) {
      const uint8_t* qp = a.qidx.rows + (qrow0 + col) * a.qidx.row_bytes;
      if (DI == 64) {
        const uint4 v = *(const uint4*)(qp + 16 * g);
        qa0 = (long long)(((unsigned long long)v.y << 32) | v.x);
        qa1 = (long long)(((unsigned long long)v.w << 32) | v.z);
      } else {
        const uint2 v = *(const uint2*)(qp + 8 * g);
        qa0 = (long long)(((unsigned long long)v.y << 32) | v.x);
      }
    }
    const float* ksc = (const float*)a.keys.scales;
    constexpr int U = 8;                    // groups in flight per wave
    for (int grp0 = wave * U; grp0 < ngroups; grp0 += kIdxWaves * U) {
      long long kb0[U], kb1[U];
      float sk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (grp0 + u) * 16 + col;
        kb0[u] = 0; kb1[u] = 0; sk[u] = 0.0f;
        if (e < cn) {
          const uint8_t* kp = a.keys.rows + (krow0 + e) * a.keys.row_bytes;
          if (DI == 64) {
            const uint4 v = *(const uint4*)(kp + 16 * g);
            kb0[u] = (long long)(((unsigned long long)v.y << 32) | v.x);
            kb1[u] = (long long)(((unsigned long long)v.w << 32) | v.z);
          } else {
            const uint2 v = *(const uint2*)(kp + 8 * g);
            kb0[u] = (long long)(((unsigned long long)v.y << 32) | v.x);
          }
          sk[u] = ksc[krow0 + e];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (grp0 + u) * 16 + col;
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qa0, kb0[u], c, 0, 0, 0);
        if (DI == 64) c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qa1, kb1[u], c, 0, 0, 0);
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wl[i], fmaxf(c[i], 0.0f), v);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0 && e < cn) s_keys[e] = score_key(v * sk[u]);
      }
    }
  } else {
    // A operand: q row `col`, k-block g (32 E2M1 = 16 bytes) and its E8M0
    i32x8 qa = {0, 0, 0, 0, 0, 0, 0, 0};
    int qs = 127;
    if (col < a.H_I && g < DI / 32) {
      const uint8_t* qp = a.qidx.rows + (qrow0 + col) * a.qidx.row_bytes;
      const uint4 v = *(const uint4*)(qp + 16 * g);
      qa[0] = (int)v.x; qa[1] = (int)v.y; qa[2] = (int)v.z; qa[3] = (int)v.w;
      qs = ((const uint8_t*)a.qidx.scales)[(qrow0 + col) * (DI / 32) + g];
    }
    const uint8_t* ksc = (const uint8_t*)a.keys.scales;
    constexpr int U = 8;
    for (int grp0 = wave * U; grp0 < ngroups; grp0 += kIdxWaves * U) {
      uint4 kv[U];
      int ks[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (grp0 + u) * 16 + col;
        kv[u] = make_uint4(0u, 0u, 0u, 0u);
        ks[u] = 127;
        if (e < cn && g < DI / 32) {
          const uint8_t* kp = a.keys.rows + (krow0 + e) * a.keys.row_bytes;
          kv[u] = *(const uint4*)(kp + 16 * g);
          ks[u] = ksc[(krow0 + e) * (DI / 32) + g];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (grp0 + u) * 16 + col;
        i32x8 kb = {(int)kv[u].x, (int)kv[u].y, (int)kv[u].z, (int)kv[u].w, 0, 0, 0, 0};
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, kb, c, 4, 4, 0, qs, 0, ks[u]);
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wl[i], fmaxf(c[i], 0.0f), v);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0 && e < cn) s_keys[e] = score_key(v);
      }
    }
  }
}

template <int FMT, int DI>
__global__ __launch_bounds__(kIdxThreads) void idx_chunk_kernel(IdxArgs a) {
  extern __shared__ uint32_t s_keys[];
  __shared__ float s_q[kMaxHI * kMaxDI];
  __shared__ float s_w[kMaxHI];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int64_t bq = blockIdx.x;             // b * Tq + q
  const int b = (int)(bq / a.Tq), q = (int)(bq % a.Tq);
  const int c = blockIdx.y;
  const int64_t t = a.q_pos ? a.q_pos[bq] : (int64_t)q;
  int64_t nt = t < 0 ? 0 : (t + 1) / a.m;
  if (nt > a.n_entries) nt = a.n_entries;
  const int64_t c0 = (int64_t)c * a.chunk;
  int64_t cn64 = nt - c0;
  const int cn = cn64 < 0 ? 0 : (cn64 > a.chunk ? a.chunk : (int)cn64);
  const int kk = cn < a.k ? cn : a.k;
  const bool direct = a.nchunk == 1;
  int32_t* out_idx = direct ? a.sel + bq * a.k : a.ws_idx + (bq * a.nchunk + c) * a.k;
  uint32_t* out_key = direct ? nullptr : a.ws_key + (bq * a.nchunk + c) * a.k;

  // pad the slots that will not be filled
  for (int i = kk + tid; i < a.k; i += kIdxThreads) {
    out_idx[i] = -1;
    if (!direct) out_key[i] = 0u;
  }
  if (kk == 0) return;                        // uniform over the workgroup

  if constexpr (FMT == CSA_F32) {
    // queries and head weights
    for (int h = tid; h < a.H_I; h += kIdxThreads) {
      decode_row<FMT>(a.qidx, (int64_t)b * a.qidx.cap + (int64_t)q * a.H_I + h, DI, s_q + h * DI);
      s_w[h] = a.head_w[bq * a.H_I + h];
    }
    __syncthreads();
    for (int e = tid; e < cn; e += kIdxThreads) {
      float kv[DI];
      decode_row<FMT>(a.keys, (int64_t)b * a.keys.cap + c0 + e, DI, kv);
      float s = 0.0f;
      for (int h = 0; h < a.H_I; ++h) {
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < DI; ++d) dot = fmaf(s_q[h * DI + d], kv[d], dot);
        s = fmaf(s_w[h], fmaxf(dot, 0.0f), s);
      }
      s_keys[e] = score_key(s);
    }
  } else {
    score_chunk_mfma<FMT, DI>(a, b, q, bq, c0, cn, s_keys, s_w);
  }
  __syncthreads();

  uint32_t thr;
  int need_eq;
  radix_select(s_keys, cn, kk, sh, thr, need_eq);
  emit_selected(s_keys, cn, thr, need_eq, sh, [&](int pos, int rank) {
    out_idx[rank] = (int32_t)(c0 + pos);
    if (!direct) out_key[rank] = s_keys[pos];
  });
}

__global__ __launch_bounds__(kIdxThreads) void idx_merge_kernel(IdxArgs a) {
  extern __shared__ uint32_t s_keys[];
  __shared__ SelShared sh;
  __shared__ uint32_t s_cnt;
  const int tid = threadIdx.x;
  const int64_t bq = blockIdx.x;
  const int n = a.nchunk * a.k;
  const uint32_t* ck = a.ws_key + bq * n;
  const int32_t* ci = a.ws_idx + bq * n;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  uint32_t mine = 0;
  for (int i = tid; i < n; i += kIdxThreads) {
    const uint32_t key = ck[i];
    s_keys[i] = key;
    mine += key != 0u;
  }
  atomicAdd(&s_cnt, mine);
  __syncthreads();
  const int valid = (int)s_cnt;
  const int kk = valid < a.k ? valid : a.k;
  int32_t* out = a.sel + bq * a.k;
  for (int i = kk + tid; i < a.k; i += kIdxThreads) out[i] = -1;
  if (kk == 0) return;
  uint32_t thr;
  int need_eq;
  radix_select(s_keys, n, kk, sh, thr, need_eq);
  emit_selected(s_keys, n, thr, need_eq, sh, [&](int pos, int rank) { out[rank] = ci[pos]; });
}

IdxPlan indexer_plan(int B, int Tq, int64_t n_entries, int k) {
  IdxPlan p{0, 0, 0, false};
  if (n_entries <= 0) { p.chunk = 1024; p.nchunk = 1; p.ok = true; return p; }
  int64_t chunk = 1024;
  const int64_t queries = (int64_t)B * Tq;
  // many queries: one chunk per query when it fits; few queries (decode):
  // chunks of at most 8192 entries for more workgroups
  const int64_t target = queries >= 256 ? n_entries : (n_entries < 8192 ? n_entries : 8192);
  while (chunk < target && chunk < kMaxChunk) chunk <<= 1;
  // the merge keeps nchunk * k candidates in LDS
  while ((n_entries + chunk - 1) / chunk * (int64_t)k > kMaxCand && chunk < kMaxChunk) chunk <<= 1;
  const int64_t nch = (n_entries + chunk - 1) / chunk;
  if (nch > 1 && nch * (int64_t)k > kMaxCand) return p;
  p.chunk = (int)chunk;
  p.nchunk = (int)nch;
  p.ws = nch > 1 ? (size_t)queries * nch * k * 8 : 0;
  p.ok = true;
  return p;
}

template <int FMT, int DI>
static hipError_t launch_idx_t(const IdxArgs& a, hipStream_t st) {
  const size_t lds = (size_t)a.chunk * 4;
  auto kfn = idx_chunk_kernel<FMT, DI>;
  hipError_t e = hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3((unsigned)((int64_t)a.B * a.Tq), a.nchunk), dim3(kIdxThreads), lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.nchunk == 1) return e;
  const size_t lds2 = (size_t)a.nchunk * a.k * 4;
  e = hipFuncSetAttribute((const void*)idx_merge_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_merge_kernel, dim3((unsigned)((int64_t)a.B * a.Tq)), dim3(kIdxThreads), lds2, st, a);
  return hipGetLastError();
}

hipError_t launch_indexer(const csa_store& qidx, const float* head_w, const csa_store& keys,
                          int64_t n_entries, const int64_t* q_pos, int B, int Tq, int H_I, int m,
                          int k, int32_t* sel, void* ws, const IdxPlan& plan, hipStream_t st) {
  IdxArgs a;
  a.qidx = view(qidx);
  a.keys = view(keys);
  a.head_w = head_w;
  a.n_entries = n_entries;
  a.q_pos = q_pos;
  a.B = B; a.Tq = Tq; a.H_I = H_I; a.m = m; a.k = k;
  a.chunk = plan.chunk; a.nchunk = plan.nchunk;
  a.sel = sel;
  const size_t half = plan.ws / 2;
  a.ws_key = (uint32_t*)ws;
  a.ws_idx = (int32_t*)((uint8_t*)ws + half);
  if ((int64_t)B * Tq == 0) return hipSuccess;
  const int d = keys.dim;
  switch (keys.fmt) {
    case CSA_F32: return d == 32 ? launch_idx_t<CSA_F32, 32>(a, st) : launch_idx_t<CSA_F32, 64>(a, st);
    case CSA_FP8_E4M3: return d == 32 ? launch_idx_t<CSA_FP8_E4M3, 32>(a, st) : launch_idx_t<CSA_FP8_E4M3, 64>(a, st);
    default: return d == 32 ? launch_idx_t<CSA_MXFP4, 32>(a, st) : launch_idx_t<CSA_MXFP4, 64>(a, st);
  }
}

}  // namespace csa
