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
  uint32_t hist[256];
  uint32_t misc[4];
  uint32_t wtot[2][kIdxWaves];
};

// Exact radix select on keys[0, n): returns the k-th largest key `thr` and how
// many keys equal to thr are to be taken (the first ones by position).
// Needs 1 <= kk <= #nonzero keys.  Called by all kIdxThreads threads.
__device__ void radix_select(const uint32_t* keys, int n, int kk, SelShared& sh, uint32_t& thr,
                             int& need_eq) {
  const int tid = threadIdx.x, lane = tid % kWave;
  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kIdxThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kIdxThreads) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = sh.hist[4 * lane + i];
      uint32_t local = c[0] + c[1] + c[2] + c[3];
      uint32_t suf = local;               // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_down(suf, o);
        if (lane + o < kWave) suf += t;
      }
      uint32_t above = suf - local;       // keys in bins of higher lanes
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < (uint32_t)remaining && above + c[i] >= (uint32_t)remaining) {
          sh.misc[0] = 4 * lane + i;
          sh.misc[1] = above;
        }
        above += c[i];
      }
    }
    __syncthreads();
    const uint32_t d = sh.misc[0];
    remaining -= (int)sh.misc[1];
    prefix |= d << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  thr = prefix;
  need_eq = remaining;
}

// Walk positions 0..n-1 in order and call emit(pos, rank) for each selected
// position; rank is its index in the ascending output.  Returns nothing; all
// threads participate.
template <typename Emit>
__device__ void emit_selected(const uint32_t* keys, int n, uint32_t thr, int need_eq, SelShared& sh,
                              Emit emit) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eq_base = 0, sel_base = 0;
  for (int r0 = 0; r0 < n; r0 += kIdxThreads) {
    const int pos = r0 + tid;
    const uint32_t key = pos < n ? keys[pos] : 0u;
    const bool eq = key != 0u && key == thr;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) sh.wtot[0][wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    int woff = 0, tot_eq = 0;
    for (int w = 0; w < kIdxWaves; ++w) {
      const int v = (int)sh.wtot[0][w];
      woff += w < wave ? v : 0;
      tot_eq += v;
    }
    const int eq_rank = eq_base + woff + __popcll(beq & lt);
    const bool take = (key != 0u && key > thr) || (eq && eq_rank < need_eq);
    const uint64_t bs = __ballot(take);
    if (lane == 0) sh.wtot[1][wave] = (uint32_t)__popcll(bs);
    __syncthreads();
    int soff = 0, tot_s = 0;
    for (int w = 0; w < kIdxWaves; ++w) {
      const int v = (int)sh.wtot[1][w];
      soff += w < wave ? v : 0;
      tot_s += v;
    }
    if (take) emit(pos, sel_base + soff + __popcll(bs & lt));
    eq_base += tot_eq;
    sel_base += tot_s;
    __syncthreads();
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

  // queries (dequantised) and head weights
  for (int h = tid; h < a.H_I; h += kIdxThreads) {
    decode_row<FMT>(a.qidx, (int64_t)b * a.qidx.cap + (int64_t)q * a.H_I + h, DI, s_q + h * DI);
    s_w[h] = a.head_w[bq * a.H_I + h];
  }
  __syncthreads();

  // score the chunk
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
