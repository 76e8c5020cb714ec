// Gathered-entry attention with sliding window and sink (CSA prefill/decode,
// HCA, swa_merge): the float32 VALU path.
//
// A workgroup owns one query row and HG heads; TPH threads share a head, each
// holding DPT dims of q and of the output accumulator.  Entries are staged
// into LDS in tiles of kTile rows, decoded to float32 once per workgroup,
// then every head computes its logits (dot + TPH-lane reduction) and updates
// its online-softmax state.  The entry list of a query is its compressed
// part (the top-k slots, or the visible range 0..n_t-1) followed by the W
// window slots.  Long lists can be split across workgroups; the partial
// (max, sum, unnormalised o) of each split is merged in a fixed order.
#include "common.h"
#include "launch.h"

namespace csa {

constexpr int kTile = 16;
constexpr int kAttnThreads = 256;

struct AttnArgs {
  const void* q; int q_f32; int B, Tq, H, D;
  Store ckv; int64_t n_entries; int mode; const int32_t* sel; int k; int m;
  Store win; int W; int ring; const int64_t* q_pos;
  const float* sink; float tau;
  const float* prior_o; const float* prior_lse;
  void* out; int out_f32; float* lse; int partial;
  int nsplit; int split_len; float* ws;
  NormRope qn;
};

__device__ __forceinline__ int64_t query_pos(const AttnArgs& a, int64_t bq) {
  return a.q_pos ? a.q_pos[bq] : (int64_t)(bq % a.Tq);
}

__device__ __forceinline__ int64_t visible(int64_t t, int m, int64_t n) {
  int64_t v = t < 0 ? 0 : (t + 1) / m;
  return v < n ? v : n;
}

// Row of list slot i of query (b, t); returns false when the slot is empty.
__device__ __forceinline__ bool list_row(const AttnArgs& a, int64_t bq, int b, int64_t t, int64_t Lc,
                                         int64_t i, const Store*& st, int64_t& row) {
  if (i < Lc) {
    int64_t j;
    if (a.mode == kModeSel) {
      j = a.sel[bq * a.k + i];
      if (j < 0 || j >= a.n_entries) return false;
    } else {
      j = i;
    }
    st = &a.ckv;
    row = (int64_t)b * a.ckv.cap + j;
    return true;
  }
  const int64_t w = i - Lc;
  const int64_t p = t - a.W + 1 + w;
  if (p < 0 || (!a.ring && p >= a.win.cap)) return false;
  st = &a.win;
  row = (int64_t)b * a.win.cap + (a.ring ? p % a.W : p);
  return true;
}

// Decode 16-byte chunk cc of a stored row into dst (float32, row layout).
__device__ __forceinline__ void decode_chunk(const Store& s, int64_t row, int cc, float* dst) {
  const uint8_t* p = s.rows + row * s.row_bytes + 16 * cc;
  const uint4 v = *(const uint4*)p;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if (s.fmt == CSA_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[4 * cc + i] = __uint_as_float(w[i]);
    return;
  }
  const int nbulk = s.dim - s.rope;
  if (16 * cc < nbulk) {
    const float sc = ((const float*)s.scales)[row];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) dst[16 * cc + 4 * i + bb] = e4m3_to_f32((w[i] >> (8 * bb)) & 255u) * sc;
  } else {
    const int d0 = nbulk + (16 * cc - nbulk) / 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[d0 + 2 * i] = bf16_to_f32(w[i] & 0xffffu);
      dst[d0 + 2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

template <int TPH, int DPT>
__global__ __launch_bounds__(kAttnThreads) void attn_valu_kernel(AttnArgs a) {
  constexpr int D = TPH * DPT;
  __shared__ float s_e[kTile][D];
  __shared__ int64_t s_row[kTile];
  __shared__ int s_src[kTile];           // 0 none, 1 ckv, 2 window
  const int tid = threadIdx.x;
  const int HG = blockDim.x / TPH;
  const int64_t bq = blockIdx.x;
  const int h = blockIdx.y * HG + tid / TPH;
  const int p = tid % TPH;
  const int b = (int)(bq / a.Tq);
  const int64_t t = query_pos(a, bq);
  const int64_t Lc = a.mode == kModeSel ? a.k : (a.mode == kModeRange ? visible(t, a.m, a.n_entries) : 0);
  const int64_t L = Lc + a.W;
  const int64_t i0 = (int64_t)blockIdx.z * a.split_len;
  const int64_t i1 = a.nsplit == 1 ? L : (i0 + a.split_len < L ? i0 + a.split_len : L);

  float qv[DPT], o[DPT];
  const int64_t qoff = (bq * a.H + h) * (int64_t)D;
#pragma unroll
  for (int r = 0; r < DPT; ++r) {
    const int d = p + TPH * r;
    qv[r] = a.q_f32 ? ((const float*)a.q)[qoff + d] : bf16_to_f32(((const uint16_t*)a.q)[qoff + d]);
    o[r] = 0.0f;
  }
  if (a.qn.gain || a.qn.rope_dims > 0) {         // uniform: RMSNorm / partial RoPE of the query row
    if (a.qn.gain) {
      float ss = 0.0f;
#pragma unroll
      for (int r = 0; r < DPT; ++r) ss = fmaf(qv[r], qv[r], ss);
#pragma unroll
      for (int off = TPH / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, TPH);
      const float rr = 1.0f / sqrtf(ss / (float)D + a.qn.eps);
#pragma unroll
      for (int r = 0; r < DPT; ++r) qv[r] = qv[r] * rr * a.qn.gain[p + TPH * r];
    }
    if (a.qn.rope_dims > 0) {                     // the pair partner of dim d is dim d ^ 1, in thread p ^ 1
      // The workgroup's rows share one position: cos / sin of each pair are
      // formed once, by a rolled loop, into the entry buffer (free until the
      // first tile), rather than by a sincos per dim in the unrolled loop.
      const int d0 = D - a.qn.rope_dims, npair = a.qn.rope_dims >> 1;
      float* const tab = &s_e[0][0];              // cos of pair i at [i], sin at [D / 2 + i]
      for (int i = tid; i < npair; i += blockDim.x) {
        float sn, cs;
        sincos_angle(__fmul_rn((float)t, a.qn.theta[i]), &sn, &cs);
        tab[i] = cs;
        tab[D / 2 + i] = sn;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < DPT; ++r) {
        const int d = p + TPH * r;
        const float other = __shfl_xor(qv[r], 1, TPH);
        if (d >= d0) {
          const float cs = tab[(d - d0) >> 1], sn = tab[D / 2 + ((d - d0) >> 1)];
          qv[r] = (d & 1) ? other * sn + qv[r] * cs : qv[r] * cs - other * sn;
        }
      }
      __syncthreads();                            // the buffer holds entries next
    }
    if (!a.q_f32) {                               // BF16 queries stay BF16
#pragma unroll
      for (int r = 0; r < DPT; ++r) qv[r] = bf16_to_f32(f32_to_bf16(qv[r]));
    }
  }
  float mrun = -INFINITY, lrun = 0.0f;
  if (a.prior_o) {
    const float lp = a.prior_lse[bq * a.H + h];
    if (lp > -INFINITY) {
      mrun = lp;
      lrun = 1.0f;
#pragma unroll
      for (int r = 0; r < DPT; ++r) o[r] = a.prior_o[qoff + p + TPH * r];
    }
  }

  const int cpr = a.ckv.rows ? a.ckv.row_bytes / 16 : a.win.row_bytes / 16;  // equal for both stores
  for (int64_t base = i0; base < i1; base += kTile) {
    if (tid < kTile) {
      const Store* st = nullptr;
      int64_t row = 0;
      const int64_t i = base + tid;
      int src = 0;
      if (i < i1 && list_row(a, bq, b, t, Lc, i, st, row)) src = (st == &a.ckv) ? 1 : 2;
      s_src[tid] = src;
      s_row[tid] = row;
    }
    __syncthreads();
    for (int c = tid; c < kTile * cpr; c += blockDim.x) {
      const int e = c / cpr, cc = c % cpr;
      const int src = s_src[e];
      if (src != 0) decode_chunk(src == 1 ? a.ckv : a.win, s_row[e], cc, s_e[e]);
    }
    __syncthreads();
    float lg[kTile];
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < kTile; ++e) {
      float dot = 0.0f;
#pragma unroll
      for (int r = 0; r < DPT; ++r) dot = fmaf(qv[r], s_e[e][p + TPH * r], dot);
#pragma unroll
      for (int off = TPH / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, TPH);
      lg[e] = s_src[e] ? a.tau * dot : -INFINITY;
      mt = fmaxf(mt, lg[e]);
    }
    const float mnew = fmaxf(mrun, mt);
    if (mnew > -INFINITY) {
      const float corr = mrun > -INFINITY ? expf(mrun - mnew) : 0.0f;
      lrun *= corr;
#pragma unroll
      for (int r = 0; r < DPT; ++r) o[r] *= corr;
#pragma unroll
      for (int e = 0; e < kTile; ++e) {
        if (!s_src[e]) continue;            // empty slot: its LDS row is stale
        const float pe = expf(lg[e] - mnew);
        lrun += pe;
#pragma unroll
        for (int r = 0; r < DPT; ++r) o[r] = fmaf(pe, s_e[e][p + TPH * r], o[r]);
      }
      mrun = mnew;
    }
    __syncthreads();
  }

  if (a.nsplit > 1) {
    float* wo = a.ws + ((bq * a.H + h) * a.nsplit + blockIdx.z) * (int64_t)D;
    float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * a.nsplit * D + ((bq * a.H + h) * a.nsplit + blockIdx.z) * 2;
#pragma unroll
    for (int r = 0; r < DPT; ++r) wo[p + TPH * r] = o[r];
    if (p == 0) { wml[0] = mrun; wml[1] = lrun; }
    return;
  }
  const float sig = (a.partial || !a.sink) ? -INFINITY : a.sink[h];
  const float M = fmaxf(mrun, sig);
  float scale = 0.0f, lse = -INFINITY;
  if (M > -INFINITY) {
    const float fm = mrun > -INFINITY ? expf(mrun - M) : 0.0f;
    const float Z = lrun * fm + (sig > -INFINITY ? expf(sig - M) : 0.0f);
    scale = fm / Z;
    lse = M + logf(Z);
  }
#pragma unroll
  for (int r = 0; r < DPT; ++r) {
    const float v = o[r] * scale;
    const int64_t idx = qoff + p + TPH * r;
    if (a.out_f32) ((float*)a.out)[idx] = v;
    else ((uint16_t*)a.out)[idx] = (uint16_t)f32_to_bf16(v);
  }
  if (a.lse && p == 0) a.lse[bq * a.H + h] = lse;
}

// Fixed-order merge of split partials, with the sink.  One wavefront per
// (query, head): lane s holds split s's (m_s, l_s), so the maximum and the
// denominator are wavefront reductions (fixed butterfly order), and each
// lane combines its dims over the splits in split order.  For D = 512 and at
// most kMergeRegs splits (the decode shapes) every partial row this lane
// needs is loaded at the start, in flight together with the statistics.
constexpr int kMaxSplit = 64;
constexpr int kMergeRegs = 8;

__global__ __launch_bounds__(64) void attn_split_merge_kernel(AttnArgs a) {
  const int64_t bq = blockIdx.x;
  const int h = blockIdx.y;
  const int D = a.D;
  const int lane = threadIdx.x;
  const int ns = a.nsplit;
  const float* wo = a.ws + (bq * a.H + h) * ns * (int64_t)D;
  const float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * ns * D + (bq * a.H + h) * ns * 2;
  const bool regs = D == 8 * kWave && ns <= kMergeRegs;          // uniform
  float4 v[kMergeRegs][2];
  if (regs) {
#pragma unroll
    for (int s = 0; s < kMergeRegs; ++s)
#pragma unroll
      for (int c = 0; c < 2; ++c)   // unused splits re-read split 0 (ignored): every load goes out
        v[s][c] = *(const float4*)(wo + (int64_t)(s < ns ? s : 0) * D + 4 * lane + 4 * kWave * c);
  }
  const float m_s = lane < ns ? wml[2 * lane] : -INFINITY;
  const float l_s = lane < ns ? wml[2 * lane + 1] : 0.0f;
  const float sig = (a.partial || !a.sink) ? -INFINITY : a.sink[h];
  const float M = fmaxf(wave_max(m_s), sig);
  float Z = 0.0f, w_s = 0.0f;
  if (M > -INFINITY) {                                            // uniform
    const float e_s = m_s > -INFINITY ? expf(m_s - M) : 0.0f;
    Z = wave_sum(l_s * e_s) + (sig > -INFINITY ? expf(sig - M) : 0.0f);
    w_s = e_s / Z;
  }
  const float lse = M > -INFINITY ? M + logf(Z) : -INFINITY;
  const int64_t qoff = (bq * a.H + h) * (int64_t)D;
  auto store4 = [&](int d, const float4& acc) {
    if (a.out_f32) {
      *(float4*)((float*)a.out + qoff + d) = acc;
    } else {
      uint2 w;
      w.x = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
      w.y = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
      *(uint2*)((uint16_t*)a.out + qoff + d) = w;
    }
  };
  if (regs) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int s = 0; s < kMergeRegs; ++s) {
        const float w = __shfl(w_s, s);
        if (s < ns) {                                             // uniform; no early exit, so v stays in registers
          acc.x = fmaf(v[s][c].x, w, acc.x); acc.y = fmaf(v[s][c].y, w, acc.y);
          acc.z = fmaf(v[s][c].z, w, acc.z); acc.w = fmaf(v[s][c].w, w, acc.w);
        }
      }
      store4(4 * lane + 4 * kWave * c, acc);
    }
  } else {
    for (int d = 4 * lane; d < D; d += 4 * kWave) {
      float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      for (int s = 0; s < ns; ++s) {
        const float w = __shfl(w_s, s);
        const float4 x = *(const float4*)(wo + (int64_t)s * D + d);
        acc.x = fmaf(x.x, w, acc.x); acc.y = fmaf(x.y, w, acc.y);
        acc.z = fmaf(x.z, w, acc.z); acc.w = fmaf(x.w, w, acc.w);
      }
      store4(d, acc);
    }
  }
  if (a.lse && lane == 0) a.lse[bq * a.H + h] = lse;
}

// ------------------------------------------------------------ host side
struct AttnShape { int tph, dpt, hg; bool ok; };

static AttnShape attn_shape(int H, int D) {
  AttnShape s{0, 0, 0, false};
  if (D == 512 && H % 32 == 0) { s.tph = 8; s.dpt = 64; s.hg = 32; s.ok = true; return s; }
  if (D != 32 && D != 64 && D != 128 && D != 256 && D != 512) return s;
  s.tph = D == 32 ? 32 : 64;
  s.dpt = D / s.tph;
  const int maxhg = kAttnThreads / s.tph;
  for (int g = maxhg; g >= 1; --g)
    if (H % g == 0) { s.hg = g; break; }
  s.ok = s.hg > 0;
  return s;
}

bool attn_supported(int H, int D) { return H >= 1 && attn_shape(H, D).ok; }

// Splits of the entry list per query: enough workgroups to cover the chip
// (about 2 per CU) when the queries alone do not, each split a whole number
// of 32-entry tiles and at least `min_len` entries.  hpw = heads per
// workgroup of the kernel that runs.
static int attn_nsplit_for(int B, int Tq, int H, int hpw, int64_t max_list, int min_len, int target,
                           int& split_len) {
  const int64_t wgs = (int64_t)B * Tq * ((H + hpw - 1) / hpw);
  split_len = 0;
  if (wgs >= target || max_list <= min_len) return 1;
  const int64_t want = (target + wgs - 1) / wgs;         // splits per query
  int64_t len = (max_list + want - 1) / want;
  len = ((len + 31) / 32) * 32;
  if (len < min_len) len = min_len;
  int64_t ns = (max_list + len - 1) / len;
  if (ns > kMaxSplit) {
    len = ((max_list + kMaxSplit - 1) / kMaxSplit + 31) / 32 * 32;
    ns = (max_list + len - 1) / len;
  }
  split_len = (int)len;
  return (int)ns;
}

// The MFMA kernel runs one workgroup per CU (its LDS tiles take most of the
// 160 KB), so decode splits aim at one round of workgroups over the 256 CUs.
constexpr int kMfmaTargetWgs = 512;
constexpr int kMfmaMinSplit = 256;

static int attn_nsplit(int B, int Tq, int H, int D, int64_t max_list, bool mfma, int& split_len) {
  if (mfma) return attn_nsplit_for(B, Tq, H, 64, max_list, kMfmaMinSplit, kMfmaTargetWgs, split_len);
  const AttnShape s = attn_shape(H, D);
  return attn_nsplit_for(B, Tq, H, s.hg ? s.hg : 1, max_list, 64, 512, split_len);
}

// Batch-invariant splits of one-query-per-sequence calls: a fixed length
// (a function of the list length only, never of the batch), so a row's
// splits, and the fixed-order merge of their partials, are the same whatever
// else is in the batch.
constexpr int kInvSplit = 512;

static int attn_nsplit_invariant(int Tq, int64_t max_list, int& split_len) {
  split_len = 0;
  if (Tq != 1 || max_list <= kInvSplit) return 1;
  int64_t len = kInvSplit, ns = (max_list + len - 1) / len;
  if (ns > kMaxSplit) {
    len = ((max_list + kMaxSplit - 1) / kMaxSplit + 31) / 32 * 32;
    ns = (max_list + len - 1) / len;
  }
  split_len = (int)len;
  return (int)ns;
}

size_t attn_workspace(int B, int Tq, int H, int D, int64_t max_list) {
  if (!attn_supported(H, D)) return 0;
  int len;
  // the larger of the two kernels' needs (the query format decides which runs)
  int ns = attn_nsplit(B, Tq, H, D, max_list, false, len);
  if (D == 512 && H % 64 == 0) {
    const int ns2 = attn_nsplit(B, Tq, H, D, max_list, true, len);
    ns = ns2 > ns ? ns2 : ns;
  }
  const int ns3 = attn_nsplit_invariant(Tq, max_list, len);   // CSA_BATCH_INVARIANT
  ns = ns3 > ns ? ns3 : ns;
  if (ns <= 1) return 0;
  return (size_t)B * Tq * H * ns * (D + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnCall& c, hipStream_t st) {
  AttnArgs a;
  a.q = c.q; a.q_f32 = c.q_fmt == CSA_F32; a.B = c.B; a.Tq = c.Tq; a.H = c.H; a.D = c.D;
  a.ckv = c.ckv.rows ? view(c.ckv) : Store{nullptr, nullptr, 0, c.D, 0, 0, 0};
  a.n_entries = c.n_entries; a.mode = c.mode; a.sel = c.sel; a.k = c.k; a.m = c.m;
  a.win = c.win.rows ? view(c.win) : Store{nullptr, nullptr, 0, c.D, 0, 0, 0};
  a.W = c.W; a.ring = c.ring; a.q_pos = c.q_pos;
  a.sink = c.sink; a.tau = c.tau; a.prior_o = c.prior_o; a.prior_lse = c.prior_lse;
  a.out = c.out; a.out_f32 = c.partial || c.q_fmt == CSA_F32; a.lse = c.lse; a.partial = c.partial;
  a.qn = c.qn;
  const int64_t max_list = (c.mode == kModeSel ? c.k : (c.mode == kModeRange ? c.n_entries : 0)) + c.W;
  int len = 0;
  const bool mfma = attn_mfma_eligible(c.q_fmt, c.H, c.D, c.ckv.rows ? c.ckv : c.win, c.prior_o != nullptr, c.tau);
  // a prior partial is merged into the final output, so its calls do not split
  a.nsplit = !c.allow_split || c.prior_o ? 1
            : (c.invariant ? attn_nsplit_invariant(c.Tq, max_list, len)
                           : attn_nsplit(c.B, c.Tq, c.H, c.D, max_list, mfma, len));
  a.split_len = len;
  a.ws = (float*)c.ws;
  if ((int64_t)c.B * c.Tq == 0) return hipSuccess;
  if (mfma) {
    hipError_t e = launch_attn_m32(c, a.nsplit, a.split_len, st);
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(attn_split_merge_kernel, dim3((unsigned)((int64_t)c.B * c.Tq), c.H), dim3(64), 0, st, a);
    return hipGetLastError();
  }
  const AttnShape s = attn_shape(c.H, c.D);
  const dim3 grid((unsigned)((int64_t)c.B * c.Tq), c.H / s.hg, a.nsplit);
  const dim3 block(s.hg * s.tph);
#define CSA_ATT(TPH, DPT) hipLaunchKernelGGL((attn_valu_kernel<TPH, DPT>), grid, block, 0, st, a)
  if (s.tph == 8) CSA_ATT(8, 64);
  else if (s.tph == 32) CSA_ATT(32, 1);
  else if (s.dpt == 1) CSA_ATT(64, 1);
  else if (s.dpt == 2) CSA_ATT(64, 2);
  else if (s.dpt == 4) CSA_ATT(64, 4);
  else CSA_ATT(64, 8);
#undef CSA_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(attn_split_merge_kernel, dim3((unsigned)((int64_t)c.B * c.Tq), c.H), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
