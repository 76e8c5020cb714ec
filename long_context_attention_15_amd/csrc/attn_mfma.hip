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
constexpr int kKsPitch = kMD + 8;        // bf16 elements per Ks row (+16 B pad)
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

// Row of list slot i; src 0 = empty, 1 = compressed store, 2 = window store.
__device__ __forceinline__ int m_list_row(const MfmaArgs& a, int64_t bq, int b, int64_t t, int64_t Lc,
                                          int64_t i, int64_t i1, int64_t& row) {
  row = 0;
  if (i >= i1) return 0;
  if (i < Lc) {
    int64_t j = i;
    if (a.mode == kModeSel) {
      j = a.sel[bq * a.k + i];
      if (j < 0 || j >= a.n_entries) return 0;
    }
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

// One staging unit: dims [8g, 8g+8) of the entry pair (2p, 2p+1).
struct StageUnit {
  u32x4 a, b;   // raw bytes: fp8 in .x/.y (bulk) or 8 bf16 (rope)
};

__global__ __launch_bounds__(kMThreads, 1) void attn_mfma_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kMT * kKsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kMD * kVtPitch];
  __shared__ __attribute__((aligned(16))) float Sx[4][16][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int rh = wave >> 1, dh = wave & 1;
  const int g32 = lane >> 5, l32 = lane & 31;
  const int64_t bq = blockIdx.x;
  const int b = (int)(bq / a.Tq);
  const int h = blockIdx.y * 64 + rh * 32 + l32;          // this lane's head
  const int64_t t = a.q_pos ? a.q_pos[bq] : (int64_t)(bq % a.Tq);
  const int64_t Lc = a.mode == kModeSel ? a.k : (a.mode == kModeRange ? m_visible(t, a.m, a.n_entries) : 0);
  const int64_t L = Lc + a.W;
  const int64_t i0 = (int64_t)blockIdx.z * a.split_len;
  const int64_t i1 = a.nsplit == 1 ? L : (i0 + a.split_len < L ? i0 + a.split_len : L);
  const int nbulk = a.ckv.dim - a.ckv.rope;                // 448
  const int gbulk = nbulk / 8;                              // dim groups in FP8

  // Q^T operand: 16 K-steps of 16 dims over this wave's 256 dims
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
  float mrun = -INFINITY, lrun = 0.0f;
  const float sc2 = a.tau * kLog2e;

  // staging assignment: entry pair p, dim groups g = gq + 16 j
  const int sp = tid & 15, gq = tid >> 4;

  auto load_tile = [&](int64_t base, StageUnit (&u)[4], float& sa, float& sb, int& va, int& vb) {
    int64_t ra, rb;
    const int srca = m_list_row(a, bq, b, t, Lc, base + 2 * sp, i1, ra);
    const int srcb = m_list_row(a, bq, b, t, Lc, base + 2 * sp + 1, i1, rb);
    const Store& sta = srca == 2 ? a.win : a.ckv;
    const Store& stb = srcb == 2 ? a.win : a.ckv;
    va = srca; vb = srcb;
    sa = srca ? ((const float*)sta.scales)[ra] : 0.0f;
    sb = srcb ? ((const float*)stb.scales)[rb] : 0.0f;
    const uint8_t* pa = sta.rows + ra * sta.row_bytes;
    const uint8_t* pb = stb.rows + rb * stb.row_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = gq + 16 * j;
      u32x4 za = {0u, 0u, 0u, 0u}, zb = {0u, 0u, 0u, 0u};
      if (g < gbulk) {
        if (srca) { u32x2 w = *(const u32x2*)(pa + 8 * g); za.x = w.x; za.y = w.y; }
        if (srcb) { u32x2 w = *(const u32x2*)(pb + 8 * g); zb.x = w.x; zb.y = w.y; }
      } else {
        const int off = nbulk + 16 * (g - gbulk);
        if (srca) za = *(const u32x4*)(pa + off);
        if (srcb) zb = *(const u32x4*)(pb + off);
      }
      u[j].a = za;
      u[j].b = zb;
    }
  };
  auto store_tile = [&](const StageUnit (&u)[4], float sa, float sb, int va, int vb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = gq + 16 * j;
      u32x4 ca, cb;
      if (g < gbulk) {
        u32x2 wa = {u[j].a.x, u[j].a.y}, wb = {u[j].b.x, u[j].b.y};
        ca = cvt8_fp8(wa, sa);
        cb = cvt8_fp8(wb, sb);
        if (!va) ca = u32x4{0u, 0u, 0u, 0u};
        if (!vb) cb = u32x4{0u, 0u, 0u, 0u};
      } else {
        ca = u[j].a;
        cb = u[j].b;
      }
      *(u32x4*)(Ks + (2 * sp) * kKsPitch + 8 * g) = ca;
      *(u32x4*)(Ks + (2 * sp + 1) * kKsPitch + 8 * g) = cb;
      const unsigned int A4[4] = {ca.x, ca.y, ca.z, ca.w};
      const unsigned int B4[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        *(unsigned int*)(Vt + (8 * g + 2 * q2) * kVtPitch + 2 * sp) = __builtin_amdgcn_perm(B4[q2], A4[q2], 0x05040100u);
        *(unsigned int*)(Vt + (8 * g + 2 * q2 + 1) * kVtPitch + 2 * sp) = __builtin_amdgcn_perm(B4[q2], A4[q2], 0x07060302u);
      }
    }
  };

  StageUnit u[4];
  float su_a, su_b;
  int sv_a, sv_b;
  if (i0 < i1) {
    load_tile(i0, u, su_a, su_b, sv_a, sv_b);
    store_tile(u, su_a, su_b, sv_a, sv_b);
  }
  __syncthreads();

  for (int64_t base = i0; base < i1; base += kMT) {
    const bool more = base + kMT < i1;
    if (more) load_tile(base + kMT, u, su_a, su_b, sv_a, sv_b);   // prefetch the next tile

    // validity of this tile's 32 slots
    int64_t rdummy;
    const bool vslot = lane < 32 && m_list_row(a, bq, b, t, Lc, base + lane, i1, rdummy) != 0;
    const unsigned int vmask = (unsigned int)__ballot(vslot);

    // S^T partial over this wave's dims: two accumulators for independent chains
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
    const uint16_t* kp = Ks + l32 * kKsPitch + dh * 256 + g32 * 8;
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
    __syncthreads();
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
    const float mnew = fmaxf(mrun, mt);
    float corr = 1.0f, psum = 0.0f;
    if (mnew > -INFINITY) {
      corr = mrun > -INFINITY ? exp2f(mrun - mnew) : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2f(p[r] - mnew);
        psum += p[r];
      }
      mrun = mnew;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = 0.0f;
    }
    psum += __shfl_xor(psum, 32);
    lrun = lrun * corr + psum;
    // P^T as the B operand of two K-steps (regs 0..7, 8..15)
    bf16x8 pb0, pb1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      pb0[r] = (__bf16)p[r];
      pb1[r] = (__bf16)p[r + 8];
    }
#pragma unroll
    for (int mt8 = 0; mt8 < 8; ++mt8)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt8][r] *= corr;
    // O^T += V^T P^T
#pragma unroll
    for (int mt8 = 0; mt8 < 8; ++mt8) {
      const uint16_t* vp = Vt + (dh * 256 + mt8 * 32 + l32) * kVtPitch + g32 * 4;
      u32x4 v0, v1;
      const u32x2 a0 = *(const u32x2*)(vp);
      const u32x2 a1 = *(const u32x2*)(vp + 8);
      const u32x2 b0 = *(const u32x2*)(vp + 16);
      const u32x2 b1 = *(const u32x2*)(vp + 24);
      v0 = u32x4{a0.x, a0.y, a1.x, a1.y};
      v1 = u32x4{b0.x, b0.y, b1.x, b1.y};
      acc[mt8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v0), pb0, acc[mt8], 0, 0, 0);
      acc[mt8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v1), pb1, acc[mt8], 0, 0, 0);
    }
    __syncthreads();                         // every wave is done with Ks / Vt / Sx
    if (more) {
      store_tile(u, su_a, su_b, sv_a, sv_b);
      __syncthreads();
    }
  }

  // ---- epilogue
  const int64_t qoff = (bq * a.H + h) * (int64_t)kMD;
  if (a.nsplit > 1) {
    // partial: m (natural log units), l, unnormalised o
    float* wo = a.ws + ((bq * a.H + h) * a.nsplit + blockIdx.z) * (int64_t)kMD;
    float* wml = a.ws + (int64_t)a.B * a.Tq * a.H * a.nsplit * kMD + ((bq * a.H + h) * a.nsplit + blockIdx.z) * 2;
#pragma unroll
    for (int mt8 = 0; mt8 < 8; ++mt8)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = dh * 256 + mt8 * 32 + (r >> 2) * 8 + g32 * 4 + (r & 3);
        wo[d] = acc[mt8][r];
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
         (kv.dim - kv.rope_dim) % 8 == 0;
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
