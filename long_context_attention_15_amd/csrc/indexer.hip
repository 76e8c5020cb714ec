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
#include <cstdlib>

#include "common.h"
#include "launch.h"

namespace csa {

constexpr int kIdxThreads = 512;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kMaxChunk = 32768;     // 128 KiB of keys in LDS
constexpr int kMaxCand = 32768;      // merge: candidates per query
constexpr int kMaxHI = 16;
constexpr int kMaxDI = 64;

// Wave-wide inclusive prefix sum / max / min in registers with DPP row
// shifts and row broadcasts (no LDS round trips).  Lane 63 ends with the
// total.
template <int OP>   // 0: add, 1: max (unsigned), 2: min (unsigned)
__device__ __forceinline__ uint32_t dpp_op(uint32_t a, uint32_t b) {
  return OP == 0 ? a + b : (OP == 1 ? (a > b ? a : b) : (a < b ? a : b));
}
template <int OP>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  constexpr uint32_t id = OP == 2 ? 0xffffffffu : 0u;
  x = dpp_op<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = dpp_op<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = dpp_op<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = dpp_op<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = dpp_op<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = dpp_op<OP>(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}
template <int OP>
__device__ __forceinline__ uint32_t wave_total(uint32_t x) {
  return __builtin_amdgcn_readlane(wave_scan<OP>(x), 63);
}

constexpr int kHistCopies = 8;                // histogram copies (lane & 7) against same-bin atomics

struct SelShared {
  uint32_t hist[256 * kHistCopies];
  uint32_t misc[4];
  uint32_t wtot[2][kIdxWaves];
};

// Exact radix select on keys[0, n) (LDS or global memory; 0 = no entry):
// returns the kk-th largest key `thr` and how many keys equal to thr are to
// be taken (the first ones by position).  The bits above the highest bit in
// which the smallest and largest keys differ are common to all keys; the
// rest is resolved in 8-bit digits, most significant first: each pass
// histograms the keys that match the digits found so far and one wavefront
// locates the digit holding the kk-th key with a DPP prefix scan.
// Needs 1 <= kk <= #nonzero keys.  Called by all kIdxThreads threads.
__device__ void radix_select(const uint32_t* keys, int n, int kk, SelShared& sh, uint32_t& thr,
                             int& need_eq) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = tid; i < n; i += kIdxThreads) {
    const uint32_t key = keys[i];
    lo = (key != 0u && key < lo) ? key : lo;
    hi = key > hi ? key : hi;
  }
  lo = wave_total<2>(lo);
  hi = wave_total<1>(hi);
  if (lane == 0) { sh.wtot[0][wave] = lo; sh.wtot[1][wave] = hi; }
  __syncthreads();
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int w = 0; w < kIdxWaves; ++w) {
    kmin = sh.wtot[0][w] < kmin ? sh.wtot[0][w] : kmin;
    kmax = sh.wtot[1][w] > kmax ? sh.wtot[1][w] : kmax;
  }
  __syncthreads();
  if (kmin >= kmax) { thr = kmax; need_eq = kk; return; }    // one distinct key value
  int hb = 31 - __builtin_clz(kmin ^ kmax);
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmax & mask;
  int remaining = kk;
  while (true) {
    const int shift = hb >= 7 ? hb - 7 : 0;
    for (int i = tid; i < 256 * kHistCopies; i += kIdxThreads) sh.hist[i] = 0u;
    __syncthreads();
    const uint32_t copy = (uint32_t)tid & (kHistCopies - 1);
    for (int i = tid; i < n; i += kIdxThreads) {
      const uint32_t key = keys[i];
      if (key != 0u && (key & mask) == prefix)
        atomicAdd(&sh.hist[((key >> shift) & 255u) * kHistCopies + copy], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l holds bins [4 (63 - l), +4): the prefix scan counts this lane's bins and all higher ones
      uint4 h = make_uint4(0u, 0u, 0u, 0u);
      const uint32_t* hb0 = sh.hist + 4 * (kWave - 1 - lane) * kHistCopies;
#pragma unroll
      for (int cpy = 0; cpy < kHistCopies; cpy += 4) {
        const uint4 x0 = *(const uint4*)(hb0 + cpy), x1 = *(const uint4*)(hb0 + kHistCopies + cpy);
        const uint4 x2 = *(const uint4*)(hb0 + 2 * kHistCopies + cpy), x3 = *(const uint4*)(hb0 + 3 * kHistCopies + cpy);
        h.x += x0.x + x0.y + x0.z + x0.w;
        h.y += x1.x + x1.y + x1.z + x1.w;
        h.z += x2.x + x2.y + x2.z + x2.w;
        h.w += x3.x + x3.y + x3.z + x3.w;
      }
      const int local = (int)(h.x + h.y + h.z + h.w);
      const int incl = (int)wave_scan<0>((uint32_t)local);
      int ab = incl - local;
      if (ab < remaining && incl >= remaining) {
        const int c[4] = {(int)h.x, (int)h.y, (int)h.z, (int)h.w};
        for (int j = 3; j >= 0; --j) {
          if (ab + c[j] >= remaining) {
            sh.misc[0] = 4 * (kWave - 1 - lane) + j;
            sh.misc[1] = (uint32_t)ab;
            break;
          }
          ab += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sh.misc[0] << shift;
    mask |= 255u << shift;
    remaining -= (int)sh.misc[1];
    __syncthreads();
    if (shift == 0) break;
    hb = shift - 1;
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
  float* sel_score;        // nullable: score of each selected entry, -inf in padded slots
  uint32_t* ws_key;
  int32_t* ws_idx;
  // long lists: per-query workspace block and the offsets inside it
  uint8_t* ws;
  size_t per_query, off_scores, off_uni, off_region, off_counts, off_skey, off_sidx, off_ctr;
  int lm, nseg, rstride;   // rstride: entries between consecutive candidate regions
  int spin_max;            // one-pass long lists: polls before a workgroup stops waiting
};

// Diagnostic event counters of this device (read and cleared by
// csa_diag_counters): one-pass indexer workgroups that stopped waiting for
// their query's other chunks, and final selections that took the
// many-candidate path.  One atomic add per event; events are rare.
__device__ unsigned long long g_diag[CSA_DIAG_COUNT];

// visible entries of query bq
__device__ __forceinline__ int64_t idx_visible(const IdxArgs& a, int64_t bq) {
  const int64_t t = a.q_pos ? a.q_pos[bq] : (int64_t)(bq % a.Tq);
  int64_t nt = t < 0 ? 0 : (t + 1) / a.m;
  return nt > a.n_entries ? a.n_entries : nt;
}

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8v;

// 8 FP8 codes (one 64-bit word) -> 8 BF16 values, exact.
__device__ __forceinline__ bf16x8v fp8x8_bf16(long long v) {
  const uint32_t w0 = (uint32_t)v, w1 = (uint32_t)((unsigned long long)v >> 32);
  uint4 r;
  r.x = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r.y = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r.z = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r.w = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8v, r);
}

// Scores of entries [c0, c0 + cn) for one query on MFMA, written to s_keys.
// Heads are the 16 rows of the A operand (H_I <= 16, the rest zero), 16
// entries are the columns; the head-weighted ReLU sum is a lane-local sum
// over 4 heads plus two cross-lane adds.
//   FP8  : the codes convert exactly to BF16 for v_mfma_f32_16x16x32_bf16,
//          whose float32 sums keep float32 accuracy (the FP8 MFMAs sum their
//          products less precisely); the row scales of q fold into the head
//          weights, the key scale multiplies the sum (powers of two).
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
    const bf16x8v qb0 = fp8x8_bf16(qa0), qb1 = fp8x8_bf16(qa1);
    const float* ksc = (const float*)a.keys.scales;
    constexpr int U = 8;                    // groups in flight per wave
    for (int grp0 = wave * U; grp0 < ngroups; grp0 += kIdxWaves * U) {
      long long kb0[U], kb1[U];
      float sk[U];
      // every load is issued (rows past the chunk read its last row, their
      // scores are never stored) so that all of them are in flight together
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int e = (grp0 + u) * 16 + col;
        e = e < cn ? e : cn - 1;
        const uint8_t* kp = a.keys.rows + (krow0 + e) * a.keys.row_bytes;
        if (DI == 64) {
          const uint4 v = *(const uint4*)(kp + 16 * g);
          kb0[u] = (long long)(((unsigned long long)v.y << 32) | v.x);
          kb1[u] = (long long)(((unsigned long long)v.w << 32) | v.z);
        } else {
          const uint2 v = *(const uint2*)(kp + 8 * g);
          kb0[u] = (long long)(((unsigned long long)v.y << 32) | v.x);
          kb1[u] = 0;
        }
        sk[u] = ksc[krow0 + e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = (grp0 + u) * 16 + col;
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb0, fp8x8_bf16(kb0[u]), c, 0, 0, 0);
        if (DI == 64) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb1, fp8x8_bf16(kb1[u]), c, 0, 0, 0);
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
        int e = (grp0 + u) * 16 + col;
        e = e < cn ? e : cn - 1;
        const int gg = g < DI / 32 ? g : 0;
        const uint8_t* kp = a.keys.rows + (krow0 + e) * a.keys.row_bytes;
        const uint4 v = *(const uint4*)(kp + 16 * gg);
        const int sv = ksc[(krow0 + e) * (DI / 32) + gg];
        kv[u] = g < DI / 32 ? v : make_uint4(0u, 0u, 0u, 0u);
        ks[u] = g < DI / 32 ? sv : 127;
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

// Scores of entries [c0, c0 + cn) for one query with 64-dim keys on 32x32
// MFMA tiles: rows = heads (H_I <= 8 of 32, the rest zero), 32 entries as
// columns, so a lane holds 4 heads of one entry and one permlane32 swap adds
// the other 4.  FP8: codes convert exactly to BF16 for four
// v_mfma_f32_32x32x16_bf16 steps, lane group g taking dims [32 g, 32 g + 32)
// (the q row scales fold into the head weights, the key scale multiplies the
// sum).  MXFP4: one v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands, lane
// group g holding the 32-element block g and its E8M0 scale.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8s;
typedef __attribute__((ext_vector_type(16))) float f32x16s;
typedef unsigned int u32x4nt __attribute__((ext_vector_type(4)));

// Streaming loads of data read once: nontemporal, so that they do not
// displace cached data (and stream at a markedly higher rate from HBM).
__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const u32x4nt v = __builtin_nontemporal_load((const u32x4nt*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int FMT>
__device__ __forceinline__ void score_chunk_mfma32(const IdxArgs& a, int b, int q, int64_t bq, int64_t c0, int cn,
                                                   uint32_t* s_keys) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t qrow0 = (int64_t)b * a.qidx.cap + (int64_t)q * a.H_I;
  // head weights of this lane's accumulator rows 4 g .. 4 g + 3
  float wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    float w = 0.0f;
    if (h < a.H_I) {
      w = a.head_w[bq * a.H_I + h];
      if (FMT == CSA_FP8_E4M3) w *= ((const float*)a.qidx.scales)[qrow0 + h];
    }
    wl[i] = w;
  }
  const bool hrow = l32 < a.H_I;
  const uint8_t* qp = a.qidx.rows + (qrow0 + (hrow ? l32 : 0)) * a.qidx.row_bytes;
  const int64_t krow0 = (int64_t)b * a.keys.cap + c0;
  const int ngroups = (cn + 31) / 32;
  constexpr int U = 8;                          // groups of 32 entries in flight per wave
  if constexpr (FMT == CSA_FP8_E4M3) {
    bf16x8s qa[4];
    {
      const uint4 v0 = hrow ? *(const uint4*)(qp + 32 * g) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 v1 = hrow ? *(const uint4*)(qp + 32 * g + 16) : make_uint4(0u, 0u, 0u, 0u);
      qa[0] = fp8x8_bf16((long long)(((unsigned long long)v0.y << 32) | v0.x));
      qa[1] = fp8x8_bf16((long long)(((unsigned long long)v0.w << 32) | v0.z));
      qa[2] = fp8x8_bf16((long long)(((unsigned long long)v1.y << 32) | v1.x));
      qa[3] = fp8x8_bf16((long long)(((unsigned long long)v1.w << 32) | v1.z));
    }
    const float* ksc = (const float*)a.keys.scales;
    for (int grp0 = wave * U; grp0 < ngroups; grp0 += kIdxWaves * U) {
      uint4 k0[U], k1[U];
      float sk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {             // every load issued (rows past the chunk read its last row)
        int e = (grp0 + u) * 32 + l32;
        e = e < cn ? e : cn - 1;
        const uint8_t* kp = a.keys.rows + (krow0 + e) * a.keys.row_bytes + 32 * g;
        k0[u] = load_nt16(kp);
        k1[u] = load_nt16(kp + 16);
        sk[u] = __builtin_nontemporal_load(ksc + krow0 + e);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f32x16s acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        const uint32_t wv[8] = {k0[u].x, k0[u].y, k0[u].z, k0[u].w, k1[u].x, k1[u].y, k1[u].z, k1[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8s kb = fp8x8_bf16((long long)(((unsigned long long)wv[2 * j + 1] << 32) | wv[2 * j]));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[j], kb, acc, 0, 0, 0);
        }
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wl[i], fmaxf(acc[i], 0.0f), v);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int e = (grp0 + u) * 32 + l32;
        if (g == 0 && e < cn) s_keys[e] = score_key(v * sk[u]);
      }
    }
  } else {
    i32x8 qa = {0, 0, 0, 0, 0, 0, 0, 0};
    int qs = 127;
    if (hrow) {
      const uint4 v = *(const uint4*)(qp + 16 * g);
      qa[0] = (int)v.x; qa[1] = (int)v.y; qa[2] = (int)v.z; qa[3] = (int)v.w;
      qs = ((const uint8_t*)a.qidx.scales)[(qrow0 + l32) * 2 + g];
    }
    const uint8_t* ksc = (const uint8_t*)a.keys.scales;
    for (int grp0 = wave * U; grp0 < ngroups; grp0 += kIdxWaves * U) {
      uint4 kv[U];
      int ks[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int e = (grp0 + u) * 32 + l32;
        e = e < cn ? e : cn - 1;
        kv[u] = load_nt16(a.keys.rows + (krow0 + e) * a.keys.row_bytes + 16 * g);
        ks[u] = __builtin_nontemporal_load(ksc + (krow0 + e) * 2 + g);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f32x16s acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        const i32x8 kb = {(int)kv[u].x, (int)kv[u].y, (int)kv[u].z, (int)kv[u].w, 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kb, acc, 4, 4, 0, qs, 0, ks[u]);
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wl[i], fmaxf(acc[i], 0.0f), v);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int e = (grp0 + u) * 32 + l32;
        if (g == 0 && e < cn) s_keys[e] = score_key(v);
      }
    }
  }
}

// FP8 keys of dim 64 for at most 8 heads (the long-list and chunk paths):
// v_mfma_f32_16x16x32_bf16 with heads as the A rows (8 used) and 16 entries
// as the columns.  Lane (col, g) reads bytes [16 g, 16 g + 16) of entry
// row col, so each wave-wide load covers 16 whole rows (1 KiB, contiguous):
// a streaming read at close to the full HBM rate, which the 32-row layout
// (every load touching half of each of 32 rows) does not reach.  Its 16
// bytes feed two K-steps (bytes 8 s .. 8 s + 8 for step s); the q operand
// takes the same byte order.  Heads 4 g .. 4 g + 3 sit in lane group g, so
// the head-weighted ReLU sum is 4 FMAs and one row-pair swap (groups 2 and 3
// carry zero weights).
__device__ __forceinline__ void score_chunk_fp8_16(const IdxArgs& a, int b, int q, int64_t bq, int64_t c0, int cn,
                                                   uint32_t* s_keys) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, g = lane >> 4;
  const int64_t qrow0 = (int64_t)b * a.qidx.cap + (int64_t)q * a.H_I;
  float wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    wl[i] = h < a.H_I ? a.head_w[bq * a.H_I + h] * ((const float*)a.qidx.scales)[qrow0 + h] : 0.0f;
  }
  long long qa0 = 0, qa1 = 0;
  if (col < a.H_I) {
    const uint4 v = *(const uint4*)(a.qidx.rows + (qrow0 + col) * a.qidx.row_bytes + 16 * g);
    qa0 = (long long)(((unsigned long long)v.y << 32) | v.x);
    qa1 = (long long)(((unsigned long long)v.w << 32) | v.z);
  }
  const bf16x8v qb0 = fp8x8_bf16(qa0), qb1 = fp8x8_bf16(qa1);
  const float* ksc = (const float*)a.keys.scales;
  const int64_t krow0 = (int64_t)b * a.keys.cap + c0;
  const int ngroups = (cn + 15) / 16;
  // double-buffered: the next batch of U groups of 16 entries is in flight
  // while the current one is scored (the last batch re-reads the chunk's
  // last row, so every issue is unconditional and the wait counts stay exact)
  constexpr int U = 4;
  uint4 kv[U];
  float sk[U];
  auto issue = [&](int g0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int e = (g0 + u) * 16 + col;
      e = e < cn ? e : cn - 1;
      kv[u] = load_nt16(a.keys.rows + (krow0 + e) * a.keys.row_bytes + 16 * g);
      sk[u] = __builtin_nontemporal_load(ksc + krow0 + e);
    }
  };
  int grp0 = wave * U;
  issue(grp0);
  for (; grp0 < ngroups; grp0 += kIdxWaves * U) {
    uint4 cv[U];
    float cs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { cv[u] = kv[u]; cs[u] = sk[u]; }
    issue(grp0 + kIdxWaves * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = (grp0 + u) * 16 + col;
      f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb0, fp8x8_bf16((long long)(((unsigned long long)cv[u].y << 32) | cv[u].x)), c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb1, fp8x8_bf16((long long)(((unsigned long long)cv[u].w << 32) | cv[u].z)), c, 0, 0, 0);
      float v = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaf(wl[i], fmaxf(c[i], 0.0f), v);
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (g == 0 && e < cn) s_keys[e] = score_key(v * cs[u]);
    }
  }
}

// Keys of entries [c0, c0 + cn) for one query into s_keys (LDS): MFMA for
// FP8 / MXFP4, float32 FMAs for F32.  Called by all kIdxThreads threads.
template <int FMT, int DI>
__device__ __forceinline__ void score_chunk(const IdxArgs& a, int b, int q, int64_t bq, int64_t c0, int cn,
                                            uint32_t* s_keys, float* s_q, float* s_w) {
  const int tid = threadIdx.x;
  if constexpr (FMT == CSA_F32) {
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
  } else if constexpr (DI == 64) {
    if (a.H_I <= 8) {
      if constexpr (FMT == CSA_FP8_E4M3) score_chunk_fp8_16(a, b, q, bq, c0, cn, s_keys);
      else score_chunk_mfma32<FMT>(a, b, q, bq, c0, cn, s_keys);
    } else {
      score_chunk_mfma<FMT, DI>(a, b, q, bq, c0, cn, s_keys, s_w);
    }
  } else {
    score_chunk_mfma<FMT, DI>(a, b, q, bq, c0, cn, s_keys, s_w);
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
  float* out_score = direct && a.sel_score ? a.sel_score + bq * a.k : nullptr;

  // pad the slots that will not be filled
  for (int i = kk + tid; i < a.k; i += kIdxThreads) {
    out_idx[i] = -1;
    if (!direct) out_key[i] = 0u;
    if (out_score) out_score[i] = -INFINITY;
  }
  if (kk == 0) return;                        // uniform over the workgroup

  score_chunk<FMT, DI>(a, b, q, bq, c0, cn, s_keys, s_q, s_w);
  __syncthreads();

  uint32_t thr;
  int need_eq;
  radix_select(s_keys, cn, kk, sh, thr, need_eq);
  emit_selected(s_keys, cn, thr, need_eq, sh, [&](int pos, int rank) {
    out_idx[rank] = (int32_t)(c0 + pos);
    if (!direct) out_key[rank] = s_keys[pos];
    if (out_score) out_score[rank] = key_score(s_keys[pos]);
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
  float* out_score = a.sel_score ? a.sel_score + bq * a.k : nullptr;
  for (int i = kk + tid; i < a.k; i += kIdxThreads) {
    out[i] = -1;
    if (out_score) out_score[i] = -INFINITY;
  }
  if (kk == 0) return;
  uint32_t thr;
  int need_eq;
  radix_select(s_keys, n, kk, sh, thr, need_eq);
  emit_selected(s_keys, n, thr, need_eq, sh, [&](int pos, int rank) {
    out[rank] = ci[pos];
    if (out_score) out_score[rank] = key_score(s_keys[pos]);
  });
}

// ------------------------------------------------- streaming top-k (prefill)
//
// Many queries, FP8 keys of 64 dims, at most 8 heads: one wavefront owns 4
// consecutive queries and streams their visible entries in ascending index
// order straight from L2 into registers (the compressed keys of a sequence
// are a few MB and stay cached), 64 entries per iteration, two iterations
// ahead.  Scores come from v_mfma_f32_32x32x16_bf16 with the 32 rows = 4
// queries x 8 heads and 32 entries as columns (FP8 codes convert to BF16
// exactly; the products and their float32 sums are as accurate as a float32
// dot product).  Each query keeps a candidate list in LDS (entry order, so
// index order) and a threshold: an entry is appended when its score beats
// the threshold.  When a list is nearly full it is compacted: radix digits
// of the keys locate a bound L with at least k keys >= L and few more; the
// keys >= L stay and the threshold becomes L, which is safe because each
// later entry with a key <= L ranks below at least k kept ones (larger key,
// or equal key and smaller index).  If no such bound exists (heavy ties) the
// exact k-th key is found and only the k best stay.  At the end an exact
// radix select over the list gives the top-k, emitted in list order =
// ascending index.  No workspace, no barriers, one pass over the keys.
constexpr int kSQW = 4;                   // queries per wavefront (= workgroup)
constexpr int kSStep = 64;                // entries per iteration (two MFMA column blocks)
constexpr int kSSlack = 96;               // a compaction keeps at most k + kSSlack entries
// Candidate slots per query.  The kernel is bound by how many wavefronts a
// CU holds, and the lists set that (one wavefront per workgroup): 736 slots
// leave room for 8 workgroups per CU, 992 for 6, so lists are kept as short
// as k allows (more frequent compactions cost less than the lost occupancy).
constexpr int kSCapSmall = 736;
constexpr int kSCapLarge = 992;
template <int CAP>
constexpr int stream_max_k() { return CAP - kSSlack - 2 * kSStep; }
constexpr int kStreamMaxK = stream_max_k<kSCapLarge>();
constexpr int64_t kStreamMaxN = 65536;    // candidate indices are 16-bit
constexpr int64_t kStreamMinQueries = 2048;
constexpr int kSRowBytes = 64;            // FP8 keys of 64 dims (indexer_stream_ok)

// list slots + one spare slot per lane
template <int CAP>
struct StreamLds {
  uint32_t ckey[kSQW][CAP + kWave];
  uint16_t cidx[kSQW][CAP + kWave];
  uint32_t hist[256];
};

typedef __attribute__((ext_vector_type(8))) __bf16 sbf16x8;
typedef __attribute__((ext_vector_type(16))) float sf32x16;

// 8 FP8 codes (two words) -> 8 BF16 values, exact.
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  uint4 r;
  r.x = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r.y = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r.z = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r.w = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

// LDS accesses of this wavefront issued so far complete before later ones.
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// max(x, 0) on the bit pattern: negative floats (and -0) become +0.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// base + the number of set bits of m below this lane.
__device__ __forceinline__ int lane_rank(uint64_t m, int base) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)base));
}

// score_key with the sign flip done arithmetically (adding +0 first folds -0).
__device__ __forceinline__ uint32_t key_of(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Float threshold equivalent to "key > thr" for every finite score.
__device__ __forceinline__ float thr_float(uint32_t thr) {
  if (thr < 0x007fffffu) return -INFINITY;
  const float f = key_score(thr);
  return (__float_as_uint(f) == 0x80000000u) ? -1.4e-45f : f;
}

// A candidate list held in registers: lane l owns positions 64 j + l; key 0
// marks an empty slot (every real key is nonzero).
template <int NS>
struct RegList {
  uint32_t key[NS];
  uint32_t id[NS];
};

template <int NS>
__device__ __forceinline__ void list_load(const uint32_t* keys, const uint16_t* ids, int n, RegList<NS>& r) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int pos = kWave * j + lane;
    r.key[j] = pos < n ? keys[pos] : 0u;
    r.id[j] = (uint32_t)ids[pos];                 // read only where the key is nonzero
  }
}

template <int NS>
__device__ __forceinline__ void list_minmax(const RegList<NS>& r, uint32_t& kmin, uint32_t& kmax) {
  // the minimum over k - 1 skips empty slots (0 wraps to the largest value)
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint32_t k = r.key[j];
    lo = min(lo, k - 1u);
    hi = max(hi, k);
  }
  kmin = wave_total<2>(lo) + 1u;
  kmax = wave_total<1>(hi);
}

// One 8-bit radix digit over the list's keys restricted to (key & mask) ==
// prefix: the digit value `bin` holding the need-th largest key, the number
// of keys in higher digits (`above`) and in that digit (`inbin`).
template <int NS>
__device__ void list_digit(const RegList<NS>& r, uint32_t prefix, uint32_t mask, int shift, int need, uint32_t* hist,
                           int& bin, int& above, int& inbin) {
  const int lane = threadIdx.x % kWave;
  *(uint4*)(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
  lds_wave_sync();
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint32_t k = r.key[j];
    if (k != 0u && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
  }
  lds_wave_sync();
  // lane l holds bins [4 (63 - l), +4): a prefix scan over lanes counts the
  // keys in this lane's bins and all higher ones
  const uint4 h = *(const uint4*)(hist + 4 * (kWave - 1 - lane));
  const int local = (int)(h.x + h.y + h.z + h.w);
  const int incl = (int)wave_scan<0>((uint32_t)local);
  const int ab = incl - local;
  const uint64_t hit = __ballot(ab < need && incl >= need);
  const int L = __ffsll((unsigned long long)hit) - 1;
  int a = __builtin_amdgcn_readlane(ab, L);
  const int c[4] = {(int)__builtin_amdgcn_readlane(h.x, L), (int)__builtin_amdgcn_readlane(h.y, L),
                    (int)__builtin_amdgcn_readlane(h.z, L), (int)__builtin_amdgcn_readlane(h.w, L)};
  int b = 0, cb = 0;
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    if (a + c[j] >= need) { b = j; cb = c[j]; break; }
    a += c[j];
  }
  bin = 4 * (kWave - 1 - L) + b;
  above = a;
  inbin = cb;
}

// A cut of the list that keeps every entry of its top kk: the entries with
// key > T plus the first need_eq entries with key == T.  Radix digits of 8
// bits are resolved from the highest bit in which the keys differ; the walk
// stops as soon as the digit bin holding the kk-th key brings the kept count
// to at most kk + slack (then T = bin lower bound - 1 and need_eq = 0: all
// keys >= the bound stay); otherwise it runs to the last bit and the cut is
// exact (kept == kk).  1 <= kk <= length.
template <int NS>
__device__ void list_cut(const RegList<NS>& r, int kk, int slack, uint32_t* hist, uint32_t& T, int& need_eq) {
  uint32_t kmin, kmax;
  list_minmax<NS>(r, kmin, kmax);
  if (kmin == kmax) { T = kmin; need_eq = kk; return; }
  int hb = 31 - __builtin_clz(kmin ^ kmax);           // highest differing bit
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = kmax & mask;
  int need = kk, above_all = 0;
  while (true) {
    const int shift = hb >= 7 ? hb - 7 : 0;
    int bin, above, inbin;
    list_digit<NS>(r, prefix, mask, shift, need, hist, bin, above, inbin);
    above_all += above;
    const uint32_t lo = prefix | ((uint32_t)bin << shift);
    if (lo > 0u && above_all + inbin <= kk + slack) { T = lo - 1u; need_eq = 0; return; }
    prefix = lo;
    mask |= 255u << shift;
    need -= above;
    if (shift == 0) break;
    hb = shift - 1;
  }
  T = prefix;
  need_eq = need;
}

// Rewrite the list with the entries of key > T plus the first need_eq of
// key == T, in order; returns the new length.
template <int NS>
__device__ int list_store_kept(const RegList<NS>& r, uint32_t T, int need_eq, uint32_t* keys, uint16_t* ids) {
  const int lane = threadIdx.x % kWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int out = 0, eqs = 0;
  if (need_eq == 0) {                                // uniform: the usual cut, at a digit boundary
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint32_t k = r.key[j];
      const bool keep = k > T;                       // T >= 0, so a kept key is nonzero
      const uint64_t bk = __builtin_amdgcn_ballot_w64(keep);
      if (keep) {
        const int d = lane_rank(bk, out);
        keys[d] = k;
        ids[d] = (uint16_t)r.id[j];
      }
      out += __popcll(bk);
    }
    lds_wave_sync();
    return __builtin_amdgcn_readfirstlane(out);
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint32_t k = r.key[j];
    const bool eq = k != 0u && k == T;
    const uint64_t beq = __ballot(eq);
    const bool keep = (k != 0u && k > T) || (eq && eqs + __popcll(beq & lt) < need_eq);
    const uint64_t bk = __ballot(keep);
    if (keep) {
      const int d = out + __popcll(bk & lt);
      keys[d] = k;
      ids[d] = (uint16_t)r.id[j];
    }
    out += __popcll(bk);
    eqs += __popcll(beq);
  }
  lds_wave_sync();
  return __builtin_amdgcn_readfirstlane(out);
}

// Mid-stream compaction of one query's list (n > k): returns the new length
// and raises thr (a strict bound: later entries need key > thr; every kept
// entry has key > T, or key == T and a smaller index, so an entry with key
// <= T ranks below at least k kept ones).
template <int NS>
__device__ int list_shrink(uint32_t* keys, uint16_t* ids, int n, int k, uint32_t* hist, uint32_t& thr) {
  RegList<NS> r;
  list_load<NS>(keys, ids, n, r);
  uint32_t T;
  int need_eq;
  list_cut<NS>(r, k, kSSlack, hist, T, need_eq);
  const uint32_t bound = need_eq == 0 ? T + 1u : T;
  thr = bound > thr ? bound : thr;
  return list_store_kept<NS>(r, T, need_eq, keys, ids);
}

struct StreamArgs {
  Store qidx, keys;
  const float* head_w;
  int64_t n_entries;
  const int64_t* q_pos;
  int B, Tq, H_I, m, k, ngroups;
  int32_t* sel;
  float* sel_score;
};

// Raw key bytes of one iteration for this lane: entry (32 blk + l32) of the
// iteration, bytes [32 g, 32 g + 32) of its FP8 row, and the row scale.
struct KeyRegs {
  uint4 w[2][2];
  float sc[2];
};

template <int CAP>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2))) void idx_stream_kernel(StreamArgs a) {
  constexpr int NS = (CAP + kWave - 1) / kWave;   // list slots per lane when a list is in registers
  constexpr int kSRowCap = CAP + kWave;
  __shared__ StreamLds<CAP> S;
  const int lane = threadIdx.x;
  const int g = lane >> 5, l32 = lane & 31;
  // heaviest groups (latest queries) first
  const int b = blockIdx.x / a.ngroups;
  const int grp = a.ngroups - 1 - (int)(blockIdx.x % a.ngroups);
  const int q0 = grp * kSQW;

  auto visible = [&](int q) -> int {
    if (q >= a.Tq) return 0;
    const int64_t bq = (int64_t)b * a.Tq + q;
    const int64_t t = a.q_pos ? a.q_pos[bq] : (int64_t)q;
    const int64_t nt = t < 0 ? 0 : (t + 1) / a.m;
    return (int)(nt < a.n_entries ? nt : a.n_entries);
  };
  int ntq[kSQW];
  int ntw = 0;                                      // the stream runs to the largest
#pragma unroll
  for (int qq = 0; qq < kSQW; ++qq) {
    ntq[qq] = visible(q0 + qq);
    ntw = max(ntw, ntq[qq]);
  }

  // A operand: row r holds query qsel(r >> 4, (r >> 2) & 1), head 4 ((r >> 3)
  // & 1) + (r & 3), so that the accumulator rows of lane half g (rows 8 j +
  // 4 g + i) are all 8 heads of query g (j < 2) and of query 2 + g (j >= 2);
  // K-step j covers dims [32 g + 8 j, +8) (the same split as the B operand)
  auto qsel = [](int hi, int half) { return hi ? 2 + half : half; };
  sbf16x8 qa[4];
  {
    const int qq = qsel(l32 >> 4, (l32 >> 2) & 1), h = 4 * ((l32 >> 3) & 1) + (l32 & 3), q = q0 + qq;
    const bool ok = q < a.Tq && h < a.H_I;
    const uint8_t* qp = a.qidx.rows + ((int64_t)b * a.qidx.cap + (int64_t)(ok ? q : 0) * a.H_I + (ok ? h : 0)) *
                                          a.qidx.row_bytes + 32 * g;
    const uint4 v0 = ok ? *(const uint4*)qp : make_uint4(0u, 0u, 0u, 0u);
    const uint4 v1 = ok ? *(const uint4*)(qp + 16) : make_uint4(0u, 0u, 0u, 0u);
    qa[0] = __builtin_bit_cast(sbf16x8, fp8x8_to_bf16(v0.x, v0.y));
    qa[1] = __builtin_bit_cast(sbf16x8, fp8x8_to_bf16(v0.z, v0.w));
    qa[2] = __builtin_bit_cast(sbf16x8, fp8x8_to_bf16(v1.x, v1.y));
    qa[3] = __builtin_bit_cast(sbf16x8, fp8x8_to_bf16(v1.z, v1.w));
  }
  // head weights of this lane's accumulator values 4 j + i (query qsel(j >> 1,
  // g), head 4 (j & 1) + i), with the query row scales folded in
  float wl[kSQW][4];
#pragma unroll
  for (int j = 0; j < kSQW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q0 + qsel(j >> 1, g), h = 4 * (j & 1) + i;
      float w = 0.0f;
      if (q < a.Tq && h < a.H_I) {
        const int64_t bq = (int64_t)b * a.Tq + q;
        w = a.head_w[bq * a.H_I + h] *
            ((const float*)a.qidx.scales)[(int64_t)b * a.qidx.cap + (int64_t)q * a.H_I + h];
      }
      wl[j][i] = w;
    }

  // lanes < 32 score queries 0 and 2, lanes >= 32 queries 1 and 3
  const int qA = g, qB = 2 + g;
  const int ntA = g ? ntq[1] : ntq[0], ntB = g ? ntq[3] : ntq[2];
  uint32_t thr[kSQW] = {0u, 0u, 0u, 0u};
  int cnt[kSQW] = {0, 0, 0, 0};
  float thrA = -INFINITY, thrB = -INFINITY;
  uint32_t* ck = &S.ckey[0][0];
  uint16_t* ci = &S.cidx[0][0];
  uint32_t* const ckA = ck + qA * kSRowCap;          // this lane's two lists
  uint32_t* const ckB = ck + qB * kSRowCap;
  uint16_t* const ciA = ci + qA * kSRowCap;
  uint16_t* const ciB = ci + qB * kSRowCap;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  const int64_t krow0 = (int64_t)b * a.keys.cap;
  const int niter = (ntw + kSStep - 1) / kSStep;
  auto load_iter = [&](int it, KeyRegs& kr) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int e = min(it * kSStep + 32 * blk + l32, ntw - 1);
      const uint8_t* kp = a.keys.rows + (krow0 + e) * kSRowBytes + 32 * g;
      kr.w[blk][0] = *(const uint4*)kp;
      kr.w[blk][1] = *(const uint4*)(kp + 16);
      kr.sc[blk] = ((const float*)a.keys.scales)[krow0 + e];
    }
  };

  // S^T block (rows: 4 queries x 8 heads, columns: the block's 32 entries)
  auto block_mfma = [&](const KeyRegs& kr, int blk) -> sf32x16 {
    sf32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint4 w0 = kr.w[blk][0], w1 = kr.w[blk][1];
    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = fp8x8_to_bf16(wv[2 * j], wv[2 * j + 1]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[j], __builtin_bit_cast(sbf16x8, v), acc, 0, 0, 0);
    }
    return acc;
  };
  // head-weighted ReLU sums, all 8 heads in the lane: lanes < 32 get queries
  // 0 and 2, lanes >= 32 queries 1 and 3
  auto block_scores = [&](const sf32x16& acc, float sk, float& sA, float& sB) {
    float va = 0.0f, vb = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        va = fmaf(wl[j][i], relu_bits(acc[4 * j + i]), va);
        vb = fmaf(wl[2 + j][i], relu_bits(acc[4 * (2 + j) + i]), vb);
      }
    sA = va * sk;
    sB = vb * sk;
  };
  // append the passing entries of one 32-entry block (entry index e for this
  // lane); a lane's slot is its list length plus the passing lanes below it
  // in its half of the wave.  Branch-free: a lane that does not pass writes
  // to its own spare slot behind the list.
  auto append = [&](float sA, float sB, int e) {
    // each mask is formed from the compares' own masks (a ballot of their
    // conjunction would first turn it into a lane value)
    const bool inA = e < ntA, inB = e < ntB, gtA = sA > thrA, gtB = sB > thrB;
    const bool pA = inA && gtA, pB = inB && gtB;
    const uint64_t mA = __builtin_amdgcn_ballot_w64(inA) & __builtin_amdgcn_ballot_w64(gtA);
    const uint64_t mB = __builtin_amdgcn_ballot_w64(inB) & __builtin_amdgcn_ballot_w64(gtB);
    const int a_lo = __popcll(mA & 0xffffffffull), a_hi = __popcll(mA >> 32);
    const int b_lo = __popcll(mB & 0xffffffffull), b_hi = __popcll(mB >> 32);
    const int rA = lane_rank(mA, g ? cnt[1] - a_lo : cnt[0]);
    const int rB = lane_rank(mB, g ? cnt[3] - b_lo : cnt[2]);
    const int dA = pA ? rA : CAP + lane;
    const int dB = pB ? rB : CAP + lane;
    ckA[dA] = key_of(sA);
    ciA[dA] = (uint16_t)e;
    ckB[dB] = key_of(sB);
    ciB[dB] = (uint16_t)e;
    cnt[0] += a_lo;
    cnt[1] += a_hi;
    cnt[2] += b_lo;
    cnt[3] += b_hi;
  };
  auto iteration = [&](int it, const KeyRegs& kr) {
    // room for one more iteration of appends in every list
    bool shrunk = false;
#pragma unroll
    for (int qq = 0; qq < kSQW; ++qq) {
      if (cnt[qq] > CAP - kSStep) {                              // uniform
        cnt[qq] = list_shrink<NS>(ck + qq * kSRowCap, ci + qq * kSRowCap, cnt[qq], a.k, S.hist, thr[qq]);
        shrunk = true;
      }
    }
    if (shrunk) {
      thrA = thr_float(g ? thr[1] : thr[0]);
      thrB = thr_float(g ? thr[3] : thr[2]);
    }
    const sf32x16 acc0 = block_mfma(kr, 0);
    const sf32x16 acc1 = block_mfma(kr, 1);
    float sA0, sB0, sA1, sB1;
    block_scores(acc0, kr.sc[0], sA0, sB0);
    block_scores(acc1, kr.sc[1], sA1, sB1);
    const int e = it * kSStep + l32;
    append(sA0, sB0, e);
    append(sA1, sB1, e + 32);
  };

  // two register sets, each reloaded right after use: iteration it + 2 is in
  // flight while it + 1 is scored
  KeyRegs r0, r1;
  if (niter > 0) load_iter(0, r0);
  if (niter > 1) load_iter(1, r1);
  for (int it = 0; it < niter; it += 2) {
    iteration(it, r0);
    if (it + 2 < niter) load_iter(it + 2, r0);
    if (it + 1 < niter) {
      iteration(it + 1, r1);
      if (it + 3 < niter) load_iter(it + 3, r1);
    }
  }
  lds_wave_sync();

  // final exact top-k of each list, emitted in list order (ascending index)
#pragma unroll
  for (int qq = 0; qq < kSQW; ++qq) {
    const int q = q0 + qq;
    if (q >= a.Tq) continue;                                        // uniform
    int32_t* out = a.sel + ((int64_t)b * a.Tq + q) * a.k;
    float* out_score = a.sel_score ? a.sel_score + ((int64_t)b * a.Tq + q) * a.k : nullptr;
    const int n = cnt[qq];
    const int kk = n < a.k ? n : a.k;
    for (int i = kk + lane; i < a.k; i += kWave) {
      out[i] = -1;
      if (out_score) out_score[i] = -INFINITY;
    }
    if (kk == 0) continue;
    const uint32_t* keys = ck + qq * kSRowCap;
    const uint16_t* ids = ci + qq * kSRowCap;
    if (n <= a.k) {
      for (int i = lane; i < n; i += kWave) {
        out[i] = (int32_t)ids[i];
        if (out_score) out_score[i] = key_score(keys[i]);
      }
      continue;
    }
    RegList<NS> r;
    list_load<NS>(keys, ids, n, r);
    uint32_t T;
    int need_eq;
    list_cut<NS>(r, kk, 0, S.hist, T, need_eq);
    int outn = 0, eqs = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint32_t k = r.key[j];
      const bool eq = k != 0u && k == T;
      const uint64_t beq = __ballot(eq);
      const bool take = (k != 0u && k > T) || (eq && eqs + __popcll(beq & lt) < need_eq);
      const uint64_t bt = __ballot(take);
      if (take) {
        out[outn + __popcll(bt & lt)] = (int32_t)r.id[j];
        if (out_score) out_score[outn + __popcll(bt & lt)] = key_score(k);
      }
      outn += __popcll(bt);
      eqs += __popcll(beq);
    }
  }
}

bool indexer_stream_ok(const csa_store& keys, int H_I, int B, int Tq, int64_t n_entries, int k) {
  return keys.fmt == CSA_FP8_E4M3 && keys.dim == 64 && keys.row_bytes == kSRowBytes && H_I <= 8 && k <= kStreamMaxK &&
         n_entries <= kStreamMaxN && (int64_t)B * Tq >= kStreamMinQueries;
}

static hipError_t launch_idx_stream(const IdxArgs& ia, hipStream_t st) {
  StreamArgs a;
  a.qidx = ia.qidx; a.keys = ia.keys; a.head_w = ia.head_w; a.n_entries = ia.n_entries; a.q_pos = ia.q_pos;
  a.B = ia.B; a.Tq = ia.Tq; a.H_I = ia.H_I; a.m = ia.m; a.k = ia.k; a.sel = ia.sel; a.sel_score = ia.sel_score;
  a.ngroups = (ia.Tq + kSQW - 1) / kSQW;
  const dim3 grid((unsigned)((int64_t)a.B * a.ngroups));
  if (a.k <= stream_max_k<kSCapSmall>()) hipLaunchKernelGGL(idx_stream_kernel<kSCapSmall>, grid, dim3(kWave), 0, st, a);
  else hipLaunchKernelGGL(idx_stream_kernel<kSCapLarge>, grid, dim3(kWave), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------ long lists (decode)
//
// Few queries over many entries (decode at long context).  Three kernels,
// exact, reading each key once at full HBM rate:
//   A  chunks of a.chunk = kLChunk entries (of the sizes measured at 262144
//      entries per query, from 4096 to 16384, this one streamed fastest):
//      the keys of the chunk's scores go to the
//      workspace, and so does the m-th largest of the maxima of kLSets
//      strided subsets of the chunk (each maximum is a real entry), m =
//      ceil(k / #chunks whose subsets are all nonempty);
//   B  per (query, segment of kLSeg entries): T = the smallest, over the
//      chunks whose subsets are all nonempty, of their m-th largest subset
//      maximum.  Each such chunk has at least m
//      entries >= T, so at least k entries have a key >= T: T is at most the
//      k-th largest key and every member of the top-k has a key >= T.  The
//      segment's entries with key >= T are compacted, in index order, into
//      the segment's region;
//   C  per query: the regions, concatenated in segment order (= index
//      order), hold every candidate; the exact top-k (ties to the smaller
//      index) is selected from them and emitted in ascending index order.
// When a query has at most kLFusedMaxChunks chunks, A and B run as one pass
// (idx_long_fused_kernel below) and the scores never leave LDS.
constexpr int kLChunk = 8192;                 // entries per chunk (32 KiB of keys in LDS, 3 workgroups per CU)
constexpr int kLSeg = 16384;
constexpr int kLPerWave = kLSeg / kIdxWaves;  // segment entries per wave in the compaction
constexpr int kLSets = 128;                   // strided sets per chunk
constexpr int kLFusedMaxChunks = 128;         // one-pass path: at most this many chunks per query
static_assert(kLFusedMaxChunks <= 2 * kWave, "one wavefront polls the chunk slots, two per lane");

template <int FMT, int DI>
__global__ __launch_bounds__(kIdxThreads) void idx_long_score_kernel(IdxArgs a) {
  extern __shared__ uint32_t s_keys[];
  __shared__ float s_q[kMaxHI * kMaxDI];
  __shared__ float s_w[kMaxHI];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int64_t bq = blockIdx.x;
  const int b = (int)(bq / a.Tq), q = (int)(bq % a.Tq);
  const int c = blockIdx.y;
  const int64_t nt = idx_visible(a, bq);
  const int64_t c0 = (int64_t)c * a.chunk;
  const int64_t cn64 = nt - c0;
  const int cn = cn64 < 0 ? 0 : (cn64 > a.chunk ? a.chunk : (int)cn64);
  uint8_t* wq = a.ws + bq * a.per_query;
  uint32_t* scores = (uint32_t*)(wq + a.off_scores);
  uint32_t* uni = (uint32_t*)(wq + a.off_uni) + c;
  if (cn == 0) return;                          // uniform (such chunks are never read)
  score_chunk<FMT, DI>(a, b, q, bq, c0, cn, s_keys, s_q, s_w);
  __syncthreads();
  for (int i = tid; i < cn; i += kIdxThreads) scores[c0 + i] = s_keys[i];
  // the largest key of each strided set {r + kLSets j} of the chunk (a real
  // entry, 0 if the set is empty); of these maxima, the one of rank m - 1
  // (descending, ties to the smaller set) goes to the workspace when the
  // chunk is full (every set nonempty: only full chunks are read), m =
  // ceil(k / #full chunks) as the compaction uses it.  Ranks are counted in
  // parallel, one set per thread.
  __shared__ uint32_t s_max[kLSets];
  for (int r = tid; r < kLSets; r += kIdxThreads) {
    uint32_t mx = 0u;
    for (int e = r; e < cn; e += kLSets) mx = s_keys[e] > mx ? s_keys[e] : mx;
    s_max[r] = mx;
  }
  __syncthreads();
  const int64_t nfull = nt >= kLSets ? (nt - kLSets) / a.chunk + 1 : 0;
  if (cn >= kLSets && nfull > 0) {
    const int64_t mm = ((int64_t)a.k + nfull - 1) / nfull;
    if (mm <= kLSets && tid < kLSets) {
      const uint32_t my = s_max[tid];
      int rank = 0;
      for (int r = 0; r < kLSets; ++r) {
        const uint32_t v = s_max[r];
        rank += (v > my || (v == my && r < tid)) ? 1 : 0;
      }
      if (rank == (int)mm - 1) *uni = my;
    }
  }
}

__global__ __launch_bounds__(kIdxThreads) void idx_long_compact_kernel(IdxArgs a) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t bq = blockIdx.x;
  const int seg = blockIdx.y;
  const int64_t nt = idx_visible(a, bq);
  uint8_t* wq = a.ws + bq * a.per_query;
  const uint32_t* scores = (const uint32_t*)(wq + a.off_scores);
  uint32_t* counts = (uint32_t*)(wq + a.off_counts);
  uint2* region = (uint2*)(wq + a.off_region);
  const int64_t s0 = (int64_t)seg * kLSeg;
  const int64_t s1 = nt < s0 + kLSeg ? nt : s0 + kLSeg;
  // uniform; short lists need no candidates unless their scores are asked for
  if (s1 <= s0 || (nt <= a.k && !a.sel_score)) {
    if (tid == 0) counts[seg] = 0u;
    return;
  }
  // T: chunk c is "full" when all its kLSets strided sets are nonempty; with
  // m = ceil(k / #full), each full chunk holds at least m entries >= its
  // m-th largest set maximum, so at least k entries are >= the smallest of
  // those (every entry when no such m exists)
  const int64_t nfull = nt >= kLSets ? (nt - kLSets) / a.chunk + 1 : 0;
  uint32_t T = 0u;
  if (nfull > 0 && ((int64_t)a.k + nfull - 1) / nfull <= kLSets) {   // uniform
    // one load per thread (all in flight together), then a workgroup minimum
    const uint32_t* uni = (const uint32_t*)(wq + a.off_uni);
    uint32_t t = 0xffffffffu;
    for (int64_t c = tid; c < nfull; c += kIdxThreads) {
      const uint32_t v = uni[c];
      t = v < t ? v : t;
    }
    t = wave_total<2>(t);
    if (lane == 0) sh.wtot[1][wave] = t;
    __syncthreads();
    T = 0xffffffffu;
    for (int w = 0; w < kIdxWaves; ++w) T = sh.wtot[1][w] < T ? sh.wtot[1][w] : T;
  }
  // compaction in index order: wave w owns the contiguous range
  // [w * kLPerWave, +kLPerWave) of the segment; its scores are loaded once,
  // all loads in flight together, and kept in registers for both passes
  const int len = (int)(s1 - s0);
  const int p0 = wave * kLPerWave;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t sv[kLPerWave / kWave];
#pragma unroll
  for (int r = 0; r < kLPerWave / kWave; ++r) {
    int pos = p0 + r * kWave + lane;
    pos = pos < len ? pos : len - 1;
    sv[r] = scores[s0 + pos];
  }
  uint32_t n_mine = 0;
#pragma unroll
  for (int r = 0; r < kLPerWave / kWave; ++r) {
    const int pos = p0 + r * kWave + lane;
    n_mine += (uint32_t)__popcll(__ballot(pos < len && sv[r] >= T));
  }
  if (lane == 0) sh.wtot[0][wave] = n_mine;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += sh.wtot[0][w];
#pragma unroll
  for (int r = 0; r < kLPerWave / kWave; ++r) {
    const int pos = p0 + r * kWave + lane;
    const bool take = pos < len && sv[r] >= T;
    const uint64_t bt = __ballot(take);
    if (take) region[s0 + base + __popcll(bt & lt)] = make_uint2(sv[r], (uint32_t)(s0 + pos));
    base += (uint32_t)__popcll(bt);
  }
  if (wave == kIdxWaves - 1 && lane == 0) counts[seg] = base;
}

// One-pass variant of A + B: the chunk's keys stay in LDS.  The workgroups of
// a query meet through per-chunk slots in the workspace (cleared by
// idx_long_zero_kernel): each nonempty chunk publishes its m-th largest set
// maximum (or "not full") in its slot and waits until every nonempty chunk
// of its query has published; the smallest statistic is T as B forms it, and
// the chunk compacts its own keys >= T, in index order, into its region
// (regions one chunk apart).  The grid
// puts the chunks of a query next to each other in dispatch order, and a
// query has far fewer chunks than the chip has resident slots, so the wait
// ends once the query's last chunk is scored.  The wait is bounded: a
// workgroup that gives up takes T = 0 (all its keys become candidates),
// which keeps the selection exact, only slower.  kLFusedMaxChunks <= 2 x 64
// (one polling wavefront, two slots per lane).
constexpr int kLSpinMax = 1 << 16;   // default polls of the chunk slots (tens of milliseconds)
constexpr int kLParts = kIdxThreads / kLSets;   // threads per strided set in the set maxima
static_assert(kLParts * kLSets == kIdxThreads && kLSets == 2 * kWave, "set maxima layout");

__global__ __launch_bounds__(256) void idx_long_zero_kernel(IdxArgs a, int64_t nq) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nq * a.nchunk) ((uint64_t*)(a.ws + (i / a.nchunk) * a.per_query + a.off_ctr))[i % a.nchunk] = 0ull;
}

template <int FMT, int DI>
__global__ __launch_bounds__(kIdxThreads) void idx_long_fused_kernel(IdxArgs a) {
  extern __shared__ uint32_t s_keys[];
  __shared__ float s_q[kMaxHI * kMaxDI];
  __shared__ float s_w[kMaxHI];
  __shared__ uint32_t s_part[kLParts][kLSets];
  __shared__ uint32_t s_wt[kIdxWaves];
  __shared__ uint32_t s_T;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c = blockIdx.x;
  const int64_t bq = blockIdx.y;
  const int b = (int)(bq / a.Tq), q = (int)(bq % a.Tq);
  const int64_t nt = idx_visible(a, bq);
  if (nt <= a.k && !a.sel_score) return;        // uniform per query: no candidates needed
  const int64_t c0 = (int64_t)c * a.chunk;
  const int64_t cn64 = nt - c0;
  const int cn = cn64 < 0 ? 0 : (cn64 > a.chunk ? a.chunk : (int)cn64);
  uint8_t* wq = a.ws + bq * a.per_query;
  uint32_t* counts = (uint32_t*)(wq + a.off_counts);
  // one slot per chunk: 0 until published, then bit 32 set and the chunk's
  // statistic (all ones when the chunk is not full) in the low word
  uint64_t* slots = (uint64_t*)(wq + a.off_ctr);
  auto publish = [&](uint64_t val) {
    const uint64_t old = __hip_atomic_exchange(slots + c, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));
  };
  if (cn == 0) {                                // uniform; never waited for
    if (tid == 0) counts[c] = 0u;
    return;
  }
  score_chunk<FMT, DI>(a, b, q, bq, c0, cn, s_keys, s_q, s_w);
  __syncthreads();
  const int64_t nfull = nt >= kLSets ? (nt - kLSets) / a.chunk + 1 : 0;
  const bool use_t = nfull > 0 && ((int64_t)a.k + nfull - 1) / nfull <= kLSets;   // uniform
  if (cn >= kLSets && use_t) {                  // uniform: a full chunk publishes its statistic
    // the maximum of each strided set {r + kLSets j}: four threads per set,
    // each over every fourth member, then one wavefront holds the kLSets
    // maxima (two per lane) and finds the m-th largest by building it bit by
    // bit from the top: the largest v with #(maxima >= v) >= m
    {
      const int r = tid % kLSets, part = tid / kLSets;
      uint32_t mx = 0u;
      for (int e = r + part * kLSets; e < cn; e += kIdxThreads) mx = s_keys[e] > mx ? s_keys[e] : mx;
      s_part[part][r] = mx;
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t va = 0u, vb = 0u;
#pragma unroll
      for (int part = 0; part < kLParts; ++part) {
        va = s_part[part][lane] > va ? s_part[part][lane] : va;
        vb = s_part[part][lane + kWave] > vb ? s_part[part][lane + kWave] : vb;
      }
      const int mm = (int)(((int64_t)a.k + nfull - 1) / nfull);
      uint32_t v = 0u;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = v | (1u << bit);
        const int cnt = __popcll(__ballot(va >= t)) + __popcll(__ballot(vb >= t));
        v = cnt >= mm ? t : v;
      }
      if (lane == 0) publish(((uint64_t)1 << 32) | v);
    }
  } else if (use_t && tid == 0) {
    publish(((uint64_t)1 << 32) | 0xffffffffu); // a nonempty chunk that is not full: arrived, no statistic
  }
  // wait for the query's other nonempty chunks: one wavefront polls all
  // their slots (two per lane) and forms T as the smallest statistic once
  // every slot is published.  Publication is an atomic exchange and the polls
  // are device-scope atomic loads, so no cache write-back or invalidation is
  // needed (those would stall the workgroups still streaming keys).  When T
  // is 0 anyway (no usable statistic) nothing is waited for.
  if (use_t && wave == 0) {                     // uniform per workgroup
    const int nact = (int)((nt + a.chunk - 1) / a.chunk);
    uint32_t t = 0u;
    bool all = false;
    for (int it = 0; !all && it < a.spin_max; ++it) {
      const uint64_t s0 = lane < nact ? __hip_atomic_load(slots + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : ((uint64_t)1 << 32) | 0xffffffffu;
      const uint64_t s1 = lane + kWave < nact
                              ? __hip_atomic_load(slots + lane + kWave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : ((uint64_t)1 << 32) | 0xffffffffu;
      all = __ballot((s0 >> 32) == 0 || (s1 >> 32) == 0) == 0ull;
      if (all) {
        const uint32_t l0 = (uint32_t)s0, l1 = (uint32_t)s1;
        t = wave_total<2>(l0 < l1 ? l0 : l1);
      } else {
        __builtin_amdgcn_s_sleep(16);
      }
    }
    if (lane == 0) {
      s_T = all ? t : 0u;
      if (!all) atomicAdd(&g_diag[CSA_DIAG_INDEXER_GIVEUPS], 1ull);
    }
  }
  __syncthreads();
  const uint32_t T = use_t ? s_T : 0u;
  // compaction in index order: wave w owns [w * per, (w + 1) * per) of the
  // chunk, counted in a first pass and written in a second
  const int per = (cn + kIdxThreads - 1) / kIdxThreads * kWave;
  const int p0 = wave * per;
  const int p1 = p0 + per < cn ? p0 + per : cn;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t n_mine = 0;
  for (int p = p0; p < p1; p += kWave) {
    const int pos = p + lane;
    n_mine += (uint32_t)__popcll(__ballot(pos < p1 && s_keys[pos] >= T));
  }
  if (lane == 0) s_wt[wave] = n_mine;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += s_wt[w];
  uint2* region = (uint2*)(wq + a.off_region) + c0;
  for (int p = p0; p < p1; p += kWave) {
    const int pos = p + lane;
    const uint32_t key = pos < p1 ? s_keys[pos] : 0u;
    const bool take = pos < p1 && key >= T;
    const uint64_t bt = __ballot(take);
    if (take) region[base + __popcll(bt & lt)] = make_uint2(key, (uint32_t)(c0 + pos));
    base += (uint32_t)__popcll(bt);
  }
  if (wave == kIdxWaves - 1 && lane == 0) counts[c] = base;
}

constexpr int kLFinalLds = 8192;

__global__ __launch_bounds__(kIdxThreads) void idx_long_final_kernel(IdxArgs a) {
  __shared__ uint32_t s_cand[kLFinalLds];
  __shared__ int32_t s_cidx[kLFinalLds];
  __shared__ SelShared sh;
  __shared__ uint32_t s_pre[kIdxThreads + 1];
  const int tid = threadIdx.x;
  const int64_t bq = blockIdx.x;
  uint8_t* wq = a.ws + bq * a.per_query;
  const uint32_t* counts = (const uint32_t*)(wq + a.off_counts);
  const uint2* region = (const uint2*)(wq + a.off_region);
  // the count load goes out together with the position load (the counts are
  // workspace memory, readable whatever nt turns out to be)
  const uint32_t cnt_ld = tid < a.nseg ? counts[tid] : 0u;
  const int64_t nt = idx_visible(a, bq);
  int32_t* out = a.sel + bq * a.k;
  float* out_score = a.sel_score ? a.sel_score + bq * a.k : nullptr;
  if (nt <= a.k && !out_score) {                // every visible entry, unscored
    for (int i = tid; i < a.k; i += kIdxThreads) out[i] = i < nt ? i : -1;
    return;
  }
  // segment offsets in the concatenated candidate list (nseg <= kIdxThreads;
  // s_pre[s] for every s <= kIdxThreads, so that segment s holds s_pre[s+1]
  // - s_pre[s] candidates)
  const int lane = tid % kWave, wave = tid / kWave;
  const uint32_t cnt_mine = cnt_ld;
  const uint32_t incl = wave_scan<0>(cnt_mine);
  if (lane == kWave - 1) sh.wtot[0][wave] = incl;
  __syncthreads();
  uint32_t wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += sh.wtot[0][w];
  s_pre[tid] = wbase + incl - cnt_mine;
  if (tid == kIdxThreads - 1) s_pre[kIdxThreads] = wbase + incl;
  __syncthreads();
  const int ncand = (int)s_pre[kIdxThreads];
  const int kk = ncand < a.k ? ncand : a.k;
  for (int i = kk + tid; i < a.k; i += kIdxThreads) {
    out[i] = -1;
    if (out_score) out_score[i] = -INFINITY;
  }
  if (kk == 0) return;
  uint32_t thr;
  int need_eq;
  if (ncand <= kLFinalLds) {
    // the usual case (about k candidates): straight from the segment
    // regions into LDS, 32 threads per segment, every load in flight together
    for (int sg = tid >> 5; sg < a.nseg; sg += kIdxThreads >> 5) {
      const uint32_t off = s_pre[sg], cnt = s_pre[sg + 1] - off;
      const uint2* rg = region + (int64_t)sg * a.rstride;
      for (uint32_t j = tid & 31; j < cnt; j += 32) {
        const uint2 v = rg[j];
        s_cand[off + j] = v.x;
        s_cidx[off + j] = (int32_t)v.y;
      }
    }
    __syncthreads();
    radix_select(s_cand, ncand, kk, sh, thr, need_eq);
    emit_selected(s_cand, ncand, thr, need_eq, sh, [&](int pos, int rank) {
      out[rank] = s_cidx[pos];
      if (out_score) out_score[rank] = key_score(s_cand[pos]);
    });
    return;
  }
  // many candidates (heavy ties, or chunks that stopped waiting): concatenated in the workspace
  if (tid == 0) atomicAdd(&g_diag[CSA_DIAG_INDEXER_WIDE_SELECT], 1ull);
  uint32_t* skey = (uint32_t*)(wq + a.off_skey);
  int32_t* sidx = (int32_t*)(wq + a.off_sidx);
  for (int sg = 0; sg < a.nseg; ++sg) {
    const uint32_t off = s_pre[sg], cnt = s_pre[sg + 1] - off;
    const uint2* rg = region + (int64_t)sg * a.rstride;
    for (uint32_t j = tid; j < cnt; j += kIdxThreads) {
      const uint2 v = rg[j];
      skey[off + j] = v.x;
      sidx[off + j] = (int32_t)v.y;
    }
  }
  __syncthreads();
  radix_select(skey, ncand, kk, sh, thr, need_eq);
  emit_selected(skey, ncand, thr, need_eq, sh, [&](int pos, int rank) {
    out[rank] = sidx[pos];
    if (out_score) out_score[rank] = key_score(skey[pos]);
  });
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Wait budget of the one-pass long-list indexer: kLSpinMax polls, or the
// value of CSA_INDEXER_SPIN_LIMIT (>= 0) for tests of the path a workgroup
// takes when it stops waiting (0: every workgroup takes it at once).
static int indexer_spin_limit() {
  const char* e = getenv("CSA_INDEXER_SPIN_LIMIT");
  if (!e || !*e) return kLSpinMax;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  return (end && *end == 0 && v >= 0 && v <= kLSpinMax) ? (int)v : kLSpinMax;
}

hipError_t diag_counters(uint64_t* out, int n, bool reset) {
  unsigned long long h[CSA_DIAG_COUNT];
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(h, HIP_SYMBOL(g_diag), sizeof(h), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  for (int i = 0; i < n && i < CSA_DIAG_COUNT; ++i) out[i] = h[i];
  if (reset) {
    unsigned long long z[CSA_DIAG_COUNT] = {};
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_diag), z, sizeof(z), 0, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  return e;
}

IdxPlan indexer_plan(int B, int Tq, int64_t n_entries, int k) {
  IdxPlan p{};
  const int64_t queries = (int64_t)B * Tq;
  if (n_entries <= 0) { p.chunk = 1024; p.nchunk = 1; p.ok = true; return p; }
  if (queries < 256 && n_entries > 8192) {
    // long lists: score / compact / final select
    const int64_t lchunk = kLChunk;
    p.nchunk = (int)((n_entries + lchunk - 1) / lchunk);
    p.lm = 1;
    // one pass (mode 2) while a query's chunks are few next to the resident
    // slots; its candidate regions are the chunks, else the kLSeg segments
    const bool fused = p.nchunk <= kLFusedMaxChunks;
    p.mode = fused ? 2 : 1;
    p.rstride = fused ? (int)lchunk : kLSeg;
    p.nseg = fused ? p.nchunk : (int)((n_entries + kLSeg - 1) / kLSeg);
    if (p.nseg > kIdxThreads) return p;                          // up to 8M entries per query
    const size_t npad = align256((size_t)p.nseg * p.rstride);
    p.off_scores = 0;
    p.off_uni = fused ? 0 : align256(npad * 4);                  // one pass keeps no scores
    p.off_region = p.off_uni + align256((size_t)p.nchunk * p.lm * 4);
    p.off_counts = p.off_region + npad * 8;
    p.off_ctr = p.off_counts + align256((size_t)p.nseg * 4);
    p.off_skey = p.off_ctr + align256((size_t)p.nchunk * 8);    // one-pass: a slot per chunk
    p.off_sidx = p.off_skey + npad * 4;
    p.per_query = p.off_sidx + npad * 4;
    p.chunk = (int)lchunk;
    p.ws = (size_t)queries * p.per_query;
    p.ok = true;
    return p;
  }
  int64_t chunk = 1024;
  // one chunk per query when it fits, else chunks whose local top-k lists are merged
  while (chunk < n_entries && chunk < kMaxChunk) chunk <<= 1;
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
static hipError_t launch_idx_long(const IdxArgs& a, bool fused, hipStream_t st) {
  const unsigned nq = (unsigned)((int64_t)a.B * a.Tq);
  if (fused) {
    hipLaunchKernelGGL(idx_long_zero_kernel, dim3((unsigned)(((int64_t)nq * a.nchunk + 255) / 256)), dim3(256), 0, st,
                       a, (int64_t)nq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // chunk index fastest: the chunks of a query are dispatched together
    hipLaunchKernelGGL((idx_long_fused_kernel<FMT, DI>), dim3(a.nchunk, nq), dim3(kIdxThreads),
                       (size_t)a.chunk * 4, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(idx_long_final_kernel, dim3(nq), dim3(kIdxThreads), 0, st, a);
    return hipGetLastError();
  }
  auto ka = idx_long_score_kernel<FMT, DI>;
  hipLaunchKernelGGL(ka, dim3(nq, a.nchunk), dim3(kIdxThreads), (size_t)a.chunk * 4, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_long_compact_kernel, dim3(nq, a.nseg), dim3(kIdxThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_long_final_kernel, dim3(nq), dim3(kIdxThreads), 0, st, a);
  return hipGetLastError();
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
                          int k, int32_t* sel, float* sel_score, void* ws, const IdxPlan& plan, hipStream_t st) {
  IdxArgs a;
  a.qidx = view(qidx);
  a.keys = view(keys);
  a.head_w = head_w;
  a.n_entries = n_entries;
  a.q_pos = q_pos;
  a.B = B; a.Tq = Tq; a.H_I = H_I; a.m = m; a.k = k;
  a.chunk = plan.chunk; a.nchunk = plan.nchunk;
  a.ws = (uint8_t*)ws;
  a.per_query = plan.per_query; a.off_scores = plan.off_scores; a.off_uni = plan.off_uni;
  a.off_region = plan.off_region; a.off_counts = plan.off_counts; a.off_skey = plan.off_skey;
  a.off_sidx = plan.off_sidx; a.off_ctr = plan.off_ctr; a.lm = plan.lm; a.nseg = plan.nseg;
  a.rstride = plan.rstride;
  a.spin_max = indexer_spin_limit();
  a.sel = sel;
  a.sel_score = sel_score;
  const size_t half = plan.ws / 2;
  a.ws_key = (uint32_t*)ws;
  a.ws_idx = (int32_t*)((uint8_t*)ws + half);
  if ((int64_t)B * Tq == 0) return hipSuccess;
  if (indexer_stream_ok(keys, H_I, B, Tq, n_entries, k)) return launch_idx_stream(a, st);
  const int d = keys.dim;
  if (plan.mode == 1 || plan.mode == 2) {
    const bool f = plan.mode == 2;
    switch (keys.fmt) {
      case CSA_F32: return d == 32 ? launch_idx_long<CSA_F32, 32>(a, f, st) : launch_idx_long<CSA_F32, 64>(a, f, st);
      case CSA_FP8_E4M3:
        return d == 32 ? launch_idx_long<CSA_FP8_E4M3, 32>(a, f, st) : launch_idx_long<CSA_FP8_E4M3, 64>(a, f, st);
      default: return d == 32 ? launch_idx_long<CSA_MXFP4, 32>(a, f, st) : launch_idx_long<CSA_MXFP4, 64>(a, f, st);
    }
  }
  switch (keys.fmt) {
    case CSA_F32: return d == 32 ? launch_idx_t<CSA_F32, 32>(a, st) : launch_idx_t<CSA_F32, 64>(a, st);
    case CSA_FP8_E4M3: return d == 32 ? launch_idx_t<CSA_FP8_E4M3, 32>(a, st) : launch_idx_t<CSA_FP8_E4M3, 64>(a, st);
    default: return d == 32 ? launch_idx_t<CSA_MXFP4, 32>(a, st) : launch_idx_t<CSA_MXFP4, 64>(a, st);
  }
}

}  // namespace csa
