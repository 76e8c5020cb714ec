// Host-side launchers of the kernels, called by the C-ABI layer (api.hip)
// after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"
#include "common.h"

namespace csa {

hipError_t launch_compress(const void* tok, int tok_fmt, int B, int64_t T, int64_t bstride, int m,
                           const float* gate, const float* bias, const csa_store& out, int64_t row0,
                           const NormRope& nr, hipStream_t st);
int compress_max_m();
hipError_t launch_decode_append(const void* tok, int tok_fmt, int B, const int64_t* pos, void* tail, int R, int m,
                                const float* gate, const float* bias, const csa_store& out, const csa_store& win,
                                int W, const NormRope& nr, hipStream_t st);
hipError_t launch_decode_rebuild(const void* tok, int tok_fmt, int B, int n, int64_t bstride, const int64_t* p0,
                                 const int32_t* n_valid, void* tail, int R, int m, const float* gate, const float* bias,
                                 const csa_store& out, const csa_store& win, int W, const NormRope& nr,
                                 hipStream_t st);

// Indexer: chunk size and chunk count chosen for a call; workspace bytes.
struct IdxPlan {
  int chunk;      // entries scored per workgroup
  int nchunk;     // chunks per query
  size_t ws;      // workspace bytes
  bool ok;
  int mode;       // 0: chunk(s) + merge, 1: long lists (score / compact / select),
                  // 2: long lists (score and compact in one pass / select)
  int lm, nseg;   // long lists: union keys per chunk, candidate regions per query
  int rstride;    // long lists: entries between consecutive candidate regions
  size_t per_query, off_scores, off_uni, off_region, off_counts, off_skey, off_sidx, off_ctr;
};
IdxPlan indexer_plan(int B, int Tq, int64_t n_entries, int k);
// Many queries over FP8 keys of 64 dims: the single-pass streaming top-k,
// which needs no workspace.
bool indexer_stream_ok(const csa_store& keys, int H_I, int B, int Tq, int64_t n_entries, int k);
// Diagnostic counters of the current device (synchronises it).
hipError_t diag_counters(uint64_t* out, int n, bool reset);
hipError_t launch_indexer(const csa_store& qidx, const float* head_w, const csa_store& keys,
                          int64_t n_entries, const int64_t* q_pos, int B, int Tq, int H_I, int m,
                          int k, int32_t* sel, float* sel_score, void* ws, const IdxPlan& plan, hipStream_t st);

// Attention: one launcher for every attention entry point.
struct AttnCall {
  const void* q; int q_fmt; int B, Tq, H, D;
  csa_store ckv; int64_t n_entries; int mode;   // 0: no compressed entries, 1: sel list, 2: range
  const int32_t* sel; int k; int m;
  csa_store win; int W; int ring;
  const int64_t* q_pos;
  const float* sink; float tau;
  const float* prior_o; const float* prior_lse;  // swa_merge: partial to merge
  void* out; float* lse; int partial;
  void* ws; size_t ws_bytes;
  int allow_split;                                 // split long lists over workgroups (needs ws)
  int invariant;                                   // splits independent of the batch (CSA_BATCH_INVARIANT)
  NormRope qn;                                     // RMSNorm / partial RoPE of the queries
};
enum { kModeNone = 0, kModeSel = 1, kModeRange = 2 };
size_t attn_workspace(int B, int Tq, int H, int D, int64_t max_list);
bool attn_supported(int H, int D);
hipError_t launch_attn(const AttnCall& c, hipStream_t st);
bool attn_mfma_eligible(int q_fmt, int H, int D, const csa_store& kv, bool has_prior, float tau);
hipError_t launch_attn_m32(const AttnCall& c, int nsplit, int split_len, hipStream_t st);

}  // namespace csa
