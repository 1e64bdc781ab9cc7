// Internal declarations shared by the libtidar translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tidar {

// Parameters of one hybrid-mask attention launch (one layer).
struct AttnParams {
  const void* q;
  const void* k_step;
  const void* v_step;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cache_len;
  void* out;
  float* lse;
  int32_t* dev_status;
  // split partials (S > 1 only): normalised output of each split over its
  // keys, [S, B, R, Hq, D] in the input precision (bf16 or fp32), and its
  // log-sum-exp in the log2 domain, [S, B, R, Hq] fp32 (-inf: no visible key)
  void* part_o;
  float* part_lse;
  int B, Hq, Hkv, D, g, R, k, num_blocks, block_len, cap, max_len;
  int S;          // number of prefix splits
  int chunk;      // prefix keys per split
  int qtiles;     // query tiles per (b, kv head)
  int nqt;        // 32-row query tiles per wave (bf16 path)
  int waves;      // waves per workgroup (bf16 path)
  float sm_scale;
  float scale_log2;  // sm_scale * log2(e)
};

struct AttnPlan {
  int S;
  int chunk;
  int qtiles;
  int nqt;
  int waves;
  int bm;          // packed query rows per workgroup
  size_t ws_bytes;
};

AttnPlan plan_attn(int dtype, int B, int Hq, int Hkv, int D, int R, int max_len, int forced_splits,
                   int local_tiles);
hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);

struct CommitParams {
  int L, B, Hkv, D, k, step_rows, cap, elem_bytes;
  const void* k_step;
  const void* v_step;
  void* k_cache;
  void* v_cache;
  const int32_t* accept_len;
  const int32_t* len_in;
  int32_t* len_out;
  int32_t* dev_status;
};
hipError_t launch_kv_commit(const CommitParams& p, hipStream_t stream);

struct RejectParams {
  int B, k, V;
  int chunk;     // vocabulary elements per stats chunk
  int nchunks;
  const float* ar;
  const float* diff;
  const int32_t* drafts;
  const float* uniforms;
  float inv_temp;
  // how the verification targets of rows 0..k-1 are formed: 0 = AR logits,
  // 1 = lam * AR + mu * diffusion (trust mixing, mu = 1 - lam), 2 = diffusion
  int mix;
  float lam, mu;
  int32_t* accept_len;
  int32_t* next_token;
  float* ratio;
  int32_t* dev_status;
  float2* row_stats;    // [B, 2k+1, nchunks] (max, sum exp) per chunk
  double* resid_sums;   // [2, B, nchunks] mass per chunk of the draw distribution, then of p_n alone
  int32_t* decision;    // [B, 2]: accept length, source row kind
  float2* row_mz;       // [B, 2k+1] merged (max, sum exp) of every row
};
size_t reject_workspace_bytes(int B, int k, int V);
int reject_max_k();
int reject_max_chunks();
void plan_reject(RejectParams& p);
hipError_t launch_reject(const RejectParams& p, hipStream_t stream);

struct LogprobParams {
  int rows, V, nchunks;
  const float* logits;     // [rows, V]
  const int32_t* targets;  // [rows]
  float* logprobs;         // [rows]
  int32_t* dev_status;
  float2* stats;           // [rows, nchunks] (max, sum exp) per vocabulary chunk
};
size_t logprob_workspace_bytes(int rows, int V);
int logprob_chunk();
hipError_t launch_logprob(const LogprobParams& p, hipStream_t stream);

}  // namespace tidar
