/*
 * tidar.h - C ABI of libtidar, the MI355X (gfx950) decode-step hot path of
 * TiDAR ("TiDAR: Think in Diffusion, Talk in Autoregression").
 *
 * One TiDAR decode step runs a single forward whose attention covers three
 * query regions at once (TiDAR review on the awesome-system-papers wiki,
 * 核心方法 section 3.2 "parallel self-speculative generation"; talk notes on
 * notes.yuuk.io, 推論パイプライン):
 *   - the committed prefix, whose KV is cached from earlier steps;
 *   - the k drafts of the previous step, verified with causal (AR) logits;
 *   - one block of mask tokens per possible accept length j = 0..k, which
 *     pre-drafts the next step conditioned on drafts d_1..d_j.
 * The AR logits then verify the drafts by rejection sampling, the pre-draft
 * block matching the accept length is kept, and the accepted drafts' KV is
 * appended to the exact cache while the rejected drafts' KV is dropped,
 * without recomputation (same section; talk notes, 厳密 KV キャッシュ対応).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host". The caller owns every
 *     buffer; the library allocates no device memory. Scratch space is passed
 *     in as `workspace`, sized by the matching *_workspace_bytes() query.
 *   - Calls only enqueue work on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and never synchronise.
 *   - Tensors are dense, row-major, in the layouts stated below. Device
 *     pointers must be 16-byte aligned.
 *   - Host-side argument checks run before any HIP call and return a negative
 *     tidar_status; nothing is launched then. A failed launch returns
 *     TIDAR_E_HIP. Problems only visible on the device (a cache length or
 *     accept length out of range, a non-finite logit row) set bits in the
 *     optional int32 `dev_status` word (bitwise OR, never cleared by the
 *     library) and the kernel clamps instead of faulting.
 *   - tidar_last_error() returns a thread-local message for the last failed
 *     call on the calling thread.
 *   - The library holds no state between calls: any number of calls may be in
 *     flight on different streams, provided their output buffers and
 *     workspaces do not overlap.
 */
#ifndef TIDAR_H_
#define TIDAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TIDAR_OK = 0,
  TIDAR_E_INVALID = -1,      /* bad argument (null pointer, bad shape, misalignment) */
  TIDAR_E_UNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim for bf16) */
  TIDAR_E_WORKSPACE = -3,    /* workspace smaller than the query returned */
  TIDAR_E_CAPACITY = -4,     /* cache capacity cannot hold the requested lengths */
  TIDAR_E_HIP = -5           /* a HIP runtime call or launch failed */
} tidar_status;

enum { TIDAR_DTYPE_F32 = 0, TIDAR_DTYPE_BF16 = 1 };

/* dev_status bits */
enum {
  TIDAR_DEV_CACHE_LEN_RANGE = 1,   /* cache_len[b] < 0 or > max_cache_len: clamped */
  TIDAR_DEV_ACCEPT_RANGE = 2,      /* accept_len[b] outside 0..k: sequence not committed */
  TIDAR_DEV_CAPACITY = 4,          /* cache_len_in[b] + n > cache_capacity: not committed */
  TIDAR_DEV_NONFINITE_ROW = 8,     /* a logit row had no finite maximum or a zero sum */
  TIDAR_DEV_DRAFT_RANGE = 16,      /* a draft token id outside 0..V-1: treated as rejected */
  TIDAR_DEV_TARGET_RANGE = 32      /* a likelihood target id outside 0..V-1: its score is NaN */
};

const char* tidar_status_string(int status);
const char* tidar_last_error(void);
/* Library version as 10000*major + 100*minor + patch. */
int tidar_version(void);

/* ------------------------------------------------------------------------
 * Hybrid-mask attention for one layer of one decode step.
 *
 * Query rows per sequence: R = k + num_blocks * block_len, ordered as
 *   r in [0, k)                    : draft d_{r+1} (region A),
 *   r = k + j*block_len + m        : mask token m of pre-draft block j
 *                                    (accept length j), j < num_blocks.
 * Visibility of step key c (0 <= c < R) from row r (computed from the region
 * indices; no mask tensor exists):
 *   draft row r        : c <= r                     (causal among drafts)
 *   block j, any m     : c < j (drafts d_1..d_j), or c inside block j
 *                        (bidirectional within the block); no other block.
 * Every row also sees the committed prefix keys [0, cache_len[b]).
 * TiDAR uses num_blocks = k + 1 and block_len = k. num_blocks = 0 gives plain
 * causal append-prefill of k tokens over the prefix (the likelihood mode of
 * the talk notes' 尤度評価 section, and the token-count sweep of the
 * free-token-slot figure).
 *
 * out[b,r,h,:] = softmax_c(sm_scale * q[b,r,h,:] . key_c) . value_c over the
 * visible keys, with query head h reading KV head h / (Hq/Hkv).
 *
 * The prefix keys are split into workgroup-sized pieces that are reduced
 * separately and merged by log-sum-exp; the result does not depend on the
 * split count beyond floating-point rounding. Each split's normalised output
 * is held in the workspace in the input precision (bf16 or fp32), with its
 * log-sum-exp in fp32. With several sequences (batch > 1, bf16, num_splits =
 * 0) the pieces are shared out per sequence on the device, in proportion to
 * each sequence's cache_len plus twice its step keys (a step-key tile costs
 * about two prefix tiles), so a ragged batch runs in one round of
 * workgroups; the per-sequence split table lives at the start of the
 * workspace and is rewritten by every launch. An optional decode-regime kernel (few packed query
 * rows per KV head, see tidar_attn_workspace_bytes) streams 128-key splits
 * plus one split of the step's keys, and the split that finishes last merges
 * them when they are small enough.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t num_q_heads;     /* Hq, multiple of num_kv_heads */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;        /* D: bf16 supports 64 and 128; f32 supports 4..256, multiple of 4 */
  int32_t k;               /* drafts verified per step (>= 0) */
  int32_t num_blocks;      /* pre-draft blocks, 0..k+1 */
  int32_t block_len;       /* mask tokens per block (>= 1 when num_blocks > 0) */
  int32_t cache_capacity;  /* cap: rows allocated per (b, kv head) in the cache */
  int32_t max_cache_len;   /* host-known bound on cache_len[b], <= cap; used to plan splits */
  float sm_scale;          /* softmax scale, > 0 (typically 1/sqrt(D)) */
  int32_t dtype;           /* TIDAR_DTYPE_F32 or TIDAR_DTYPE_BF16 for q, k/v, out */
  int32_t num_splits;      /* 0 = library chooses; otherwise the prefix split count (the same
                              for every sequence) */
} tidar_attn_desc;

/* Workspace bytes tidar_attn_step needs for this descriptor (0 if none).
 * The decode-regime kernel (bf16, head_dim 128, num_splits = 0, few packed
 * query rows per KV head) is chosen by itself for Hq/Hkv * R <= 32 when
 * B * Hkv * (ceil(max_cache_len / 128) + 1) <= 256; environment
 * TIDAR_ATTN_DECODE=1 selects it up to Hq/Hkv * R <= 128 (R <= 128), =0
 * never. Its workspace leads with one arrival counter per (sequence, KV
 * head). They are used only when TIDAR_ATTN_FUSED_MERGE=1 asks it to merge
 * its splits itself: then the workspace must be zero-filled before its first
 * use (hipMemset, or torch.zeros), and every launch returns the counters to
 * zero. Otherwise the workspace needs no clearing. */
size_t tidar_attn_workspace_bytes(const tidar_attn_desc* desc);

/*
 * q        [B, R, Hq, D]    dtype
 * k_step   [B, R, Hkv, D]   dtype   keys of this step's R tokens
 * v_step   [B, R, Hkv, D]   dtype
 * k_cache  [B, Hkv, cap, D] dtype   this layer's cache. Rows at or past cache_len[b] never
 *                                  affect the result: bf16 k_cache rows below max_cache_len
 *                                  may be loaded (any bit pattern, NaN included, is masked
 *                                  out); bf16 v_cache rows below max_cache_len may be loaded
 *                                  by the decode-regime kernel, which clears them before use;
 *                                  rows at or past max_cache_len are never read
 * v_cache  [B, Hkv, cap, D] dtype
 * cache_len[B] int32        committed prefix length per sequence (device)
 * out      [B, R, Hq, D]    dtype   written
 * lse      [B, R, Hq] f32 or NULL   natural-log normaliser of each row
 * dev_status int32 or NULL
 * The cache is not modified (appending is tidar_kv_commit's job).
 */
int tidar_attn_step(const tidar_attn_desc* desc, const void* q, const void* k_step,
                    const void* v_step, const void* k_cache, const void* v_cache,
                    const int32_t* cache_len, void* out, float* lse, int32_t* dev_status,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * KV commit: append the accepted drafts' KV, evict the rejected ones.
 * For every layer l, sequence b, KV head h and i < n_b = accept_len[b]:
 *   k_cache[l,b,h,cache_len_in[b]+i,:] = k_step[l,b,i,h,:]   (same for v)
 *   cache_len_out[b] = cache_len_in[b] + n_b
 * Draft rows i >= n_b and all pre-draft rows (i >= k) are never written, so
 * the valid cache stays one contiguous run per sequence. No recomputation.
 *
 * k_step/v_step  [L, B, step_rows, Hkv, D] dtype (rows 0..k-1 are the drafts)
 * k_cache/v_cache [L, B, Hkv, cap, D] dtype   updated in place
 * accept_len [B] int32 (device, e.g. straight from tidar_reject_sample)
 * cache_len_in [B], cache_len_out [B] int32; must not alias
 * max_cache_len: host bound on cache_len_in; max_cache_len + k <= cap is checked.
 * A sequence whose accept_len is outside 0..k, or whose new length would pass
 * cap, is left unchanged (cache_len_out = cache_len_in) and flagged in dev_status.
 * ---------------------------------------------------------------------- */
int tidar_kv_commit(int32_t num_layers, int32_t batch, int32_t num_kv_heads, int32_t head_dim,
                    int32_t k, int32_t step_rows, int32_t cache_capacity, int32_t max_cache_len,
                    int32_t dtype, const void* k_step, const void* v_step, void* k_cache,
                    void* v_cache, const int32_t* accept_len, const int32_t* cache_len_in,
                    int32_t* cache_len_out, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------
 * AR rejection sampling of the diffusion drafts (speculative-sampling rule,
 * Leviathan et al. 2023 / Chen et al. 2023, which the TiDAR pages name as AR
 * rejection sampling of the drafts):
 *   p_i = softmax(ar_logits[b,i,:] / T), i = 0..k     (row i verifies d_{i+1}; row k = bonus)
 *   q_i = softmax(diff_logits[b,i,:] / T), i = 0..k-1
 *   n = number of leading i with uniforms[b,i] < min(1, p_i(d_{i+1}) / q_i(d_{i+1}))
 *   if n < k: next_token ~ normalised max(0, p_n - q_n)  (all-zero residual -> p_n)
 *   else:     next_token ~ p_k                          (bonus token)
 * The draw is the inverse CDF with uniforms[b,k]: the smallest token id whose
 * running sum of weights exceeds u * (sum of weights), scanning in id order.
 * The pre-draft block for the next step is rows [k + n*k, k + (n+1)*k) of the
 * step, i.e. block index n = accept_len[b] (no copy is made).
 *
 * ar_logits [B, k+1, V] f32, diff_logits [B, k, V] f32, drafts [B, k] int32,
 * uniforms [B, k+1] f32 in [0, 1). Outputs: accept_len [B] int32 in 0..k,
 * next_token [B] int32, ratio [B, k] f32 or NULL (p_i(d)/q_i(d) for every i,
 * +inf where q_i(d) = 0). temperature > 0.
 * ---------------------------------------------------------------------- */
size_t tidar_reject_workspace_bytes(int32_t batch, int32_t k, int32_t vocab);

int tidar_reject_sample(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits,
                        const float* diff_logits, const int32_t* drafts, const float* uniforms,
                        float temperature, int32_t* accept_len, int32_t* next_token, float* ratio,
                        int32_t* dev_status, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * The same sampler with trust mixing of the verification targets (TiDAR
 * review, awesome-system-papers wiki, section 设计取舍: trust AR vs trust
 * diffusion logits, Fig. 6 — the AR and diffusion logits are mixed with a
 * weight lambda at verification time):
 *   p_i = softmax((trust_ar * ar_logits[b,i,:] + (1 - trust_ar) * diff_logits[b,i,:]) / T),
 *         i = 0..k-1, mixed on the diffusion row that proposed d_{i+1};
 *   p_k = softmax(ar_logits[b,k,:] / T)  (the bonus row has no diffusion row);
 *   q_i, the acceptance rule, the residual and the draws are unchanged.
 * trust_ar in [0, 1] (else TIDAR_E_INVALID): 1 reproduces tidar_reject_sample
 * bit for bit (the AR logits are used as they are), 0 uses the diffusion
 * logits as the targets (every in-range draft is then accepted). Each mixed
 * logit is formed in fp32 as fmaf(trust_ar, a, (1 - trust_ar) * d).
 * Arguments, layouts, ownership, workspace (tidar_reject_workspace_bytes)
 * and errors are those of tidar_reject_sample; ratio holds the mixed
 * p_i(d) / q_i(d).
 * ---------------------------------------------------------------------- */
int tidar_reject_sample_trust(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits,
                              const float* diff_logits, const int32_t* drafts, const float* uniforms,
                              float temperature, float trust_ar, int32_t* accept_len,
                              int32_t* next_token, float* ratio, int32_t* dev_status, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The sampler with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments, layouts, results and errors
 * are those of tidar_reject_sample_trust (trust_ar = 1 is
 * tidar_reject_sample); it runs the same kernels and gives the same bits.
 * The workspace is a static device array inside the library, of
 * tidar_reject_noalloc_max_bytes() bytes (1 MiB) per GPU, held until the
 * process ends; its device address is looked up once per device, on the
 * first call there. Calls whose tidar_reject_workspace_bytes(batch, k,
 * vocab) exceeds that size return TIDAR_E_WORKSPACE before any launch
 * (1 MiB covers e.g. batch 64 at k = 16, vocab 151936). No allocation and no
 * allocating library routine is called. Every call on one GPU uses the same
 * array and overwrites all of it that it reads, so nothing needs clearing;
 * calls that overlap on one GPU (different streams, or host threads)
 * race on it and must be serialised by the caller. The stream's device is
 * the GPU used (NULL stream: the current device).
 * ---------------------------------------------------------------------- */
int tidar_reject_sample_noalloc(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits,
                                const float* diff_logits, const int32_t* drafts, const float* uniforms,
                                float temperature, float trust_ar, int32_t* accept_len,
                                int32_t* next_token, float* ratio, int32_t* dev_status, void* stream);

/* Bytes of the static scratch behind tidar_reject_sample_noalloc. */
size_t tidar_reject_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------
 * Likelihood mode: per-token AR log-probabilities (talk notes on
 * notes.yuuk.io, 尤度評価: with the attention mask set to causal, TiDAR
 * scores a sequence as an AR model in one forward, no Monte-Carlo sampling;
 * review, 实验与结果: one NFE with a pure causal mask). The causal forward
 * is tidar_attn_step with num_blocks = 0 (append-prefill rows, causal among
 * themselves over the full prefix); this call turns the resulting logits
 * into scores:
 *   logprobs[r] = logits[r, targets[r]] - log(sum_v exp(logits[r, v]))
 * (temperature 1; fp32 statistics per 4096-token chunk merged in a fixed
 * order, so results are run-to-run deterministic).
 *
 * logits [rows, V] f32 (e.g. [B, R, V] flattened; 16-byte aligned),
 * targets [rows] int32 (the next token of each row), logprobs [rows] f32
 * output. A target outside 0..V-1 scores NaN and sets
 * TIDAR_DEV_TARGET_RANGE; a row with no finite maximum or a zero sum scores
 * NaN and sets TIDAR_DEV_NONFINITE_ROW. Workspace: at least
 * tidar_logprob_workspace_bytes(rows, V) bytes, 256-byte aligned (0 is
 * returned for rows < 1 or V < 1). Errors: TIDAR_E_INVALID (shape, NULL,
 * alignment), TIDAR_E_UNSUPPORTED (rows * V >= 2^31), TIDAR_E_WORKSPACE,
 * TIDAR_E_HIP.
 * ---------------------------------------------------------------------- */
size_t tidar_logprob_workspace_bytes(int32_t rows, int32_t vocab);

int tidar_token_logprobs(int32_t rows, int32_t vocab, const float* logits, const int32_t* targets,
                         float* logprobs, int32_t* dev_status, void* workspace, size_t workspace_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TIDAR_H_ */
