// C ABI of libtidar: argument validation, workspace sizing, split planning
// and kernel launches. Every check runs on the host before any HIP call, so
// a bad argument never reaches the device.
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "tidar.h"
#include "tidar_ceilings.h"
#include "tidar_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TIDAR_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr long kMaxElems = 0x7fffffffL;

// a * b, saturated at LONG_MAX (size checks multiply untrusted extents)
long sat_mul(long a, long b) {
  long r;
  return __builtin_mul_overflow(a, b, &r) ? LONG_MAX : r;
}

// 64-key tiles of step keys a query tile may see: the whole causal run in
// append-prefill mode, else the drafts plus one block
int local_tiles_of(const tidar_attn_desc* d) {
  const long R = (long)d->k + (long)d->num_blocks * (d->num_blocks > 0 ? d->block_len : 0);
  return d->num_blocks == 0 ? (int)((R + 63) / 64) : (d->k + 63) / 64 + (d->block_len + 63) / 64;
}

int check_desc(const tidar_attn_desc* d, tidar::AttnPlan* plan) {
  if (!d) return fail(TIDAR_E_INVALID, "desc is NULL");
  if (d->dtype != TIDAR_DTYPE_F32 && d->dtype != TIDAR_DTYPE_BF16)
    return fail(TIDAR_E_INVALID, "dtype %d is neither f32 (0) nor bf16 (1)", d->dtype);
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(TIDAR_E_INVALID, "batch, num_q_heads and num_kv_heads must be >= 1");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(TIDAR_E_INVALID, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->k < 0 || d->num_blocks < 0) return fail(TIDAR_E_INVALID, "k and num_blocks must be >= 0");
  if ((long)d->num_blocks > (long)d->k + 1)
    return fail(TIDAR_E_INVALID, "num_blocks (%d) exceeds k + 1 (%ld): block j needs drafts d_1..d_j", d->num_blocks,
                (long)d->k + 1);
  if (d->num_blocks > 0 && d->block_len < 1) return fail(TIDAR_E_INVALID, "block_len must be >= 1");
  const long R = (long)d->k + (long)d->num_blocks * (d->num_blocks > 0 ? d->block_len : 0);
  if (R < 1) return fail(TIDAR_E_INVALID, "no query rows (k + num_blocks * block_len == 0)");
  if (R > 65536) return fail(TIDAR_E_UNSUPPORTED, "R = %ld query rows exceeds 65536", R);
  if (d->cache_capacity < 1) return fail(TIDAR_E_INVALID, "cache_capacity must be >= 1");
  if (d->max_cache_len < 0) return fail(TIDAR_E_INVALID, "max_cache_len must be >= 0");
  if (d->max_cache_len > d->cache_capacity)
    return fail(TIDAR_E_CAPACITY, "max_cache_len %d exceeds cache_capacity (%d)", d->max_cache_len,
                d->cache_capacity);
  if (!(d->sm_scale > 0.f) || !isfinite(d->sm_scale))
    return fail(TIDAR_E_INVALID, "sm_scale must be positive and finite");
  if (d->num_splits < 0) return fail(TIDAR_E_INVALID, "num_splits must be >= 0");
  const int D = d->head_dim;
  if (d->dtype == TIDAR_DTYPE_BF16) {
    if (D != 64 && D != 128) return fail(TIDAR_E_UNSUPPORTED, "bf16 path supports head_dim 64 or 128, got %d", D);
  } else {
    if (D < 4 || D > 256 || D % 4) return fail(TIDAR_E_UNSUPPORTED, "f32 path needs head_dim in 4..256, multiple of 4");
  }
  const long qe = sat_mul(sat_mul(sat_mul(d->batch, R), d->num_q_heads), D);
  const long ce = sat_mul(sat_mul(sat_mul(d->batch, d->num_kv_heads), d->cache_capacity), D);
  if (qe > kMaxElems || ce > kMaxElems) return fail(TIDAR_E_UNSUPPORTED, "tensor too large for 32-bit indexing");
  const int local_tiles = local_tiles_of(d);
  if (d->dtype == TIDAR_DTYPE_BF16 && (d->num_kv_heads > 0xffff || d->num_q_heads / d->num_kv_heads > 0xffff ||
                                        d->k > 0xffff || (d->num_blocks > 0 && d->block_len > 0xffff)))
    return fail(TIDAR_E_UNSUPPORTED, "bf16 path: KV heads, group size, k and block_len must be below 65536");
  *plan = tidar::plan_attn(d->dtype, d->batch, d->num_q_heads, d->num_kv_heads, D, (int)R, d->max_cache_len,
                           d->num_splits, local_tiles);
  // the bf16 kernel receives the tile and split counts packed in 16 bits
  if (d->dtype == TIDAR_DTYPE_BF16 && (plan->qtiles > 0xffff || plan->S > 0xffff))
    return fail(TIDAR_E_UNSUPPORTED, "bf16 path: %d query tiles x %d splits exceed 65535", plan->qtiles, plan->S);
  if ((long)d->batch * d->num_kv_heads * (long)plan->qtiles * plan->S > kMaxElems)
    return fail(TIDAR_E_UNSUPPORTED, "attention grid too large");
  return TIDAR_OK;
}

// Shared by the sampler entry points. With noalloc the workspace is the
// library's static device scratch (no caller buffer, no allocation).
int reject_common(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits, const float* diff_logits,
                  const int32_t* drafts, const float* uniforms, float temperature, float trust_ar,
                  int32_t* accept_len, int32_t* next_token, float* ratio, int32_t* dev_status, void* workspace,
                  size_t workspace_bytes, bool noalloc, void* stream) {
  if (batch < 1 || k < 0 || vocab < 1) return fail(TIDAR_E_INVALID, "need batch >= 1, k >= 0, vocab >= 1");
  if (k > tidar::reject_max_k()) return fail(TIDAR_E_UNSUPPORTED, "k = %d exceeds %d", k, tidar::reject_max_k());
  tidar::RejectParams p{};
  p.B = batch;
  p.k = k;
  p.V = vocab;
  tidar::plan_reject(p);
  if (p.nchunks > tidar::reject_max_chunks())
    return fail(TIDAR_E_UNSUPPORTED, "vocab %d too large (max %d)", vocab, tidar::reject_max_chunks() * p.chunk);
  if ((long)batch * (k + 1) * (long)vocab > 0x7fffffffL || (long)batch * (2 * k + 1) * p.nchunks > 0x7fffffffL)
    return fail(TIDAR_E_UNSUPPORTED, "logits too large");
  if (!(temperature > 0.f) || !isfinite(temperature)) return fail(TIDAR_E_INVALID, "temperature must be > 0");
  if (!(trust_ar >= 0.f && trust_ar <= 1.f)) return fail(TIDAR_E_INVALID, "trust_ar must lie in [0, 1]");
  if (!ar_logits || !uniforms || !accept_len || !next_token)
    return fail(TIDAR_E_INVALID, "a required pointer is NULL");
  if (k > 0 && (!diff_logits || !drafts)) return fail(TIDAR_E_INVALID, "diff_logits and drafts required when k > 0");
  if (!aligned(ar_logits, 16) || (diff_logits && !aligned(diff_logits, 16)))
    return fail(TIDAR_E_INVALID, "logit pointers must be 16-byte aligned");
  const size_t need = tidar::reject_workspace_bytes(batch, k, vocab);
  if (noalloc) {
    if (need > tidar::kRejectScratchBytes)
      return fail(TIDAR_E_WORKSPACE, "batch %d, k %d, vocab %d need %zu bytes of scratch; the allocation-free "
                  "sampler holds %zu", batch, k, vocab, need, tidar::kRejectScratchBytes);
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "device of the stream");
    if ((e = tidar::reject_scratch(dev, &workspace)) != hipSuccess) return hip_fail(e, "sampler scratch address");
    workspace_bytes = tidar::kRejectScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(TIDAR_E_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(TIDAR_E_INVALID, "workspace must be 256-byte aligned");
  p.ar = ar_logits;
  p.diff = diff_logits;
  p.drafts = drafts;
  p.uniforms = uniforms;
  p.inv_temp = 1.f / temperature;
  p.mix = trust_ar == 1.f ? 0 : trust_ar == 0.f ? 2 : 1;
  p.lam = trust_ar;
  p.mu = 1.f - trust_ar;
  p.accept_len = accept_len;
  p.next_token = next_token;
  p.ratio = ratio;
  p.dev_status = dev_status;
  char* ws = static_cast<char*>(workspace);
  const size_t a = ((size_t)batch * (2 * k + 1) * p.nchunks * sizeof(float2) + 255) / 256 * 256;
  const size_t bsz = ((size_t)2 * batch * p.nchunks * sizeof(double) + 255) / 256 * 256;
  p.row_stats = reinterpret_cast<float2*>(ws);
  p.resid_sums = reinterpret_cast<double*>(ws + a);
  p.arrive = reinterpret_cast<int32_t*>(ws + a + bsz);
  const size_t dsz = ((size_t)batch * sizeof(int32_t) + 255) / 256 * 256;
  p.gathered = reinterpret_cast<float*>(ws + a + bsz + dsz);
  hipError_t e = tidar::launch_reject(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reject launch");
  return TIDAR_OK;
}

}  // namespace

extern "C" {

const char* tidar_status_string(int status) {
  switch (status) {
    case TIDAR_OK: return "TIDAR_OK";
    case TIDAR_E_INVALID: return "TIDAR_E_INVALID";
    case TIDAR_E_UNSUPPORTED: return "TIDAR_E_UNSUPPORTED";
    case TIDAR_E_WORKSPACE: return "TIDAR_E_WORKSPACE";
    case TIDAR_E_CAPACITY: return "TIDAR_E_CAPACITY";
    case TIDAR_E_HIP: return "TIDAR_E_HIP";
    default: return "unknown tidar status";
  }
}

const char* tidar_last_error(void) { return g_err.c_str(); }

int tidar_version(void) { return 100; }

int tidar_attn_stamps(uint64_t* dst, int max_workgroups) {
  if (!dst || max_workgroups < 0) return -1;
  return tidar::read_attn_stamps(reinterpret_cast<unsigned long long*>(dst), max_workgroups) == hipSuccess ? 0 : -5;
}

size_t tidar_attn_workspace_bytes(const tidar_attn_desc* desc) {
  tidar::AttnPlan plan;
  if (check_desc(desc, &plan) != TIDAR_OK) return 0;
  return plan.ws_bytes;
}

int tidar_attn_step(const tidar_attn_desc* desc, const void* q, const void* k_step, const void* v_step,
                    const void* k_cache, const void* v_cache, const int32_t* cache_len, void* out, float* lse,
                    int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream) {
  tidar::AttnPlan plan;
  int st = check_desc(desc, &plan);
  if (st != TIDAR_OK) return st;
  if (!q || !k_step || !v_step || !k_cache || !v_cache || !cache_len || !out)
    return fail(TIDAR_E_INVALID, "a required pointer is NULL");
  const void* ptrs[] = {q, k_step, v_step, k_cache, v_cache, out};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(TIDAR_E_INVALID, "tensor pointers must be 16-byte aligned");
  if (!aligned(cache_len, 4) || (lse && !aligned(lse, 4)) || (dev_status && !aligned(dev_status, 4)))
    return fail(TIDAR_E_INVALID, "cache_len, lse and dev_status must be 4-byte aligned");
  if (plan.ws_bytes > 0) {
    if (!workspace) return fail(TIDAR_E_WORKSPACE, "workspace of %zu bytes required", plan.ws_bytes);
    if (workspace_bytes < plan.ws_bytes)
      return fail(TIDAR_E_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, plan.ws_bytes);
    if (!aligned(workspace, 256)) return fail(TIDAR_E_INVALID, "workspace must be 256-byte aligned");
  }
  tidar::AttnParams p{};
  p.q = q;
  p.k_step = k_step;
  p.v_step = v_step;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.cache_len = cache_len;
  p.out = out;
  p.lse = lse;
  p.dev_status = dev_status;
  p.B = desc->batch;
  p.Hq = desc->num_q_heads;
  p.Hkv = desc->num_kv_heads;
  p.D = desc->head_dim;
  p.g = p.Hq / p.Hkv;
  p.k = desc->k;
  p.num_blocks = desc->num_blocks;
  p.block_len = desc->num_blocks > 0 ? desc->block_len : 1;
  p.R = p.k + desc->num_blocks * (desc->num_blocks > 0 ? desc->block_len : 0);
  p.cap = desc->cache_capacity;
  p.max_len = desc->max_cache_len;
  p.S = plan.S;
  p.chunk = plan.chunk;
  p.qtiles = plan.qtiles;
  p.nqt = plan.nqt;
  p.waves = plan.waves;
  p.decode = plan.decode;
  p.fused_merge = plan.fused_merge;
  p.ragged = plan.ragged;
  p.stamps = plan.stamps;
  p.local_tiles = local_tiles_of(desc);
  p.sm_scale = desc->sm_scale;
  p.scale_log2 = desc->sm_scale * 1.4426950408889634f;
  if (plan.S > 1 || plan.decode) {
    // [arrival counters (decode path) or split table (ragged)] [split outputs] [split log-sum-exps]
    const size_t rows = (size_t)plan.S * (plan.ragged ? 1 : p.B) * p.R * p.Hq;
    const size_t elem = desc->dtype == TIDAR_DTYPE_BF16 ? 2 : 4;
    char* ws = static_cast<char*>(workspace);
    p.counters = reinterpret_cast<int32_t*>(ws);
    p.split_tab = plan.ragged ? reinterpret_cast<int32_t*>(ws) : nullptr;
    p.part_o = ws + plan.counter_bytes;
    const size_t o_bytes = (rows * p.D * elem + 255) / 256 * 256;
    p.part_lse = reinterpret_cast<float*>(ws + plan.counter_bytes + o_bytes);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = desc->dtype == TIDAR_DTYPE_BF16 ? tidar::launch_attn_bf16(p, s) : tidar::launch_attn_f32(p, s);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return TIDAR_OK;
}

int tidar_kv_commit(int32_t num_layers, int32_t batch, int32_t num_kv_heads, int32_t head_dim, int32_t k,
                    int32_t step_rows, int32_t cache_capacity, int32_t max_cache_len, int32_t dtype,
                    const void* k_step, const void* v_step, void* k_cache, void* v_cache, const int32_t* accept_len,
                    const int32_t* cache_len_in, int32_t* cache_len_out, int32_t* dev_status, void* stream) {
  if (dtype != TIDAR_DTYPE_F32 && dtype != TIDAR_DTYPE_BF16) return fail(TIDAR_E_INVALID, "bad dtype %d", dtype);
  if (num_layers < 1 || batch < 1 || num_kv_heads < 1 || head_dim < 1)
    return fail(TIDAR_E_INVALID, "num_layers, batch, num_kv_heads and head_dim must be >= 1");
  if (k < 0 || step_rows < k) return fail(TIDAR_E_INVALID, "need 0 <= k <= step_rows");
  const int eb = dtype == TIDAR_DTYPE_BF16 ? 2 : 4;
  const long row_bytes = (long)head_dim * eb;
  if (row_bytes % 16) return fail(TIDAR_E_UNSUPPORTED, "row of head_dim elements must be a multiple of 16 bytes");
  // a workgroup walks its k rows in 16-byte pieces with 32-bit counters
  if (sat_mul(k, row_bytes / 16) > kMaxElems) return fail(TIDAR_E_UNSUPPORTED, "k rows of head_dim too large");
  if (cache_capacity < 1) return fail(TIDAR_E_INVALID, "cache_capacity must be >= 1");
  if (max_cache_len < 0) return fail(TIDAR_E_INVALID, "max_cache_len must be >= 0");
  if ((long)max_cache_len + k > cache_capacity)
    return fail(TIDAR_E_CAPACITY, "max_cache_len (%d) + k (%d) exceeds cache_capacity (%d)", max_cache_len, k,
                cache_capacity);
  if (!k_step || !v_step || !k_cache || !v_cache || !accept_len || !cache_len_in || !cache_len_out)
    return fail(TIDAR_E_INVALID, "a required pointer is NULL");
  if (cache_len_in == cache_len_out) return fail(TIDAR_E_INVALID, "cache_len_in must not alias cache_len_out");
  const void* ptrs[] = {k_step, v_step, k_cache, v_cache};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(TIDAR_E_INVALID, "tensor pointers must be 16-byte aligned");
  if (sat_mul(sat_mul(num_layers, batch), num_kv_heads) > kMaxElems) return fail(TIDAR_E_UNSUPPORTED, "grid too large");
  tidar::CommitParams p{};
  p.L = num_layers;
  p.B = batch;
  p.Hkv = num_kv_heads;
  p.D = head_dim;
  p.k = k;
  p.step_rows = step_rows;
  p.cap = cache_capacity;
  p.elem_bytes = eb;
  p.k_step = k_step;
  p.v_step = v_step;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.accept_len = accept_len;
  p.len_in = cache_len_in;
  p.len_out = cache_len_out;
  p.dev_status = dev_status;
  hipError_t e = tidar::launch_kv_commit(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv commit launch");
  return TIDAR_OK;
}

size_t tidar_reject_workspace_bytes(int32_t batch, int32_t k, int32_t vocab) {
  if (batch < 1 || k < 0 || vocab < 1 || k > tidar::reject_max_k()) return 0;
  return tidar::reject_workspace_bytes(batch, k, vocab);
}

int tidar_reject_sample(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits, const float* diff_logits,
                        const int32_t* drafts, const float* uniforms, float temperature, int32_t* accept_len,
                        int32_t* next_token, float* ratio, int32_t* dev_status, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return tidar_reject_sample_trust(batch, k, vocab, ar_logits, diff_logits, drafts, uniforms, temperature, 1.0f,
                                   accept_len, next_token, ratio, dev_status, workspace, workspace_bytes, stream);
}

int tidar_reject_sample_trust(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits,
                              const float* diff_logits, const int32_t* drafts, const float* uniforms,
                              float temperature, float trust_ar, int32_t* accept_len, int32_t* next_token,
                              float* ratio, int32_t* dev_status, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return reject_common(batch, k, vocab, ar_logits, diff_logits, drafts, uniforms, temperature, trust_ar, accept_len,
                       next_token, ratio, dev_status, workspace, workspace_bytes, false, stream);
}

int tidar_reject_sample_noalloc(int32_t batch, int32_t k, int32_t vocab, const float* ar_logits,
                                const float* diff_logits, const int32_t* drafts, const float* uniforms,
                                float temperature, float trust_ar, int32_t* accept_len, int32_t* next_token,
                                float* ratio, int32_t* dev_status, void* stream) {
  return reject_common(batch, k, vocab, ar_logits, diff_logits, drafts, uniforms, temperature, trust_ar, accept_len,
                       next_token, ratio, dev_status, nullptr, 0, true, stream);
}

size_t tidar_reject_noalloc_max_bytes(void) { return tidar::kRejectScratchBytes; }


size_t tidar_logprob_workspace_bytes(int32_t rows, int32_t vocab) {
  if (rows < 1 || vocab < 1) return 0;
  return tidar::logprob_workspace_bytes(rows, vocab);
}

int tidar_token_logprobs(int32_t rows, int32_t vocab, const float* logits, const int32_t* targets, float* logprobs,
                         int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 1 || vocab < 1) return fail(TIDAR_E_INVALID, "need rows >= 1 and vocab >= 1");
  const long nchunks = ((long)vocab + tidar::logprob_chunk() - 1) / tidar::logprob_chunk();
  if ((long)rows * vocab > 0x7fffffffL || (long)rows * nchunks > 0x7fffffffL)
    return fail(TIDAR_E_UNSUPPORTED, "logits too large");
  if (!logits || !targets || !logprobs) return fail(TIDAR_E_INVALID, "a required pointer is NULL");
  if (!aligned(logits, 16)) return fail(TIDAR_E_INVALID, "logits must be 16-byte aligned");
  const size_t need = tidar::logprob_workspace_bytes(rows, vocab);
  if (!workspace || workspace_bytes < need)
    return fail(TIDAR_E_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(TIDAR_E_INVALID, "workspace must be 256-byte aligned");
  tidar::LogprobParams p{};
  p.rows = rows;
  p.V = vocab;
  p.nchunks = (int)nchunks;
  p.logits = logits;
  p.targets = targets;
  p.logprobs = logprobs;
  p.dev_status = dev_status;
  p.stats = static_cast<float2*>(workspace);
  hipError_t e = tidar::launch_logprob(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "logprob launch");
  return TIDAR_OK;
}

}  // extern "C"
