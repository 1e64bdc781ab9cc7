// AR rejection sampling of the diffusion drafts, fused with the vocab-wide
// softmax it needs (TiDAR review, awesome-system-papers wiki, 核心方法
// section 3.2; acceptance rule of speculative sampling, Leviathan et al. 2023
// and Chen et al. 2023: keep d_{i+1} with probability min(1, p_i/q_i), on the
// first rejection draw from normalised max(0, p_i - q_i), after k acceptances
// draw a bonus token from p_k).
//
// Three HBM-streaming launches, all with a fixed reduction order so results
// are run-to-run deterministic:
//   1. rej_stats : per (row, vocab chunk) max and sum of exp over the 2k+1
//                  logit rows of each sequence (one read of all logits);
//   2. rej_resid : every workgroup of a sequence merges the row statistics,
//                  evaluates the acceptance chain from the gathered p_i(d),
//                  q_i(d) (identical in all of them) and sums the residual
//                  (or bonus) weights of its vocab chunk, and p_n alone for
//                  the rounding fallback, in fp64;
//   3. rej_pick  : per sequence, locates the chunk whose running mass passes
//                  u * total, then the token inside it (inverse CDF in token
//                  id order).
// Trust mixing (TiDAR review, 设计取舍: trust AR vs trust diffusion logits,
// Fig. 6) replaces the target logits of rows 0..k-1 by lam * AR +
// (1 - lam) * diffusion of the same position; the statistics, the gathered
// draft probabilities and the draw weights all evaluate the mixed logit the
// same way, fmaf(lam, a, mu * d). lam = 1 and lam = 0 read the AR or the
// diffusion row as it is.
#include "tidar_internal.h"

#include <math.h>

namespace tidar {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;            // vocab elements per chunk = 16 per thread
constexpr int kPer = kChunk / kThreads;
constexpr int kMaxK = 128;
constexpr int kMaxChunks = 1024;
constexpr int kStage = 4096;            // (row, chunk) statistics staged in LDS per sequence
constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sumf(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ double wave_sumd(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Block reductions with a fixed combination order (waves 0..3 in sequence).
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sumf(float x, float* red) {
  x = wave_sumf(x);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = x;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}
__device__ __forceinline__ double block_sumd(double x, double* red) {
  x = wave_sumd(x);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = x;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ const float* row_ptr(const RejectParams& p, int b, int rr) {
  // rows 0..k: AR logits (row i verifies d_{i+1}; row k is the bonus row);
  // rows k+1..2k: diffusion logits of drafts 0..k-1
  return rr <= p.k ? p.ar + ((size_t)b * (p.k + 1) + rr) * p.V
                   : p.diff + ((size_t)b * p.k + (rr - p.k - 1)) * p.V;
}

// Load this thread's kPer elements of a chunk (scaled by 1/T); -inf past the end.
__device__ __forceinline__ void load_chunk(const float* x, int e0, int e1, float inv_t, bool vec4,
                                           float (&v)[kPer]) {
  if (vec4 && e0 + kChunk <= e1) {
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(x + e0 + 4 * (threadIdx.x + kThreads * j));
      v[4 * j + 0] = f.x * inv_t;
      v[4 * j + 1] = f.y * inv_t;
      v[4 * j + 2] = f.z * inv_t;
      v[4 * j + 3] = f.w * inv_t;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = e0 + threadIdx.x + kThreads * j;
      v[j] = idx < e1 ? x[idx] * inv_t : kNegInf;
    }
  }
}

// The three sampler kernels take the fields their first loads need as
// leading scalar arguments, which the dispatch preloads into scalar registers
// (this file is built with kernel-argument preloading): the logit, draft and
// statistics loads then go out without first waiting for the argument block.
// a_k_nch packs k | nchunks << 16 (k <= 128, nchunks <= 1024).
__device__ __forceinline__ const float* row_ptr_a(const float* ar, const float* diff, int k, int V, int b, int rr) {
  return rr <= k ? ar + ((size_t)b * (k + 1) + rr) * V : diff + ((size_t)b * k + (rr - k - 1)) * V;
}

__global__ __launch_bounds__(kThreads) void rej_stats_kernel(const float* __restrict__ a_ar,
                                                             const float* __restrict__ a_diff, int a_V,
                                                             uint32_t a_k_nch, int a_mix, float a_inv_t, float a_lam,
                                                             float a_mu, RejectParams p) {
  __shared__ float red[4];
  const int k = (int)(a_k_nch & 0xffff), nch = (int)(a_k_nch >> 16);
  const int c = blockIdx.x % nch;
  const int row = blockIdx.x / nch;
  const int nrows = 2 * k + 1;
  const int b = row / nrows, rr = row % nrows;
  const bool target = rr < k;  // a verification target (not the bonus row)
  const float* x = row_ptr_a(a_ar, a_diff, k, a_V, b, target && a_mix == 2 ? k + 1 + rr : rr);
  const int e0 = c * kChunk, e1 = min(e0 + kChunk, a_V);
  const bool vec4 = (a_V & 3) == 0;
  float v[kPer];
  if (target && a_mix == 1) {
    // mixed target: (lam * a + mu * d) / T, formed exactly as in the draws
    float w[kPer];
    load_chunk(x, e0, e1, 1.f, vec4, v);
    load_chunk(row_ptr_a(a_ar, a_diff, k, a_V, b, k + 1 + rr), e0, e1, 1.f, vec4, w);
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = fmaf(a_lam, v[j], a_mu * w[j]) * a_inv_t;
  } else {
    load_chunk(x, e0, e1, a_inv_t, vec4, v);
  }
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < kPer; ++j) mx = fmaxf(mx, v[j]);
  mx = block_max(mx, red);
  float s = 0.f;
  if (mx != kNegInf) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) s += expf(v[j] - mx);
  }
  s = block_sumf(s, red);
  if (threadIdx.x == 0) p.row_stats[((size_t)b * nrows + rr) * nch + c] = make_float2(mx, s);
}

// The mixed logit of a verification target (mix == 1), as rej_stats forms it.
__device__ __forceinline__ float mix_logit(const RejectParams& p, float a, float d) {
  return fmaf(p.lam, a, p.mu * d);
}

// Weight of token t for the final draw: residual max(0, p_n - q_n) after a
// rejection, p_k for the bonus draw, p_n for the all-zero-residual fallback.
// Probabilities are evaluated as 2^(y * s - m * log2 e) / z from the merged
// row statistics (m, z) of the temperature-scaled logits, y being the
// target's logit (AR, mixed, or diffusion; the bonus row is always AR).
struct DrawRows {
  const float* a;  // AR row (unused when the target is the diffusion row)
  const float* q;  // diffusion row of the same position, or nullptr for the bonus draw
  bool sub;        // subtract q: the residual after a rejection
  int mix;         // target logits: 0 = a, 1 = lam * a + mu * q, 2 = q
  float lam, mu;
  float s;         // log2(e) / T
  float ba, ra;    // m_target * log2(e), 1 / z_target
  float bq, rq;
  __device__ __forceinline__ void init(const RejectParams& p, int b, int n, const float2* mz) {
    const float l2e = 1.4426950408889634f;
    const int k = p.k;
    a = row_ptr(p, b, n);
    q = n < k ? row_ptr(p, b, k + 1 + n) : nullptr;
    sub = n < k;
    mix = n < k ? p.mix : 0;
    lam = p.lam;
    mu = p.mu;
    s = p.inv_temp * l2e;
    const float2 sa = mz[n], sq = n < k ? mz[k + 1 + n] : make_float2(0.f, 1.f);
    ba = sa.x * l2e;
    ra = 1.f / sa.y;
    bq = q ? sq.x * l2e : 0.f;
    rq = q ? 1.f / sq.y : 0.f;
  }
  __device__ __forceinline__ bool needs_a() const { return mix != 2; }
  __device__ __forceinline__ float target(float xa, float xq) const {
    return mix == 0 ? xa : mix == 2 ? xq : fmaf(lam, xa, mu * xq);
  }
  __device__ __forceinline__ float pt(float y) const { return __builtin_amdgcn_exp2f(fmaf(y, s, -ba)) * ra; }
  __device__ __forceinline__ float pq(float x) const { return __builtin_amdgcn_exp2f(fmaf(x, s, -bq)) * rq; }
};

// Merge the per-chunk statistics of row rr across one wave: lane l takes
// chunks l, l + 64, ... (a fixed order, so the result is deterministic).
__device__ __forceinline__ float2 merge_row_wave(const RejectParams& p, int b, int rr, int lane) {
  const float2* st = p.row_stats + ((size_t)b * (2 * p.k + 1) + rr) * p.nchunks;
  float m = kNegInf;
  for (int c = lane; c < p.nchunks; c += 64) m = fmaxf(m, st[c].x);
  m = wave_max(m);
  float z = 0.f;
  if (m != kNegInf)
    for (int c = lane; c < p.nchunks; c += 64)
      if (st[c].x != kNegInf) z += st[c].y * expf(st[c].x - m);
  return make_float2(m, wave_sumf(z));
}

// Merge the staged per-chunk statistics of every row at once: kGroup lanes
// per row, lane j of a group taking chunks j, j + kGroup, ... (a fixed order,
// so the result is deterministic). Returns the row's (max, sum exp) in the
// group's lane 0 for row `rr` (rr >= nrows: no row).
constexpr int kGroup = 8;
__device__ __forceinline__ float2 merge_row_group(const float2* st, int nchunks, int rr, int nrows, int gl) {
  float m = kNegInf;
  if (rr < nrows)
    for (int c = gl; c < nchunks; c += kGroup) m = fmaxf(m, st[rr * nchunks + c].x);
#pragma unroll
  for (int o = kGroup / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kGroup));
  float z = 0.f;
  if (rr < nrows && m != kNegInf)
    for (int c = gl; c < nchunks; c += kGroup) {
      const float2 v = st[rr * nchunks + c];
      if (v.x != kNegInf) z += v.y * expf(v.x - m);
    }
#pragma unroll
  for (int o = kGroup / 2; o > 0; o >>= 1) z += __shfl_xor(z, o, kGroup);
  return make_float2(m, z);
}

// Inclusive prefix sum over the block in thread order (fp64); `tot` gets the
// block total. Uses red[0..3].
__device__ __forceinline__ double block_scan_incl(double x, double* red, double* tot) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (l >= o) x += y;
  }
  __syncthreads();
  if (l == 63) red[w] = x;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += red[i];
  *tot = ((red[0] + red[1]) + red[2]) + red[3];
  return x + off;
}

__global__ __launch_bounds__(kThreads) void rej_resid_kernel(const int32_t* __restrict__ a_drafts,
                                                             const float* __restrict__ a_uni,
                                                             const float2* __restrict__ a_stats, uint32_t a_k_nch,
                                                             RejectParams p) {
  __shared__ float2 mz[2 * kMaxK + 1];
  __shared__ float2 st_lds[kStage];
  __shared__ float rho[kMaxK];
  __shared__ float uni[kMaxK];
  __shared__ int n_sh;
  __shared__ double redd[4];
  const int k = (int)(a_k_nch & 0xffff), nch = (int)(a_k_nch >> 16);
  const int c = blockIdx.x % nch, b = blockIdx.x / nch;
  const int nrows = 2 * k + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the draft tokens' logits are gathered first so their latency overlaps
  // the statistics merge
  const int i = threadIdx.x;
  int d = -1;
  float da = 0.f, dq = 0.f;  // logits of draft i under its target and diffusion rows
  if (i < k) {
    d = a_drafts[(size_t)b * k + i];
    uni[i] = a_uni[(size_t)b * (k + 1) + i];
    if (d >= 0 && d < p.V) {
      dq = row_ptr(p, b, k + 1 + i)[d];
      da = p.mix == 2 ? dq : row_ptr(p, b, i)[d];
      if (p.mix == 1) da = mix_logit(p, da, dq);  // the target's logit at the draft
    }
  }
  // per-row statistics: stage every (row, chunk) pair of this sequence in
  // LDS with one round of loads, then merge each row across one wave
  const int total = nrows * nch;
  if (total <= kStage) {
    const float2* g = a_stats + (size_t)b * total;
    float2 v[kStage / kThreads];
#pragma unroll
    for (int j = 0; j < kStage / kThreads; ++j) {
      const int t = threadIdx.x + kThreads * j;
      if (t < total) v[j] = g[t];
    }
#pragma unroll
    for (int j = 0; j < kStage / kThreads; ++j) {
      const int t = threadIdx.x + kThreads * j;
      if (t < total) st_lds[t] = v[j];
    }
    __syncthreads();
  }
  // each row merged by a group of kGroup lanes (all rows at once when the
  // statistics fit in LDS), else by one wave per row from global memory
  const bool staged = total <= kStage;
  const int nr_pass = staged ? kThreads / kGroup : kThreads / 64;
  for (int rr0 = 0; rr0 < nrows; rr0 += nr_pass) {
    const int rr = rr0 + (staged ? (int)threadIdx.x / kGroup : wave);
    const float2 v = staged ? merge_row_group(st_lds, p.nchunks, rr, nrows, threadIdx.x % kGroup)
                            : (rr < nrows ? merge_row_wave(p, b, rr, lane) : make_float2(0.f, 0.f));
    if (rr < nrows && (staged ? threadIdx.x % kGroup == 0 : lane == 0)) {
      mz[rr] = v;
      if (c == 0) p.row_mz[(size_t)b * nrows + rr] = v;
      if (!(isfinite(v.x) && v.y > 0.f && isfinite(v.y)) && c == 0 && p.dev_status) atomicOr(p.dev_status, 8);
    }
  }
  __syncthreads();
  if (i < k) {
    float r = 0.f;
    if (d < 0 || d >= p.V) {
      if (c == 0 && p.dev_status) atomicOr(p.dev_status, 16);
    } else {
      const float2 sa = mz[i], sq = mz[k + 1 + i];
      const float pa = expf(da * p.inv_temp - sa.x) / sa.y;
      const float pq = expf(dq * p.inv_temp - sq.x) / sq.y;
      r = pq > 0.f ? pa / pq : INFINITY;
    }
    rho[i] = r;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < k && uni[n] < fminf(1.f, rho[n])) ++n;
    n_sh = n;
  }
  __syncthreads();
  const int n = n_sh;
  if (c == 0) {
    for (int i = threadIdx.x; i < k; i += kThreads)
      if (p.ratio) p.ratio[(size_t)b * k + i] = rho[i];
    if (threadIdx.x == 0) {
      p.accept_len[b] = n;
      p.decision[2 * b] = n;
      p.decision[2 * b + 1] = 0;
    }
  }
  DrawRows dr;
  dr.init(p, b, n, mz);
  // per chunk: mass of the draw distribution, and of p_n alone (the
  // fallback when the residual vanishes through rounding)
  const int e0 = c * kChunk, e1 = min(e0 + kChunk, p.V);
  float xa[kPer], xq[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int t = min(e0 + threadIdx.x + kThreads * j, e1 - 1);
    xa[j] = dr.needs_a() ? dr.a[t] : 0.f;
    xq[j] = dr.q ? dr.q[t] : 0.f;
  }
  double acc = 0.0, acc_a = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (e0 + (int)threadIdx.x + kThreads * j < e1) {
      const float pt = dr.pt(dr.target(xa[j], xq[j]));
      const float w = dr.sub ? fmaxf(0.f, pt - dr.pq(xq[j])) : pt;
      acc += (double)w;
      acc_a += (double)pt;
    }
  }
  acc = block_sumd(acc, redd);
  acc_a = block_sumd(acc_a, redd);
  if (threadIdx.x == 0) {
    p.resid_sums[(size_t)b * p.nchunks + c] = acc;
    p.resid_sums[((size_t)p.B + b) * p.nchunks + c] = acc_a;
  }
}

__global__ __launch_bounds__(kThreads) void rej_pick_kernel(const int32_t* __restrict__ a_decision,
                                                            const double* __restrict__ a_sums, uint32_t a_k_nch,
                                                            int a_B, RejectParams p) {
  __shared__ double red[4];
  __shared__ double sums[kMaxChunks];
  __shared__ int pick_c, last_c, first_t, last_t;
  __shared__ double pick_base;
  const int k = (int)(a_k_nch & 0xffff), nch = (int)(a_k_nch >> 16);
  const int b = blockIdx.x, nrows = 2 * k + 1;
  // thread t owns chunks [cpt*t, cpt*t + cpt)
  const int cpt = (nch + kThreads - 1) / kThreads;
  const int c0 = cpt * threadIdx.x, c1 = min(c0 + cpt, nch);
  double mine = 0.0;
  for (int c = c0; c < c1; ++c) mine += (sums[c] = a_sums[(size_t)b * nch + c]);
  const int n = a_decision[2 * b];
  DrawRows dr;
  dr.init(p, b, n, p.row_mz + (size_t)b * nrows);
  double total;
  double incl = block_scan_incl(mine, red, &total);
  if (!(total > 0.0)) {
    // the residual vanished through rounding: draw from p_n instead
    dr.sub = false;
    mine = 0.0;
    for (int c = c0; c < c1; ++c) mine += (sums[c] = a_sums[((size_t)a_B + b) * nch + c]);
    incl = block_scan_incl(mine, red, &total);
  }
  const double target = (double)p.uniforms[(size_t)b * (k + 1) + k] * total;
  if (threadIdx.x == 0) {
    pick_c = 0x7fffffff;
    last_c = -1;
    first_t = 0x7fffffff;
    last_t = -1;
  }
  __syncthreads();
  // first chunk whose running mass passes the target; last chunk with mass
  // (the fallback when rounding leaves the target at the total)
  {
    double run = incl - mine;
    int mf = 0x7fffffff, ml = -1;
    for (int c = c0; c < c1; ++c) {
      if (sums[c] > 0.0) ml = c;
      if (mf == 0x7fffffff && run + sums[c] > target) mf = c;
      run += sums[c];
    }
    // one LDS atomic per wave (per-thread atomics on one word serialise)
    mf = wave_min_i(mf);
    ml = wave_max_i(ml);
    if ((threadIdx.x & 63) == 0) {
      if (mf != 0x7fffffff) atomicMin(&pick_c, mf);
      if (ml >= 0) atomicMax(&last_c, ml);
    }
  }
  __syncthreads();
  const int cp = pick_c != 0x7fffffff ? pick_c : max(last_c, 0);
  if (threadIdx.x == 0) {
    double base = 0.0;
    for (int c = 0; c < cp; ++c) base += sums[c];
    pick_base = base;
  }
  // inverse CDF inside the chosen chunk: thread t owns kPer consecutive tokens
  const int e0 = cp * kChunk, e1 = min(e0 + kChunk, p.V);
  float w[kPer], xq[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int t = min(e0 + (int)threadIdx.x * kPer + j, e1 - 1);
    w[j] = dr.needs_a() ? dr.a[t] : 0.f;
    xq[j] = dr.q ? dr.q[t] : 0.f;
  }
  double tsum = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const float pt = dr.pt(dr.target(w[j], xq[j]));
    w[j] = e0 + (int)threadIdx.x * kPer + j < e1 ? (dr.sub ? fmaxf(0.f, pt - dr.pq(xq[j])) : pt) : 0.f;
    tsum += (double)w[j];
  }
  double ctot;
  double run = block_scan_incl(tsum, red, &ctot) - tsum;  // its barriers also publish pick_base
  run += pick_base;
  int mine_first = 0x7fffffff, mine_last = -1;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int t = e0 + (int)threadIdx.x * kPer + j;
    run += (double)w[j];
    if (t < e1) {
      if (run > target && mine_first == 0x7fffffff) mine_first = t;
      if (w[j] > 0.f) mine_last = t;
    }
  }
  mine_first = wave_min_i(mine_first);
  mine_last = wave_max_i(mine_last);
  if ((threadIdx.x & 63) == 0) {
    if (mine_first != 0x7fffffff) atomicMin(&first_t, mine_first);
    if (mine_last >= 0) atomicMax(&last_t, mine_last);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.next_token[b] = first_t != 0x7fffffff ? first_t : max(last_t, 0);
}

}  // namespace

size_t reject_workspace_bytes(int B, int k, int V) {
  const size_t nchunks = ((size_t)V + kChunk - 1) / kChunk;
  size_t bytes = 0;
  bytes += ((size_t)B * (2 * k + 1) * nchunks * sizeof(float2) + 255) / 256 * 256;
  bytes += ((size_t)2 * B * nchunks * sizeof(double) + 255) / 256 * 256;
  bytes += ((size_t)B * 2 * sizeof(int32_t) + 255) / 256 * 256;
  bytes += ((size_t)B * (2 * k + 1) * sizeof(float2) + 255) / 256 * 256;
  return bytes;
}

void plan_reject(RejectParams& p) {
  p.chunk = kChunk;
  p.nchunks = (int)(((long)p.V + kChunk - 1) / kChunk);
}

int reject_max_k() { return kMaxK; }
int reject_max_chunks() { return kMaxChunks; }

hipError_t launch_reject(const RejectParams& p, hipStream_t stream) {
  const unsigned stats_grid = (unsigned)((size_t)p.nchunks * p.B * (2 * p.k + 1));
  const uint32_t k_nch = (uint32_t)p.k | ((uint32_t)p.nchunks << 16);
  hipLaunchKernelGGL(rej_stats_kernel, dim3(stats_grid), dim3(kThreads), 0, stream, p.ar, p.diff, p.V, k_nch, p.mix,
                     p.inv_temp, p.lam, p.mu, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rej_resid_kernel, dim3((unsigned)((size_t)p.nchunks * p.B)), dim3(kThreads), 0, stream, p.drafts,
                     p.uniforms, p.row_stats, k_nch, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rej_pick_kernel, dim3(p.B), dim3(kThreads), 0, stream, p.decision, p.resid_sums, k_nch, p.B, p);
  return hipGetLastError();
}

}  // namespace tidar
