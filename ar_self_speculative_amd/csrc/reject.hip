// AR rejection sampling of the diffusion drafts, fused with the vocab-wide
// softmax it needs (TiDAR review, awesome-system-papers wiki, 核心方法
// section 3.2; acceptance rule of speculative sampling, Leviathan et al. 2023
// and Chen et al. 2023: keep d_{i+1} with probability min(1, p_i/q_i), on the
// first rejection draw from normalised max(0, p_i - q_i), after k acceptances
// draw a bonus token from p_k).
//
// Two HBM-streaming launches, all with a fixed reduction order so results
// are run-to-run deterministic:
//   1. rej_stats : per (row, vocab chunk) max and sum of exp over the 2k+1
//                  logit rows of each sequence (one read of all logits),
//                  and the drafts' own logits, stored by the threads that
//                  hold them;
//   2. rej_draw  : every workgroup of a sequence merges the row statistics,
//                  evaluates the acceptance chain from the gathered p_i(d),
//                  q_i(d) (identical in all of them) and sums the residual
//                  (or bonus) weights of its vocab chunk, and p_n alone for
//                  the rounding fallback, in fp64; the last of them to
//                  finish locates the chunk whose running mass passes
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

#include <mutex>

namespace tidar {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;            // vocab elements per chunk = 16 per thread
constexpr int kPer = kChunk / kThreads;
constexpr int kMaxK = 128;
constexpr int kMaxChunks = 1024;
constexpr int kStage = 4096;            // (row, chunk) statistics staged in LDS per sequence
constexpr float kNegInf = -INFINITY;

// Cross-lane reductions and scans by DPP lane moves (register to register,
// no trip through the LDS unit as a shuffle takes). dpp<CTRL, ROWS, BANKS>(x,
// id): each lane's value from the lane that CTRL names; lanes outside the
// ROWS / BANKS masks, and lanes whose source lies outside their row, get id.
// CTRL: quad_perm (0x00-0xff), row_shr:n (0x110 + n), row_mirror (0x140),
// row_half_mirror (0x141), row_bcast:15 (0x142), row_bcast:31 (0x143).
template <int CTRL, int ROWS = 0xf, int BANKS = 0xf>
__device__ __forceinline__ float dpp(float x, float id) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), CTRL, ROWS, BANKS, false));
}
template <int CTRL, int ROWS = 0xf, int BANKS = 0xf>
__device__ __forceinline__ double dpp(double x, double id) {
  const long long v = __double_as_longlong(x), w = __double_as_longlong(id);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp((int)w, (int)v, CTRL, ROWS, BANKS, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp((int)(w >> 32), (int)(v >> 32), CTRL, ROWS, BANKS, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ float lane63(float x) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63)); }
__device__ __forceinline__ double lane63(double x) {
  const long long v = __double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)v, 63);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(v >> 32), 63);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Reduction over each aligned group of 8 lanes, the result in all 8: pairs
// (xor 1), quads (xor 2), then the two quads (mirror within the 8).
template <typename T, typename Op>
__device__ __forceinline__ T group8(T x, T id, Op op) {
  x = op(x, dpp<0xb1>(x, id));   // quad_perm [1,0,3,2]
  x = op(x, dpp<0x4e>(x, id));   // quad_perm [2,3,0,1]
  x = op(x, dpp<0x141>(x, id));  // row_half_mirror
  return x;
}
// Reduction over the wave, the result in every lane: groups of 8, rows of 16
// (mirror), then rows 0+1 into row 1 and 2+3 into row 3 (row_bcast:15), all
// four into row 3 (row_bcast:31), read from lane 63.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, T id, Op op) {
  x = group8(x, id, op);
  x = op(x, dpp<0x140>(x, id));
  x = op(x, dpp<0x142, 0xa>(x, id));
  x = op(x, dpp<0x143, 0xc>(x, id));
  return lane63(x);
}
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
__device__ __forceinline__ float wave_max(float x) { return wave_reduce(x, kNegInf, MaxOp()); }
__device__ __forceinline__ float wave_sumf(float x) { return wave_reduce(x, 0.f, AddOp()); }
__device__ __forceinline__ double wave_sumd(double x) { return wave_reduce(x, 0.0, AddOp()); }

// Inclusive prefix sum over the wave in lane order: within each row of 16 by
// right shifts of 1, 2, 3 (of the inputs), then 4 and 8 (of the partial
// sums, into the banks that have such a source), then across rows by the
// row broadcasts of lanes 15 and 31.
__device__ __forceinline__ double wave_scan_incl(double x) {
  const double x0 = x;
  x += dpp<0x111>(x0, 0.0);
  x += dpp<0x112>(x0, 0.0);
  x += dpp<0x113>(x0, 0.0);
  x += dpp<0x114, 0xf, 0xe>(x, 0.0);
  x += dpp<0x118, 0xf, 0xc>(x, 0.0);
  x += dpp<0x142, 0xa>(x, 0.0);
  x += dpp<0x143, 0xc>(x, 0.0);
  return x;
}

// Minimum over the wave of per-lane values that grow with the lane index
// wherever they are set (INT_MAX: not set): the value of the lowest lane that
// has one, found by ballot rather than a shuffle tree.
__device__ __forceinline__ int wave_first_i(int x) {
  const unsigned long long m = __ballot(x != 0x7fffffff);
  return m ? __builtin_amdgcn_readlane(x, (int)__builtin_ctzll(m)) : 0x7fffffff;
}
// Maximum of such values (-1: not set): the value of the highest lane with one.
__device__ __forceinline__ int wave_last_i(int x) {
  const unsigned long long m = __ballot(x >= 0);
  return m ? __builtin_amdgcn_readlane(x, 63 - (int)__builtin_clzll(m)) : -1;
}

// Two block sums at once, each with a fixed combination order (waves 0..3 in
// sequence). red holds 8 doubles.
__device__ __forceinline__ void block_sumd2(double& x, double& y, double* red) {
  x = wave_sumd(x);
  y = wave_sumd(y);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) {
    red[w] = x;
    red[4 + w] = y;
  }
  __syncthreads();
  x = ((red[0] + red[1]) + red[2]) + red[3];
  y = ((red[4] + red[5]) + red[6]) + red[7];
}

__device__ __forceinline__ const float* row_ptr(const RejectParams& p, int b, int rr) {
  // rows 0..k: AR logits (row i verifies d_{i+1}; row k is the bonus row);
  // rows k+1..2k: diffusion logits of drafts 0..k-1
  return rr <= p.k ? p.ar + ((size_t)b * (p.k + 1) + rr) * p.V
                   : p.diff + ((size_t)b * p.k + (rr - p.k - 1)) * p.V;
}

// The three sampler kernels take the fields their first loads need as
// leading scalar arguments, which the dispatch preloads into scalar registers
// (this file is built with kernel-argument preloading): the logit, draft and
// statistics loads then go out without first waiting for the argument block.
// a_k_nch packs k | nchunks << 16 (k <= 128, nchunks <= 1024).
__device__ __forceinline__ const float* row_ptr_a(const float* ar, const float* diff, int k, int V, int b, int rr) {
  return rr <= k ? ar + ((size_t)b * (k + 1) + rr) * V : diff + ((size_t)b * k + (rr - k - 1)) * V;
}

// Element `off` of a chunk (0 <= off < chunk length): the thread that holds
// it after load_chunk, and its index in that thread's kPer values.
__device__ __forceinline__ void chunk_owner(int off, bool vec, int& thread, int& slot) {
  if (vec) {
    const int j = off / (4 * kThreads), rem = off % (4 * kThreads);
    thread = rem / 4;
    slot = 4 * j + rem % 4;
  } else {
    thread = off % kThreads;
    slot = off / kThreads;
  }
}

// Statistics pass: each workgroup takes kPPW consecutive (row, chunk) pairs
// of one sequence and issues all their loads in straight-line code before
// any arithmetic (past-the-end elements load a valid address and are masked
// to -inf), so one memory round trip covers all of them. One pair per
// workgroup measured fastest (two or four per workgroup leave some CUs with
// twice the bytes of others at the Qwen3 vocabulary). Per pair: the
// maximum and the sum of exponentials of the temperature-scaled logits. The
// thread that holds a draft's token in a pair also stores that logit
// (scaled; the mixed one for a mixed target), so the accept chain needs no
// gather of its own. Workgroup 0 of each sequence clears that sequence's
// arrival counter for the draw pass that follows in stream order.
//
// MIX: how the targets of rows 0..k-1 are formed (0 AR, 1 mixed, 2
// diffusion); VEC: the vocabulary is a multiple of 4, so each thread loads
// float4s (element 4 * (thread + kThreads * j) + e of a chunk), else single
// floats (element thread + kThreads * j).
constexpr int kPPW = 1;

template <bool VEC>
__device__ __forceinline__ void load_chunk_masked(const float* x, int e0, int e1, float (&v)[kPer]) {
  if (VEC) {
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const int idx = e0 + 4 * ((int)threadIdx.x + kThreads * j);
      const float4 f = *reinterpret_cast<const float4*>(x + (idx < e1 ? idx : 0));
      v[4 * j + 0] = f.x;
      v[4 * j + 1] = f.y;
      v[4 * j + 2] = f.z;
      v[4 * j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = e0 + (int)threadIdx.x + kThreads * j;
      v[j] = x[idx < e1 ? idx : 0];
    }
  }
}

template <bool VEC>
__device__ __forceinline__ bool chunk_elem_valid(int e0, int e1, int j) {
  return VEC ? e0 + 4 * ((int)threadIdx.x + kThreads * (j / 4)) < e1 : e0 + (int)threadIdx.x + kThreads * j < e1;
}

template <int MIX, bool VEC>
__global__ __launch_bounds__(kThreads) void rej_stats_kernel(const float* __restrict__ a_ar,
                                                             const float* __restrict__ a_diff, int a_V,
                                                             uint32_t a_k_nch, float a_inv_t, float a_lam, float a_mu,
                                                             RejectParams p) {
  __shared__ float red[kThreads / 64][kPPW];
  const int k = (int)(a_k_nch & 0xffff), nch = (int)(a_k_nch >> 16);
  const int nrows = 2 * k + 1, npairs = nrows * nch;
  const int G = (npairs + kPPW - 1) / kPPW;
  const int b = blockIdx.x / G, g0 = (blockIdx.x % G) * kPPW;
  float v[kPPW][kPer];
  float w[MIX == 1 ? kPPW : 1][kPer];
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const int pair = min(g0 + pp, npairs - 1);  // a short last group repeats its last pair (not stored)
    const int rr = pair / nch, c = pair % nch;
    const bool target = rr < k;  // a verification target (not the bonus row)
    const int e0 = c * kChunk, e1 = min(e0 + kChunk, a_V);
    load_chunk_masked<VEC>(row_ptr_a(a_ar, a_diff, k, a_V, b, MIX == 2 && target ? k + 1 + rr : rr), e0, e1, v[pp]);
    // mixed target: the diffusion row of the same position (other rows load their own row again)
    if (MIX == 1)
      load_chunk_masked<VEC>(row_ptr_a(a_ar, a_diff, k, a_V, b, target ? k + 1 + rr : rr), e0, e1, w[pp]);
  }
  // keep the arithmetic below the loads: the scheduler would otherwise start
  // scaling the first values as they arrive, stalling the loads behind them
  __builtin_amdgcn_sched_barrier(0);
  // the draft proposed on each pair's row (-1: the bonus row, or past the end)
  int dsel[kPPW];
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const int pair = g0 + pp, rr = pair / nch;
    dsel[pp] = (pair < npairs && rr != k) ? p.drafts[(size_t)b * k + (rr < k ? rr : rr - k - 1)] : -1;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // scale (and mix) in the same order as the draws, mask past-the-end elements,
  // then the block maxima of the kPPW pairs (waves combined in a fixed order)
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const int pair = min(g0 + pp, npairs - 1);
    const int c = pair % nch;
    const bool mixed = MIX == 1 && pair / nch < k;
    const int e0 = c * kChunk, e1 = min(e0 + kChunk, a_V);
    float m = kNegInf;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      float x = v[pp][j];
      if (MIX == 1) x = mixed ? fmaf(a_lam, x, a_mu * w[pp][j]) : x;
      x *= a_inv_t;
      v[pp][j] = chunk_elem_valid<VEC>(e0, e1, j) ? x : kNegInf;
      m = fmaxf(m, v[pp][j]);
    }
    m = wave_max(m);
    if (lane == 0) red[wave][pp] = m;
  }
  __syncthreads();
  float mx[kPPW];
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) mx[pp] = fmaxf(fmaxf(red[0][pp], red[1][pp]), fmaxf(red[2][pp], red[3][pp]));
  // the drafts' logits, by the threads that hold them
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    const int pair = g0 + pp, rr = pair / nch, c = pair % nch;
    const int d = dsel[pp];
    const int e0 = c * kChunk, e1 = min(e0 + kChunk, a_V);
    if (d >= e0 && d < e1) {
      int t, slot;
      chunk_owner(d - e0, VEC, t, slot);
      if ((int)threadIdx.x == t) {
        float val = 0.f;
#pragma unroll
        for (int j = 0; j < kPer; ++j) val = j == slot ? v[pp][j] : val;
        const int i = rr < k ? rr : rr - k - 1;
        p.gathered[(size_t)b * 2 * k + (rr < k ? i : k + i)] = val;
      }
    }
  }
  if (g0 == 0 && threadIdx.x == 0) p.arrive[b] = 0;
  float sm[kPPW];
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp) {
    float s = 0.f;
    if (mx[pp] != kNegInf) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) s += expf(v[pp][j] - mx[pp]);
    }
    sm[pp] = wave_sumf(s);
  }
  __syncthreads();  // every wave has read the maxima
#pragma unroll
  for (int pp = 0; pp < kPPW; ++pp)
    if (lane == 0) red[wave][pp] = sm[pp];
  __syncthreads();
  if (threadIdx.x < kPPW && g0 + (int)threadIdx.x < npairs) {
    const int pp = threadIdx.x, pair = g0 + pp;
    float m = kNegInf, s = 0.f;
#pragma unroll
    for (int q = 0; q < kPPW; ++q)
      if (q == pp) {
        m = mx[q];
        s = ((red[0][q] + red[1][q]) + red[2][q]) + red[3][q];
      }
    p.row_stats[((size_t)b * nrows + pair / nch) * nch + pair % nch] = make_float2(m, s);
  }
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
  // sa, sq: merged (max, sum exp) of the target row n and of its diffusion row
  __device__ __forceinline__ void init(const RejectParams& p, int b, int n, float2 sa, float2 sq) {
    const float l2e = 1.4426950408889634f;
    const int k = p.k;
    a = row_ptr(p, b, n);
    q = n < k ? row_ptr(p, b, k + 1 + n) : nullptr;
    sub = n < k;
    mix = n < k ? p.mix : 0;
    lam = p.lam;
    mu = p.mu;
    s = p.inv_temp * l2e;
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
constexpr int kGroup = 8;  // the group8 reduction spans exactly 8 lanes
__device__ __forceinline__ float2 merge_row_group(const float2* st, int nchunks, int rr, int nrows, int gl) {
  float m = kNegInf;
  if (rr < nrows)
    for (int c = gl; c < nchunks; c += kGroup) m = fmaxf(m, st[rr * nchunks + c].x);
  m = group8(m, kNegInf, MaxOp());
  float z = 0.f;
  if (rr < nrows && m != kNegInf)
    for (int c = gl; c < nchunks; c += kGroup) {
      const float2 v = st[rr * nchunks + c];
      if (v.x != kNegInf) z += v.y * expf(v.x - m);
    }
  z = group8(z, 0.f, AddOp());
  return make_float2(m, z);
}

// The same merge with each lane's chunk statistics already in registers
// (lane j of a group holds chunks j, j + kGroup, ...; chunks past the end
// and rows past the last hold (-inf, 0)): the same order and arithmetic as
// merge_row_group, without a round of LDS reads per chunk.
constexpr int kRegChunks = 8;
__device__ __forceinline__ float2 merge_row_regs(const float2 (&v)[kRegChunks]) {
  float m = kNegInf;
#pragma unroll
  for (int j = 0; j < kRegChunks; ++j) m = fmaxf(m, v[j].x);
  m = group8(m, kNegInf, MaxOp());
  float z = 0.f;
  if (m != kNegInf)
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j)
      if (v[j].x != kNegInf) z += v[j].y * expf(v[j].x - m);
  z = group8(z, 0.f, AddOp());
  return make_float2(m, z);
}

// Inclusive prefix sum over the block in thread order (fp64); `tot` gets the
// block total. Uses red[0..3].
__device__ __forceinline__ double block_scan_incl(double x, double* red, double* tot) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  x = wave_scan_incl(x);
  __syncthreads();
  if (l == 63) red[w] = x;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += red[i];
  *tot = ((red[0] + red[1]) + red[2]) + red[3];
  return x + off;
}

// Token pick for sequence b, run by the last draw-pass workgroup of the
// sequence once every chunk's masses are visible: inverse CDF in token-id
// order, first over the chunk masses, then inside the chosen chunk.
__device__ __forceinline__ void pick_token(const RejectParams& p, int b, int k, int nch, DrawRows dr) {
  __shared__ double red[4];
  __shared__ double sums[kMaxChunks];
  __shared__ int pick_c, last_c, first_t, last_t;
  __shared__ double pick_base;
  // thread t owns chunks [cpt*t, cpt*t + cpt)
  const int cpt = (nch + kThreads - 1) / kThreads;
  const int c0 = cpt * threadIdx.x, c1 = min(c0 + cpt, nch);
  double* a_sums = p.resid_sums;
  double mine = 0.0;
  for (int c = c0; c < c1; ++c)
    mine += (sums[c] = __hip_atomic_load(a_sums + (size_t)b * nch + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  double total;
  double incl = block_scan_incl(mine, red, &total);
  if (!(total > 0.0)) {
    // the residual vanished through rounding: draw from p_n instead
    dr.sub = false;
    mine = 0.0;
    for (int c = c0; c < c1; ++c)
      mine += (sums[c] = __hip_atomic_load(a_sums + ((size_t)p.B + b) * nch + c, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
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
    mf = wave_first_i(mf);  // thread t's chunks follow thread t - 1's
    ml = wave_last_i(ml);
    if ((threadIdx.x & 63) == 0) {
      if (mf != 0x7fffffff) atomicMin(&pick_c, mf);
      if (ml >= 0) atomicMax(&last_c, ml);
    }
  }
  __syncthreads();
  const int cp = pick_c != 0x7fffffff ? pick_c : max(last_c, 0);
  // mass before the chosen chunk, summed by its owner in the order of the search above
  if (c0 <= cp && cp < c1) {
    double base = incl - mine;
    for (int c = c0; c < cp; ++c) base += sums[c];
    pick_base = base;
  }
  // inverse CDF inside the chosen chunk: thread t owns kPer consecutive tokens
  // (rows loaded unconditionally, as in the draw pass)
  const int e0 = cp * kChunk, e1 = min(e0 + kChunk, p.V);
  const int t0 = e0 + (int)threadIdx.x * kPer;
  const float* qrow = dr.q ? dr.q : dr.a;
  float w[kPer], xq[kPer];
  if ((p.V & 3) == 0) {
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const int off = t0 + 4 * j < e1 ? t0 + 4 * j : e0;
      const float4 fa = *reinterpret_cast<const float4*>(dr.a + off);
      const float4 fq = *reinterpret_cast<const float4*>(qrow + off);
      w[4 * j] = fa.x, w[4 * j + 1] = fa.y, w[4 * j + 2] = fa.z, w[4 * j + 3] = fa.w;
      xq[4 * j] = fq.x, xq[4 * j + 1] = fq.y, xq[4 * j + 2] = fq.z, xq[4 * j + 3] = fq.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = min(t0 + j, e1 - 1);
      w[j] = dr.a[t];
      xq[j] = qrow[t];
    }
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
  mine_first = wave_first_i(mine_first);  // thread t's tokens follow thread t - 1's
  mine_last = wave_last_i(mine_last);
  if ((threadIdx.x & 63) == 0) {
    if (mine_first != 0x7fffffff) atomicMin(&first_t, mine_first);
    if (mine_last >= 0) atomicMax(&last_t, mine_last);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.next_token[b] = first_t != 0x7fffffff ? first_t : max(last_t, 0);
}

__global__ __launch_bounds__(kThreads) void rej_draw_kernel(const int32_t* __restrict__ a_drafts,
                                                             const float* __restrict__ a_uni,
                                                             const float2* __restrict__ a_stats, uint32_t a_k_nch,
                                                             RejectParams p) {
  __shared__ float2 mz[2 * kMaxK + 1];
  __shared__ float2 st_lds[kStage];
  __shared__ int nw[kMaxK / 64];
  __shared__ int last_sh;
  __shared__ double redd[8];
  const int k = (int)(a_k_nch & 0xffff), nch = (int)(a_k_nch >> 16);
  const int c = blockIdx.x % nch, b = blockIdx.x / nch;
  const int nrows = 2 * k + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the drafts, their scaled logits under the target and diffusion rows
  // (stored by the statistics pass) and the uniforms: independent loads that
  // go out together with the statistics below
  const int i = threadIdx.x;
  int d = -1;
  float da = 0.f, dq = 0.f, u = 0.f;
  if (i < k) {
    d = a_drafts[(size_t)b * k + i];
    u = a_uni[(size_t)b * (k + 1) + i];
    da = p.gathered[(size_t)b * 2 * k + i];
    dq = p.gathered[(size_t)b * 2 * k + k + i];
  }
  const int total = nrows * nch;
  const auto put_row = [&](int rr, float2 v) {
    mz[rr] = v;
    if (!(isfinite(v.x) && v.y > 0.f && isfinite(v.y)) && c == 0 && p.dev_status) atomicOr(p.dev_status, 8);
  };
  // per-row statistics. Up to 64 rows of up to 64 chunks: every lane loads
  // its two rows' share straight into registers (one round of loads) and
  // kGroup lanes merge each row.
  if (nrows <= 2 * (kThreads / kGroup) && nch <= kGroup * kRegChunks) {
    const float2* g = a_stats + (size_t)b * total;
    const int gl = (int)threadIdx.x % kGroup, r0 = (int)threadIdx.x / kGroup, r1 = r0 + kThreads / kGroup;
    float2 v0[kRegChunks], v1[kRegChunks];
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const int cc = gl + kGroup * j;
      v0[j] = cc < nch && r0 < nrows ? g[r0 * nch + cc] : make_float2(kNegInf, 0.f);
      v1[j] = cc < nch && r1 < nrows ? g[r1 * nch + cc] : make_float2(kNegInf, 0.f);
    }
    const float2 m0 = merge_row_regs(v0), m1 = merge_row_regs(v1);
    if (gl == 0) {
      if (r0 < nrows) put_row(r0, m0);
      if (r1 < nrows) put_row(r1, m1);
    }
  } else {
    // larger shapes: stage every (row, chunk) pair of this sequence in LDS with
    // one round of loads when they fit, then merge each row across kGroup
    // lanes; else one wave per row from global memory
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
    const bool staged = total <= kStage;
    const int nr_pass = staged ? kThreads / kGroup : kThreads / 64;
    for (int rr0 = 0; rr0 < nrows; rr0 += nr_pass) {
      const int rr = rr0 + (staged ? (int)threadIdx.x / kGroup : wave);
      const float2 v = staged ? merge_row_group(st_lds, p.nchunks, rr, nrows, threadIdx.x % kGroup)
                              : (rr < nrows ? merge_row_wave(p, b, rr, lane) : make_float2(0.f, 0.f));
      if (rr < nrows && (staged ? threadIdx.x % kGroup == 0 : lane == 0)) put_row(rr, v);
    }
  }
  __syncthreads();
  // thread i < k: the ratio p_i(d) / q_i(d) and whether d_{i+1} is rejected
  // (u_i >= min(1, ratio)); the accept length n is the first rejection, found
  // by ballot (k <= 128: waves 0 and 1), or k
  bool rej = false;
  if (i < k) {
    float r = 0.f;
    if (d < 0 || d >= p.V) {
      if (c == 0 && p.dev_status) atomicOr(p.dev_status, 16);
    } else {
      const float2 sa = mz[i], sq = mz[k + 1 + i];
      const float pa = expf(da - sa.x) / sa.y;
      const float pq = expf(dq - sq.x) / sq.y;
      r = pq > 0.f ? pa / pq : INFINITY;
    }
    rej = !(u < fminf(1.f, r));
    if (c == 0 && p.ratio) p.ratio[(size_t)b * k + i] = r;
  }
  const unsigned long long rb = __ballot(rej);
  if (wave < kMaxK / 64 && lane == 0) nw[wave] = rb ? wave * 64 + (int)__builtin_ctzll(rb) : k;
  __syncthreads();
  int n = k;
#pragma unroll
  for (int w = 0; w < kMaxK / 64; ++w) n = min(n, nw[w]);
  if (c == 0 && threadIdx.x == 0) p.accept_len[b] = n;
  DrawRows dr;
  dr.init(p, b, n, mz[n], n < k ? mz[k + 1 + n] : make_float2(0.f, 1.f));
  // per chunk: mass of the draw distribution, and of p_n alone (the
  // fallback when the residual vanishes through rounding)
  const int e0 = c * kChunk, e1 = min(e0 + kChunk, p.V);
  // both rows loaded unconditionally (the bonus draw has no diffusion row and
  // reads its AR row twice; a diffusion target reads the unused AR row)
  const float* qrow = dr.q ? dr.q : dr.a;
  float xa[kPer], xq[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int t = min(e0 + (int)threadIdx.x + kThreads * j, e1 - 1);
    xa[j] = dr.a[t];
    xq[j] = qrow[t];
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
  block_sumd2(acc, acc_a, redd);
  // Publish this chunk's masses; the last of the sequence's workgroups to
  // arrive sees all of them and draws the token. The masses are stored at
  // device scope (written through this XCD's L2), and the arrival count goes
  // out once those stores are complete: no release fence, which would write
  // back the XCD's whole L2 in every workgroup. Only the drawing workgroup
  // acquires, and it reads the masses with device-scope loads.
  if (threadIdx.x == 0) {
    __hip_atomic_store(p.resid_sums + (size_t)b * nch + c, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.resid_sums + ((size_t)p.B + b) * nch + c, acc_a, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): both stores are complete
    const int prev = __hip_atomic_fetch_add(p.arrive + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_sh = prev == nch - 1;
  }
  __syncthreads();
  if (!last_sh) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  pick_token(p, b, k, nch, dr);
}

}  // namespace

// Scratch of the allocation-free entry point: the sampler's workspace (per
// (row, chunk) statistics, per-chunk draw masses, arrival counters, the
// drafts' gathered logits) lives in this file-scope device array instead of a caller
// buffer. Each GPU holds its own copy for the life of the process. Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in); it passes the device address hipGetSymbolAddress returns,
// looked up once per device with that device current.
}  // namespace tidar

static __device__ __align__(256) unsigned char scratch[tidar::kRejectScratchBytes];

namespace tidar {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t reject_scratch(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

size_t reject_workspace_bytes(int B, int k, int V) {
  const size_t nchunks = ((size_t)V + kChunk - 1) / kChunk;
  size_t bytes = 0;
  bytes += ((size_t)B * (2 * k + 1) * nchunks * sizeof(float2) + 255) / 256 * 256;  // row_stats
  bytes += ((size_t)2 * B * nchunks * sizeof(double) + 255) / 256 * 256;            // resid_sums
  bytes += ((size_t)B * sizeof(int32_t) + 255) / 256 * 256;                          // arrive
  bytes += ((size_t)B * 2 * k * sizeof(float) + 255) / 256 * 256;                    // gathered
  return bytes;
}

void plan_reject(RejectParams& p) {
  p.chunk = kChunk;
  p.nchunks = (int)(((long)p.V + kChunk - 1) / kChunk);
}

int reject_max_k() { return kMaxK; }
int reject_max_chunks() { return kMaxChunks; }

hipError_t launch_reject(const RejectParams& p, hipStream_t stream) {
  const unsigned stats_grid =
      (unsigned)((size_t)p.B * (((size_t)(2 * p.k + 1) * p.nchunks + kPPW - 1) / kPPW));
  const uint32_t k_nch = (uint32_t)p.k | ((uint32_t)p.nchunks << 16);
  const bool vec = (p.V & 3) == 0;
#define TIDAR_STATS(MIX, VEC)                                                                                    \
  hipLaunchKernelGGL((rej_stats_kernel<MIX, VEC>), dim3(stats_grid), dim3(kThreads), 0, stream, p.ar, p.diff, p.V, \
                     k_nch, p.inv_temp, p.lam, p.mu, p)
  if (p.mix == 1) {
    if (vec) TIDAR_STATS(1, true); else TIDAR_STATS(1, false);
  } else if (p.mix == 2) {
    if (vec) TIDAR_STATS(2, true); else TIDAR_STATS(2, false);
  } else {
    if (vec) TIDAR_STATS(0, true); else TIDAR_STATS(0, false);
  }
#undef TIDAR_STATS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rej_draw_kernel, dim3((unsigned)((size_t)p.nchunks * p.B)), dim3(kThreads), 0, stream, p.drafts,
                     p.uniforms, p.row_stats, k_nch, p);
  return hipGetLastError();
}

}  // namespace tidar
