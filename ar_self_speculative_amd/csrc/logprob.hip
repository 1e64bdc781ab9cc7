// Per-token AR log-likelihood for TiDAR's likelihood mode (talk notes on
// notes.yuuk.io, 尤度評価: with the attention mask set to causal, the model
// scores a sequence as an AR model in one forward, without Monte-Carlo
// sampling; review on the awesome-system-papers wiki, 实验与结果: one NFE
// with a pure causal mask). The causal forward is the attention's
// append-prefill mode (num_blocks = 0); this file turns its logits into
// log p(x_{t+1} | x_<=t) = logits[t, x_{t+1}] - log sum_v exp(logits[t, v]).
//
// Two HBM-streaming launches with a fixed reduction order (run-to-run
// deterministic):
//   1. lp_stats : per (row, 4096-token chunk) maximum and sum of exp;
//   2. lp_final : one wave per row merges its chunks in chunk order, gathers
//                 the target's logit and writes the log-probability.
#include "tidar_internal.h"

#include <math.h>

namespace tidar {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;
constexpr int kPer = kChunk / kThreads;
constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(kThreads) void lp_stats_kernel(LogprobParams p) {
  __shared__ float red[4];
  const int c = blockIdx.x % p.nchunks;
  const size_t row = blockIdx.x / p.nchunks;
  const float* x = p.logits + row * p.V;
  const int e0 = c * kChunk, e1 = min(e0 + kChunk, p.V);
  float v[kPer];
  if ((p.V & 3) == 0 && e0 + kChunk <= e1) {
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(x + e0 + 4 * (threadIdx.x + kThreads * j));
      v[4 * j] = f.x;
      v[4 * j + 1] = f.y;
      v[4 * j + 2] = f.z;
      v[4 * j + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = e0 + threadIdx.x + kThreads * j;
      v[j] = idx < e1 ? x[idx] : kNegInf;
    }
  }
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < kPer; ++j) mx = fmaxf(mx, v[j]);
  mx = wave_max(mx);
  if (l == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = 0.f;
  if (mx != kNegInf) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) s += expf(v[j] - mx);
  }
  s = wave_sum(s);
  __syncthreads();
  if (l == 0) red[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) p.stats[row * p.nchunks + c] = make_float2(mx, ((red[0] + red[1]) + red[2]) + red[3]);
}

__global__ __launch_bounds__(kThreads) void lp_final_kernel(LogprobParams p) {
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= (size_t)p.rows) return;
  const int t = p.targets[row];
  const float2* st = p.stats + row * p.nchunks;
  // merge the chunks: lane l takes chunks l, l + 64, ... (fixed order)
  float m = kNegInf;
  for (int c = lane; c < p.nchunks; c += 64) m = fmaxf(m, st[c].x);
  m = wave_max(m);
  float z = 0.f;
  if (m != kNegInf)
    for (int c = lane; c < p.nchunks; c += 64)
      if (st[c].x != kNegInf) z += st[c].y * expf(st[c].x - m);
  z = wave_sum(z);
  if (lane == 0) {
    float out = NAN;
    if (!(isfinite(m) && z > 0.f && isfinite(z))) {
      if (p.dev_status) atomicOr(p.dev_status, 8);
    } else if (t < 0 || t >= p.V) {
      if (p.dev_status) atomicOr(p.dev_status, 32);
    } else {
      out = p.logits[row * p.V + t] - (m + logf(z));
    }
    p.logprobs[row] = out;
  }
}

}  // namespace

size_t logprob_workspace_bytes(int rows, int V) {
  const size_t nchunks = ((size_t)V + kChunk - 1) / kChunk;
  return ((size_t)rows * nchunks * sizeof(float2) + 255) / 256 * 256;
}

int logprob_chunk() { return kChunk; }

hipError_t launch_logprob(const LogprobParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(lp_stats_kernel, dim3((unsigned)((size_t)p.rows * p.nchunks)), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lp_final_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tidar
