// Exact-KV commit after verification (TiDAR review, awesome-system-papers
// wiki, 核心方法 section 3.2: surplus draft KV is evicted without
// recomputation; talk notes on notes.yuuk.io, 厳密 KV キャッシュ対応).
//
// The accepted drafts are always a prefix d_1..d_n of the step's draft rows,
// so committing them is one contiguous ragged copy per (layer, sequence, KV
// head): step rows 0..n-1 go to cache rows len_in .. len_in+n-1. Rejected
// draft rows and pre-draft rows are simply never written. The accept length
// is read on the device, so the sampler's output feeds this kernel with no
// host round trip.
#include "tidar_internal.h"

namespace tidar {
namespace {

// Each workgroup loads the first kCommitThreads 16-byte pieces of its
// (layer, sequence, KV head)'s k candidate draft rows together with the
// accept length, and stores those among the first n rows: the row loads need
// not wait for the accept length (one memory round trip instead of two).
// Pieces past n are read and dropped; pieces past the first kCommitThreads
// (k * head_dim * elem_bytes > kCommitThreads * 16) are copied once n is known.
constexpr int kCommitThreads = 256;

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(CommitParams p) {
  int idx = blockIdx.x;
  const int h = idx % p.Hkv;
  idx /= p.Hkv;
  const int b = idx % p.B;
  const int l = idx / p.B;

  const size_t row_bytes = (size_t)p.D * p.elem_bytes;
  const int cpr = (int)(row_bytes / 16);  // 16-byte chunks per row
  const size_t src0 = ((((size_t)l * p.B + b) * p.step_rows) * p.Hkv + h) * row_bytes;
  const size_t src_row_stride = (size_t)p.Hkv * row_bytes;
  const char* ks = reinterpret_cast<const char*>(p.k_step);
  const char* vs = reinterpret_cast<const char*>(p.v_step);
  char* kc = reinterpret_cast<char*>(p.k_cache);
  char* vc = reinterpret_cast<char*>(p.v_cache);
  // this thread's candidate piece first: its address does not depend on the accept length
  const int c = threadIdx.x;
  const int total = p.k * cpr;
  uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
  if (c < total) {
    const size_t so = src0 + (size_t)(c / cpr) * src_row_stride + (size_t)(c % cpr) * 16;
    kr = *reinterpret_cast<const uint4*>(ks + so);
    vr = *reinterpret_cast<const uint4*>(vs + so);
  }

  const int n = p.accept_len[b];
  const int start = p.len_in[b];
  bool ok = true;
  if (n < 0 || n > p.k) {
    ok = false;
    if (threadIdx.x == 0 && l == 0 && h == 0 && p.dev_status) atomicOr(p.dev_status, 2);
  } else if (start < 0 || start + n > p.cap) {
    ok = false;
    if (threadIdx.x == 0 && l == 0 && h == 0 && p.dev_status) atomicOr(p.dev_status, 4);
  }
  if (l == 0 && h == 0 && threadIdx.x == 0) p.len_out[b] = ok ? start + n : start;
  if (!ok) return;

  const size_t dst0 = ((((size_t)l * p.B + b) * p.Hkv + h) * p.cap + start) * row_bytes;
  const int keep = n * cpr;
  if (c < keep) {
    const size_t d0 = dst0 + (size_t)(c / cpr) * row_bytes + (size_t)(c % cpr) * 16;
    *reinterpret_cast<uint4*>(kc + d0) = kr;
    *reinterpret_cast<uint4*>(vc + d0) = vr;
  }
  for (int cc = kCommitThreads + threadIdx.x; cc < keep; cc += kCommitThreads) {
    const int i = cc / cpr, q = cc % cpr;
    const size_t so = src0 + i * src_row_stride + (size_t)q * 16;
    const size_t d0 = dst0 + (size_t)i * row_bytes + (size_t)q * 16;
    *reinterpret_cast<uint4*>(kc + d0) = *reinterpret_cast<const uint4*>(ks + so);
    *reinterpret_cast<uint4*>(vc + d0) = *reinterpret_cast<const uint4*>(vs + so);
  }
}

}  // namespace

hipError_t launch_kv_commit(const CommitParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.L * p.B * p.Hkv);
  hipLaunchKernelGGL(kv_commit_kernel, dim3(grid), dim3(kCommitThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tidar
