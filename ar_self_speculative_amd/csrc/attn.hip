// Hybrid-mask decode-step attention for gfx950 (MI355X).
//
// One TiDAR decode step attends, in one pass, from three query regions
// (TiDAR review, awesome-system-papers wiki, 核心方法 section 3.2): the k
// drafts of the previous step (causal over the prefix and each other) and one
// pre-draft block per accept length j (prefix + drafts d_1..d_j + its own
// block, bidirectional inside the block). The mask is evaluated from region
// indices; no mask tensor exists.
//
// bf16 path (the hot one): a workgroup owns 128 packed query rows of one
// (sequence, KV head) - the g query heads of the group share every K/V tile -
// and one split of the prefix keys. Scores are computed transposed,
// S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16, so each lane owns one query
// row and 16 keys per 32-key sub-tile: the row maximum is an in-lane max
// plus one half-wave swap (v_permlane32_swap), and the probabilities are
// already in the B-operand layout of the O^T = V^T . P^T product. K tiles are
// staged row-major in LDS, V tiles transposed. The prefix is split across
// workgroups; partial (max, sum, unnormalised output) triples are merged by
// log-sum-exp in a second kernel. The split that owns the last prefix keys
// also processes the step's own keys under the region predicate.
#include "tidar_internal.h"

#include <math.h>

#include <algorithm>

namespace tidar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // packed query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  // permlane32_swap exchanges the value between lane l and l^32; r[0] holds the
  // swapped-in value in this lane's copy and r[1] the original (for our use
  // both operands are x, so the pair is {x, partner} in some order).
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
}

// Visibility of step key c from a query row, given the row's (dlim, blo, bhi):
// drafts c < dlim, or the row's own pre-draft block [blo, bhi).
struct RowRule {
  int dlim, blo, bhi;
  __device__ __forceinline__ bool sees(int c) const { return c < dlim || (c >= blo && c < bhi); }
};

__device__ __forceinline__ RowRule row_rule(int r, int k, int block_len) {
  RowRule rr;
  if (r < k) {  // draft d_{r+1}: causal over the drafts, itself included
    rr.dlim = r + 1;
    rr.blo = 0;
    rr.bhi = 0;
  } else {      // block j = accept length j: drafts d_1..d_j plus its own block
    const int j = (r - k) / block_len;
    rr.dlim = j;
    rr.blo = k + j * block_len;
    rr.bhi = rr.blo + block_len;
  }
  return rr;
}

// Local key ranges needed by packed rows [m_lo, m_hi] (inclusive): drafts
// [0, dend) and the pre-draft blocks [blk_lo, blk_hi).
struct LocalRanges {
  int c0[2], c1[2];
  int n;
};

__device__ __forceinline__ LocalRanges local_ranges(int r_lo, int r_hi, int k, int bl) {
  int dend = 0;
  if (r_lo < k) dend = min(r_hi, k - 1) + 1;
  int blk_lo = 0, blk_hi = 0;
  if (r_hi >= k) {
    const int j_hi = (r_hi - k) / bl;
    dend = max(dend, j_hi);
    const int j_lo = (max(r_lo, k) - k) / bl;
    blk_lo = k + j_lo * bl;
    blk_hi = k + (j_hi + 1) * bl;
  }
  LocalRanges lr;
  lr.n = 0;
  if (blk_hi > blk_lo && blk_lo <= dend) {
    lr.c0[0] = 0;
    lr.c1[0] = max(dend, blk_hi);
    lr.n = 1;
  } else {
    if (dend > 0) { lr.c0[lr.n] = 0; lr.c1[lr.n] = dend; lr.n++; }
    if (blk_hi > blk_lo) { lr.c0[lr.n] = blk_lo; lr.c1[lr.n] = blk_hi; lr.n++; }
  }
  return lr;
}

__device__ __forceinline__ int remap_xcd(int i, int n) {
  // Workgroups are dealt to the 8 XCDs round-robin. Give each XCD a
  // contiguous range of work items so the query tiles that share a K/V chunk
  // run on the same XCD and hit its L2.
  const int n8 = n & ~7;
  return i < n8 ? (i & 7) * (n8 >> 3) + (i >> 3) : i;
}

template <int D>
struct BfTile {
  static constexpr int KSTR = D + 8;    // K row stride in LDS (elements), +16 B pad
  static constexpr int VSTR = kBN + 4;  // V^T row stride in LDS (elements), +8 B pad
};

// Stage one tile of up to kBN keys: K row-major, V transposed. Rows at or
// beyond nvalid are written as zeros so that no stale or invalid value can
// reach the MFMA (0 * NaN would poison the product).
template <int D>
__device__ __forceinline__ void stage_tile(const u16* __restrict__ ksrc, const u16* __restrict__ vsrc,
                                           size_t row_stride, int nvalid, u16* ks, u16* vt, int tid) {
  constexpr int KSTR = BfTile<D>::KSTR, VSTR = BfTile<D>::VSTR;
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int ITER = kBN * CPR / kThreads;
  static_assert(kBN * CPR % kThreads == 0, "tile does not divide");
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int c = tid + kThreads * it;
    const int key = c / CPR, dc = c % CPR;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < nvalid) val = *reinterpret_cast<const uint4*>(ksrc + key * row_stride + dc * 8);
    *reinterpret_cast<uint4*>(ks + key * KSTR + dc * 8) = val;
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int c = tid + kThreads * it;
    const int key = c % kBN, dc = c / kBN;        // lanes run along keys: conflict-free transposed stores
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < nvalid) val = *reinterpret_cast<const uint4*>(vsrc + key * row_stride + dc * 8);
    const u16* e = reinterpret_cast<const u16*>(&val);
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[(dc * 8 + j) * VSTR + key] = e[j];
  }
}

// Per-wave online-softmax state and the MFMA work on one staged tile.
template <int D>
struct WaveState {
  static constexpr int DSTEPS = D / 16;
  static constexpr int DT = D / 32;
  bf16x8 qf[DSTEPS];
  f32x16 o[DT];
  float mrow;  // running max, log2 domain
  float lrow;  // this lane's share of the running sum

  // MODE 0: all keys valid; 1: keys >= nvalid masked; 2: step keys under the region rule
  template <int MODE>
  __device__ __forceinline__ void tile(const u16* ks, const u16* vt, int lane, float scale_log2,
                                       int nvalid, int c_base, const RowRule& rule) {
    constexpr int KSTR = BfTile<D>::KSTR, VSTR = BfTile<D>::VSTR;
    const int l32 = lane & 31, half = lane >> 5;
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x16{};
      const u16* kr = ks + (32 * mt + l32) * KSTR + 8 * half;
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 16 * st);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[mt], 0, 0, 0);
      }
    }
    // s[mt][v] is the score of key 32*mt + 8*(v/4) + 4*half + (v%4) for this lane's row
    if (MODE != 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * mt + 8 * (v >> 2) + 4 * half + (v & 3);
          bool ok = kk < nvalid;
          if (MODE == 2) ok = ok && rule.sees(c_base + kk);
          if (!ok) s[mt][v] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[mt][v]);
    mx = half_max(mx);
    const float mnew = fmaxf(mrow, mx * scale_log2);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(mrow - muse);
    mrow = mnew;
    lrow *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    // probabilities, packed as the B operand of O^T = V^T P^T
    bf16x8 pb[4];
    float lsum = 0.f;
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
      const int mt = ks4 >> 1, vb = 8 * (ks4 & 1);
      f32x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[mt][vb + e], scale_log2, -muse));
        pv[e] = pe;
        lsum += pe;
      }
      pb[ks4] = __builtin_convertvector(pv, bf16x8);
    }
    lrow += lsum;
    // B-operand index 8*half + e of k-step ks4 is key 16*ks4 + 8*(e/4) + 4*half + (e%4);
    // the V^T operand must use the same key order.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u16* vr = vt + (32 * dt + l32) * VSTR + 4 * half;
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + 16 * ks4);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 16 * ks4 + 8);
        uint4 w4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 a = __builtin_bit_cast(bf16x8, w4);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks4], o[dt], 0, 0, 0);
      }
    }
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnParams p) {
  constexpr int KSTR = BfTile<D>::KSTR, VSTR = BfTile<D>::VSTR;
  constexpr int DSTEPS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) u16 ks[kBN * KSTR];
  __shared__ __attribute__((aligned(16))) u16 vt[D * VSTR];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, half = lane >> 5;

  int w = remap_xcd(blockIdx.x, gridDim.x);
  const int qt = w % p.qtiles;
  w /= p.qtiles;
  const int s = w % p.S;
  w /= p.S;
  const int kvh = w % p.Hkv;
  const int b = w / p.Hkv;

  int len = p.cache_len[b];
  if (len < 0 || len > p.max_len) {
    if (tid == 0 && p.dev_status) atomicOr(p.dev_status, 1);
    len = min(max(len, 0), p.max_len);
  }
  const bool last = (s == p.S - 1);
  const int kbeg = s * p.chunk;
  const int kend = last ? len : min(kbeg + p.chunk, len);

  const int M = p.R * p.g;
  const int m = qt * kBM + wave * 32 + l32;
  const bool row_ok = m < M;
  const int r = row_ok ? m / p.g : 0;
  const int h = kvh * p.g + (row_ok ? m - r * p.g : 0);
  const RowRule rule = row_rule(r, p.k, p.block_len);

  WaveState<D> st;
  {
    const u16* qp = reinterpret_cast<const u16*>(p.q) + ((size_t)(b * p.R + r) * p.Hq + h) * D + 8 * half;
#pragma unroll
    for (int i = 0; i < DSTEPS; ++i) {
      st.qf[i] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * i) : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < DT; ++i) st.o[i] = f32x16{};
    st.mrow = kNegInf;
    st.lrow = 0.f;
  }

  const size_t head_off = (size_t)(b * p.Hkv + kvh) * p.cap * D;
  const u16* kc = reinterpret_cast<const u16*>(p.k_cache) + head_off;
  const u16* vc = reinterpret_cast<const u16*>(p.v_cache) + head_off;

  for (int t0 = kbeg; t0 < kend; t0 += kBN) {
    const int nvalid = min(kBN, kend - t0);
    __syncthreads();
    stage_tile<D>(kc + (size_t)t0 * D, vc + (size_t)t0 * D, D, nvalid, ks, vt, tid);
    __syncthreads();
    if (nvalid == kBN)
      st.template tile<0>(ks, vt, lane, p.scale_log2, nvalid, 0, rule);
    else
      st.template tile<1>(ks, vt, lane, p.scale_log2, nvalid, 0, rule);
  }

  if (last) {
    const int m_lo = qt * kBM;
    const int m_hi = min(M, m_lo + kBM) - 1;
    const LocalRanges lr = local_ranges(m_lo / p.g, m_hi / p.g, p.k, p.block_len);
    const size_t step_stride = (size_t)p.Hkv * D;
    const u16* kst = reinterpret_cast<const u16*>(p.k_step) + ((size_t)b * p.R * p.Hkv + kvh) * D;
    const u16* vst = reinterpret_cast<const u16*>(p.v_step) + ((size_t)b * p.R * p.Hkv + kvh) * D;
    for (int seg = 0; seg < lr.n; ++seg) {
      for (int c0 = lr.c0[seg]; c0 < lr.c1[seg]; c0 += kBN) {
        const int nvalid = min(kBN, lr.c1[seg] - c0);
        __syncthreads();
        stage_tile<D>(kst + c0 * step_stride, vst + c0 * step_stride, step_stride, nvalid, ks, vt, tid);
        __syncthreads();
        st.template tile<2>(ks, vt, lane, p.scale_log2, nvalid, c0, rule);
      }
    }
  }

  // o[dt][v] holds O^T[d = 32*dt + 8*(v/4) + 4*half + v%4][this lane's row]
  const float ltot = half_sum(st.lrow);
  if (!row_ok) return;
  const size_t orow = ((size_t)(b * p.R + r) * p.Hq + h);
  if (p.S == 1) {
    const float inv = 1.f / ltot;
    u16* op = reinterpret_cast<u16*>(p.out) + orow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * half;
        ushort4 pk;
        pk.x = f32_to_bf16_bits(st.o[dt][4 * i + 0] * inv);
        pk.y = f32_to_bf16_bits(st.o[dt][4 * i + 1] * inv);
        pk.z = f32_to_bf16_bits(st.o[dt][4 * i + 2] * inv);
        pk.w = f32_to_bf16_bits(st.o[dt][4 * i + 3] * inv);
        *reinterpret_cast<ushort4*>(op + d) = pk;
      }
    if (p.lse && half == 0) p.lse[orow] = (st.mrow + log2f(ltot)) * 0.69314718055994531f;
  } else {
    const size_t prow = (size_t)s * p.B * p.R * p.Hq + orow;
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * half;
        *reinterpret_cast<float4*>(po + d) =
            make_float4(st.o[dt][4 * i + 0], st.o[dt][4 * i + 1], st.o[dt][4 * i + 2], st.o[dt][4 * i + 3]);
      }
    if (half == 0) *reinterpret_cast<float2*>(p.part_ml + prow * 2) = make_float2(st.mrow, ltot);
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per (packed query row, split). Plain VALU arithmetic in
// fp32 with an online softmax in the log2 domain; same split/merge scheme.
// ---------------------------------------------------------------------------
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

constexpr int kF32MaxD = 256;

__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
  __shared__ float qs[kF32MaxD];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int D = p.D;
  int w = blockIdx.x;
  const int M = p.R * p.g;
  const int m = w % M;
  w /= M;
  const int s = w % p.S;
  w /= p.S;
  const int kvh = w % p.Hkv;
  const int b = w / p.Hkv;
  const int r = m / p.g;
  const int h = kvh * p.g + (m - r * p.g);
  int len = p.cache_len[b];
  if (len < 0 || len > p.max_len) {
    if (lane == 0 && p.dev_status) atomicOr(p.dev_status, 1);
    len = min(max(len, 0), p.max_len);
  }
  const bool last = (s == p.S - 1);
  const int kbeg = s * p.chunk;
  const int kend = last ? len : min(kbeg + p.chunk, len);
  const RowRule rule = row_rule(r, p.k, p.block_len);

  const float* qrow = reinterpret_cast<const float*>(p.q) + ((size_t)(b * p.R + r) * p.Hq + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
  __syncthreads();

  float o[kF32MaxD / 64];
#pragma unroll
  for (int j = 0; j < kF32MaxD / 64; ++j) o[j] = 0.f;
  float mrow = kNegInf, lrow = 0.f;

  auto run = [&](const float* kb, const float* vb, size_t stride, int c0, int c1, bool local) {
    for (int t0 = c0; t0 < c1; t0 += 64) {
      const int c = t0 + lane;
      float sc = kNegInf;
      if (c < c1 && (!local || rule.sees(c))) {
        const float* kr = kb + (size_t)c * stride;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kr[d], acc);
        sc = acc * p.scale_log2;
      }
      const float mx = wave_max(sc);
      const float mnew = fmaxf(mrow, mx);
      const float muse = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = exp2f(mrow - muse);
      const float pe = exp2f(sc - muse);
      mrow = mnew;
      lrow = lrow * alpha + wave_sum(pe);
      __syncthreads();
      ps[lane] = pe;
      __syncthreads();
      const int n = min(64, c1 - t0);
#pragma unroll
      for (int j = 0; j < kF32MaxD / 64; ++j) {
        const int d = lane + 64 * j;
        if (d < D) {
          float acc = o[j] * alpha;
          for (int cc = 0; cc < n; ++cc) {
            const float pc = ps[cc];
            if (pc != 0.f) acc = fmaf(pc, vb[(size_t)(t0 + cc) * stride + d], acc);
          }
          o[j] = acc;
        }
      }
    }
  };

  const size_t head_off = (size_t)(b * p.Hkv + kvh) * p.cap * D;
  run(reinterpret_cast<const float*>(p.k_cache) + head_off, reinterpret_cast<const float*>(p.v_cache) + head_off,
      D, kbeg, kend, false);
  if (last) {
    const size_t stride = (size_t)p.Hkv * D;
    const float* kst = reinterpret_cast<const float*>(p.k_step) + ((size_t)b * p.R * p.Hkv + kvh) * D;
    const float* vst = reinterpret_cast<const float*>(p.v_step) + ((size_t)b * p.R * p.Hkv + kvh) * D;
    const LocalRanges lr = local_ranges(r, r, p.k, p.block_len);
    for (int seg = 0; seg < lr.n; ++seg) run(kst, vst, stride, lr.c0[seg], lr.c1[seg], true);
  }

  const size_t orow = ((size_t)(b * p.R + r) * p.Hq + h);
  if (p.S == 1) {
    const float inv = 1.f / lrow;
    float* op = reinterpret_cast<float*>(p.out) + orow * D;
#pragma unroll
    for (int j = 0; j < kF32MaxD / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < D) op[d] = o[j] * inv;
    }
    if (p.lse && lane == 0) p.lse[orow] = (mrow + log2f(lrow)) * 0.69314718055994531f;
  } else {
    const size_t prow = (size_t)s * p.B * p.R * p.Hq + orow;
#pragma unroll
    for (int j = 0; j < kF32MaxD / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < D) p.part_o[prow * D + d] = o[j];
    }
    if (lane == 0) *reinterpret_cast<float2*>(p.part_ml + prow * 2) = make_float2(mrow, lrow);
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials: m = max_s m_s,
// l = sum_s l_s 2^(m_s - m), O = sum_s o_s 2^(m_s - m) / l.
// One thread per 4 output elements of a row.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  const int D = p.D;
  const int tpr = D / 4;  // threads per row
  const size_t rows = (size_t)p.B * p.R * p.Hq;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t row = gid / tpr;
  const int d = (int)(gid % tpr) * 4;
  if (row >= rows) return;
  float mmax = kNegInf;
  for (int s = 0; s < p.S; ++s) mmax = fmaxf(mmax, p.part_ml[((size_t)s * rows + row) * 2]);
  const float muse = (mmax == kNegInf) ? 0.f : mmax;
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < p.S; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + ((size_t)s * rows + row) * 2);
    if (ml.y == 0.f) continue;
    const float wgt = exp2f(ml.x - muse);
    l += ml.y * wgt;
    const float4 o = *reinterpret_cast<const float4*>(p.part_o + ((size_t)s * rows + row) * D + d);
    acc.x = fmaf(o.x, wgt, acc.x);
    acc.y = fmaf(o.y, wgt, acc.y);
    acc.z = fmaf(o.z, wgt, acc.z);
    acc.w = fmaf(o.w, wgt, acc.w);
  }
  const float inv = 1.f / l;
  if (BF16) {
    ushort4 pk;
    pk.x = f32_to_bf16_bits(acc.x * inv);
    pk.y = f32_to_bf16_bits(acc.y * inv);
    pk.z = f32_to_bf16_bits(acc.z * inv);
    pk.w = f32_to_bf16_bits(acc.w * inv);
    *reinterpret_cast<ushort4*>(reinterpret_cast<u16*>(p.out) + row * D + d) = pk;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * D + d) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (p.lse && d == 0) p.lse[row] = (mmax + log2f(l)) * 0.69314718055994531f;
}

hipError_t launch_merge(const AttnParams& p, bool bf16, hipStream_t stream) {
  const size_t threads = (size_t)p.B * p.R * p.Hq * (p.D / 4);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(attn_merge_kernel<true>, dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_merge_kernel<false>, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attn(int dtype, int B, int Hq, int Hkv, int D, int R, int max_len, int forced_splits) {
  AttnPlan pl{};
  const int g = Hq / Hkv;
  const long M = (long)R * g;
  long base;
  if (dtype == 1) {
    pl.bm = kBM;
    pl.qtiles = (int)((M + kBM - 1) / kBM);
    base = (long)B * Hkv * pl.qtiles;
  } else {
    pl.bm = 1;
    pl.qtiles = (int)M;
    base = (long)B * Hkv * M;
  }
  const int ntiles = (max_len + kBN - 1) / kBN;
  int S;
  if (forced_splits > 0) {
    S = forced_splits;
  } else {
    // Aim for about two resident workgroups per CU on the 256-CU part,
    // with at least two key tiles per split.
    const long target = 512;
    S = (int)((target + base - 1) / base);
    S = std::max(1, std::min(S, std::max(1, ntiles / 2)));
  }
  S = std::max(1, std::min(S, std::max(1, ntiles)));
  int chunk = ntiles > 0 ? ((ntiles + S - 1) / S) * kBN : kBN;
  S = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  pl.S = S;
  pl.chunk = chunk;
  pl.ws_bytes = S > 1 ? (size_t)S * B * R * Hq * (size_t)(D + 2) * sizeof(float) + 256 : 0;
  return pl;
}

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.B * p.Hkv * p.qtiles * p.S);
  if (p.D == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.D == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, p);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  return launch_merge(p, true, stream);
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.B * p.Hkv * (size_t)p.R * p.g * p.S);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(grid), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  return launch_merge(p, false, stream);
}

}  // namespace tidar
