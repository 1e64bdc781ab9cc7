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
// already in the B-operand layout of the O^T = V^T . P^T product. K and V
// tiles are staged row-major in LDS; V fragments are read with the
// transposing ds_read_tr16_b64. The prefix is split across workgroups; each
// split stores its normalised output (in the input precision) and its
// log-sum-exp, and a second kernel merges them. The split that owns the last
// prefix keys also processes the step's own keys under the region predicate.
#include "tidar_internal.h"

#include <math.h>

#include <stdlib.h>

#include <algorithm>

namespace tidar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
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
  __device__ __forceinline__ bool sees(int c) const { return (c < dlim) | ((c >= blo) & (c < bhi)); }
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

// Local key ranges needed by packed rows whose step rows are r_lo..r_hi:
// drafts [0, dend) and the pre-draft blocks [blk_lo, blk_hi), merged into one
// range when they touch. n = number of ranges (0, 1 or 2).
struct LocalRanges {
  int a0, a1, b0, b1;
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
  LocalRanges lr{0, 0, 0, 0, 0};
  if (blk_hi > blk_lo && blk_lo <= dend) {
    lr.a1 = max(dend, blk_hi);
    lr.n = 1;
  } else if (dend > 0 && blk_hi > blk_lo) {
    lr.a1 = dend;
    lr.b0 = blk_lo;
    lr.b1 = blk_hi;
    lr.n = 2;
  } else if (dend > 0) {
    lr.a1 = dend;
    lr.n = 1;
  } else if (blk_hi > blk_lo) {
    lr.a0 = blk_lo;
    lr.a1 = blk_hi;
    lr.n = 1;
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

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0): loads at byte offsets >= bytes return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D>
struct Cfg {
  // K rows padded to 272 B (D=128): 16 consecutive rows start in distinct
  // 4-bank groups, so the 128-bit A-operand reads are conflict-free.
  static constexpr int KSTR = D + 8;
  // V rows padded to 320 B: the four rows read together by one transposing
  // ds_read_tr16_b64 land in disjoint 16-bank ranges.
  static constexpr int VSTR = D + 32;
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int LD_ITER = kBN * CPR / kThreads;   // chunks per thread per tile
  static constexpr int KBUF = kBN * KSTR;
  static constexpr int VBUF = kBN * VSTR;
  static_assert(kBN * CPR % kThreads == 0, "tile does not divide");
};

// Global -> register -> LDS staging of K and V tiles. Buffer loads return
// zero past the end of the valid range, so partial tiles (and prefetches past
// the last tile) need no branches, and no invalid value can reach the MFMAs
// (0 * NaN would poison them).
template <int D>
struct Stage {
  static constexpr int ROWS_PER_IT = kThreads / Cfg<D>::CPR;  // tile rows covered per load round
  uint4 k[Cfg<D>::LD_ITER], v[Cfg<D>::LD_ITER];

  // per-thread part of the byte offset; the row part goes in the scalar offset
  __device__ __forceinline__ static uint32_t voff(int tid, uint32_t row_bytes) {
    return (uint32_t)(tid / Cfg<D>::CPR) * row_bytes + (uint32_t)(tid % Cfg<D>::CPR) * 16u;
  }
  __device__ __forceinline__ static int lds_off(int tid, int stride) {
    return (tid / Cfg<D>::CPR) * stride + (tid % Cfg<D>::CPR) * 8;
  }
  __device__ __forceinline__ void load_k(__amdgpu_buffer_rsrc_t r, uint32_t vo, int row0, uint32_t row_bytes) {
#pragma unroll
    for (int it = 0; it < Cfg<D>::LD_ITER; ++it)
      k[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, vo, (row0 + it * ROWS_PER_IT) * row_bytes, 0));
  }
  __device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t r, uint32_t vo, int row0, uint32_t row_bytes) {
#pragma unroll
    for (int it = 0; it < Cfg<D>::LD_ITER; ++it)
      v[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, vo, (row0 + it * ROWS_PER_IT) * row_bytes, 0));
  }
  __device__ __forceinline__ void store_k(u16* ks, int lo) const {
#pragma unroll
    for (int it = 0; it < Cfg<D>::LD_ITER; ++it)
      *reinterpret_cast<uint4*>(ks + lo + it * ROWS_PER_IT * Cfg<D>::KSTR) = k[it];
  }
  __device__ __forceinline__ void store_v(u16* vs, int lo) const {
#pragma unroll
    for (int it = 0; it < Cfg<D>::LD_ITER; ++it)
      *reinterpret_cast<uint4*>(vs + lo + it * ROWS_PER_IT * Cfg<D>::VSTR) = v[it];
  }
};

// Per-wave state: NQT tiles of 32 query rows, online softmax in the log2
// domain. The running maximum is only raised when a tile exceeds it by more
// than kSlack (probabilities then stay below 2^kSlack), which skips the
// rescale of the accumulators on almost every tile.
constexpr float kSlack = 8.f;

template <int D, int NQT>
struct Wave {
  static constexpr int DSTEPS = D / 16;
  static constexpr int DT = D / 32;
  using S = f32x16[NQT][2];
  using P = bf16x8[NQT][4];
  bf16x8 qf[NQT][DSTEPS];
  f32x16 o[NQT][DT];
  float m[NQT];  // reference maximum (log2 domain), per lane = per query row
  float l[NQT];  // this lane's share of the running sum

  // S^T = K Q^T for one 64-key tile: s[nt][mt][v] is the score of key
  // 32*mt + 8*(v/4) + 4*half + (v%4) for this lane's row of query tile nt.
  __device__ __forceinline__ void qk(const u16* ks, int lane, S& s) const {
    constexpr int KSTR = Cfg<D>::KSTR;
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) s[nt][0] = s[nt][1] = f32x16{};
#pragma unroll
    for (int st = 0; st < DSTEPS; ++st) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (32 * mt + l32) * KSTR + 8 * half + 16 * st);
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt)
          s[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[nt][st], s[nt][mt], 0, 0, 0);
      }
    }
  }

  // keys at tile positions >= nvalid, or (step keys) outside the row's region, get -inf
  template <bool REGION>
  __device__ __forceinline__ static void mask(S& s, int lane, int nvalid, int c_base, const RowRule (&rules)[NQT]) {
    const int half = lane >> 5;
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // branch-free on purpose: a divergent element store into the
          // score vector is easy to mis-lower, a select is not
          const int kk = 32 * mt + 8 * (v >> 2) + 4 * half + (v & 3);
          bool ok = kk < nvalid;
          if (REGION) ok = ok & rules[nt].sees(c_base + kk);
          s[nt][mt][v] = ok ? s[nt][mt][v] : kNegInf;
        }
  }

  // Row maxima of the tile; raise the reference maximum (and rescale the
  // accumulators) only where the tile exceeds it by more than kSlack.
  __device__ __forceinline__ void update_max(const S& s, float sl2) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      float mx = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[nt][mt][v]);
      mx = half_max(mx) * sl2;
      const bool raise = mx > m[nt] + kSlack;
      if (__ballot(raise)) {
        const float mnew = raise ? mx : m[nt];
        const float alpha = raise ? __builtin_amdgcn_exp2f(m[nt] - mnew) : 1.f;  // m = -inf gives 0
        m[nt] = mnew;
        l[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[nt][dt] *= alpha;
      }
    }
  }

  // p = 2^(s*sl2 - m), summed into l and packed (bf16, RNE) as the B operand of O^T = V^T P^T
  __device__ __forceinline__ void probs(const S& s, float sl2, P& pb) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      const float muse = (m[nt] == kNegInf) ? 0.f : m[nt];
      float lsum = 0.f;
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const int mt = ks4 >> 1, vb = 8 * (ks4 & 1);
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(s[nt][mt][vb + e], sl2, -muse));
          pv[e] = pe;
          lsum += pe;
        }
        pb[nt][ks4] = __builtin_convertvector(pv, bf16x8);
      }
      l[nt] += lsum;
    }
  }

  // O^T += V^T P^T. B-operand index 8*half + e of k-step ks4 is key
  // 16*ks4 + 8*(e/4) + 4*half + (e%4). The V^T fragment comes from the
  // row-major V tile through two transposing reads: within each group of
  // 16 lanes, lane j points at 4 consecutive d of key row j/4, and lane i
  // receives d = (its column) for 4 consecutive keys.
  __device__ __forceinline__ void pv(const u16* vs, int lane, const P& pb) {
    constexpr int VSTR = Cfg<D>::VSTR;
    const int half = lane >> 5, g16 = lane & 15;
    const u16* vb0 = vs + (4 * half + (g16 >> 2)) * VSTR + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u16* vp = vb0 + 16 * ks4 * VSTR + 32 * dt;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * VSTR));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt)
          o[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[nt][ks4], o[nt][dt], 0, 0, 0);
      }
    }
  }
};

// Interleave the next tile's QK^T MFMAs with this tile's exponentials so the
// matrix and vector pipes work at the same time within one wave.
__device__ __forceinline__ void interleave_qk_softmax() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read (K fragment)
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
  }
}

template <int D, int NQT>
__global__ __launch_bounds__(kThreads, NQT == 1 ? 2 : 1) void attn_bf16_kernel(AttnParams p) {
  using C = Cfg<D>;
  using W = Wave<D, NQT>;
  constexpr int DSTEPS = D / 16, DT = D / 32;
  constexpr int WROWS = 32 * NQT;       // query rows per wave
  constexpr int BM = kWaves * WROWS;    // query rows per workgroup
  __shared__ __attribute__((aligned(16))) u16 ks[2][C::KBUF];
  __shared__ __attribute__((aligned(16))) u16 vs[2][C::VBUF];

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
  const int nk = max(0, kend - kbeg);

  const int M = p.R * p.g;
  W st;
  RowRule rules[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int m = qt * BM + wave * WROWS + 32 * nt + l32;
    const bool ok = m < M;
    const int r = ok ? m / p.g : 0;
    const int h = kvh * p.g + (ok ? m - r * p.g : 0);
    rules[nt] = row_rule(r, p.k, p.block_len);
    const u16* qp = reinterpret_cast<const u16*>(p.q) + ((size_t)(b * p.R + r) * p.Hq + h) * D + 8 * half;
#pragma unroll
    for (int i = 0; i < DSTEPS; ++i)
      st.qf[nt][i] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * i) : bf16x8{};
#pragma unroll
    for (int i = 0; i < DT; ++i) st.o[nt][i] = f32x16{};
    st.m[nt] = kNegInf;
    st.l[nt] = 0.f;
  }
  const float sl2 = p.scale_log2;

  // ---- prefix keys [kbeg, kend) ----
  // Software pipeline over 64-key tiles, one barrier per tile. At the top of
  // iteration t the scores of tile t are in registers, K[t+1] is in
  // ks[(t+1)&1] and V[t] in vs[t&1]; the loads of K[t+2] and V[t+1] are in
  // flight while the wave computes QK^T(t+1), softmax(t) and PV(t).
  const size_t head_off = (size_t)(b * p.Hkv + kvh) * p.cap * D + (size_t)kbeg * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(reinterpret_cast<const u16*>(p.k_cache) + head_off, (uint32_t)nk * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(reinterpret_cast<const u16*>(p.v_cache) + head_off, (uint32_t)nk * D * 2);
  const int ntile = (nk + kBN - 1) / kBN;
  const uint32_t rb = D * 2;
  const uint32_t vo = Stage<D>::voff(tid, rb);
  const int klo = Stage<D>::lds_off(tid, C::KSTR), vlo = Stage<D>::lds_off(tid, C::VSTR);
  Stage<D> stg;
  typename W::S s_cur, s_next;
  typename W::P pb;
  if (ntile > 0) {
    stg.load_k(kr, vo, 0, rb);
    stg.load_v(vr, vo, 0, rb);
    stg.store_k(ks[0], klo);
    stg.store_v(vs[0], vlo);
    stg.load_k(kr, vo, kBN, rb);
    stg.store_k(ks[1], klo);
    __syncthreads();
    st.qk(ks[0], lane, s_cur);
  }
  for (int t = 0; t < ntile; ++t) {
    // all reads of ks[t&1] (QK^T of tile t, issued in the previous iteration
    // or the prologue) and of vs[(t+1)&1] (PV of tile t-1) are done before
    // this iteration overwrites them
    __syncthreads();
    stg.load_k(kr, vo, (t + 2) * kBN, rb);
    stg.load_v(vr, vo, (t + 1) * kBN, rb);
    const int nvalid = nk - t * kBN;
    if (nvalid < kBN) W::template mask<false>(s_cur, lane, nvalid, 0, rules);
    st.update_max(s_cur, sl2);
    if (t + 1 < ntile) {
      st.qk(ks[(t + 1) & 1], lane, s_next);
      st.probs(s_cur, sl2, pb);
      interleave_qk_softmax();
    } else {
      st.probs(s_cur, sl2, pb);
    }
    st.pv(vs[t & 1], lane, pb);
    stg.store_k(ks[t & 1], klo);
    stg.store_v(vs[(t + 1) & 1], vlo);
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      s_cur[nt][0] = s_next[nt][0];
      s_cur[nt][1] = s_next[nt][1];
    }
  }
  __syncthreads();

  // ---- the step's own keys under the region rule (last split only) ----
  if (last) {
    const int m_lo = qt * BM;
    const int m_hi = min(M, m_lo + BM) - 1;
    const LocalRanges lr = local_ranges(m_lo / p.g, m_hi / p.g, p.k, p.block_len);
    const uint32_t row_bytes = (uint32_t)p.Hkv * D * 2;
    const size_t step_off = ((size_t)b * p.R * p.Hkv + kvh) * D;
    const u16* kst = reinterpret_cast<const u16*>(p.k_step) + step_off;
    const u16* vst = reinterpret_cast<const u16*>(p.v_step) + step_off;
    for (int seg = 0; seg < lr.n; ++seg) {
      const int c_lo = seg == 0 ? lr.a0 : lr.b0;
      const int c_hi = seg == 0 ? lr.a1 : lr.b1;
      const uint32_t bytes = (uint32_t)(c_hi - 1) * row_bytes + D * 2;  // rows < c_hi are valid
      const __amdgpu_buffer_rsrc_t lkr = make_rsrc(kst, bytes);
      const __amdgpu_buffer_rsrc_t lvr = make_rsrc(vst, bytes);
      const uint32_t lvo = Stage<D>::voff(tid, row_bytes);
      for (int c0 = c_lo; c0 < c_hi; c0 += kBN) {
        stg.load_k(lkr, lvo, c0, row_bytes);
        stg.load_v(lvr, lvo, c0, row_bytes);
        stg.store_k(ks[0], klo);
        stg.store_v(vs[0], vlo);
        __syncthreads();
        st.qk(ks[0], lane, s_cur);
        W::template mask<true>(s_cur, lane, min(kBN, c_hi - c0), c0, rules);
        st.update_max(s_cur, sl2);
        st.probs(s_cur, sl2, pb);
        st.pv(vs[0], lane, pb);
        __syncthreads();
      }
    }
  }

  // o[nt][dt][v] holds O^T[d = 32*dt + 8*(v/4) + 4*half + v%4][this lane's row]
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const float ltot = half_sum(st.l[nt]);
    const int m = qt * BM + wave * WROWS + 32 * nt + l32;
    if (m >= M) continue;
    const int r = m / p.g;
    const int h = kvh * p.g + (m - r * p.g);
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
          pk.x = f32_to_bf16_bits(st.o[nt][dt][4 * i + 0] * inv);
          pk.y = f32_to_bf16_bits(st.o[nt][dt][4 * i + 1] * inv);
          pk.z = f32_to_bf16_bits(st.o[nt][dt][4 * i + 2] * inv);
          pk.w = f32_to_bf16_bits(st.o[nt][dt][4 * i + 3] * inv);
          *reinterpret_cast<ushort4*>(op + d) = pk;
        }
      if (p.lse && half == 0) p.lse[orow] = (st.m[nt] + log2f(ltot)) * 0.69314718055994531f;
    } else {
      // normalised partial in bf16 plus its log2-domain log-sum-exp
      const size_t prow = (size_t)s * p.B * p.R * p.Hq + orow;
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      u16* po = reinterpret_cast<u16*>(p.part_o) + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * dt + 8 * i + 4 * half;
          ushort4 pk;
          pk.x = f32_to_bf16_bits(st.o[nt][dt][4 * i + 0] * inv);
          pk.y = f32_to_bf16_bits(st.o[nt][dt][4 * i + 1] * inv);
          pk.z = f32_to_bf16_bits(st.o[nt][dt][4 * i + 2] * inv);
          pk.w = f32_to_bf16_bits(st.o[nt][dt][4 * i + 3] * inv);
          *reinterpret_cast<ushort4*>(po + d) = pk;
        }
      if (half == 0) p.part_lse[prow] = ltot > 0.f ? st.m[nt] + log2f(ltot) : kNegInf;
    }
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
    if (lr.n > 0) run(kst, vst, stride, lr.a0, lr.a1, true);
    if (lr.n > 1) run(kst, vst, stride, lr.b0, lr.b1, true);
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
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
    float* po = reinterpret_cast<float*>(p.part_o) + prow * D;
#pragma unroll
    for (int j = 0; j < kF32MaxD / 64; ++j) {
      const int d = lane + 64 * j;
      if (d < D) po[d] = o[j] * inv;
    }
    if (lane == 0) p.part_lse[prow] = lrow > 0.f ? mrow + log2f(lrow) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials (normalised outputs o_s with
// log2-domain log-sum-exps e_s): with w_s = 2^(e_s - max e),
// O = sum_s w_s o_s / sum_s w_s and LSE = max e + log2(sum_s w_s).
// One thread per 8 (bf16) or 4 (fp32) output elements of a row.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int D = p.D;
  const int tpr = D / VEC;  // threads per row
  const size_t rows = (size_t)p.B * p.R * p.Hq;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t row = gid / tpr;
  const int d = (int)(gid % tpr) * VEC;
  if (row >= rows) return;
  float emax = kNegInf;
  for (int s = 0; s < p.S; ++s) emax = fmaxf(emax, p.part_lse[(size_t)s * rows + row]);
  const float euse = (emax == kNegInf) ? 0.f : emax;
  float wsum = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
#pragma unroll 4
  for (int s = 0; s < p.S; ++s) {
    const size_t prow = (size_t)s * rows + row;
    const float wgt = __builtin_amdgcn_exp2f(p.part_lse[prow] - euse);  // 0 for an empty split
    wsum += wgt;
    if (BF16) {
      const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(p.part_o) + prow * D + d);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(__uint_as_float(w4[i] << 16), wgt, acc[2 * i]);
        acc[2 * i + 1] = fmaf(__uint_as_float(w4[i] & 0xffff0000u), wgt, acc[2 * i + 1]);
      }
    } else {
      const float4 o = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.part_o) + prow * D + d);
      acc[0] = fmaf(o.x, wgt, acc[0]);
      acc[1] = fmaf(o.y, wgt, acc[1]);
      acc[2] = fmaf(o.z, wgt, acc[2]);
      acc[VEC - 1] = fmaf(o.w, wgt, acc[VEC - 1]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (BF16) {
    uint4 pk;
    uint32_t* w4 = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w4[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1] * inv) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<u16*>(p.out) + row * D + d) = pk;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * D + d) =
        make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[VEC - 1] * inv);
  }
  if (p.lse && d == 0) p.lse[row] = (emax + log2f(wsum)) * 0.69314718055994531f;
}

hipError_t launch_merge(const AttnParams& p, bool bf16, hipStream_t stream) {
  const size_t threads = (size_t)p.B * p.R * p.Hq * (p.D / (bf16 ? 8 : 4));
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
    // 32 or 64 query rows per wave; TIDAR_ATTN_WAVE_ROWS overrides the choice (tuning knob)
    pl.nqt = 1;
    if (const char* e = getenv("TIDAR_ATTN_WAVE_ROWS")) pl.nqt = atoi(e) >= 64 ? 2 : 1;
    pl.bm = kWaves * 32 * pl.nqt;
    pl.qtiles = (int)((M + pl.bm - 1) / pl.bm);
    base = (long)B * Hkv * pl.qtiles;
  } else {
    pl.nqt = 1;
    pl.bm = 1;
    pl.qtiles = (int)M;
    base = (long)B * Hkv * M;
  }
  const int ntiles = (max_len + kBN - 1) / kBN;
  int S;
  if (forced_splits > 0) {
    S = forced_splits;
  } else {
    // Fill the resident workgroup slots (two per CU on the 256-CU part) in
    // one round: a second, partial round would cost as much as the first.
    // Keep at least two key tiles per split.
    long slots = 512;
    if (const char* e = getenv("TIDAR_ATTN_TARGET_WG")) slots = std::max(1L, atol(e));
    S = (int)std::max(1L, slots / base);
    S = std::max(1, std::min(S, std::max(1, ntiles / 2)));
  }
  S = std::max(1, std::min(S, std::max(1, ntiles)));
  int chunk = ntiles > 0 ? ((ntiles + S - 1) / S) * kBN : kBN;
  S = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  pl.S = S;
  pl.chunk = chunk;
  // partial outputs in the input precision, then one fp32 log-sum-exp per row
  const size_t prow = (size_t)S * B * R * Hq;
  const size_t elem = dtype == 1 ? 2 : 4;
  pl.ws_bytes = S > 1 ? (prow * D * elem + 255) / 256 * 256 + prow * sizeof(float) : 0;
  return pl;
}

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.B * p.Hkv * p.qtiles * p.S);
  if (p.D == 128 && p.nqt == 1)
    hipLaunchKernelGGL((attn_bf16_kernel<128, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.D == 128 && p.nqt == 2)
    hipLaunchKernelGGL((attn_bf16_kernel<128, 2>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.D == 64 && p.nqt == 1)
    hipLaunchKernelGGL((attn_bf16_kernel<64, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.D == 64 && p.nqt == 2)
    hipLaunchKernelGGL((attn_bf16_kernel<64, 2>), dim3(grid), dim3(kThreads), 0, stream, p);
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
