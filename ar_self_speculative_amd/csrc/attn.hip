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
#include <type_traits>

namespace tidar {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kBM = 128;          // packed query rows per workgroup (bf16 path)
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

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// inclusive prefix sum over the wave's lanes
__device__ __forceinline__ int wave_incl_scan_int(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
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
  // raw buffer (stride 0): loads at byte offsets >= bytes return zero. The
  // fields go through readfirstlane so the descriptor is known to be uniform
  // and stays in scalar registers.
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// LDS tile layout: 64 keys x D bf16 held as D/16 column pairs of 32 B per
// key. Element (key r, dim d) sits at byte
//   (d/16)*kCPS + r*32 + (((d%16)/8) ^ ((r/8)%2))*16 + (d%8)*2,
// i.e. the two 16-B halves of a key's slot swap places every 8 keys, and
// column pairs are kCPS = 2048 + 128 bytes apart. Then
//  * a wave's A-operand read of K (32 keys x 16 dims, 16 B per lane) touches
//    all 64 banks once per 16 lanes (the swap moves keys 8..15 of each group
//    of 16 onto the other half of the banks), and
//  * a transposing V read (8 keys x 32 dims, two column pairs) puts its two
//    column pairs 128 B apart in bank space,
// so neither conflicts, with one or two address registers per lane. The
// global->LDS copies write 1 KB (32 keys x one column pair) per instruction.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kCPS = 2048 + 128;  // bytes per column pair in LDS

// cache-policy operand of the buffer-store builtins: sc1 (device scope)
constexpr int kStoreDevice = 16;

template <int D>
struct Lay {
  static constexpr int NCP = D / 16;             // column pairs
  static constexpr int TILE_BYTES = NCP * kCPS;  // 64 keys
  static constexpr int NLD = 2 * NCP;            // 1 KB copies per tile
};

// Copy i (0 <= i < NLD / WAVES) of this wave's share of a tile copy (the
// scalar offset is wave-uniform by construction; readfirstlane tells the
// compiler so).
template <int D, int WAVES>
__device__ __forceinline__ void copy_one(__amdgpu_buffer_rsrc_t r, uint32_t vo, int row0, uint32_t row_bytes,
                                         lds_u8* dst, int wave, int i) {
  const int j = wave + WAVES * i;
  const int cp = j >> 1, h = j & 1;
  const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)(row0 + 32 * h) * row_bytes + 32u * cp);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + cp * kCPS + h * 1024),
                                           16, vo, so, 0, 0);
}

// Global -> LDS copy of one 64-key tile (rows row0 .. row0+63 of a buffer
// resource whose rows are row_bytes apart), without passing through
// registers. Copy j moves column pair j/2 of keys 32*(j%2) .. +31; lane l
// fetches 16 B of key l/2. Rows past the resource's end arrive as zeros, so
// partial tiles need no branches and no invalid value reaches the MFMAs.
template <int D, int WAVES>
__device__ __forceinline__ void copy_tile(__amdgpu_buffer_rsrc_t r, uint32_t vo, int row0, uint32_t row_bytes,
                                          lds_u8* dst, int wave) {
#pragma unroll
  for (int i = 0; i < Lay<D>::NLD / WAVES; ++i) copy_one<D, WAVES>(r, vo, row0, row_bytes, dst, wave, i);
}

// Lane l of a copy lands on LDS slot half (l%2) of key l/2; it fetches the
// logical half that the swap puts there.
__device__ __forceinline__ uint32_t copy_voff(int lane, uint32_t row_bytes) {
  return (uint32_t)(lane >> 1) * row_bytes + (uint32_t)((lane & 1) ^ ((lane >> 4) & 1)) * 16u;
}

// wait for this wave's outstanding global->LDS copies
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads()
// it does not wait for this wave's global loads (a workgroup-scope release
// for all address spaces waits on vmcnt(0)). Global-to-LDS copies are
// vector-memory operations: each wave waits for its own with an explicit
// vmcnt before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-wave state: NQT tiles of 32 query rows, online softmax in the log2
// domain. The running maximum is only raised when a tile exceeds it by more
// than kSlack (probabilities then stay below 2^kSlack), which skips the
// rescale of the accumulators on almost every tile.
constexpr float kSlack = 8.f;

// LSE32: accumulate the row sum in fp32 from the unrounded probabilities
// (used when the caller asks for the log-sum-exp); otherwise from the
// bf16-rounded ones that also feed P V, with one packed dot per pair.
template <int D, int NQT, bool LSE32 = false>
struct Wave {
  static constexpr int DSTEPS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int SPS = 32 / DSTEPS;  // scores per row turned into P per QK k-step
  using S = f32x16[NQT][2];
  using P = bf16x8[NQT][4];
  bf16x8 qf[NQT][DSTEPS];
  f32x16 o[NQT][DT];
  float m[NQT];  // reference maximum (log2 domain), per lane = per query row
  float l[NQT];  // this lane's share of the running sum (of the bf16-rounded P)
  uint32_t ka;        // LDS byte offset of this lane's K fragment inside a tile
  uint32_t va0, va1;  // ... of its V^T fragment, keys 0..7 and 8..15 of a k-step

  __device__ __forceinline__ void init_addr(int lane) {
    const int l32 = lane & 31, half = lane >> 5, g16 = lane & 15, gbit = (lane >> 4) & 1;
    ka = (uint32_t)(l32 * 32 + (half ^ ((l32 >> 3) & 1)) * 16);
    const int row = 4 * half + (g16 >> 2), lhalf = (g16 & 3) >> 1;
    va0 = (uint32_t)(gbit * kCPS + row * 32 + lhalf * 16 + (g16 & 1) * 8);
    va1 = (uint32_t)(gbit * kCPS + (row + 8) * 32 + (lhalf ^ 1) * 16 + (g16 & 1) * 8);
  }

  // K fragment: keys 32*mt + l32, dims 16*st + 8*half .. +7 (A operand of S^T = K Q^T)
  __device__ __forceinline__ bf16x8 kfrag(const lds_u8* kb, int st, int mt) const {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kb + ka + st * kCPS + mt * 1024);
  }
  // V^T fragment for k-step ks4 (keys 16*ks4 .. +15) and dims 32*dt .. +31:
  // two transposing reads; within each group of 16 lanes, lane j points at
  // 4 consecutive dims of one key and lane i receives one dim of 4 keys.
  __device__ __forceinline__ bf16x8 vfrag(const lds_u8* vb, int ks4, int dt) const {
    const int off = dt * 2 * kCPS + ks4 * 512;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + va0 + off));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + va1 + off));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // S^T = K Q^T for one tile, not interleaved (first tile and step keys).
  // s[nt][mt][v] is the score of key 32*mt + 8*(v/4) + 4*half + (v%4).
  __device__ __forceinline__ void qk(const lds_u8* kb, S& s) const {
    // Standalone S^T = K Q^T (tiles that are not interleaved with a step):
    // the K fragments are read QLA MFMA slots ahead so the LDS latency
    // overlaps the matrix work.
    constexpr int N = 2 * DSTEPS, QLA = 4;
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) s[nt][0] = s[nt][1] = f32x16{};
    bf16x8 a[N];
#pragma unroll
    for (int j = 0; j < QLA; ++j) a[j] = kfrag(kb, j >> 1, j & 1);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (j + QLA < N) a[j + QLA] = kfrag(kb, (j + QLA) >> 1, (j + QLA) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt)
        s[nt][j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], qf[nt][j >> 1], s[nt][j & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // keys at tile positions >= nvalid, or (step keys) outside the row's region, get -inf
  template <bool REGION>
  __device__ __forceinline__ static void mask(S& s, int lane, int nvalid, int c_base, const RowRule (&rules)[NQT]) {
    // The key index of score v is a compile-time offset from 4*half. The
    // empty asm keeps the compiler from hoisting 32 such per-lane constants
    // out of the tile loop (they would occupy 32 registers for its length).
    int h4 = (lane >> 5) * 4;
    asm volatile("" : "+v"(h4));
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // branch-free on purpose: a divergent element store into the
          // score vector is easy to mis-lower, a select is not
          const int kk = h4 + (32 * mt + 8 * (v >> 2) + (v & 3));
          bool ok = kk < nvalid;
          if (REGION) ok = ok & rules[nt].sees(c_base + kk);
          s[nt][mt][v] = ok ? s[nt][mt][v] : kNegInf;
        }
  }

  // in-lane maximum of 8 scores of score group g (0..3) into mx
  __device__ __forceinline__ static void max8(const S& s, int nt, int g, float& mx) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) mx = fmaxf(mx, fmaxf(s[nt][g >> 1][8 * (g & 1) + e], s[nt][g >> 1][8 * (g & 1) + e + 1]));
  }

  // Raise the reference maximum (and rescale the accumulators) where the
  // tile's row maximum (log2 domain, mx holds the in-lane part of the raw
  // score maximum) exceeds it by more than kSlack.
  __device__ __forceinline__ void update_max(float (&mx)[NQT], float sl2) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      const float t = half_max(mx[nt]) * sl2;
      const bool raise = t > m[nt] + kSlack;
      if (__ballot(raise)) {
        const float mnew = raise ? t : m[nt];
        const float alpha = raise ? __builtin_amdgcn_exp2f(m[nt] - mnew) : 1.f;  // m = -inf gives 0
        m[nt] = mnew;
        l[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[nt][dt] *= alpha;
      }
    }
  }

  // P for scores [i0, i0 + n) of row tile nt (n even): each pair is rounded
  // to bf16 (nearest even), added to the row sum and stored straight into
  // the B operand of O^T = V^T P^T.
  __device__ __forceinline__ void probs(const S& s, int nt, int i0, int n, float muse, float sl2, P& pb) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int j = 0; j < n; j += 2) {
      const int i = i0 + j;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[nt][i >> 4][i & 15], sl2, -muse));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[nt][(i + 1) >> 4][(i + 1) & 15], sl2, -muse));
      const f32x2 pp = {p0, p1};
      const bf16x2 h = __builtin_convertvector(pp, bf16x2);
      if (LSE32)
        l[nt] += p0 + p1;
      else
        l[nt] = __builtin_amdgcn_fdot2_f32_bf16(h, one, l[nt], false);
      pb[nt][i >> 3][i & 7] = h[0];
      pb[nt][i >> 3][(i & 7) + 1] = h[1];
    }
  }

  // One tile step in a fixed instruction order:
  //   phase A: the next tile's S^T = K Q^T MFMAs (QK) interleaved with this
  //            tile's probabilities (from s_cur);
  //   phase B: this tile's O^T += V^T P^T MFMAs interleaved with the row
  //            maxima of the next tile (NEXT).
  // Operand fragments are read LA (K, phase A) and LB (V, phase B) MFMA
  // slots ahead; sched_barrier(0) pins each slot so the LDS, matrix and
  // vector pipes overlap.
  static constexpr int LA = 2, LB = 2;
  // There is no branch between the phases: code motion across one would undo
  // the interleaving.
  // With MASK, the next tile's scores are masked between the phases (before
  // their maxima are taken): keys past nvalid, and for a tile of step keys
  // (local) the keys outside each row's region.
  template <bool QK, bool NEXT, bool MASK = false>
  __device__ __forceinline__ void step(const lds_u8* kb_next, const lds_u8* vb_cur, const S& s_cur, S& s_next,
                                       float sl2, bool local = false, int nvalid = kBN, int c_base = 0,
                                       int lane = 0, const RowRule (*rules)[NQT] = nullptr) {
    float muse[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) muse[nt] = (m[nt] == kNegInf) ? 0.f : m[nt];
    P pb;
    // ---- phase A: slot j = (k-step j/2, key half j%2) ----
    constexpr int NA = 2 * DSTEPS;
    bf16x8 kf[NA];
    if (QK) {
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) s_next[nt][0] = s_next[nt][1] = f32x16{};
#pragma unroll
      for (int j = 0; j < LA; ++j) kf[j] = kfrag(kb_next, j >> 1, j & 1);
    }
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      if (QK && j + LA < NA) kf[j + LA] = kfrag(kb_next, (j + LA) >> 1, (j + LA) & 1);
      __builtin_amdgcn_sched_barrier(0);
      if (QK) {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt)
          s_next[nt][j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[nt][j >> 1], s_next[nt][j & 1], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) probs(s_cur, nt, (SPS / 2) * j, SPS / 2, muse[nt], sl2, pb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (MASK) {
      if (local)
        mask<true>(s_next, lane, nvalid, c_base, *rules);
      else if (nvalid < kBN)
        mask<false>(s_next, lane, nvalid, 0, *rules);
    }
    // ---- phase B: slot j = (k-step j/DT, dim tile j%DT) ----
    float mx[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) mx[nt] = kNegInf;
    constexpr int NB = 4 * DT;
    bf16x8 vf[NB];
#pragma unroll
    for (int j = 0; j < LB; ++j) vf[j] = vfrag(vb_cur, j / DT, j % DT);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j + LB < NB) vf[j + LB] = vfrag(vb_cur, (j + LB) / DT, (j + LB) % DT);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt)
        o[nt][j % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], pb[nt][j / DT], o[nt][j % DT], 0, 0, 0);
      if (NEXT && (j % (NB / 4)) == 0) {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) max8(s_next, nt, j / (NB / 4), mx[nt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT) update_max(mx, sl2);
  }

  // max of a whole (masked) tile, then the reference maximum update
  __device__ __forceinline__ void tile_max(const S& s, float sl2) {
    float mx[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      mx[nt] = kNegInf;
#pragma unroll
      for (int g = 0; g < 4; ++g) max8(s, nt, g, mx[nt]);
    }
    update_max(mx, sl2);
  }
};

// Where the keys of tile u of a workgroup come from: first the prefix tiles
// (KV cache rows, row stride D), then, for the split that owns the last
// prefix keys, the step's own keys visible to its rows (k_step / v_step
// rows, stride Hkv*D) in at most two contiguous ranges.
struct TileSrc {
  const void* k;       // K rows of the range (resource base)
  const void* v;       // V rows of the range
  uint32_t bytes;      // resource size: rows past it load as zeros
  int row0;            // first row of the tile in the resource
  uint32_t row_bytes;
  uint32_t vo;         // per-lane part of the copy offsets
  int nvalid;          // rows of the tile that exist
  int c_base;          // step-key index of the tile's first key (local tiles)
  bool local;
};

struct TileSeq {
  int np;                             // prefix tiles
  int nl0, nl1;                       // local tiles of the two ranges
  int nk;                             // prefix keys
  int c_lo0, c_hi0, c_lo1, c_hi1;     // the local ranges
  const void *pk, *pv, *lk, *lv;      // prefix and step-key bases
  uint32_t pbytes, lbytes0, lbytes1;
  uint32_t prb, lrb, pvo, lvo;
  __device__ __forceinline__ int count() const { return __builtin_amdgcn_readfirstlane(np + nl0 + nl1); }
  __device__ __forceinline__ TileSrc at(int u) const {
    // scalar arithmetic only (no selection between fields): the struct then
    // stays in registers
    TileSrc t;
    const int pre = u < np;                 // 1 for a prefix tile
    const int sec = (u >= np + nl0);        // 1 for the second local range
    const int loc = u - np - sec * nl0;     // tile index inside its local range
    const int c_lo = c_lo0 + sec * (c_lo1 - c_lo0);
    const int c_hi = c_hi0 + sec * (c_hi1 - c_hi0);
    const int c0 = c_lo + loc * kBN;
    // every field is wave-uniform; readfirstlane lets the compiler keep the
    // tile loop's control flow scalar
    t.local = !pre;
    t.row0 = __builtin_amdgcn_readfirstlane(pre ? u * kBN : c0);
    t.c_base = __builtin_amdgcn_readfirstlane(pre ? 0 : c0);
    t.nvalid = __builtin_amdgcn_readfirstlane(pre ? min(kBN, nk - u * kBN) : min(kBN, c_hi - c0));
    t.bytes = __builtin_amdgcn_readfirstlane(pre ? pbytes : (lbytes0 + (uint32_t)sec * (lbytes1 - lbytes0)));
    t.row_bytes = __builtin_amdgcn_readfirstlane(pre ? prb : lrb);
    t.vo = pre ? pvo : lvo;
    t.k = pre ? pk : lk;
    t.v = pre ? pv : lv;
    return t;
  }
};

// Iteration t of the tile loop when tile t+1 is a full prefix tile: the
// fully interleaved step with no other path, so the accumulators keep their
// registers across iterations. The scores of tile t are in s_cur, those of
// tile t+1 land in s_next (the caller alternates the two). All of the
// iteration's copies go out first: issued one at a time from inside the
// step instead, they stalled the waves that issued them there and the CU's
// throughput did not rise.
template <int D, int NQT, int WAVES, bool LSE32>
__device__ __forceinline__ void main_iter(Wave<D, NQT, LSE32>& st, lds_u8* __restrict__ kb_dst,
                                          const lds_u8* __restrict__ kb_next, const lds_u8* __restrict__ vb_cur,
                                          lds_u8* __restrict__ vb_dst, const TileSeq& seq, int t, int wave,
                                          float sl2, const typename Wave<D, NQT, LSE32>::S& s_cur,
                                          typename Wave<D, NQT, LSE32>::S& s_next) {
  if (t + 2 < seq.count()) {
    const TileSrc a = seq.at(t + 2);
    copy_tile<D, WAVES>(make_rsrc(a.k, a.bytes), a.vo, a.row0, a.row_bytes, kb_dst, wave);
  }
  copy_tile<D, WAVES>(make_rsrc(seq.pv, seq.pbytes), seq.pvo, (t + 1) * kBN, seq.prb, vb_dst, wave);
  st.template step<true, true>(kb_next, vb_cur, s_cur, s_next, sl2);
  wait_copies();
}

// The copies of main-loop iteration t alone, for a wave with no rows to
// compute: the same instructions as main_iter issues, so every tile still
// arrives whole.
template <int D, int WAVES>
__device__ __forceinline__ void main_iter_copies(lds_u8* __restrict__ kb_dst, lds_u8* __restrict__ vb_dst,
                                                 const TileSeq& seq, int t, int wave) {
  if (t + 2 < seq.count()) {
    const TileSrc a = seq.at(t + 2);
    copy_tile<D, WAVES>(make_rsrc(a.k, a.bytes), a.vo, a.row0, a.row_bytes, kb_dst, wave);
  }
  copy_tile<D, WAVES>(make_rsrc(seq.pv, seq.pbytes), seq.pvo, (t + 1) * kBN, seq.prb, vb_dst, wave);
  wait_copies();
}

// One iteration t of the tile loop: copies of K[t+2] (into kb_dst) and
// V[t+1] (into vb_dst) are issued, then the tile step runs on K[t+1]
// (kb_next) and V[t] (vb_cur). The four buffers are distinct; passing them as
// restrict pointers lets the compiler see that the reads do not wait for the
// copies in flight. The next tile's scores are masked between the step's
// phases when it needs it (the partial last prefix tile, or step keys under
// the region rule); the loop's last tile (P V only) is peeled by the caller.
template <int D, int NQT, int WAVES, bool LSE32>
__device__ __forceinline__ void tile_iter(Wave<D, NQT, LSE32>& st, lds_u8* __restrict__ kb_dst,
                                          const lds_u8* __restrict__ kb_next, const lds_u8* __restrict__ vb_cur,
                                          lds_u8* __restrict__ vb_dst, const TileSeq& seq, int t, int wave, int lane,
                                          const RowRule (&rules)[NQT], float sl2,
                                          typename Wave<D, NQT, LSE32>::S& sA, typename Wave<D, NQT, LSE32>::S& sB,
                                          bool live) {
  // t + 1 < count(): the next tile exists (the caller peels the last tile)
  if (t + 2 < seq.count()) {
    const TileSrc a = seq.at(t + 2);
    copy_tile<D, WAVES>(make_rsrc(a.k, a.bytes), a.vo, a.row0, a.row_bytes, kb_dst, wave);
  }
  const TileSrc n = seq.at(t + 1);
  copy_tile<D, WAVES>(make_rsrc(n.v, n.bytes), n.vo, n.row0, n.row_bytes, vb_dst, wave);
  if (live)
    st.template step<true, true, true>(kb_next, vb_cur, sA, sB, sl2, n.local, n.nvalid, n.c_base, lane, &rules);
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    sA[nt][0] = sB[nt][0];
    sA[nt][1] = sB[nt][1];
  }
  wait_copies();
}

// The first kernel arguments are the fields the prologue needs before its
// first loads, as plain scalars: this file is built with kernel-argument
// preloading, so the dispatch places them in scalar registers and the Q, K[0]
// and cache-length loads go out without first waiting for a load of the
// argument block (at launch every workgroup waits on memory at once, and that
// wait is a large part of a workgroup's life). Small fields come packed two
// to a dword (each below 2^16, checked on the host): a_qt_s = qtiles | S << 16,
// a_hkv_g = Hkv | g << 16, a_k_bl = k | block_len << 16; a_nwg is the grid size.

// RAG: ragged batch (split slots apportioned per sequence); PAD: the last
// query tile is only partly filled. Template parameters, so that launches
// without them carry none of their code.
// Per-workgroup timestamps of the STAMP instantiation (a measurement build
// of the launch that computes exactly what the plain one does; only the
// 128-dim, four-wave, non-ragged launch without LSE has it): wave 0 of
// workgroup w writes record w of kStampFields 64-bit words.
constexpr int kStampFields = 8;
constexpr int kStampMaxWG = 4096;
__device__ unsigned long long g_attn_stamps[kStampMaxWG * kStampFields];

template <int D, int NQT, int WAVES, bool LSE32, bool RAG, bool PAD, bool STAMP = false>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void attn_bf16_kernel(
    const int32_t* __restrict__ a_len, const void* __restrict__ a_q, const void* __restrict__ a_kc, uint32_t a_qt_s,
    uint32_t a_hkv_g, uint32_t a_k_bl, int a_R, int a_nwg, int a_cap, int a_chunk, int a_max_len, AttnParams p) {
  // shader-clock counter and the 100 MHz reference at entry
  unsigned long long st_entry = 0, st_rentry = 0, st_pro = 0, st_loop = 0;
  if (STAMP) {
    st_entry = __builtin_amdgcn_s_memtime();
    st_rentry = __builtin_amdgcn_s_memrealtime();
  }
  using W = Wave<D, NQT, LSE32>;
  using L = Lay<D>;
  constexpr int DSTEPS = D / 16, DT = D / 32;
  constexpr int WROWS = 32 * NQT;      // query rows per wave
  constexpr int BM = WAVES * WROWS;    // query rows per workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[L::TILE_BYTES];
  lds_u8* const KB[2] = {(lds_u8*)kb0, (lds_u8*)kb1};
  lds_u8* const VB[2] = {(lds_u8*)vb0, (lds_u8*)vb1};

  // Work-item and workgroup ids come from the intrinsics (this file is built
  // with the IEEE mode bit clear, which keeps the device-library accessors
  // behind threadIdx/blockIdx from being inlined, and a call would hide that
  // the workgroup id is uniform).
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;

  const int qtiles = (int)(a_qt_s & 0xffff), S = (int)(a_qt_s >> 16);
  const int Hkv = (int)(a_hkv_g & 0xffff), g = (int)(a_hkv_g >> 16);
  const int kdr = (int)(a_k_bl & 0xffff), bl = (int)(a_k_bl >> 16);
  int w = remap_xcd((int)__builtin_amdgcn_workgroup_id_x(), a_nwg);
  const int qt = w % qtiles;
  w /= qtiles;
  int s, kvh, b, Sb, chunk, len = 0;
  size_t prow_off;  // partial rows of this split: [prow_off, prow_off + rows) of part_o / part_lse, in output rows
  if (RAG && p.B <= 64) {
    // The sequence and split of slot `slot`: every workgroup shares the S
    // slots out the same way from the clamped lengths. Sequence i weighs
    // w_i = its prefix tiles plus twice the step-key tiles of its last split
    // (a step-key tile goes through the region rule and the masked tile
    // path, and costs about two prefix tiles) and takes S_i = max(1,
    // ceil(w_i / c)) slots, c being the smallest weight per split with
    // sum S_i <= S (a binary search between ceil(sum w / S) and
    // ceil(sum w / (S - B)), which always fits). Its splits but the last
    // take ceil(w_i / S_i) prefix tiles each when that still makes S_i
    // splits, else ceil(tiles_i / S_i). Lane i holds sequence i.
    const int slot = w % S;
    kvh = w / S;
    const int B = p.B, lt = p.local_tiles;
    const int raw_l = lane < B ? a_len[lane] : 0;
    const int li = min(max(raw_l, 0), a_max_len);
    const int wl = lane < B ? (li + kBN - 1) / kBN + 2 * lt : 0;
    const int wsum = __builtin_amdgcn_readfirstlane(wave_sum_int(wl));
    int lo = max(1, (wsum + S - 1) / S), hi = (wsum + (S - B) - 1) / (S - B);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int n = __builtin_amdgcn_readfirstlane(wave_sum_int(lane < B ? max(1, (wl + mid - 1) / mid) : 0));
      if (n <= S)
        hi = mid;
      else
        lo = mid + 1;
    }
    const int sl = lane < B ? max(1, (wl + lo - 1) / lo) : 0;
    const int incl = wave_incl_scan_int(sl, lane);
    if (qt == 0 && kvh == 0 && slot == 0 && wave == 0 && lane < B) {
      p.split_tab[2 * lane] = incl - sl;
      p.split_tab[2 * lane + 1] = sl;
    }
    const unsigned long long over = __ballot(lane < B && incl > slot);
    if (over == 0) return;  // a slot no sequence needed
    b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(over));
    Sb = __builtin_amdgcn_readlane(sl, b);
    const int bstart = __builtin_amdgcn_readlane(incl, b) - Sb;
    s = __builtin_amdgcn_readfirstlane(slot - bstart);
    const int raw = __builtin_amdgcn_readlane(raw_l, b);
    if (raw < 0 || raw > a_max_len) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, 1);
    }
    len = __builtin_amdgcn_readlane(li, b);
    {  // the last split's step-key tiles count towards its share, as in the weights
      const int pt = (len + kBN - 1) / kBN, chb = (pt + 2 * lt + Sb - 1) / Sb;
      chunk = __builtin_amdgcn_readfirstlane(((pt + chb - 1) / max(chb, 1) == Sb ? chb : (pt + Sb - 1) / Sb) * kBN);
    }
    prow_off = (size_t)(bstart + s - b) * a_R * Hkv * g;
  } else if (RAG) {
    // More than 64 sequences: the same sharing with c = ceil(sum w / (S - B))
    // (sum S_i <= S), from a scalar pass over the lengths.
    const int slot = w % S;
    kvh = w / S;
    const int B = p.B, lt = p.local_tiles;
    int wsum = 0;
    for (int i = 0; i < B; ++i) {
      const int li = min(max(a_len[i], 0), a_max_len);
      wsum += (li + kBN - 1) / kBN + 2 * lt;
    }
    const int E = S - B;  // > 0 by the plan
    const int c = (wsum + E - 1) / E;
    const bool writer = qt == 0 && kvh == 0 && slot == 0 && tid == 0;
    int start = 0, bstart = 0;
    b = -1;
    Sb = 1;
    for (int i = 0; i < B; ++i) {
      const int li = min(max(a_len[i], 0), a_max_len);
      const int si = max(1, ((li + kBN - 1) / kBN + 2 * lt + c - 1) / c);
      if (writer) {
        p.split_tab[2 * i] = start;
        p.split_tab[2 * i + 1] = si;
      }
      if (b < 0 && slot < start + si) {
        b = i;
        bstart = start;
        Sb = si;
      }
      start += si;
    }
    b = __builtin_amdgcn_readfirstlane(b);
    if (b < 0) return;  // a slot no sequence needed
    s = __builtin_amdgcn_readfirstlane(slot - bstart);
    Sb = __builtin_amdgcn_readfirstlane(Sb);
    const int raw = a_len[b];
    if (raw < 0 || raw > a_max_len) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, 1);
    }
    len = __builtin_amdgcn_readfirstlane(min(max(raw, 0), a_max_len));
    {  // the last split's step-key tiles count towards its share, as in the weights
      const int pt = (len + kBN - 1) / kBN, chb = (pt + 2 * lt + Sb - 1) / Sb;
      chunk = __builtin_amdgcn_readfirstlane(((pt + chb - 1) / max(chb, 1) == Sb ? chb : (pt + Sb - 1) / Sb) * kBN);
    }
    prow_off = (size_t)(bstart + s - b) * a_R * Hkv * g;
  } else {
    s = w % S;
    w /= S;
    kvh = w % Hkv;
    b = w / Hkv;
    Sb = S;
    chunk = a_chunk;
    prow_off = (size_t)s * p.B * a_R * Hkv * g;
  }

  // The first prefix tile's K rows do not depend on the cache length: their
  // copy goes out first, bounded by the host's max_len instead (rows below
  // max_len lie inside the cache). Rows at or past the length that it brings
  // in are masked to -inf before any use; V rows past the length are never
  // loaded (their copies are bounded by the length), so P V sees only zeros
  // there. (Ragged batches already know the length: no early copy.)
  const bool last = (s == Sb - 1);
  const int kbeg = s * chunk;
  const int nk_hint = RAG ? 0
                          : __builtin_amdgcn_readfirstlane(
                                max(0, (last ? a_max_len : min(kbeg + chunk, a_max_len)) - kbeg));
  const size_t head_off = (size_t)(b * Hkv + kvh) * a_cap * D + (size_t)kbeg * D;
  const uint32_t pvo = copy_voff(lane, D * 2);
  if (nk_hint > 0)
    copy_tile<D, WAVES>(make_rsrc(reinterpret_cast<const u16*>(a_kc) + head_off, (uint32_t)nk_hint * (D * 2)), pvo, 0,
                        D * 2, KB[0], wave);

  // Q next: its loads do not depend on the cache length either, so they are
  // in flight while the length is fetched. Rows past M load row 0 (in
  // bounds) and are zeroed, which keeps the eight loads free of branches.
  const int M = a_R * g;
  const int Hq = Hkv * g;
  // A wave whose rows all lie past M (the padded part of the last query
  // tile) skips the matrix and softmax work; it still issues its share of the
  // tile copies and takes part in every barrier.
  const bool live = !PAD || qt * BM + wave * WROWS < M;
  W st;
  st.init_addr(lane);
  RowRule rules[NQT];
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int m = qt * BM + wave * WROWS + 32 * nt + l32;
    const bool ok = m < M;
    const int r = ok ? m / g : 0;
    const int h = kvh * g + (ok ? m - r * g : 0);
    rules[nt] = row_rule(r, kdr, bl);
    const u16* qp = reinterpret_cast<const u16*>(a_q) + ((size_t)(b * a_R + r) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int i = 0; i < DSTEPS; ++i) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * i);
      st.qf[nt][i] = ok ? v : bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < DT; ++i) st.o[nt][i] = f32x16{};
    st.m[nt] = kNegInf;
    st.l[nt] = 0.f;
  }

  if (!RAG) {
    len = __builtin_amdgcn_readfirstlane(a_len[b]);  // uniform: keeps the tile loop scalar
    if (len < 0 || len > a_max_len) {
      if (tid == 0 && p.dev_status) atomicOr(p.dev_status, 1);
      len = min(max(len, 0), a_max_len);
    }
  }
  const int kend = last ? len : min(kbeg + chunk, len);
  const int nk = max(0, kend - kbeg);

  // In a ragged batch a split can hold no prefix keys (a sequence shorter
  // than its share of slots): it records an empty partial (log-sum-exp -inf,
  // which the merge weighs by exactly zero without reading the partial) and
  // leaves, skipping the prologue's waits and the epilogue's 32 KB partial
  // store. (With one split count for every sequence such splits run through
  // and store an all-zero partial, as every other split does.)
  if (RAG && !last && nk == 0) {
    wait_copies();
    if (half == 0) {
      const __amdgpu_buffer_rsrc_t lrsrc = make_rsrc(p.part_lse + prow_off, 0xFFFFFFFFu);
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        const int m = qt * BM + wave * WROWS + 32 * nt + l32;
        if (m < M) {
          const int r = m / g;
          const uint32_t orow = (uint32_t)((b * a_R + r) * Hq + kvh * g + (m - r * g));
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(kNegInf), lrsrc, (int)(orow * 4u), 0, kStoreDevice);
        }
      }
    }
    return;
  }

  const float sl2 = p.scale_log2;

  // ---- the tile sequence: prefix keys [kbeg, kend), then (last split only)
  // the step's own keys under the region rule ----
  TileSeq seq;
  seq.nk = __builtin_amdgcn_readfirstlane(nk);
  seq.np = __builtin_amdgcn_readfirstlane((nk + kBN - 1) / kBN);
  seq.prb = D * 2;
  seq.pvo = pvo;
  seq.pk = reinterpret_cast<const u16*>(a_kc) + head_off;
  seq.pv = reinterpret_cast<const u16*>(p.v_cache) + head_off;
  seq.pbytes = (uint32_t)nk * seq.prb;
  seq.nl0 = seq.nl1 = 0;
  seq.c_lo0 = seq.c_hi0 = seq.c_lo1 = seq.c_hi1 = 0;
  seq.lrb = (uint32_t)Hkv * D * 2;
  seq.lvo = copy_voff(lane, seq.lrb);
  const size_t step_off = ((size_t)b * a_R * Hkv + kvh) * D;
  seq.lk = reinterpret_cast<const u16*>(p.k_step) + step_off;
  seq.lv = reinterpret_cast<const u16*>(p.v_step) + step_off;
  seq.lbytes0 = seq.lbytes1 = 0;
  if (last) {
    const int m_lo = qt * BM;
    const int m_hi = min(M, m_lo + BM) - 1;
    const LocalRanges lr = local_ranges(m_lo / g, m_hi / g, kdr, bl);
    // uniform by construction; readfirstlane keeps the tile loop scalar
    const int n = __builtin_amdgcn_readfirstlane(lr.n);
    if (n > 0) {
      seq.c_lo0 = __builtin_amdgcn_readfirstlane(lr.a0);
      seq.c_hi0 = __builtin_amdgcn_readfirstlane(lr.a1);
      seq.nl0 = __builtin_amdgcn_readfirstlane((seq.c_hi0 - seq.c_lo0 + kBN - 1) / kBN);
      seq.lbytes0 = (uint32_t)(seq.c_hi0 - 1) * seq.lrb + D * 2;  // rows < c_hi are valid
    }
    if (n > 1) {
      seq.c_lo1 = __builtin_amdgcn_readfirstlane(lr.b0);
      seq.c_hi1 = __builtin_amdgcn_readfirstlane(lr.b1);
      seq.nl1 = __builtin_amdgcn_readfirstlane((seq.c_hi1 - seq.c_lo1 + kBN - 1) / kBN);
      seq.lbytes1 = (uint32_t)(seq.c_hi1 - 1) * seq.lrb + D * 2;
    }
  }
  const int ntot = __builtin_amdgcn_readfirstlane(seq.count());

  // Software pipeline over 64-key tiles, one barrier per tile. At the top of
  // iteration t the scores of tile t are in registers (masked, with the
  // reference maximum already raised for them), K[t+1] is in KB[(t+1)&1]
  // and V[t] in VB[t&1]; the copies of K[t+2] and V[t+1] fly while the wave
  // computes QK^T(t+1), P(t) and PV(t).
  typename W::S sA, sB;
  if (ntot > 0) {
    // Only Q and K[0] are waited for before the first QK^T; V[0] and K[1]
    // arrive while it and the first maxima run (every workgroup starts at
    // once, so this start-up burst is what the first wait pays for).
    const TileSrc t0 = seq.at(0);
    if (nk == 0 || nk_hint == 0) {
      // tile 0 is not the first prefix tile: replace whatever the early copy
      // brought (once it has landed) with the right one
      wait_copies();
      copy_tile<D, WAVES>(make_rsrc(t0.k, t0.bytes), t0.vo, t0.row0, t0.row_bytes, KB[0], wave);
    }
    wait_copies();
    __syncthreads();
    copy_tile<D, WAVES>(make_rsrc(t0.v, t0.bytes), t0.vo, t0.row0, t0.row_bytes, VB[0], wave);
    if (ntot > 1) {
      const TileSrc t1 = seq.at(1);
      copy_tile<D, WAVES>(make_rsrc(t1.k, t1.bytes), t1.vo, t1.row0, t1.row_bytes, KB[1], wave);
    }
    if (live) {
      st.qk(KB[0], sA);
      if (t0.local)
        W::template mask<true>(sA, lane, t0.nvalid, t0.c_base, rules);
      else if (t0.nvalid < kBN)
        W::template mask<false>(sA, lane, t0.nvalid, 0, rules);
      st.tile_max(sA, sl2);
    }
    wait_copies();
  }
  if (ntot == 0) wait_copies();  // the early copy lands before KB[0] is reused for staging
  if (STAMP) st_pro = __builtin_amdgcn_s_memtime();  // tile 0's scores and maxima are in registers
  // iterations whose next tile is a full prefix tile run a loop of their own
  const int tmain = __builtin_amdgcn_readfirstlane(max(0, min(nk / kBN, ntot) - 1));
  // Unrolled by two: the scores of the current tile alternate between sA
  // and sB, so no register copies are needed between iterations. Each
  // barrier: all reads of K[t] (QK^T of tile t) and V[t-1] (PV of tile t-1)
  // are done before this iteration's copies overwrite their buffers.
  int t = 0;
  if (live) {
    for (; t + 1 < tmain; t += 2) {
      __syncthreads();
      main_iter<D, NQT, WAVES, LSE32>(st, KB[0], KB[1], VB[0], VB[1], seq, t, wave, sl2, sA, sB);
      __syncthreads();
      main_iter<D, NQT, WAVES, LSE32>(st, KB[1], KB[0], VB[1], VB[0], seq, t + 1, wave, sl2, sB, sA);
    }
    if (t < tmain) {  // an odd count: one more (t even), then the scores move back to sA
      __syncthreads();
      main_iter<D, NQT, WAVES, LSE32>(st, KB[0], KB[1], VB[0], VB[1], seq, t, wave, sl2, sA, sB);
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        sA[nt][0] = sB[nt][0];
        sA[nt][1] = sB[nt][1];
      }
      ++t;
    }
  } else {
    // the same barriers and copies, no compute (a loop of its own, so the
    // computing waves' loop carries no branch)
    for (; t < tmain; ++t) {
      __syncthreads();
      main_iter_copies<D, WAVES>((t & 1) ? KB[1] : KB[0], (t & 1) ? VB[0] : VB[1], seq, t, wave);
    }
  }
  for (; t + 1 < ntot; ++t) {
    const int par = t & 1;
    __syncthreads();
    tile_iter<D, NQT, WAVES, LSE32>(st, par ? KB[1] : KB[0], par ? KB[0] : KB[1], par ? VB[1] : VB[0],
                             par ? VB[0] : VB[1], seq, t, wave, lane, rules, sl2, sA, sB, live);
  }
  if (t < ntot) {  // the last tile: P V only (its V is in VB[t & 1])
    __syncthreads();
    if (live) st.template step<false, false>(nullptr, (t & 1) ? VB[1] : VB[0], sA, sB, sl2);
  }

  if (STAMP) st_loop = __builtin_amdgcn_s_memtime();  // this wave's last tile is done
  // o[nt][dt][v] holds O^T[d = 32*dt + 8*(v/4) + 4*half + v%4][this lane's row].
  // Each 32-row group is normalised, rounded to bf16 and staged row-major in
  // LDS (row pitch 2*D + 16 bytes; the row's output index sits in the
  // padding), then written back as whole rows with 16-byte stores: a store
  // instruction covers complete 128-byte lines instead of 8-byte pieces of
  // 32 different rows. WAVES * NQT == 4, so the four groups take one tile
  // buffer each.
  constexpr int PITCH = 2 * D + 16;
  constexpr int CHUNKS = D / 8;                 // 16-byte pieces per row
  constexpr int PASSES = 32 * CHUNKS / 64;      // store instructions per group
  constexpr int GROUPS = WAVES * NQT;  // 32-row groups of the workgroup, GROUPS / 4 per tile buffer
  static_assert((GROUPS == 4 || GROUPS == 8) && (GROUPS / 4) * 32 * PITCH <= L::TILE_BYTES, "staging does not fit");
  __syncthreads();  // every wave is done with the last tile's K and V
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const int grp = wave * NQT + nt, gb = grp % 4;
    lds_u8* const stage = (gb == 0 ? KB[0] : gb == 1 ? KB[1] : gb == 2 ? VB[0] : VB[1]) + (grp / 4) * 32 * PITCH;
    const float ltot = half_sum(st.l[nt]);
    const int m = qt * BM + wave * WROWS + 32 * nt + l32;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (half == 0) {
      const int r = m / g;
      const uint32_t orow = (uint32_t)((b * a_R + r) * Hq + kvh * g + (m - r * g));
      *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(stage + l32 * PITCH + 2 * D) =
          m < M ? orow : 0xFFFFFFFFu;
    }
    if (m < M && half == 0) {
      const int r = m / g;
      const size_t orow = ((size_t)(b * a_R + r) * Hq + kvh * g + (m - r * g));
      if (S == 1) {
        if (p.lse) p.lse[orow] = (st.m[nt] + log2f(ltot)) * 0.69314718055994531f;
      } else {
        // log2-domain log-sum-exp of this split's partial, written through like the partial
        const float e = ltot > 0.f ? st.m[nt] + log2f(ltot) : kNegInf;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), make_rsrc(p.part_lse + prow_off, 0xFFFFFFFFu),
                                              (int)(orow * 4u), 0, kStoreDevice);
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * half;
        bf16x4 v;
        v[0] = (__bf16)(st.o[nt][dt][4 * i + 0] * inv);
        v[1] = (__bf16)(st.o[nt][dt][4 * i + 1] * inv);
        v[2] = (__bf16)(st.o[nt][dt][4 * i + 2] * inv);
        v[3] = (__bf16)(st.o[nt][dt][4 * i + 3] * inv);
        *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(stage + l32 * PITCH + 2 * d) = v;
      }
    __syncthreads();  // the group's rows are complete in LDS (cheap: once per workgroup)
    // The stores carry device scope (sc1), which writes them through the
    // XCD's L2 as they retire. Plain stores would leave the whole output
    // dirty in L2 (16.5 MB of split partials at the Qwen3-8B step shape),
    // and the end of the kernel writes every dirty line back before the
    // merge may start; written through, that traffic drains while other
    // workgroups still compute. Offsets stay below 2^32: the output holds
    // fewer than 2^31 elements of 2 bytes (checked on the host).
    u16* const obase = S == 1 ? reinterpret_cast<u16*>(p.out) : reinterpret_cast<u16*>(p.part_o) + prow_off * D;
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(obase, 0xFFFFFFFFu);
#pragma unroll
    for (int j = 0; j < PASSES; ++j) {
      const int f = j * 64 + lane;
      const int row = f / CHUNKS, c = f % CHUNKS;
      const uint32_t orow = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(stage + row * PITCH + 2 * D);
      if (orow == 0xFFFFFFFFu) continue;  // past the last query row
      const u32x4 val = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(stage + row * PITCH + 16 * c);
      __builtin_amdgcn_raw_buffer_store_b128(val, orsrc, (int)(orow * (uint32_t)(2 * D) + 16u * (uint32_t)c), 0,
                                             kStoreDevice);
    }
  }
  if (STAMP) {
    // end: this wave's stores acknowledged
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const unsigned long long st_end = __builtin_amdgcn_s_memtime();
    const unsigned long long st_rend = __builtin_amdgcn_s_memrealtime();
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    if (wave == 0 && lane == 0 && wg < kStampMaxWG) {
      const unsigned hw = __builtin_amdgcn_s_getreg(0xF804);   // HW_ID: wave, SIMD, CU, SA, SE
      const unsigned xcc = __builtin_amdgcn_s_getreg(0xF814);  // XCC_ID
      unsigned long long* r = g_attn_stamps + (size_t)wg * kStampFields;
      r[0] = st_entry;
      r[1] = st_rentry;
      r[2] = st_pro;
      r[3] = st_loop;
      r[4] = st_end;
      r[5] = st_rend;
      r[6] = (unsigned long long)hw | ((unsigned long long)xcc << 32);
      r[7] = (unsigned long long)(unsigned)ntot | ((unsigned long long)(unsigned)s << 16) |
             ((unsigned long long)(unsigned)a_nwg << 32);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-regime kernel: few packed query rows per KV head (M = R * g <= 128,
// R <= 128), where the step is bound by streaming the prefix K/V from HBM and
// by latency, not by the matrix work. A workgroup owns one (sequence, KV
// head) and one split: 128 prefix keys (two 64-key tiles), or, for the last
// split, the step's own R keys under the region rule. It issues the copies
// of all its K and V tiles into LDS at entry and then:
//   phase 1: S^T = K Q^T per (32-row tile, 64-key tile) unit, spread over the
//            four waves; row maxima are exchanged through LDS, and the
//            probabilities (rounded to bf16, the row sums from the rounded
//            values as in the main kernel) are written to LDS in the
//            B-operand layout of the P V product, over the K tiles;
//   phase 2: O^T = V^T P^T per (32-row tile, 32-dim tile) unit.
// Each split stores its normalised output (bf16) and log2-domain LSE like
// the main kernel's splits. When the partials of a (sequence, KV head) are
// small, the split that arrives last merges them (arrival counter in the
// workspace, acquire-release at device scope, reset to zero by the merger);
// otherwise the merge kernel runs after this one.
// ---------------------------------------------------------------------------
constexpr int kDecChunk = 128;   // prefix keys per split
constexpr int kDecMaxRows = 128; // packed query rows per (sequence, KV head)
constexpr int kDecMergeLoads = 34;  // partials one thread of the in-kernel merge loads at once

// The body of the decode kernel. The two LDS buffers arrive as restrict
// pointers: the compiler then knows that the V copies in flight do not write
// what phase 1 reads. LSE32 as in the main kernel: the row sums in fp32 from
// the unrounded probabilities when the caller wants the log-sum-exp.
template <int D, bool LSE32>
__device__ __forceinline__ void attn_dec_body(lds_u8* __restrict__ kb, lds_u8* __restrict__ vb,
                                              float (*__restrict__ rmax)[2][32], float (*__restrict__ rsum)[2][32],
                                              int* __restrict__ last_sh, const int32_t* a_len, const void* a_q,
                                              const void* a_kc, const void* a_vc, int a_R, int a_cap, int a_max_len,
                                              int b, int kvh, int s, int NS, int Hkv, int g, int kdr, int bl,
                                              const AttnParams& p) {
  using W = Wave<D, 1, LSE32>;
  using L = Lay<D>;
  constexpr int DSTEPS = D / 16, DT = D / 32;
  const int tid = (int)__builtin_amdgcn_workitem_id_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const bool local = (s == NS - 1);
  const int M = a_R * g, Hq = Hkv * g;
  const int RT = (M + 31) / 32;

  // The keys of this split: [kbeg, kbeg + nk) of the prefix, or the R step
  // keys. The K and V copies go out before the cache length arrives, bounded
  // by the host's max_len. Rows past the length that they bring in may hold
  // anything (NaN included): their scores are masked before any use, and
  // their V rows are cleared in LDS before P V reads the tile.
  const uint32_t prb = D * 2, lrb = (uint32_t)Hkv * D * 2;
  const int kbeg = s * kDecChunk;
  const uint16_t* kbase;
  const uint16_t* vbase;
  uint32_t rb;
  if (local) {
    const size_t off = ((size_t)b * a_R * Hkv + kvh) * D;
    kbase = reinterpret_cast<const u16*>(p.k_step) + off;
    vbase = reinterpret_cast<const u16*>(p.v_step) + off;
    rb = lrb;
  } else {
    const size_t off = ((size_t)(b * Hkv + kvh) * a_cap + kbeg) * D;
    kbase = reinterpret_cast<const u16*>(a_kc) + off;
    vbase = reinterpret_cast<const u16*>(a_vc) + off;
    rb = prb;
  }
  const uint32_t vo = copy_voff(lane, rb);
  const int nk_hint = __builtin_amdgcn_readfirstlane(local ? a_R : max(0, min(kDecChunk, a_max_len - kbeg)));
  const auto bytes_of = [&](int n) { return local ? (uint32_t)(n - 1) * lrb + D * 2 : (uint32_t)n * prb; };
  // Both K tiles and both V tiles are always copied: copies past the
  // resource's end return zeros without touching memory.
  {
    const uint32_t nb = nk_hint > 0 ? bytes_of(nk_hint) : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, nb);
    copy_tile<D, 4>(rk, vo, 0, rb, kb, wave);
    copy_tile<D, 4>(rk, vo, kBN, rb, kb + L::TILE_BYTES, wave);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, nb);
    copy_tile<D, 4>(rv, vo, 0, rb, vb, wave);
    copy_tile<D, 4>(rv, vo, kBN, rb, vb + L::TILE_BYTES, wave);
  }

  // phase 1 units of this wave: u = wave and wave + 4, (row tile, key tile) = (u / 2, u % 2)
  W st[2];
  RowRule rules[2][1];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rt = (wave + 4 * i) >> 1;
    st[i].init_addr(lane);
    st[i].l[0] = 0.f;
    const int m = rt * 32 + l32;
    const bool ok = m < M;
    const int r = ok ? m / g : 0;
    const int h = kvh * g + (ok ? m - r * g : 0);
    rules[i][0] = row_rule(r, kdr, bl);
    // rows past M (and units with no rows) load row 0, which is in bounds, and
    // are zeroed: the loads carry no branch, so they all fly together
    const u16* qp = reinterpret_cast<const u16*>(a_q) + ((size_t)(b * a_R + r) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int d = 0; d < DSTEPS; ++d) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * d);
      st[i].qf[0][d] = ok ? v : bf16x8{};
    }
  }

  int len = __builtin_amdgcn_readfirstlane(a_len[b]);
  if (len < 0 || len > a_max_len) {
    if (tid == 0 && p.dev_status) atomicOr(p.dev_status, 1);
    len = min(max(len, 0), a_max_len);
  }
  const int nk = __builtin_amdgcn_readfirstlane(local ? a_R : max(0, min(kDecChunk, len - kbeg)));
  const int ntiles = (nk + kBN - 1) / kBN;
  bool has[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = wave + 4 * i;
    has[i] = (u >> 1) < RT && (u & 1) < ntiles;
  }
  const float sl2 = p.scale_log2;
  wait_copies();  // this wave's K and V copies and Q rows have landed
  lds_barrier();  // every K and V tile is in LDS

  // Clear the V rows [nk, ntiles * 64) of the last tile in use: copied from
  // past the length, they may hold anything, and P V reads whole tiles (a
  // zero probability times a NaN would still be NaN). Key j of a tile holds
  // 32 bytes in each column pair, at half j / 32, slot j % 32. Nothing reads
  // the V tiles before the barriers that follow phase 1. (The step keys'
  // copies end at the last step key, so their tail arrives as zeros.)
  if (!local && nk < ntiles * kBN) {
    constexpr int PIECES = 2 * L::NCP;  // 16-byte pieces per key
    for (int it = tid; it < (ntiles * kBN - nk) * PIECES; it += 256) {
      const int key = nk + it / PIECES, pc = it % PIECES;
      const int kt = key / kBN, j = key % kBN;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          vb + kt * L::TILE_BYTES + (pc >> 1) * kCPS + (j >> 5) * 1024 + (j & 31) * 32 + (pc & 1) * 16) =
          u32x4{0u, 0u, 0u, 0u};
    }
  }

  typename W::S sc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = wave + 4 * i, rt = u >> 1, kt = u & 1;
    if (rt >= RT) continue;
    float t = kNegInf;
    if (has[i]) {
      st[i].qk(kb + kt * L::TILE_BYTES, sc[i]);
      const int nv = min(kBN, nk - kt * kBN);
      if (local)
        W::template mask<true>(sc[i], lane, nv, kt * kBN, rules[i]);
      else if (nv < kBN)
        W::template mask<false>(sc[i], lane, nv, 0, rules[i]);
      float mx = kNegInf;
#pragma unroll
      for (int q = 0; q < 4; ++q) W::max8(sc[i], 0, q, mx);
      t = half_max(mx) * sl2;
    }
    if (half == 0) rmax[rt][kt][l32] = t;
  }
  lds_barrier();  // row maxima published; every read of the K tiles is done

  // P over the K tiles: slot (row tile, key tile, k-step) of 1 KB, one 16-byte B fragment per lane
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = wave + 4 * i, rt = u >> 1, kt = u & 1;
    if (!has[i]) continue;
    const float mrow = fmaxf(rmax[rt][0][l32], rmax[rt][1][l32]);
    const float muse = mrow == kNegInf ? 0.f : mrow;
    typename W::P pb;
    st[i].probs(sc[i], 0, 0, 32, muse, sl2, pb);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(kb + ((rt * 2 + kt) * 4 + ks) * 1024 +
                                                                  lane * 16) = pb[0][ks];
    const float lsum = half_sum(st[i].l[0]);
    if (half == 0) rsum[rt][kt][l32] = lsum;
  }
  lds_barrier();  // P and the row sums are in LDS

  // phase 2: units (row tile, dim tile), u = wave + 4 j
  W vw;
  vw.init_addr(lane);
  u16* const obase = reinterpret_cast<u16*>(p.part_o) + (size_t)s * p.B * a_R * Hq * D;
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(obase, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t lrsrc = make_rsrc(p.part_lse + (size_t)s * p.B * a_R * Hq, 0xFFFFFFFFu);
  for (int u = wave; u < RT * DT; u += 4) {
    const int rt = u / DT, dt = u % DT;
    f32x16 o = {};
    for (int kt = 0; kt < ntiles; ++kt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 pf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            kb + ((rt * 2 + kt) * 4 + ks) * 1024 + lane * 16);
        o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vw.vfrag(vb + kt * L::TILE_BYTES, ks, dt), pf, o,
                                                    0, 0, 0);
      }
    }
    const int m = rt * 32 + l32;
    if (m >= M) continue;
    const float ltot = (ntiles > 0 ? rsum[rt][0][l32] : 0.f) + (ntiles > 1 ? rsum[rt][1][l32] : 0.f);
    const float mrow = fmaxf(rmax[rt][0][l32], rmax[rt][1][l32]);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const int r = m / g;
    const uint32_t orow = (uint32_t)((b * a_R + r) * Hq + kvh * g + (m - r * g));
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * dt + 8 * i4 + 4 * half;
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(o[4 * i4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16_bits(o[4 * i4 + 1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(o[4 * i4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16_bits(o[4 * i4 + 3] * inv) << 16);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, orsrc, (int)(orow * (uint32_t)(2 * D) + 2u * (uint32_t)d), 0,
                                            kStoreDevice);
    }
    if (dt == 0 && half == 0) {
      const float e = ltot > 0.f ? mrow + log2f(ltot) : kNegInf;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), lrsrc, (int)(orow * 4u), 0, kStoreDevice);
    }
  }
  if (!p.fused_merge) return;

  // ---- merge by the split that arrives last ----
  // The partials were written through to device scope (sc1); once every
  // wave's stores are complete, a device-scope arrival count publishes them.
  // No release fence is needed for that (it would write back the whole L2 of
  // this XCD in every workgroup); only the merging workgroup acquires, and it
  // reads the partials with device-scope loads.
  wait_copies();    // this wave's partial stores are complete
  __syncthreads();  // ... and every wave's
  if (tid == 0) {
    int32_t* ctr = p.counters + (b * Hkv + kvh);
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int is_last = old == NS - 1;
    if (is_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last_sh = is_last;
  }
  __syncthreads();
  if (!*last_sh) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // Every split's partial of this (sequence, KV head): item = (row m < M, 8
  // dims); T threads share an item, thread `sub` of them taking splits sub,
  // sub + T, ... (the host guarantees at most kDecMergeLoads each), all of
  // whose loads are issued before any is used, so the merge costs one memory
  // round trip. The T partial merges are then combined in LDS, in a fixed
  // order (results do not depend on which split arrived last).
  const int items = M * (D / 8);
  const int T = items >= 256 ? 1 : 256 / items;
  const int item = tid / T, sub = tid % T;
  const size_t split_rows = (size_t)p.B * a_R * Hq;
  const __amdgpu_buffer_rsrc_t prsrc = make_rsrc(p.part_o, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t plsrc = make_rsrc(p.part_lse, 0xFFFFFFFFu);
  typedef __attribute__((address_space(3))) float lds_f32;
  lds_f32* const red = reinterpret_cast<lds_f32*>(vb);  // [T][256 / T][10] partial merges
  for (int it0 = 0; it0 < items; it0 += 256 / T) {
    const int it = it0 + item;
    const bool live = it < items;
    const int m = live ? it / (D / 8) : 0, d = live ? (it % (D / 8)) * 8 : 0;
    const int r = m / g;
    const uint32_t orow = (uint32_t)((b * a_R + r) * Hq + kvh * g + (m - r * g));
    float e[kDecMergeLoads];
    u32x4 raw[kDecMergeLoads];
#pragma unroll
    for (int j = 0; j < kDecMergeLoads; ++j) {
      const int sj = sub + j * T;
      const bool in = live && sj < NS;
      const uint32_t prow = (uint32_t)((size_t)(in ? sj : 0) * split_rows + orow);
      e[j] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(plsrc, (int)(prow * 4u), 0, kStoreDevice))
                : kNegInf;
      raw[j] = in ? __builtin_amdgcn_raw_buffer_load_b128(prsrc, (int)(prow * (uint32_t)(2 * D) + 2u * d), 0,
                                                          kStoreDevice)
                  : u32x4{0u, 0u, 0u, 0u};
    }
    float emax = kNegInf;
#pragma unroll
    for (int j = 0; j < kDecMergeLoads; ++j) emax = fmaxf(emax, e[j]);
    float wsum = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (emax != kNegInf) {
#pragma unroll
      for (int j = 0; j < kDecMergeLoads; ++j) {
        const float wgt = __builtin_amdgcn_exp2f(e[j] - emax);  // 0 for an empty or absent split
        wsum += wgt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(__uint_as_float(raw[j][i] << 16), wgt, acc[2 * i]);
          acc[2 * i + 1] = fmaf(__uint_as_float(raw[j][i] & 0xffff0000u), wgt, acc[2 * i + 1]);
        }
      }
    }
    if (T > 1) {
      __syncthreads();  // the previous round's reads of `red` are done
      lds_f32* slot = red + ((size_t)sub * (256 / T) + item) * 10;
      slot[0] = emax;
      slot[1] = wsum;
#pragma unroll
      for (int i = 0; i < 8; ++i) slot[2 + i] = acc[i];
      __syncthreads();
      if (sub != 0) continue;
      // thread 0 of the item folds the others in, in order
      for (int q = 1; q < T; ++q) {
        const lds_f32* o2 = red + ((size_t)q * (256 / T) + item) * 10;
        const float e2 = o2[0];
        const float mx = fmaxf(emax, e2);
        if (mx == kNegInf) continue;
        const float a1 = __builtin_amdgcn_exp2f(emax - mx), a2 = __builtin_amdgcn_exp2f(e2 - mx);
        wsum = wsum * a1 + o2[1] * a2;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] * a1 + o2[2 + i] * a2;
        emax = mx;
      }
    }
    if (!live) continue;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pk[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1] * inv) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<u16*>(p.out) + (size_t)orow * D + d) = pk;
    if (p.lse && d == 0) p.lse[orow] = (emax + log2f(wsum)) * 0.69314718055994531f;
  }
}

template <int D, bool LSE32>
__global__ __launch_bounds__(256, 2) void attn_dec_kernel(
    const int32_t* __restrict__ a_len, const void* __restrict__ a_q, const void* __restrict__ a_kc,
    const void* __restrict__ a_vc, uint32_t a_hkv_g, uint32_t a_k_bl, int a_R, int a_ns, int a_cap,
    int a_max_len, int a_nwg, AttnParams p) {
  using L = Lay<D>;
  static_assert(D == 128, "the decode kernel is built for head_dim 128");
  static_assert(4 * 2 * 4 * 1024 <= 2 * L::TILE_BYTES, "P does not fit over the K tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t kb[2 * L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb[2 * L::TILE_BYTES];
  __shared__ float rmax[4][2][32];  // log2-domain row maxima per (row tile, key tile)
  __shared__ float rsum[4][2][32];  // row sums (of the rounded P) per (row tile, key tile)
  __shared__ int last_sh;
  const int Hkv = (int)(a_hkv_g & 0xffff), g = (int)(a_hkv_g >> 16);
  const int kdr = (int)(a_k_bl & 0xffff), bl = (int)(a_k_bl >> 16);
  const int NS = a_ns;
  int w = remap_xcd((int)__builtin_amdgcn_workgroup_id_x(), a_nwg);
  const int s = w % NS;
  w /= NS;
  const int kvh = w % Hkv;
  const int b = w / Hkv;
  attn_dec_body<D, LSE32>((lds_u8*)kb, (lds_u8*)vb, rmax, rsum, &last_sh, a_len, a_q, a_kc, a_vc, a_R, a_cap, a_max_len, b,
                   kvh, s, NS, Hkv, g, kdr, bl, p);
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
  const int lane = (int)__builtin_amdgcn_workitem_id_x();
  const int D = p.D;
  int w = (int)__builtin_amdgcn_workgroup_id_x();
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
// Arguments are plain scalars so that they are preloaded into scalar registers
// at dispatch and the partial loads need not wait for the argument block.
// Split partials of an output row: with RAG (ragged batches), sequence b's
// splits sit in partial blocks tab[2b] .. tab[2b] + tab[2b+1] - 1 of
// seq_rows rows each; without, split s of every row is block s of `rows`.
//
// Many splits over few rows (the decode regime) would make one thread fold
// its partials in many dependent rounds of loads. There T = 2^lt adjacent
// lanes share an output vector instead: lane `sub` takes splits sub,
// sub + T, ..., all of whose loads (up to CH) go out together, and the T
// partial merges are combined by xor shuffles in a fixed tree, so results
// depend only on T, which the host derives from the plan.
constexpr int kMergeCH = 8;       // splits whose loads one thread has in flight together
constexpr int kMergeMaxLanes = 16;  // lanes that may share one output vector

// log2 of the lanes sharing an output vector for S splits: the fewest that
// keep every thread's partial loads in one round (up to kMergeMaxLanes).
inline int merge_lanes_log2(int S) {
  int lt = 0;
  while ((1 << lt) < kMergeMaxLanes && (long)kMergeCH << lt < (long)S) ++lt;
  return lt;
}

template <bool BF16, bool RAG>
__global__ __launch_bounds__(256) void attn_merge_kernel(const void* __restrict__ part_o,
                                                        const float* __restrict__ part_lse, void* __restrict__ out,
                                                        float* __restrict__ lse, uint32_t rows, uint32_t D,
                                                        uint32_t S, const int32_t* __restrict__ tab,
                                                        uint32_t seq_rows, uint32_t lt) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int CH = kMergeCH;
  const uint32_t tpr = D / VEC;  // output vectors per row
  const uint32_t T = 1u << lt;
  // rows * tpr * T < 2^31 (checked by the host)
  const uint32_t gid = __builtin_amdgcn_workgroup_id_x() * 256u + __builtin_amdgcn_workitem_id_x();
  const uint32_t sub = gid & (T - 1), vid = gid >> lt;
  const uint32_t row = vid / tpr;
  const uint32_t d = (vid - row * tpr) * VEC;
  // the T lanes of a vector share its row, so they leave (or stay) together
  if (row >= rows) return;
  uint32_t s_lo = 0, s_n = S;
  size_t stride = rows, pbase = row;
  if (RAG) {
    const uint32_t b = row / seq_rows;
    s_lo = (uint32_t)tab[2 * b];
    s_n = (uint32_t)tab[2 * b + 1];
    stride = seq_rows;
    pbase = row - b * seq_rows;
  }
  // running merge (reference emax, weight sum, weighted sum), CH splits at a time
  float emax = kNegInf, wsum = 0.f;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  for (uint32_t s0 = 0; s0 < s_n; s0 += CH * T) {
    float e[CH];
    float x[CH][VEC];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t sj = s0 + j * T + sub;
      const bool in = sj < s_n;
      const size_t prow = (size_t)(s_lo + (in ? sj : 0)) * stride + pbase;
      e[j] = in ? part_lse[prow] : kNegInf;
      if (BF16) {
        const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const u16*>(part_o) + prow * D + d);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[j][2 * i] = __uint_as_float(w4[i] << 16);
          x[j][2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
        }
      } else {
        const float4 o = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(part_o) + prow * D + d);
        x[j][0] = o.x;
        x[j][1] = o.y;
        x[j][2] = o.z;
        x[j][VEC - 1] = o.w;
      }
    }
    float cmax = emax;
#pragma unroll
    for (int j = 0; j < CH; ++j) cmax = fmaxf(cmax, e[j]);
    if (cmax == kNegInf) continue;  // nothing visible yet
    const float alpha = __builtin_amdgcn_exp2f(emax - cmax);  // 0 when emax = -inf
    wsum *= alpha;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] *= alpha;
    emax = cmax;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float wgt = __builtin_amdgcn_exp2f(e[j] - cmax);  // 0 for an empty or absent split
      wsum += wgt;
      // in a ragged batch an empty split writes no partial: weigh it by
      // exactly zero, whatever its partial slot holds
      const bool live = !RAG || e[j] != kNegInf;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = fmaf(live ? x[j][i] : 0.f, wgt, acc[i]);
    }
  }
  // combine the T lanes' merges; lane sub = 0 ends with the whole in a fixed order
  for (uint32_t o = 1; o < T; o <<= 1) {
    const float e2 = __shfl_xor(emax, (int)o), w2 = __shfl_xor(wsum, (int)o);
    float a2[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) a2[i] = __shfl_xor(acc[i], (int)o);
    const float mx = fmaxf(emax, e2);
    if (mx == kNegInf) continue;  // neither side has a visible key
    const float c1 = __builtin_amdgcn_exp2f(emax - mx), c2 = __builtin_amdgcn_exp2f(e2 - mx);
    wsum = wsum * c1 + w2 * c2;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = acc[i] * c1 + a2[i] * c2;
    emax = mx;
  }
  if (sub != 0) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (BF16) {
    uint4 pk;
    uint32_t* w4 = reinterpret_cast<uint32_t*>(&pk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w4[i] = (uint32_t)f32_to_bf16_bits(acc[2 * i] * inv) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1] * inv) << 16);
    // written through L2 as in the main kernel's epilogue (byte offsets < 2^32)
    const u32x4 pv = {pk.x, pk.y, pk.z, pk.w};
    __builtin_amdgcn_raw_buffer_store_b128(pv, make_rsrc(out, 0xFFFFFFFFu), (int)((row * D + d) * 2u), 0,
                                           kStoreDevice);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)row * D + d) =
        make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[VEC - 1] * inv);
  }
  if (lse && d == 0) lse[row] = (emax + log2f(wsum)) * 0.69314718055994531f;
}

hipError_t launch_merge(const AttnParams& p, bool bf16, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.R * p.Hq;
  const int32_t* tab = p.ragged ? p.split_tab : nullptr;
  // a ragged batch's per-sequence split counts are known on the device only
  // and stay small; it keeps one lane per output vector
  const int lt = tab ? 0 : merge_lanes_log2(p.S);
  const size_t threads = (rows * (p.D / (bf16 ? 8 : 4))) << lt;
  if (threads > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  const uint32_t seq_rows = (uint32_t)((size_t)p.R * p.Hq);
  if (bf16 && tab)
    hipLaunchKernelGGL((attn_merge_kernel<true, true>), dim3(grid), dim3(256), 0, stream, p.part_o, p.part_lse, p.out,
                       p.lse, (uint32_t)rows, (uint32_t)p.D, (uint32_t)p.S, tab, seq_rows, (uint32_t)lt);
  else if (bf16)
    hipLaunchKernelGGL((attn_merge_kernel<true, false>), dim3(grid), dim3(256), 0, stream, p.part_o, p.part_lse, p.out,
                       p.lse, (uint32_t)rows, (uint32_t)p.D, (uint32_t)p.S, tab, seq_rows, (uint32_t)lt);
  else
    hipLaunchKernelGGL((attn_merge_kernel<false, false>), dim3(grid), dim3(256), 0, stream, p.part_o, p.part_lse,
                       p.out, p.lse, (uint32_t)rows, (uint32_t)p.D, (uint32_t)p.S, tab, seq_rows, (uint32_t)lt);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attn(int dtype, int B, int Hq, int Hkv, int D, int R, int max_len, int forced_splits,
                   int local_tiles) {
  AttnPlan pl{};
  const int g = Hq / Hkv;
  const long M = (long)R * g;
  long base;
  // Decode regime (few packed rows per KV head): a latency-bound kernel that
  // copies a whole 128-key split into LDS at once. On MI355X it beats the
  // main kernel for up to 32 packed rows per KV head when its workgroups fit
  // one per CU (256) in one round; past that (e.g. 8 KV heads at 4096
  // prefix keys: 264 workgroups) and for more rows the main kernel is
  // faster. TIDAR_ATTN_DECODE=1 selects it wherever it applies (up to 128
  // rows), =0 never. Its splits are merged by the merge kernel;
  // TIDAR_ATTN_FUSED_MERGE=1 merges them inside the kernel instead (by the
  // last-arriving split, within its load bound), which measured slower.
  const long dec_S = (max_len + kDecChunk - 1) / kDecChunk + 1;  // prefix splits, then the step keys
  const char* dec_env = getenv("TIDAR_ATTN_DECODE");
  const bool dec_auto = M <= 32 && (long)B * Hkv * dec_S <= 256;
  const bool dec_on = dec_env ? atoi(dec_env) == 1 : dec_auto;
  if (dtype == 1 && D == 128 && M <= kDecMaxRows && R <= 128 && forced_splits == 0 && dec_on) {
    pl.decode = 1;
    pl.nqt = 1;
    pl.waves = 4;
    pl.bm = kBM;
    pl.qtiles = 1;
    pl.chunk = kDecChunk;
    pl.S = (int)dec_S;
    const long items = M * (D / 8);
    const long T = items >= 256 ? 1 : 256 / items;
    const bool fits = (pl.S + T - 1) / T <= kDecMergeLoads;
    pl.fused_merge = 0;
    if (const char* e = getenv("TIDAR_ATTN_FUSED_MERGE")) pl.fused_merge = fits && atoi(e) != 0;
    pl.counter_bytes = ((size_t)B * Hkv * sizeof(int32_t) + 255) / 256 * 256;
    const size_t prow = (size_t)pl.S * B * R * Hq;
    pl.ws_bytes = pl.counter_bytes + (prow * D * 2 + 255) / 256 * 256 + prow * sizeof(float);
    return pl;
  }
  if (dtype == 1) {
    // 32 query rows per wave, four waves; TIDAR_ATTN_WAVES=8 selects 8-wave
    // workgroups of 256 rows (a tuning knob, built for head_dim 128 only)
    pl.nqt = 1;
    pl.waves = 4;
    if (const char* e = getenv("TIDAR_ATTN_WAVES")) pl.waves = (atoi(e) == 8 && D == 128) ? 8 : 4;
    pl.bm = pl.waves == 8 ? 2 * kBM : kBM;
    pl.qtiles = (int)((M + pl.bm - 1) / pl.bm);
    base = (long)B * Hkv * pl.qtiles;
  } else {
    pl.nqt = 1;
    pl.bm = 1;
    pl.qtiles = (int)M;
    base = (long)B * Hkv * M;
  }
  const int ntiles = (max_len + kBN - 1) / kBN;
  // Batches of several sequences (bf16, no forced split count): the split
  // slots are shared out on the device in proportion to each sequence's key
  // tiles, so short sequences take few workgroups and long ones many, in one
  // round of resident workgroups. TIDAR_ATTN_RAGGED=0 keeps one split count
  // for every sequence instead.
  const char* ragged_env = getenv("TIDAR_ATTN_RAGGED");
  if (dtype == 1 && B > 1 && forced_splits == 0 && !(ragged_env && atoi(ragged_env) == 0)) {
    const long slots = pl.waves == 8 ? 256 : 512;
    long ns = slots / ((long)Hkv * pl.qtiles);
    ns = std::min(ns, (long)B * (ntiles + local_tiles));
    ns = std::min(ns, 0xffffL);
    if (ns > B) {
      pl.ragged = 1;
      pl.S = (int)ns;
      pl.chunk = 0;
      pl.counter_bytes = ((size_t)B * 2 * sizeof(int32_t) + 255) / 256 * 256;
      const size_t prow = (size_t)pl.S * R * Hq;
      pl.ws_bytes = pl.counter_bytes + (prow * D * 2 + 255) / 256 * 256 + prow * sizeof(float);
      return pl;
    }
  }
  int S;
  int bal_ch = 0;  // split size in tiles that counts the step-key tiles into the last split's share (0: none)
  const char* target_env = getenv("TIDAR_ATTN_TARGET_WG");
  if (forced_splits > 0) {
    S = forced_splits;
  } else if (dtype == 1 && !target_env) {
    // bf16: pick the split count from a cost model in shader cycles whose
    // constants were measured on this kernel (head_dim 128, MI355X):
    //  - a workgroup costs F (prologue and epilogue) plus t per 64-key tile;
    //    t is lower when the workgroup has its CU to itself (at most 256
    //    workgroups) than when two share it; past 512 the workgroups run in
    //    further rounds;
    //  - the split that owns the last prefix keys also has the step's keys;
    //  - the merge of S > 1 partials costs a fixed part (its launch and the
    //    kernel boundary), a part that grows by 2500 cycles per 8 splits and
    //    a part per partial element (~3.3 TB/s). The second term was fitted
    //    when the merge folded 8 partials per memory round trip; the merge
    //    now loads up to 128 at once, but a sweep of forced split counts on
    //    the append-prefill shapes still puts the best counts where this
    //    term does (it also stands for the costs of more, shorter splits).
    const double F = 16000.0, t1 = 2650.0 * D / 128, t2 = 3300.0 * D / 128;
    const double part_elems = (double)B * R * Hq * D;
    double best = 0.0;
    S = 1;
    for (int st = 1; st <= std::max(1, std::min(ntiles, 64)); ++st) {
      const int ch = ntiles > 0 ? (ntiles + st - 1) / st : 1;
      const int se = ntiles > 0 ? (ntiles + ch - 1) / ch : 1;
      if (se != st) continue;  // the same plan as a smaller count
      const long wgs = base * se;
      // 8-wave workgroups: one per CU, two waves per SIMD already
      const long slots = pl.waves == 8 ? 256 : 512;
      const long rounds = (wgs + slots - 1) / slots;
      const double t = (pl.waves == 8 || wgs > 256) ? t2 : t1;
      const int n_last = ntiles - (se - 1) * ch + local_tiles;
      const double cost = rounds * (F + std::max(ch, n_last) * t) +
                          (se > 1 ? 6000.0 + 2500.0 * ((se + 7) / 8) + se * part_elems * 1.26e-3 : 0.0);
      if (st == 1 || cost < best) {
        best = cost;
        S = se;
      }
    }
    // Same split count, boundaries moved so that the last split's step-key
    // tiles count towards its share: ceil((prefix + w * step-key tiles) / S)
    // prefix tiles for every split but the last, with w = 2 (a step-key tile
    // goes through the region rule and the masked tile path, and costs about
    // two prefix tiles), else w = 1, whichever first still makes S splits.
    // With 512 causal rows over 4096 keys, 8 step-key tiles: splits of 20,
    // 20, 20 and 4 + 8 tiles instead of 16, 16, 16 and 16 + 8.
    for (int wl = 2; wl >= 1 && bal_ch == 0 && ntiles > 0 && local_tiles > 0; --wl) {
      const int ch = (ntiles + wl * local_tiles + S - 1) / S;
      if ((ntiles + ch - 1) / ch == S) bal_ch = ch;
    }
  } else {
    // Fill the resident workgroup slots (two per CU on the 256-CU part) in
    // one round: a second, partial round would cost as much as the first.
    // Keep at least two key tiles per split. TIDAR_ATTN_TARGET_WG sets the
    // slot count (and selects this rule for bf16 too).
    long slots = 512;
    if (target_env) slots = std::max(1L, atol(target_env));
    S = (int)std::max(1L, slots / base);
    S = std::max(1, std::min(S, std::max(1, ntiles / 2)));
  }
  S = std::max(1, std::min(S, std::max(1, ntiles)));
  int chunk = ntiles > 0 ? (bal_ch > 0 ? bal_ch : (ntiles + S - 1) / S) * kBN : kBN;
  S = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  pl.S = S;
  pl.chunk = chunk;
  // TIDAR_ATTN_STAMPS=1: the timestamped instantiation where it exists
  if (const char* e = getenv("TIDAR_ATTN_STAMPS")) pl.stamps = dtype == 1 && atoi(e) == 1;
  // partial outputs in the input precision, then one fp32 log-sum-exp per row
  const size_t prow = (size_t)S * B * R * Hq;
  const size_t elem = dtype == 1 ? 2 : 4;
  pl.ws_bytes = S > 1 ? (prow * D * elem + 255) / 256 * 256 + prow * sizeof(float) : 0;
  return pl;
}

hipError_t launch_attn_bf16(const AttnParams& p, hipStream_t stream) {
  if (p.decode) {
    const size_t grid = (size_t)p.B * p.Hkv * p.S;
    if (grid > 0x7fffffff || p.Hkv > 0xffff || p.g > 0xffff || p.k > 0xffff || p.block_len > 0xffff || p.D != 128)
      return hipErrorInvalidValue;
    const uint32_t hkv_g = (uint32_t)p.Hkv | ((uint32_t)p.g << 16);
    const uint32_t k_bl = (uint32_t)p.k | ((uint32_t)p.block_len << 16);
    if (p.lse)
      hipLaunchKernelGGL((attn_dec_kernel<128, true>), dim3((unsigned)grid), dim3(256), 0, stream, p.cache_len, p.q,
                         p.k_cache, p.v_cache, hkv_g, k_bl, p.R, p.S, p.cap, p.max_len, (int)grid, p);
    else
      hipLaunchKernelGGL((attn_dec_kernel<128, false>), dim3((unsigned)grid), dim3(256), 0, stream, p.cache_len, p.q,
                         p.k_cache, p.v_cache, hkv_g, k_bl, p.R, p.S, p.cap, p.max_len, (int)grid, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.fused_merge) return e;
    return launch_merge(p, true, stream);
  }
  const size_t grid = (size_t)(p.ragged ? 1 : p.B) * p.Hkv * p.qtiles * p.S;
  if (grid > 0x7fffffff || p.qtiles > 0xffff || p.S > 0xffff || p.Hkv > 0xffff || p.g > 0xffff || p.k > 0xffff ||
      p.block_len > 0xffff || (p.ragged && (!p.split_tab || p.S <= p.B)))
    return hipErrorInvalidValue;
  const uint32_t qt_s = (uint32_t)p.qtiles | ((uint32_t)p.S << 16);
  const uint32_t hkv_g = (uint32_t)p.Hkv | ((uint32_t)p.g << 16);
  const uint32_t k_bl = (uint32_t)p.k | ((uint32_t)p.block_len << 16);
#define TIDAR_ATTN_ARGS                                                                                       \
  p.cache_len, p.q, p.k_cache, qt_s, hkv_g, k_bl, p.R, (int)grid, p.cap, p.chunk, p.max_len, p
  // 128 query rows per workgroup (four waves of 32 rows), or 256 (eight
  // waves, head_dim 128); the row sums in fp32 when the caller wants the LSE
  const bool l32 = p.lse != nullptr;
#define TIDAR_LAUNCH2(D_, W_, L_, R_, P_)                                                                        \
  hipLaunchKernelGGL((attn_bf16_kernel<D_, 1, W_, L_, R_, P_>), dim3((unsigned)grid), dim3(64 * W_), 0, stream, \
                     TIDAR_ATTN_ARGS)
#define TIDAR_LAUNCH1(D_, W_, L_, R_)          \
  do {                                         \
    if (pad)                                   \
      TIDAR_LAUNCH2(D_, W_, L_, R_, true);     \
    else                                       \
      TIDAR_LAUNCH2(D_, W_, L_, R_, false);    \
  } while (0)
#define TIDAR_LAUNCH(D_, W_, L_)        \
  do {                                  \
    if (p.ragged)                       \
      TIDAR_LAUNCH1(D_, W_, L_, true);  \
    else                                \
      TIDAR_LAUNCH1(D_, W_, L_, false); \
  } while (0)
  // packed query rows that leave the last tile (32 rows per wave) partly empty
  const bool pad = ((size_t)p.R * p.g) % (size_t)(32 * p.waves * p.nqt) != 0;
  if (p.stamps && p.D == 128 && p.waves == 4 && !l32 && !p.ragged && !pad && grid <= (size_t)kStampMaxWG) {
    hipLaunchKernelGGL((attn_bf16_kernel<128, 1, 4, false, false, false, true>), dim3((unsigned)grid), dim3(256), 0,
                       stream, TIDAR_ATTN_ARGS);
  } else if (p.D == 128 && p.waves == 8) {
    if (l32) TIDAR_LAUNCH(128, 8, true); else TIDAR_LAUNCH(128, 8, false);
  } else if (p.D == 128 && p.waves == 4) {
    if (l32) TIDAR_LAUNCH(128, 4, true); else TIDAR_LAUNCH(128, 4, false);
  } else if (p.D == 64 && p.waves == 4) {
    if (l32) TIDAR_LAUNCH(64, 4, true); else TIDAR_LAUNCH(64, 4, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef TIDAR_LAUNCH
#undef TIDAR_LAUNCH1
#undef TIDAR_LAUNCH2
#undef TIDAR_ATTN_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  return launch_merge(p, true, stream);
}

hipError_t read_attn_stamps(unsigned long long* host_dst, int max_workgroups) {
  const int n = std::min(std::max(max_workgroups, 0), kStampMaxWG);
  if (n == 0) return hipSuccess;
  return hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(g_attn_stamps), (size_t)n * kStampFields * sizeof(unsigned long long),
                             0, hipMemcpyDeviceToHost);
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.B * p.Hkv * (size_t)p.R * p.g * p.S);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(grid), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  return launch_merge(p, false, stream);
}

}  // namespace tidar
