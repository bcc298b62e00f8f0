// Stage 2: max-based dynamic threshold plus sink / window / recent blocks,
// emitted as a CSR index ("FlashPrefill V2", Sec. 3.1 threshold paragraph and
// the CSR paragraph; thresh_I = alpha * max_J Score_IJ is printed in the
// core-method section of the FlashPrefill summary page).
//
// Three launches, no scratch memory:
//   count  four segments per workgroup, one per wave: row max, threshold,
//          |Sel| via ballots, with the exact re-decision below (all four
//          waves evaluate any wave's uncertain blocks together);
//   scan   one workgroup: exclusive prefix of the counts -> cu;
//   emit   one wave per segment: the count pass's decisions, survivors
//          written ascending at cu[s] (ballot + lane prefix = in-order
//          compaction).
// The count pass hands its exact decisions to the emit pass in the scores
// themselves: an uncertain block it drops gets its score negated (scores are
// positive, so every other pass reads them through fabsf), and the emit pass
// takes the sign as the decision and restores the score.
//
// Exact decisions near the threshold.  The scores carry a small relative
// error (the block-score kernel's bf16 split of kbar and float32
// accumulation: below kScoreErr).  A block whose score lies within
// 2 kScoreErr of thresh_I, relative, is re-decided in float64: its energy
// E_J = sum_r exp(s_rJ - m) over the tile's rows, s_rJ = scale q_r . kbar_J,
// against alpha max_K E_K, the maximum taken exactly over every block whose
// score is within 2 kScoreErr of the largest.  Normalisation and the common
// reference m cancel in Score_IJ >= alpha max_K Score_IK, so this is the
// threshold comparison of the definition, evaluated exactly.
#include "common.hpp"
#include "launch.hpp"

namespace bslp {

// Bound on the relative error of a block score (checked by the tests).
constexpr float kScoreErr = 1e-3f;

struct SegPos {
  int b, h, I;
  int64_t off;  // first score element
};

// What the exact re-decision reads: the query rows and the pooled keys.
struct RefineArgs {
  const void* q;       // [T, Hq, d] in the problem dtype
  const float* kbar;   // [pooled rows, Hkv, d]
  int dtype;
  float lscale;        // softmax_scale * q_scale (host scales)
};

__device__ __forceinline__ SegPos segment_position(const Plan& p, int64_t seg) {
  SegPos r;
  r.b = seq_of_segment(p, seg);
  const SeqInfo& s = p.seq[r.b];
  segment_tile(s, (int)(seg - s.seg_base), r.h, r.I);
  r.off = score_offset(s, r.h, r.I);
  return r;
}

// Blocks forced into every selection of tile I: sink = [0, sink), and the
// window + recent band = [I - recent - window + 1, I].
__device__ __forceinline__ bool forced(int J, int I, const SelectArgs& a) {
  return J < a.sink || J >= I - a.recent - a.window + 1;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}


__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmax(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ---- exact evaluation of block energies, shared by a workgroup
//
// A workgroup holds four segments, one per wave.  Every wave walks its own
// segment; the blocks that need an exact energy (the candidates for the
// largest, then the blocks in the uncertain band) are posted in LDS, up to
// kItems per wave at a time, and all 256 threads evaluate the posted blocks
// of the four waves together: thread t takes the tile's rows t, t + 256, ...,
// loads each row once for all of its wave's posted blocks, and keeps an
// online (max, sum of exp) pair per block; the pairs meet in a fixed order.
// The result is log E_J = m + log(sum_r exp(s_rJ - m)) in float64.

constexpr int kWaves = 4;
constexpr int kItems = 4;

struct SegShared {
  int n_items[kWaves];              // posted blocks per wave
  int h[kWaves], q0[kWaves], R[kWaves];
  int64_t row0[kWaves];             // Q row of query position 0 of the wave's request
  float kd[kWaves][kItems][128];    // kbar of the posted blocks
  double pm[kWaves][kItems][kWaves], pe[kWaves][kItems][kWaves];  // [.][.][evaluating wave]
};

__device__ __forceinline__ void lse_merge(double& m, double& e, double m2, double e2) {
  const double M = fmax(m, m2);
  if (M == -INFINITY) return;  // both empty
  e = e * exp(m - M) + e2 * exp(m2 - M);
  m = M;
}

__device__ __forceinline__ void lse_add(double& m, double& e, double x) {
  if (x > m) {
    e = e * exp(m - x) + 1.0;  // exp(-inf) = 0 on the first logit
    m = x;
  } else {
    e += exp(x - m);
  }
}

// Query dims taken per load batch, all loads of a batch in flight together:
// at most 64 registers of raw data (128 bf16 or e4m3 dims, 64 float32 ones).
template <int DT, int D>
constexpr int kBatchDims = (DT == kF32 || D < 128) ? 64 : 128;

// One query element of a raw batch as float (bf16 / e4m3 / float32 words).
template <int DT>
__device__ __forceinline__ float raw_elem(const uint32_t* w, int c) {
  if constexpr (DT == kF32) {
    return __uint_as_float(w[c]);
  } else if constexpr (DT == kBF16) {
    return __uint_as_float((c & 1) ? (w[c >> 1] & 0xffff0000u) : (w[c >> 1] << 16));
  } else {
    const uint32_t x = w[c >> 2];
    switch (c & 3) {  // the byte select must be a constant (c is, once unrolled)
      case 0: return __builtin_amdgcn_cvt_f32_fp8(x, 0);
      case 1: return __builtin_amdgcn_cvt_f32_fp8(x, 1);
      case 2: return __builtin_amdgcn_cvt_f32_fp8(x, 2);
      default: return __builtin_amdgcn_cvt_f32_fp8(x, 3);
    }
  }
}

// Dot products of one batch of query dims with the posted kbar rows,
// accumulated in float64: every product of a float32 kbar element and a
// query element is exact there.
template <int DT, int BD>
__device__ __forceinline__ void dot_batch(const typename Elem<DT>::T* __restrict__ q, int64_t off,
                                          const float* kd, int c0, int n,
                                          double (&acc)[kItems]) {
  constexpr int W = BD * (int)sizeof(typename Elem<DT>::T) / 4;  // 32-bit words
  uint32_t w[W];
  const uint4* src = reinterpret_cast<const uint4*>(q + off);
#pragma unroll
  for (int i = 0; i < W / 4; ++i) {
    const uint4 u = src[i];
    w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
  }
#pragma unroll 1
  for (int k = 0; k < n; ++k) {
    // the raw words pass an empty asm per block, so their float64 forms are
    // made inside this loop rather than kept for every block at once
#pragma unroll
    for (int i = 0; i < W; ++i) asm volatile("" : "+v"(w[i]));
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int c = 0; c < BD; c += 2) {
      a0 = fma((double)raw_elem<DT>(w, c), (double)kd[k * 128 + c0 + c], a0);
      a1 = fma((double)raw_elem<DT>(w, c + 1), (double)kd[k * 128 + c0 + c + 1], a1);
    }
    switch (k) {  // registers cannot be indexed at run time
      case 0: acc[0] += a0 + a1; break;
      case 1: acc[1] += a0 + a1; break;
      case 2: acc[2] += a0 + a1; break;
      default: acc[3] += a0 + a1; break;
    }
  }
}

template <int DT, int D>
__device__ void evaluate_posted(int g, int hq, const RefineArgs& ra, double lscale, SegShared& sh,
                                int tid) {
  const auto* q = static_cast<const typename Elem<DT>::T*>(ra.q);
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll 1
  for (int w = 0; w < kWaves; ++w) {
    const int n = sh.n_items[w];  // uniform
    if (n == 0) continue;
    const int h = sh.h[w], q0 = sh.q0[w], R = sh.R[w];  // rows of PackGQA group g
    const int64_t row0 = sh.row0[w];
    double m[kItems], e[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      m[k] = -INFINITY;
      e[k] = 0.0;
    }
#pragma unroll 1
    for (int r = tid; r < R; r += kWaves * 64) {
      const int64_t off = ((row0 + q0 + r / g) * hq + h * g + r % g) * D;
      double acc[kItems];
#pragma unroll
      for (int k = 0; k < kItems; ++k) acc[k] = 0.0;
      // an offset the compiler cannot see through, so that the kbar reads
      // stay in the loop (hoisted, they would take 4 x 128 registers)
      int opaque = 0;
      asm volatile("" : "+v"(opaque));
      const float* kd = &sh.kd[w][0][0] + opaque;
      constexpr int BD = kBatchDims<DT, D>;
#pragma unroll 1
      for (int c0 = 0; c0 < D; c0 += BD) dot_batch<DT, BD>(q, off + c0, kd, c0, n, acc);
#pragma unroll
      for (int k = 0; k < kItems; ++k)
        if (k < n) lse_add(m[k], e[k], acc[k] * lscale);
    }
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      if (k >= n) break;
      double mk = m[k], ek = e[k];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double m2 = __shfl_xor(mk, off), e2 = __shfl_xor(ek, off);
        lse_merge(mk, ek, m2, e2);
      }
      if (lane == 0) {
        sh.pm[w][k][wave] = mk;
        sh.pe[w][k][wave] = ek;
      }
    }
  }
}

// Kernel arguments stay out of the call: a Plan passed by reference to a
// function that is not inlined would be copied to scratch first.
__device__ void evaluate_dispatch(int d, int g, int hq, const RefineArgs& ra, double lscale,
                                  SegShared& sh, int tid) {
  if (ra.dtype == kBF16) {
    if (d == 128) evaluate_posted<kBF16, 128>(g, hq, ra, lscale, sh, tid);
    else evaluate_posted<kBF16, 64>(g, hq, ra, lscale, sh, tid);
  } else if (ra.dtype == kFP8) {
    if (d == 128) evaluate_posted<kFP8, 128>(g, hq, ra, lscale, sh, tid);
    else evaluate_posted<kFP8, 64>(g, hq, ra, lscale, sh, tid);
  } else {
    if (d == 128) evaluate_posted<kF32, 128>(g, hq, ra, lscale, sh, tid);
    else evaluate_posted<kF32, 64>(g, hq, ra, lscale, sh, tid);
  }
}

// ---- one segment's walk, shared by the count and emit passes
//
// Two cursors over the segment's 64-block chunks.  The gather cursor lists,
// in order, the candidates for the largest energy (score within 2 kScoreErr
// of the largest score; phase 0) and then the blocks in the uncertain band
// (phase 1); they are posted kItems at a time.  The decide cursor builds each
// chunk's keep mask from the scores, overwrites the uncertain blocks' bits
// with their exact decisions (log E_J >= log alpha + max log E over the
// candidates) as they arrive, and hands every finished chunk to the pass.
// Threshold and the uncertain band of a segment with largest score smax,
// computed identically by both passes.
struct Band {
  float thresh, lo, hi, top;
};
__device__ __forceinline__ Band band_of(float smax, float alpha) {
  Band b;
  b.thresh = alpha * smax;
  b.lo = b.thresh * (1.f - 2.f * kScoreErr);
  b.hi = b.thresh * (1.f + 2.f * kScoreErr);
  b.top = smax * (1.f - 2.f * kScoreErr);
  return b;
}

struct Walk {
  float thresh, lo, hi, top;
  int n, I;
  int gphase, gJ0;     // gather cursor
  uint64_t gmask;      // its blocks of chunk gJ0 not yet posted
  int dJ0;             // decide cursor: the chunk being built
  uint64_t keep, pend; // its keep mask; its uncertain blocks not yet decided
  double lemax, lalpha;
  bool refine;
};

// Scores are read through fabsf: the count pass negates the scores of the
// uncertain blocks it drops (see select_count_kernel).
__device__ __forceinline__ float score_at(const float* row, int J) { return fabsf(row[J]); }

__device__ __forceinline__ bool is_candidate(const Walk& w, const float* row, int J) {
  return J < w.n && score_at(row, J) >= w.top;
}

__device__ __forceinline__ bool is_uncertain(const Walk& w, const SelectArgs& a, const float* row,
                                             int J) {
  if (J >= w.n || forced(J, w.I, a)) return false;
  const float sc = score_at(row, J);
  return sc >= w.lo && sc <= w.hi;
}

__device__ __forceinline__ void decide_start(Walk& w, const SelectArgs& a, const float* row,
                                             int lane) {
  const int J = w.dJ0 + lane;
  const bool in = J < w.n;
  w.keep = __ballot(in && (score_at(row, J) >= w.thresh || forced(J, w.I, a)));
  w.pend = w.refine ? __ballot(is_uncertain(w, a, row, J)) : 0ull;
}

__device__ __forceinline__ Walk walk_begin(const SelectArgs& a, const SegPos& sp,
                                           const float* row, int lane) {
  Walk w;
  w.n = sp.I + 1;
  w.I = sp.I;
  float mx = -INFINITY;
  for (int J = lane; J < w.n; J += 64) mx = fmaxf(mx, score_at(row, J));
  const Band bd = band_of(wave_max(mx), a.alpha);
  w.thresh = bd.thresh;
  w.lo = bd.lo;
  w.hi = bd.hi;
  w.top = bd.top;
  w.refine = false;
  if (a.alpha > 0.f) {
    bool unc = false;
    for (int J = lane; J < w.n; J += 64) unc |= is_uncertain(w, a, row, J);
    w.refine = __ballot(unc) != 0ull;
  }
  w.lemax = -INFINITY;
  w.lalpha = a.alpha > 0.f ? log((double)a.alpha) : 0.0;
  w.gphase = w.refine ? 0 : 2;
  w.gJ0 = 0;
  w.gmask = w.refine ? __ballot(is_candidate(w, row, lane)) : 0ull;
  w.dJ0 = 0;
  decide_start(w, a, row, lane);
  return w;
}

// Next block for the gather cursor, -1 when both phases are exhausted.
__device__ int gather_next(Walk& w, const SelectArgs& a, const float* row, int lane) {
  for (;;) {
    if (w.gphase == 2) return -1;
    if (w.gmask) {
      const int J = w.gJ0 + __builtin_ctzll(w.gmask);
      w.gmask &= w.gmask - 1;
      return J;
    }
    w.gJ0 += 64;
    if (w.gJ0 >= w.n) {
      if (++w.gphase == 2) return -1;
      w.gJ0 = 0;
    }
    const int J = w.gJ0 + lane;
    w.gmask = __ballot(w.gphase == 0 ? is_candidate(w, row, J) : is_uncertain(w, a, row, J));
  }
}

// Hands finished chunks to the pass: every chunk before block J (J = n: all).
template <class F>
__device__ void decide_until(Walk& w, const SelectArgs& a, const float* row, int lane, int J,
                             F&& consume) {
  while (w.dJ0 < w.n && J >= w.dJ0 + 64) {
    consume(w.dJ0, w.keep);
    w.dJ0 += 64;
    if (w.dJ0 < w.n) decide_start(w, a, row, lane);
  }
  if (J >= w.n && w.dJ0 < w.n) {
    consume(w.dJ0, w.keep);
    w.dJ0 = w.n;
  }
}

// The workgroup loop: every wave walks its segment; posted blocks are
// evaluated by all threads between two barriers.
template <class F>
__device__ void select_segments(const Plan& p, const SelectArgs& a, const RefineArgs& ra,
                                float* scores, SegShared& sh, int64_t seg, F&& consume) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool active = seg < p.num_segments;
  SegPos sp{0, 0, 0, 0};
  if (active) sp = segment_position(p, seg);
  float* row = scores + sp.off;
  const double lscale = (double)ra.lscale * (p.dscale ? (double)p.dscale[0] : 1.0);
  Walk w;
  bool more = false;
  if (active) {
    w = walk_begin(a, sp, row, lane);
    more = w.refine;
    if (!more) decide_until(w, a, row, lane, w.n, consume);
  }
  const SeqInfo s = p.seq[sp.b];
  if (lane == 0) {
    sh.h[wave] = sp.h;
    sh.q0[wave] = tile_q0(s, sp.I, p.B);
    sh.R[wave] = p.g * tile_nq(s, sp.I, p.B);
    sh.row0[wave] = q_row(s, 0);
  }
  const float* kb_head = ra.kbar + ((int64_t)s.pool_base * p.hkv + sp.h) * p.d;
  while (__syncthreads_or(more)) {
    int items[kItems], phases[kItems];
    int n = 0;
    if (more) {
      for (; n < kItems; ++n) {
        items[n] = gather_next(w, a, row, lane);
        phases[n] = w.gphase;  // the phase of the returned block (the call may advance it)
        if (items[n] < 0) break;
        for (int c = lane; c < p.d; c += 64)
          sh.kd[wave][n][c] = kb_head[(int64_t)items[n] * p.hkv * p.d + c];
      }
    }
    if (lane == 0) sh.n_items[wave] = n;
    __syncthreads();
    evaluate_dispatch(p.d, p.g, p.hq, ra, lscale, sh, tid);
    __syncthreads();
    for (int k = 0; k < n; ++k) {
      double m = sh.pm[wave][k][0], e = sh.pe[wave][k][0];
#pragma unroll
      for (int v = 1; v < kWaves; ++v) lse_merge(m, e, sh.pm[wave][k][v], sh.pe[wave][k][v]);
      const double lE = m + log(e);
      if (phases[k] == 0) {
        w.lemax = fmax(w.lemax, lE);
      } else {
        decide_until(w, a, row, lane, items[k], consume);
        const uint64_t bit = 1ull << (items[k] - w.dJ0);
        if (lE >= w.lalpha + w.lemax) {
          w.keep |= bit;
        } else {
          w.keep &= ~bit;
          // the drop is handed to the emit pass as a negated score
          if (lane == 0) row[items[k]] = -score_at(row, items[k]);
        }
        w.pend &= ~bit;
      }
    }
    if (more && w.gphase == 2) {
      decide_until(w, a, row, lane, w.n, consume);
      more = false;
    }
  }
}

// Count pass: the whole decision, exact near the threshold.  An uncertain
// block that the exact comparison drops has its score negated, so the emit
// pass reads every decision from the scores alone (and restores them).
__global__ __launch_bounds__(256, 2) void select_count_kernel(Plan p, SelectArgs a, RefineArgs ra,
                                                           float* scores,
                                                           int32_t* __restrict__ counts) {
  __shared__ SegShared sh;
  const int64_t seg = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  int cnt = 0;
  select_segments(p, a, ra, scores, sh, seg,
                  [&](int, uint64_t keep) { cnt += __popcll(keep); });
  if (seg < p.num_segments && (threadIdx.x & 63) == 0) counts[seg] = cnt;
}

// Exclusive prefix sum over all segment counts, one workgroup of 1024 threads;
// each thread owns ITEMS consecutive counts per sweep.
__global__ __launch_bounds__(1024) void select_scan_kernel(int64_t n, const int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ cu) {
  constexpr int ITEMS = 8;
  constexpr int NT = 1024;
  __shared__ int32_t wsum[NT / 64];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += (int64_t)NT * ITEMS) {
    int32_t v[ITEMS];
    int32_t tsum = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t e = base + (int64_t)tid * ITEMS + i;
      v[i] = e < n ? counts[e] : 0;
      tsum += v[i];
    }
    // inclusive scan of tsum across the wave
    int32_t x = tsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int32_t w = lane < NT / 64 ? wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < NT / 64; off <<= 1) {
        const int32_t y = __shfl_up(w, off);
        if (lane >= off) w += y;
      }
      if (lane < NT / 64) wsum[lane] = w;  // inclusive over waves
    }
    __syncthreads();
    const int32_t carry = carry_s;
    int32_t run = carry + (wave ? wsum[wave - 1] : 0) + x - tsum;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t e = base + (int64_t)tid * ITEMS + i;
      if (e < n) cu[e] = run;
      run += v[i];
    }
    __syncthreads();
    if (tid == NT - 1) carry_s = run;
    __syncthreads();
  }
  if (tid == 0) cu[n] = carry_s;
}

// Emit pass, one wave per segment: the count pass's decisions, written
// ascending at cu[s] (ballot + lane prefix = in-order compaction).  In the
// uncertain band the sign of the score is the decision; negated scores are
// restored, so the scores leave the call as they came in.
__global__ __launch_bounds__(256) void select_emit_kernel(Plan p, SelectArgs a,
                                                          float* __restrict__ scores,
                                                          const int32_t* __restrict__ cu,
                                                          int32_t* __restrict__ idx) {
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (seg >= p.num_segments) return;
  const SegPos sp = segment_position(p, seg);
  float* row = scores + sp.off;
  const int n = sp.I + 1;
  float mx = -INFINITY;
  for (int J = lane; J < n; J += 64) mx = fmaxf(mx, score_at(row, J));
  const Band bd = band_of(wave_max(mx), a.alpha);
  int32_t* out = idx + cu[seg];
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int written = 0;
  for (int J0 = 0; J0 < n; J0 += 64) {
    const int J = J0 + lane;
    const bool in = J < n;
    const float sv = in ? row[J] : 0.f;
    const float sc = fabsf(sv);
    const bool frc = in && forced(J, sp.I, a);
    const bool unc = in && a.alpha > 0.f && !frc && sc >= bd.lo && sc <= bd.hi;
    const bool keep = unc ? !signbit(sv) : in && (sc >= bd.thresh || frc);
    if (unc && signbit(sv)) row[J] = sc;
    const uint64_t m = __ballot(keep);
    if (keep) out[written + __popcll(m & below)] = J;
    written += __popcll(m);
  }
}

hipError_t launch_select(const Plan& p, const SelectArgs& a, const void* q, const float* kbar,
                         int dtype, float lscale, float* scores, int32_t* counts, int32_t* cu,
                         int32_t* idx, hipStream_t st) {
  const RefineArgs ra{q, kbar, dtype, lscale};
  const unsigned nblk = (unsigned)((p.num_segments + kWaves - 1) / kWaves);
  if (p.num_segments > 0) {
    hipLaunchKernelGGL(select_count_kernel, dim3(nblk), dim3(kWaves * 64), 0, st, p, a, ra, scores,
                       counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_scan_kernel, dim3(1), dim3(1024), 0, st, (int64_t)p.num_segments,
                     (const int32_t*)counts, cu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_segments == 0) return e;
  hipLaunchKernelGGL(select_emit_kernel, dim3(nblk), dim3(kWaves * 64), 0, st, p, a, scores,
                     (const int32_t*)cu, idx);
  return hipGetLastError();
}

}  // namespace bslp
