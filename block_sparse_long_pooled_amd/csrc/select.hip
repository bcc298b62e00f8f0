// Stage 2: max-based dynamic threshold plus sink / window / recent blocks,
// emitted as a CSR index ("FlashPrefill V2", Sec. 3.1 threshold paragraph and
// the CSR paragraph; thresh_I = alpha * max_J Score_IJ is printed in the
// core-method section of the FlashPrefill summary page).
//
// Three launches, no scratch memory:
//   count  one wave per segment: row max, threshold, |Sel| via ballots;
//   scan   one workgroup: exclusive prefix of the counts -> cu;
//   emit   one wave per segment: the same comparisons again, survivors written
//          ascending at cu[s] (ballot + lane prefix = in-order compaction).
// Both passes evaluate the identical float comparisons, so count and emitted
// list always agree.
#include "common.hpp"
#include "launch.hpp"

namespace bslp {

struct SegPos {
  int b, h, I;
  int64_t off;  // first score element
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

__device__ __forceinline__ float row_threshold(const float* row, int n, float alpha, int lane) {
  float mx = -INFINITY;
  for (int J = lane; J < n; J += 64) mx = fmaxf(mx, row[J]);
  return alpha * wave_max(mx);
}

__global__ __launch_bounds__(256) void select_count_kernel(Plan p, SelectArgs a,
                                                           const float* __restrict__ scores,
                                                           int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= p.num_segments) return;
  const SegPos sp = segment_position(p, seg);
  const float* row = scores + sp.off;
  const int n = sp.I + 1;
  const float thresh = row_threshold(row, n, a.alpha, lane);
  int cnt = 0;
  for (int J0 = 0; J0 < n; J0 += 64) {
    const int J = J0 + lane;
    const bool keep = J < n && (row[J] >= thresh || forced(J, sp.I, a));
    cnt += __popcll(__ballot(keep));
  }
  if (lane == 0) counts[seg] = cnt;
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

__global__ __launch_bounds__(256) void select_emit_kernel(Plan p, SelectArgs a,
                                                          const float* __restrict__ scores,
                                                          const int32_t* __restrict__ cu,
                                                          int32_t* __restrict__ idx) {
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= p.num_segments) return;
  const SegPos sp = segment_position(p, seg);
  const float* row = scores + sp.off;
  const int n = sp.I + 1;
  const float thresh = row_threshold(row, n, a.alpha, lane);
  int32_t* out = idx + cu[seg];
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int written = 0;
  for (int J0 = 0; J0 < n; J0 += 64) {
    const int J = J0 + lane;
    const bool keep = J < n && (row[J] >= thresh || forced(J, sp.I, a));
    const uint64_t m = __ballot(keep);
    if (keep) out[written + __popcll(m & below)] = J;
    written += __popcll(m);
  }
}

hipError_t launch_select(const Plan& p, const SelectArgs& a, const float* scores, int32_t* counts,
                         int32_t* cu, int32_t* idx, hipStream_t st) {
  const unsigned nblk = (unsigned)((p.num_segments + 3) / 4);
  if (p.num_segments > 0) {
    hipLaunchKernelGGL(select_count_kernel, dim3(nblk), dim3(256), 0, st, p, a, scores, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_scan_kernel, dim3(1), dim3(1024), 0, st, (int64_t)p.num_segments,
                     (const int32_t*)counts, cu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_segments == 0) return e;
  hipLaunchKernelGGL(select_emit_kernel, dim3(nblk), dim3(256), 0, st, p, a, scores,
                     (const int32_t*)cu, idx);
  return hipGetLastError();
}

}  // namespace bslp
