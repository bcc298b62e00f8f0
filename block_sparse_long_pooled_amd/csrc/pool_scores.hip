// Stage 1 of the FlashPrefill V2 hot path: mean-pooled keys/values and the
// fused block-score reduction ("FlashPrefill V2", Sec. 3.1; score formulas
// printed in the method-steps section of the FlashPrefill summary page).
#include "common.hpp"
#include "launch.hpp"

namespace bslp {

// ------------------------------------------------------------------ pooling
// One workgroup per (pooled row, group of HC KV heads, K-or-V): a token row
// of HC heads is HC*D contiguous elements, read by TPR = HC*D/8 threads with
// one 8-element (16-byte for bf16) load each, so every load instruction of a
// wave covers a contiguous 1 KB.  The RG = 256/TPR row groups take the
// block's rows r, r + RG, ...; each thread sums its 8 columns over its rows,
// and the groups are combined in fixed order, so results are deterministic.
// HBM-bound: the block's K (or V) rows are read once.
constexpr int kPoolThreads = 256;
constexpr int kRowsInFlight = 8;  // token rows a thread loads before adding them

template <int D>
constexpr int pool_heads() { return kPoolThreads * 8 / D; }  // heads per workgroup

template <int DT, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(Plan p, KVDesc kv,
                                                            const typename Elem<DT>::T* __restrict__ k,
                                                            const typename Elem<DT>::T* __restrict__ v,
                                                            float k_scale, float v_scale,
                                                            float* __restrict__ kbar,
                                                            float* __restrict__ vbar) {
  __shared__ __attribute__((aligned(16))) float part[kPoolThreads * 8];
  const int prow = blockIdx.x;
  const int h0 = blockIdx.y * pool_heads<D>();
  const bool is_v = blockIdx.z != 0;
  const int hc = min(pool_heads<D>(), p.hkv - h0);
  const int tpr = hc * D / 8;          // threads per token row (D % 8 == 0)
  const int rg_n = kPoolThreads / tpr; // row groups
  const int tid = threadIdx.x;
  const int rg = tid / tpr, col8 = tid % tpr;
  const bool active = rg < rg_n;
  int b = 0;
  while (b + 1 < p.num_seqs && p.seq[b + 1].pool_base <= prow) ++b;
  const SeqInfo s = p.seq[b];
  const int J = prow - s.pool_base;
  const int j0 = J * p.B;
  const int cnt = min(p.B, s.len - j0);
  const typename Elem<DT>::T* x = is_v ? v : k;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    // kRowsInFlight rows' loads in flight at a time, added in row order as
    // one by one (the sum is the same as a row-by-row loop's)
    constexpr int U = kRowsInFlight;
    int r = rg;
    for (; r + (U - 1) * rg_n < cnt; r += U * rg_n) {
      // all U rows first (their page-table entries in one batch of loads),
      // then the data
      int64_t rows[U];
      if (kv.page_table != nullptr) {
        int32_t phys[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          phys[u] = kv.page_table[(int64_t)b * kv.max_pages + ((j0 + r + u * rg_n) >> kv.page_shift)];
#pragma unroll
        for (int u = 0; u < U; ++u)
          rows[u] = ((int64_t)phys[u] << kv.page_shift) |
                    (int64_t)((j0 + r + u * rg_n) & ((1 << kv.page_shift) - 1));
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) rows[u] = (int64_t)s.kv_start + j0 + r + u * rg_n;
      }
      float e[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) load8<DT>(x, (rows[u] * p.hkv + h0) * D + col8 * 8, e[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += e[u][i];
      }
    }
    for (; r < cnt; r += rg_n) {
      const int64_t row = kv.row(b, s.kv_start, j0 + r);
      float e[8];
      load8<DT>(x, (row * p.hkv + h0) * D + col8 * 8, e);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += e[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[rg * tpr * 8 + col8 * 8 + i] = acc[i];
  }
  __syncthreads();
  if (tid < tpr) {
    const float sc = p.dscale ? p.dscale[is_v ? 2 : 1] : (is_v ? v_scale : k_scale);
    float* out = (is_v ? vbar : kbar) + ((int64_t)prow * p.hkv + h0) * D + tid * 8;
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = part[tid * 8 + i];
      for (int g2 = 1; g2 < rg_n; ++g2) t += part[g2 * tpr * 8 + tid * 8 + i];
      m[i] = t / (float)cnt * sc;
    }
    *reinterpret_cast<float4*>(out) = make_float4(m[0], m[1], m[2], m[3]);
    *reinterpret_cast<float4*>(out + 4) = make_float4(m[4], m[5], m[6], m[7]);
  }
}

// ------------------------------------------------------------------ scores
// One workgroup per segment (b, h, I).  Key blocks are processed in chunks of
// CH = 32; thread t owns block J0 + (t % 32) of the chunk (its pooled key in
// registers) and the tile rows r = t/32, t/32 + 8, ... of the tile's
// R = g*|tile| query rows:
//   * s_rJ = lscale * q_r . kbar_J is accumulated in float64 (q and kbar are
//     exact in float32, so every product is exact);
//   * each thread keeps a running (max m_J, sum S_J = sum_r exp(s_rJ - m_J));
//   * the (m_J, S_J) pairs of the 8 row groups are merged in fixed order;
//   * the chunk writes S_J * exp(m_J - M_c) (M_c = chunk max) into the score
//     row and keeps (M_c, chunk sum) in LDS - the per-chunk maximum of the V2
//     index buffer (FlashPrefill V2, scoring/threshold fusion paragraph).
// A final pass rescales every entry by exp(M_c - M_I) / sum, giving
// Score_IJ = S'_IJ / sum_K S'_IK as defined on the FlashPrefill summary page.
template <int DT, int D>
__global__ __launch_bounds__(256) void scores_kernel(Plan p,
                                                     const typename Elem<DT>::T* __restrict__ q,
                                                     const float* __restrict__ kbar, double lscale,
                                                     float* __restrict__ scores) {
  if (p.dscale) lscale *= (double)p.dscale[0];
  constexpr int CH = 32;
  constexpr int NT = 256;
  constexpr int RG = NT / CH;  // row groups
  extern __shared__ double dyn[];
  double* cmax = dyn;                               // [chunks]
  double* csum = dyn + ((p.max_nblk + CH - 1) / CH);  // [chunks]
  __shared__ double wm[NT / 64][CH];
  __shared__ float wsum[NT / 64][CH];
  __shared__ double fin[2];

  const int tid = threadIdx.x;
  const int jj = tid % CH;
  const int rg = tid / CH;
  const int wave = tid >> 6;
  const int64_t seg = p.num_segments - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int b = seq_of_segment(p, seg);
  const SeqInfo s = p.seq[b];
  int h, I;
  segment_tile(s, (int)(seg - s.seg_base), h, I);
  const int q0 = tile_q0(s, I, p.B);
  const int R = p.g * tile_nq(s, I, p.B);
  const int nJ = I + 1;
  const int nch = (nJ + CH - 1) / CH;
  float* row_out = scores + score_offset(s, h, I);

  for (int c = 0; c < nch; ++c) {
    const int J = c * CH + jj;
    const bool validJ = J < nJ;
    double m = -INFINITY;
    float S = 0.f;
    if (validJ) {
      float kr[D];
      const float* kp = kbar + ((int64_t)(s.pool_base + J) * p.hkv + h) * D;
#pragma unroll
      for (int cc = 0; cc < D; cc += 4) {
        const float4 t4 = *reinterpret_cast<const float4*>(kp + cc);
        kr[cc] = t4.x; kr[cc + 1] = t4.y; kr[cc + 2] = t4.z; kr[cc + 3] = t4.w;
      }
      for (int r = rg; r < R; r += RG) {
        const int pos = q0 + r / p.g;
        const int hq = h * p.g + r % p.g;
        const int64_t qoff = (q_row(s, pos) * p.hq + hq) * D;
        double acc = 0.0;
#pragma unroll
        for (int cc = 0; cc < D; cc += 8) {
          float qv[8];
          load8<DT>(q, qoff + cc, qv);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fma((double)qv[e], (double)kr[cc + e], acc);
        }
        const double sv = acc * lscale;
        if (sv > m) {
          S = S * expf((float)(m - sv)) + 1.f;
          m = sv;
        } else {
          S += expf((float)(sv - m));
        }
      }
    }
    // merge the two row groups of this wave (lanes t and t^32 share J)
    {
      const double mo = __shfl_xor(m, 32);
      const float so = __shfl_xor(S, 32);
      const double mx = fmax(m, mo);
      const double ms = (mx == -INFINITY) ? 0.0 : mx;  // both empty: stays (-inf, 0)
      S = S * expf((float)(m - ms)) + so * expf((float)(mo - ms));
      m = mx;
    }
    if ((tid & 63) < CH) { wm[wave][jj] = m; wsum[wave][jj] = S; }
    __syncthreads();
    if (tid < CH) {
      double mm = -INFINITY;
      float ss = 0.f;
      for (int w = 0; w < NT / 64; ++w) {
        const double mo = wm[w][jj];
        const float so = wsum[w][jj];
        const double mx = fmax(mm, mo);
        const double ms = (mx == -INFINITY) ? 0.0 : mx;
        ss = ss * expf((float)(mm - ms)) + so * expf((float)(mo - ms));
        mm = mx;
      }
      double Mc = validJ ? mm : -INFINITY;
      for (int off = 16; off >= 1; off >>= 1) Mc = fmax(Mc, __shfl_xor(Mc, off, 32));
      const double t = validJ ? (double)ss * exp(mm - Mc) : 0.0;
      double tsum = t;
      for (int off = 16; off >= 1; off >>= 1) tsum += __shfl_xor(tsum, off, 32);
      if (validJ) row_out[J] = (float)t;
      if (jj == 0) { cmax[c] = Mc; csum[c] = tsum; }
    }
    __syncthreads();
  }
  if (tid == 0) {
    double M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmax(M, cmax[c]);
    double tot = 0.0;
    for (int c = 0; c < nch; ++c) tot += csum[c] * exp(cmax[c] - M);
    fin[0] = M;
    fin[1] = tot;
  }
  __syncthreads();
  if (tid < CH) {
    // each of these threads re-reads only the entries it wrote itself
    const double M = fin[0], inv = 1.0 / fin[1];
    for (int c = 0; c < nch; ++c) {
      const int J = c * CH + tid;
      if (J < nJ) row_out[J] = (float)((double)row_out[J] * exp(cmax[c] - M) * inv);
    }
  }
}

template <int DT, int D>
static hipError_t launch_stage1_t(const Plan& p, const KVDesc& kv, const void* q, const void* k,
                                  const void* v, float q_scale, float k_scale, float v_scale,
                                  float softmax_scale, float* kbar, float* vbar, float* scores,
                                  int parts, hipStream_t st) {
  using T = typename Elem<DT>::T;
  if ((parts & kStagePool) && p.pooled_rows > 0) {
    const int groups = (p.hkv + pool_heads<D>() - 1) / pool_heads<D>();
    // a d-major (fp8) V is pooled by its own kernel; the grid then covers K
    const bool vrows = !(DT == kFP8 && p.v_dmajor);
    dim3 grid((unsigned)p.pooled_rows, (unsigned)groups, vrows ? 2 : 1);
    hipLaunchKernelGGL((pool_kernel<DT, D>), grid, dim3(kPoolThreads), 0, st, p, kv, (const T*)k,
                       (const T*)v, k_scale, v_scale, kbar, vbar);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!vrows) {
      e = launch_pool_v_dmajor(p, kv, v, v_scale, vbar, nullptr, st);
      if (e != hipSuccess) return e;
    }
  }
  if (!(parts & kStageScores)) return hipSuccess;
  if (p.num_segments > 0 && scores_mfma_supported(p, DT)) {
    const double c2 = (double)softmax_scale * (double)q_scale * 1.4426950408889634;
    return launch_scores_mfma(p, DT, q, kbar, (float)c2, scores, st);
  }
  if (p.num_segments > 0) {
    const int nch = (p.max_nblk + 31) / 32;
    const size_t lds = sizeof(double) * (2 * nch);
    const double lscale = (double)softmax_scale * (double)q_scale;
    hipLaunchKernelGGL((scores_kernel<DT, D>), dim3((unsigned)p.num_segments), dim3(256), lds, st,
                       p, (const T*)q, (const float*)kbar, lscale, scores);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_stage1(const Plan& p, const KVDesc& kv, int dtype, const void* q, const void* k,
                         const void* v, float q_scale, float k_scale, float v_scale,
                         float softmax_scale, float* kbar, float* vbar, float* scores,
                         int parts, hipStream_t st) {
#define BSLP_S1(DT, D) \
  return launch_stage1_t<DT, D>(p, kv, q, k, v, q_scale, k_scale, v_scale, softmax_scale, kbar, \
                                vbar, scores, parts, st)
  if (p.d == 128) {
    if (dtype == kF32) BSLP_S1(kF32, 128);
    if (dtype == kBF16) BSLP_S1(kBF16, 128);
    BSLP_S1(kFP8, 128);
  } else {
    if (dtype == kF32) BSLP_S1(kF32, 64);
    if (dtype == kBF16) BSLP_S1(kBF16, 64);
    BSLP_S1(kFP8, 64);
  }
#undef BSLP_S1
}

}  // namespace bslp
