// Stage 3, vector-ALU form: block-sparse causal online-softmax attention
// with mean correction, one query row per lane ("FlashPrefill V2", Sec. 3.1
// last sentence, Sec. 3.2 / Fig. 3 correction path, PackGQA and CSR
// paragraphs).  This form serves float32 inputs only (exact fp32
// arithmetic, no matrix cores); bf16 and fp8 inputs always take the
// matrix-core kernels.
//
// Work unit: (segment (b, h, I), 64 consecutive PackGQA rows of tile I).
// Packed row r of the tile is position I*B + r / g of query head h*g + r % g.
// K/V of each selected block are staged, dequantised, in LDS 32 keys at a
// time and shared by all 64 rows (every row of the unit has the same KV head).
// The selected list is walked backwards (descending blocks); then the pruned,
// fully visible blocks J <= I-1 (found by a two-pointer walk of the ascending
// list) enter as pooled keys/values with logit + ln|B_J|.
#include "common.hpp"
#include "launch.hpp"

namespace bslp {

template <int D>
struct ValuState {
  float o[D];
  float m, l;
};

// Online-softmax update of one lane with nk staged keys.
template <int D>
__device__ __forceinline__ void valu_update(ValuState<D>& st, const float (&qr)[D],
                                            const float (*Ks)[D], const float (*Vs)[D], int nk,
                                            const int* kpos, const float* bias, int qpos,
                                            float lscale) {
  float sc[32];
  float mx = -INFINITY;
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    float t = -INFINITY;
    if (kk < nk && kpos[kk] <= qpos) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = fmaf(qr[c], Ks[kk][c], acc);
      t = acc * lscale + bias[kk];
    }
    sc[kk] = t;
    mx = fmaxf(mx, t);
  }
  const float m_new = fmaxf(st.m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __expf(st.m - m_use);
  st.l *= alpha;
#pragma unroll
  for (int c = 0; c < D; ++c) st.o[c] *= alpha;
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    if (kk < nk) {
      const float pr = __expf(sc[kk] - m_use);
      st.l += pr;
#pragma unroll
      for (int c = 0; c < D; ++c) st.o[c] = fmaf(pr, Vs[kk][c], st.o[c]);
    }
  }
  st.m = m_new;
}

template <int DT, int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(
    Plan p, KVDesc kv, const typename Elem<DT>::T* __restrict__ q,
    const typename Elem<DT>::T* __restrict__ k, const typename Elem<DT>::T* __restrict__ v,
    const float* __restrict__ kbar, const float* __restrict__ vbar,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ idx, float lscale, float k_scale,
    float v_scale, int correction, int dense, int units_per_seg, void* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ float Ks[32][D];
  __shared__ float Vs[32][D];
  __shared__ int kpos_s[32];
  __shared__ float bias_s[32];
  __shared__ int todo_s[32];

  const int lane = threadIdx.x;
  const int64_t unit = (int64_t)gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int64_t seg = unit / units_per_seg;
  const int mt = (int)(unit % units_per_seg);
  const int b = seq_of_segment(p, seg);
  const SeqInfo s = p.seq[b];
  int h, I;
  segment_tile(s, (int)(seg - s.seg_base), h, I);
  const int R = p.g * tile_nq(s, I, p.B);
  if (mt * 64 >= R) return;  // uniform: tile shorter than this unit
  const int r = mt * 64 + lane;
  const bool valid = r < R;
  const int qpos = valid ? tile_q0(s, I, p.B) + r / p.g : -1;
  const int hq = h * p.g + (r % p.g);

  float qr[D];
  if (valid) {
    const int64_t qoff = (q_row(s, qpos) * p.hq + hq) * D;
#pragma unroll
    for (int c = 0; c < D; c += 8) load8<DT>(q, qoff + c, qr + c);
  } else {
#pragma unroll
    for (int c = 0; c < D; ++c) qr[c] = 0.f;
  }
  ValuState<D> st;
#pragma unroll
  for (int c = 0; c < D; ++c) st.o[c] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;

  // CSR walked backwards; the dense path walks every block J <= I
  const int beg = dense ? 0 : cu[seg], end = dense ? I + 1 : cu[seg + 1];
  for (int t = end - 1; t >= beg; --t) {
    const int J = dense ? t : idx[t];
    const int j0 = J * p.B;
    const int cnt = min(p.B, s.len - j0);
    for (int sub = 0; sub < cnt; sub += 32) {
      const int nk = min(32, cnt - sub);
      for (int e = lane; e < 32 * D; e += 64) {
        const int kk = e / D, c = e % D;
        float kvv = 0.f, vvv = 0.f;
        if (kk < nk) {
          const int64_t row = kv.row(b, s.kv_start, j0 + sub + kk);
          const int64_t off = (row * p.hkv + h) * D + c;
          kvv = Elem<DT>::load(k, off) * k_scale;
          vvv = Elem<DT>::load(v, off) * v_scale;
        }
        Ks[kk][c] = kvv;
        Vs[kk][c] = vvv;
      }
      if (lane < 32) { kpos_s[lane] = j0 + sub + lane; bias_s[lane] = 0.f; }
      __syncthreads();
      valu_update<D>(st, qr, Ks, Vs, nk, kpos_s, bias_s, qpos, lscale);
      __syncthreads();
    }
  }

  if (correction && I > 0) {
    // todo = valid & ~selected with valid = {0 .. I-1}; two-pointer walk of
    // the ascending selected list, 32 corrected blocks per staging round.
    int ptr = beg, J = 0;
    while (J < I) {
      int n = 0;
      while (J < I && n < 32) {
        while (ptr < end && idx[ptr] < J) ++ptr;
        if (!(ptr < end && idx[ptr] == J)) {
          if (lane == 0) todo_s[n] = J;
          ++n;
        }
        ++J;
      }
      if (n == 0) break;
      __syncthreads();
      for (int e = lane; e < 32 * D; e += 64) {
        const int kk = e / D, c = e % D;
        float kvv = 0.f, vvv = 0.f;
        if (kk < n) {
          const int64_t off = ((int64_t)(s.pool_base + todo_s[kk]) * p.hkv + h) * D + c;
          kvv = kbar[off];
          vvv = vbar[off];
        }
        Ks[kk][c] = kvv;
        Vs[kk][c] = vvv;
      }
      if (lane < 32) {
        kpos_s[lane] = -1;  // pooled terms are visible to every row
        bias_s[lane] = lane < n ? logf((float)min(p.B, s.len - todo_s[lane] * p.B)) : 0.f;
      }
      __syncthreads();
      valu_update<D>(st, qr, Ks, Vs, n, kpos_s, bias_s, qpos, lscale);
      __syncthreads();
    }
  }

  if (!valid) return;
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
  const int64_t ooff = (q_row(s, qpos) * p.hq + hq) * D;
  if constexpr (DT == kF32) {
    float* o = reinterpret_cast<float*>(out) + ooff;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = st.o[c] * inv;
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + ooff;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = f32_to_bf16(st.o[c] * inv);
  }
  if (lse) lse[(int64_t)hq * p.total_tokens + q_row(s, qpos)] =
      st.l > 0.f ? st.m + logf(st.l) : -INFINITY;
}

template <int DT, int D>
static hipError_t launch_attn_valu_t(const Plan& p, const KVDesc& kv, const AttnArgs& a,
                                     hipStream_t st) {
  using T = typename Elem<DT>::T;
  const int units_per_seg = (p.g * p.B + 63) / 64;
  const int64_t units = p.num_segments * units_per_seg;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_valu_kernel<DT, D>), dim3((unsigned)units), dim3(64), 0, st, p, kv,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, a.kbar, a.vbar, a.cu, a.idx,
                     a.lscale, a.k_scale, a.v_scale, a.correction && !a.dense, a.dense, units_per_seg,
                     a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_attn_valu(const Plan& p, const KVDesc& kv, int dtype, const AttnArgs& a,
                            hipStream_t st) {
  if (dtype != kF32) return hipErrorInvalidValue;  // bf16 / fp8 run on the matrix cores
  return p.d == 128 ? launch_attn_valu_t<kF32, 128>(p, kv, a, st)
                    : launch_attn_valu_t<kF32, 64>(p, kv, a, st);
}

}  // namespace bslp
