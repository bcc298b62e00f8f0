// Stage 3 on the matrix cores: block-sparse causal online-softmax attention
// with mean correction and PackGQA rows, bf16 inputs ("FlashPrefill V2",
// Sec. 3.1 last sentence, Sec. 3.2 / Fig. 3 correction path, PackGQA, CSR
// and paged-KV paragraphs).  Written for gfx950 wave64 MFMA.
//
// Work unit: (segment (b, h, I), 128 consecutive PackGQA rows of tile I);
// 4 waves x 32 rows.  Packed row r of the tile is position I*B + r / g of
// query head h*g + r % g, so one staged K/V block serves all g heads.
//
// Per wave the scores are computed transposed, S^T[key, row] = K Q^T, with
// v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims of K (from LDS), B = the
// wave's Q rows (kept in registers).  In the 32x32 accumulator every lane
// then owns one query row (column) and 16 keys, the other 16 keys of the
// 32-key tile sitting in lane ^ 32; row max and row sum are in-lane plus one
// v_permlane32_swap.  The probabilities stay in registers and feed the PV
// product O^T[d, row] += V^T P^T as the B operand directly: the 8 values a
// lane holds for 16 consecutive keys are keys {0-3, 8-11} (lanes 0-31) or
// {4-7, 12-15} (lanes 32-63), so V^T is staged in LDS with its key columns
// permuted the same way, and every MFMA operand is one 16-byte LDS read.
//
// LDS layout (bytes): K tile [BLK][D] bf16 and V^T tile [D][BLK] bf16, both
// in 16-byte units XOR-swizzled by row so that the 32 lanes of an operand read
// and the transposing writes hit distinct banks; plus a selected-block bitmap
// for the correction chunks.
//
// Selected blocks are walked backwards (CSR order reversed); the pruned blocks
// that every row of the tile sees completely (J <= I-1, not selected) then
// enter in chunks of BLK pooled keys kbar_J / values vbar_J through the same
// MFMA pipeline, their logits shifted by log|B_J| and unselected or invisible
// columns masked; chunks without such blocks are skipped uniformly.
#include "common.hpp"
#include "launch.hpp"

namespace bslp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;  // packed query rows per unit
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int kperm(int key) {  // V^T column of a key
  return (key & ~15) | ((key & 4) << 1) | ((key & 8) >> 1) | (key & 3);
}
__device__ __forceinline__ int kswz(int key) { return key & 7; }
__device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 3)) & 7; }

// v_permlane32_swap exchanges the src0 of lanes 0-31 with the vdst of lanes
// 32-63; with both operands = x every lane ends up holding {own x, x of
// lane ^ 32} in its two results (order depending on the half), so max / sum
// of the pair combine the two halves of a row in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace

template <int D, int BLK>
struct MfmaTile {
  static constexpr int KT = BLK / 32;    // 32-key tiles of S^T
  static constexpr int KS = D / 16;      // k-steps of Q K^T
  static constexpr int DT = D / 32;      // 32-dim tiles of O^T
  static constexpr int PT = BLK / 16;    // k-steps of P V
  static constexpr int KU = D / 8;       // 16-byte units per K row
  static constexpr int VU = BLK / 8;     // 16-byte units per V^T row
  static constexpr int KTOTAL = BLK * KU;        // 16-byte K chunks per tile
  static constexpr int VTOTAL = (BLK / 4) * KU;  // 4-key x 8-dim V groups per tile
  static constexpr int KCHUNKS = (KTOTAL + kThreads - 1) / kThreads;
  static constexpr int VGROUPS = (VTOTAL + kThreads - 1) / kThreads;
};

// K tile: element (key, d) at key*D + ((d/8) ^ kswz(key))*8 + d%8
// V^T tile: element (d, key) at d*BLK + ((kperm(key)/8) ^ vswz(d))*8 + kperm(key)%8

template <int D, int BLK>
__device__ __forceinline__ void store_k_unit(uint16_t* Ks, int key, int unit, uint4 val) {
  *reinterpret_cast<uint4*>(Ks + key * D + ((unit ^ kswz(key)) << 3)) = val;
}

// 4 consecutive keys (4a .. 4a+3) x 8 dims (8e .. 8e+7) -> V^T rows 8e..8e+7.
template <int D, int BLK>
__device__ __forceinline__ void store_v_group(uint16_t* Vt, int a, int e, const uint4 (&w)[4]) {
  const int col = kperm(4 * a);  // 4-aligned, the 4 keys stay adjacent
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&w[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&w[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&w[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&w[3]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high / low halves
    const uint32_t lo = __builtin_amdgcn_perm(w1[i >> 1], w0[i >> 1], sel);
    const uint32_t hi = __builtin_amdgcn_perm(w3[i >> 1], w2[i >> 1], sel);
    const int d = 8 * e + i;
    uint16_t* dst = Vt + d * BLK + ((((col >> 3) ^ vswz(d))) << 3) + (col & 7);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
}

// Stage exact key block: keys j0 .. j0+cnt-1 of request b, head h.
template <int D, int BLK>
__device__ __forceinline__ void stage_kv_block(uint16_t* Ks, uint16_t* Vt, const uint16_t* k,
                                               const uint16_t* v, const KVDesc& kv, int b,
                                               int tok_start, int hkv, int h, int j0, int cnt) {
  using C = MfmaTile<D, BLK>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KCHUNKS; ++i) {
    const int c = tid + i * kThreads;
    if (C::KTOTAL % kThreads != 0 && c >= C::KTOTAL) break;
    const int key = c / C::KU, unit = c % C::KU;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < cnt) {
      const int64_t row = kv.row(b, tok_start, j0 + key);
      val = *reinterpret_cast<const uint4*>(k + (row * hkv + h) * D + unit * 8);
    }
    store_k_unit<D, BLK>(Ks, key, unit, val);
  }
#pragma unroll
  for (int i = 0; i < C::VGROUPS; ++i) {
    const int s = tid + i * kThreads;
    if (C::VTOTAL % kThreads != 0 && s >= C::VTOTAL) break;
    const int a = s / C::KU, e = s % C::KU;
    uint4 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int key = 4 * a + c;
      w[c] = make_uint4(0, 0, 0, 0);
      if (key < cnt) {
        const int64_t row = kv.row(b, tok_start, j0 + key);
        w[c] = *reinterpret_cast<const uint4*>(v + (row * hkv + h) * D + e * 8);
      }
    }
    store_v_group<D, BLK>(Vt, a, e, w);
  }
}

__device__ __forceinline__ uint4 f32x8_to_bf16x8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                    pack_bf16x2(b.z, b.w));
}

// Stage pooled rows J0 .. J0+n-1 (float32 kbar / vbar, rounded to bf16).
template <int D, int BLK>
__device__ __forceinline__ void stage_pooled(uint16_t* Ks, uint16_t* Vt, const float* kbar,
                                             const float* vbar, int64_t row0, int hkv, int h,
                                             int n) {
  using C = MfmaTile<D, BLK>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KCHUNKS; ++i) {
    const int c = tid + i * kThreads;
    if (C::KTOTAL % kThreads != 0 && c >= C::KTOTAL) break;
    const int key = c / C::KU, unit = c % C::KU;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < n) val = f32x8_to_bf16x8(kbar + ((row0 + key) * hkv + h) * D + unit * 8);
    store_k_unit<D, BLK>(Ks, key, unit, val);
  }
#pragma unroll
  for (int i = 0; i < C::VGROUPS; ++i) {
    const int s = tid + i * kThreads;
    if (C::VTOTAL % kThreads != 0 && s >= C::VTOTAL) break;
    const int a = s / C::KU, e = s % C::KU;
    uint4 w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int key = 4 * a + c;
      w[c] = key < n ? f32x8_to_bf16x8(vbar + ((row0 + key) * hkv + h) * D + e * 8)
                     : make_uint4(0, 0, 0, 0);
    }
    store_v_group<D, BLK>(Vt, a, e, w);
  }
}

// One wave's S^T = K Q^T over the staged tile.
template <int D, int BLK>
__device__ __forceinline__ void qk_tile(const uint16_t* Ks, const bf16x8_t (&qf)[D / 16],
                                        f32x16_t (&sacc)[BLK / 32], int lane) {
  using C = MfmaTile<D, BLK>;
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
  }
  const int key_l = lane & 31, half = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      const int key = kt * 32 + key_l;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
          Ks + key * D + (((2 * ks + half) ^ kswz(key)) << 3));
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kt], 0, 0, 0);
    }
  }
}

// Online softmax on the masked, scaled logits in sacc (log2 domain), then
// O^T += V^T P^T.
template <int D, int BLK>
__device__ __forceinline__ void softmax_pv(const uint16_t* Vt, f32x16_t (&sacc)[BLK / 32],
                                           f32x16_t (&oacc)[D / 32], float& m_run, float& l_run,
                                           int lane) {
  using C = MfmaTile<D, BLK>;
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
  }
  mx = halves_max(mx);
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  float lsum = 0.f;
  bf16x8_t pb[C::PT];
#pragma unroll
  for (int t = 0; t < C::PT; ++t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(sacc[t >> 1][8 * (t & 1) + j] - m_use);
      lsum += p;
      pb[t][j] = (__bf16)p;
    }
  }
  l_run = l_run * alpha + lsum;
  m_run = m_new;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
  }
  const int d_l = lane & 31, half = lane >> 5;
#pragma unroll
  for (int t = 0; t < C::PT; ++t) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int d = dt * 32 + d_l;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
          Vt + d * BLK + (((2 * t + half) ^ vswz(d)) << 3));
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t], oacc[dt], 0, 0, 0);
    }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_bf16_kernel(
    Plan p, KVDesc kv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ kbar,
    const float* __restrict__ vbar, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ idx, float scale_log2, int correction, int units_per_seg,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  using C = MfmaTile<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * BLK];
  __shared__ uint32_t selbits[kMaxBlocksPerSeq / 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t unit = (int64_t)gridDim.x - 1 - blockIdx.x;  // longest rows first
  const int64_t seg = unit / units_per_seg;
  const int mt = (int)(unit % units_per_seg);
  const int b = seq_of_segment(p, seg);
  const SeqInfo s = p.seq[b];
  const int local = (int)(seg - s.seg_base);
  const int h = local / s.nblk;
  const int I = local % s.nblk;
  const int nb = min(p.B, s.len - I * p.B);
  const int R = p.g * nb;
  if (mt * kRows >= R) return;  // uniform

  // this lane's query row
  const int r = mt * kRows + wave * 32 + (lane & 31);
  const bool valid = r < R;
  const int qpos = I * p.B + (valid ? r / p.g : 0);
  const int hq = h * p.g + r % p.g;
  const int half = lane >> 5;
  bf16x8_t qf[C::KS];
  {
    const int64_t qoff = ((int64_t)(s.tok_start + qpos) * p.hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (valid) u = *reinterpret_cast<const uint4*>(q + qoff + ks * 16 + half * 8);
      qf[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  f32x16_t oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) oacc[dt][rr] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t sacc[C::KT];

  const int beg = cu[seg], end = cu[seg + 1];
  for (int t = end - 1; t >= beg; --t) {
    const int J = idx[t];
    const int j0 = J * p.B;
    const int cnt = min(BLK, s.len - j0);
    __syncthreads();  // previous tile fully consumed
    stage_kv_block<D, BLK>(Ks, Vt, k, v, kv, b, s.tok_start, p.hkv, h, j0, cnt);
    __syncthreads();
    qk_tile<D, BLK>(Ks, qf, sacc, lane);
    const bool diag = (J == I);
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = kt * 32 + (rr >> 2) * 8 + half * 4 + (rr & 3);
        float x = sacc[kt][rr] * scale_log2;
        if (diag && (j0 + key > qpos || key >= cnt)) x = -INFINITY;
        sacc[kt][rr] = x;
      }
    }
    softmax_pv<D, BLK>(Vt, sacc, oacc, m_run, l_run, lane);
  }

  if (correction && I > 0) {
    const int nwords = (I + 31) >> 5;
    __syncthreads();
    for (int w = tid; w < nwords; w += kThreads) selbits[w] = 0u;
    __syncthreads();
    for (int t = beg + tid; t < end; t += kThreads) {
      const int J = idx[t];
      if (J < I) atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    const float bias = __log2f((float)p.B);  // every J <= I-1 is a full block
    for (int J0 = 0; J0 < I; J0 += BLK) {
      const int n = min(BLK, I - J0);
      bool any = false;  // identical decision in every thread
      for (int w = 0; w < (n + 31) / 32; ++w) {
        const int rem = n - 32 * w;
        const uint32_t validm = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
        any |= ((~selbits[(J0 >> 5) + w]) & validm) != 0u;
      }
      if (!any) continue;
      __syncthreads();
      stage_pooled<D, BLK>(Ks, Vt, kbar, vbar, (int64_t)s.pool_base + J0, p.hkv, h, n);
      __syncthreads();
      qk_tile<D, BLK>(Ks, qf, sacc, lane);
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = kt * 32 + (rr >> 2) * 8 + half * 4 + (rr & 3);
          const int J = J0 + key;
          const bool todo = key < n && !((selbits[J >> 5] >> (J & 31)) & 1u);
          sacc[kt][rr] = todo ? sacc[kt][rr] * scale_log2 + bias : -INFINITY;
        }
      }
      softmax_pv<D, BLK>(Vt, sacc, oacc, m_run, l_run, lane);
    }
  }

  // epilogue: l over all keys of the row = both lane halves
  const float l_tot = halves_sum(l_run);
  if (!valid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t ooff = ((int64_t)(s.tok_start + qpos) * p.hq + hq) * D;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = dt * 32 + g4 * 8 + half * 4;
      const uint32_t lo = pack_bf16x2(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv);
      const uint32_t hi = pack_bf16x2(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
      *reinterpret_cast<uint2*>(out + ooff + d) = make_uint2(lo, hi);
    }
  }
  if (lse && half == 0)
    lse[(int64_t)hq * p.total_tokens + s.tok_start + qpos] =
        l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
}

template <int D, int BLK>
static hipError_t launch_mfma_t(const Plan& p, const KVDesc& kv, const AttnArgs& a,
                                hipStream_t st) {
  const int units_per_seg = (p.g * p.B + kRows - 1) / kRows;
  const int64_t units = p.num_segments * units_per_seg;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_mfma_bf16_kernel<D, BLK>), dim3((unsigned)units), dim3(kThreads), 0,
                     st, p, kv, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.kbar, a.vbar, a.cu, a.idx, a.lscale * kLog2e, a.correction, units_per_seg,
                     (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_bf16(const Plan& p, const KVDesc& kv, const AttnArgs& a,
                                 hipStream_t st) {
  if (p.d == 128 && p.B == 128) return launch_mfma_t<128, 128>(p, kv, a, st);
  if (p.d == 128 && p.B == 64) return launch_mfma_t<128, 64>(p, kv, a, st);
  if (p.d == 64 && p.B == 128) return launch_mfma_t<64, 128>(p, kv, a, st);
  return launch_mfma_t<64, 64>(p, kv, a, st);
}

}  // namespace bslp
