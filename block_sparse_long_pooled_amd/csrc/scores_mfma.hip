// Stage 1 block scores on the matrix cores (bf16 and fp8 inputs).
//
// Computes, for every segment (b, h, I), the FlashPrefill block scores over
// the mean-pooled keys ("FlashPrefill V2", Sec. 3.1 and the paragraph that
// fuses scoring and thresholding; formulas printed in the method-steps
// section of the FlashPrefill summary page):
//   s_rJ     = softmax_scale * q_r . kbar_J        (r: the g*|tile| PackGQA rows)
//   M_I      = max_{r, J<=I} s_rJ
//   Score_IJ = sum_r exp(s_rJ - M_I) / sum_{K<=I} sum_r exp(s_rK - M_I)
//
// Accuracy.  q is exact in bf16 (bf16 input, or an e4m3 code, whose 4
// significant bits fit).  kbar (float32) is split into two bf16 terms,
// hi = bf16(x) and lo = bf16(x - hi), both rounded to nearest, so hi + lo is
// x to within 2^-18 |x|; every bf16 x bf16 product is exact in float32 and
// the MFMA sums are accumulated lo first, then hi.  The scores then carry a
// relative error of order 1e-5 (well below the 1e-3 that selection assumes:
// it re-decides every block within 2e-3 of the threshold exactly in
// float64), for two thirds of the matrix work of an exact 3-term split.
//
// Work layout.  One workgroup per segment, NW waves (up to 16); wave w owns
// RT row tiles of 32 packed rows (Q in registers as the A operand of
// v_mfma_f32_32x32x16_bf16).  Key blocks are processed in chunks of 32: the
// chunk's split kbar rows are staged in LDS (double buffered, next chunk
// prefetched into registers while the current one is multiplied) and read
// as the B operand, so in the 32x32 accumulator every lane owns one key
// block J (its column) and 16 rows.  Each lane reduces its rows in-lane
// (max, then sum of exp2), the two lane halves combine with
// v_permlane32_swap, and the waves' partials (m, S) meet in LDS, where each
// wave merges 32/NW of the chunk's blocks over the NW partials with
// shuffles, so no wave does more of it than another.  The per-block maxima
// m_J stay in LDS and the sums S_J in the score row.  Each combine group
// also keeps a running pair (largest m_J so far, float64 sum of its
// S_J 2^(m_J - that maximum)); at the end every thread merges the 32 pairs
// into M_I = max_J m_J and the total sum_J S_J 2^(m_J - M_I), and writes
// the scores S_J 2^(m_J - M_I) / total.
#include "common.hpp"
#include "launch.hpp"

namespace bslp {

typedef __bf16 sbf16x8_t __attribute__((ext_vector_type(8)));
typedef float sf32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kChunk = 32;  // key blocks per chunk = MFMA N
constexpr int kScRsrcWord3 = 0x00020000;  // raw buffer descriptor, 32-bit data format

__device__ __forceinline__ int sc_uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const float* sc_uniform_ptr(const float* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)sc_uni((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)sc_uni((int)(uint32_t)(x >> 32));
  return reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x from lane ^ OFF (OFF < 32): ds_swizzle in its xor mode needs no lane-index
// registers, which a loop that holds the query rows cannot spare.
template <int OFF>
__device__ __forceinline__ float swz_xor(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (OFF << 10) | 0x1f));
}

// max over aligned groups of N lanes (N = 4, 8 or 16), in a fixed order
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 16) x = fmaxf(x, swz_xor<8>(x));
  if constexpr (N >= 8) x = fmaxf(x, swz_xor<4>(x));
  x = fmaxf(x, swz_xor<2>(x));
  return fmaxf(x, swz_xor<1>(x));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 16) x += swz_xor<8>(x);
  if constexpr (N >= 8) x += swz_xor<4>(x);
  x += swz_xor<2>(x);
  return x + swz_xor<1>(x);
}

// Two-term split of two floats into packed bf16 pairs, every term rounded to
// nearest even by v_cvt_pk_bf16_f32: x = hi + lo + r with |r| <= 2^-18 |x|
// (x - hi is exact).  Returns (hi pair, lo pair), element a in the low half.
__device__ __forceinline__ uint2 split2_pair(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const bf2 h = __builtin_convertvector(f2{a, b}, bf2);
  const uint32_t hu = __builtin_bit_cast(uint32_t, h);
  const float ha = __uint_as_float(hu << 16), hb = __uint_as_float(hu & 0xffff0000u);
  const bf2 l = __builtin_convertvector(f2{a - ha, b - hb}, bf2);
  return make_uint2(hu, __builtin_bit_cast(uint32_t, l));
}

// 8 e4m3 codes (two little-endian words) as 8 bf16, exactly.  An e4m3 value
// has 4 significant bits, so its float32 bits end in 16 zeros and the upper
// halves of two v_cvt_pk_f32_fp8 results pack into bf16 pairs.
__device__ __forceinline__ uint4 widen_e4m3x8(uint2 u) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(u.x, false);  // bytes 0, 1
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(u.x, true);   // bytes 2, 3
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(u.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(u.y, true);
  constexpr uint32_t hi16 = 0x07060302u;  // upper half of src1, then of src0
  return make_uint4(__builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), hi16),
                    __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), hi16),
                    __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), hi16),
                    __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), hi16));
}

}  // namespace

// Two row tiles per wave at 8 waves (512-row tiles) fit in 128 VGPRs, i.e.
// 4 waves per SIMD: two 8-wave workgroups share a CU, so one workgroup's
// per-chunk barrier and combine overlap the other's MFMAs.
template <int DT, int D, int RT, int NW>
__global__ __launch_bounds__(NW * 64, (RT == 2 && NW == 8) ? 4 : 1)
void scores_mfma_kernel(Plan p,
                                                              const typename Elem<DT>::T* __restrict__ q,
                                                              const float* __restrict__ kbar,
                                                              float c2, float* __restrict__ scores) {
  if (p.dscale) c2 *= p.dscale[0];  // fp8 q scale kept on the device
  c2 = __builtin_bit_cast(float, sc_uni(__builtin_bit_cast(int, c2)));  // uniform: a scalar register
  constexpr int NT = NW * 64;
  constexpr int KS = D / 16;            // k-steps of 16 dims
  constexpr int LD = D + 8;             // padded LDS row (bf16), 16-byte multiple
  constexpr int F4 = kChunk * D / 4;    // float4 per kbar chunk
  constexpr int PF = (F4 + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t kb[2][2][kChunk * LD];
  __shared__ float part_m[2][NW][kChunk];
  __shared__ float part_s[2][NW][kChunk];
  __shared__ float red_m[kChunk];
  __shared__ double red_s[kChunk];
  extern __shared__ float dyn[];  // m_J[nch * 32]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int jj = lane & 31;
  const int64_t seg = p.num_segments - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int b = seq_of_segment(p, seg);
  const SeqInfo s = p.seq[b];
  int h, I;
  segment_tile(s, (int)(seg - s.seg_base), h, I);
  const int q0 = tile_q0(s, I, p.B);
  const int R = p.g * tile_nq(s, I, p.B);
  const int nJ = I + 1;
  const int nch = (nJ + kChunk - 1) / kChunk;
  float* mJ = dyn;
  float* row_out = scores + score_offset(s, h, I);
  const float* kb_head = kbar + ((int64_t)s.pool_base * p.hkv + h) * D;
  const int64_t kb_stride = (int64_t)p.hkv * D;  // floats between pooled rows

  // ---- this wave's query rows (A operands), zero beyond R
  const int row0 = wave * RT * 32;
  const bool wave_active = row0 < R;
  sbf16x8_t qa[RT][KS];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = row0 + t * 32 + jj;
    const bool ok = r < R;
    const int pos = q0 + (ok ? r / p.g : 0);
    const int hq = h * p.g + (ok ? r % p.g : 0);
    const int64_t qoff = (q_row(s, pos) * p.hq + hq) * D;
    if constexpr (DT == kFP8) {
      // every lane loads (a padding row reads the tile's first row), so the
      // loads issue back to back instead of one round trip per widening
      uint2 cw[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        cw[ks] = *reinterpret_cast<const uint2*>(q + qoff + ks * 16 + half * 8);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 u = widen_e4m3x8(cw[ks]);
        if (!ok) u = make_uint4(0, 0, 0, 0);
        qa[t][ks] = __builtin_bit_cast(sbf16x8_t, u);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (ok) u = *reinterpret_cast<const uint4*>(q + qoff + ks * 16 + half * 8);
        qa[t][ks] = __builtin_bit_cast(sbf16x8_t, u);
      }
    }
  }

  // ---- kbar chunk staging: global float32 -> registers -> split bf16 in LDS.
  // Raw buffer loads from one scalar descriptor per chunk: the descriptor
  // ends after the chunk's last block, so the rows past it read as zero.
  uint32_t foff[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int f = tid + i * NT;
    foff[i] = (F4 % NT == 0 || f < F4)
                  ? (uint32_t)(f / (D / 4)) * (uint32_t)kb_stride * 4u + (uint32_t)(f % (D / 4)) * 16u
                  : 0x80000000u;  // past every descriptor: reads zero, never stored
  }
  float4 pf[PF];
  auto fetch = [&](int c) __attribute__((always_inline)) {
    const int last = min(kChunk, nJ - c * kChunk) - 1;
    const float* base = kb_head + (int64_t)c * kChunk * kb_stride;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)sc_uniform_ptr(base), (short)0, sc_uni((last * (int)kb_stride + D) * 4), kScRsrcWord3);
#pragma unroll
    for (int i = 0; i < PF; ++i)
      pf[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)foff[i], 0, 0));
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int f = tid + i * NT;
      if (F4 % NT != 0 && f >= F4) break;
      const int j = f / (D / 4);
      const int d0 = (f % (D / 4)) * 4;
      const uint2 p01 = split2_pair(pf[i].x, pf[i].y), p23 = split2_pair(pf[i].z, pf[i].w);
      const int o = j * LD + d0;
      *reinterpret_cast<uint2*>(&kb[buf][0][o]) = make_uint2(p01.x, p23.x);
      *reinterpret_cast<uint2*>(&kb[buf][1][o]) = make_uint2(p01.y, p23.y);
    }
  };

  fetch(0);
  store(0);
  __syncthreads();

  // merge of chunk cc's row partials: wave w takes blocks w*BPW .. +BPW-1 of
  // the chunk, a lane (of each half) the partial of row wave sw for block jl,
  // and groups of NW lanes reduce (max, then the rescaled sum) in a fixed
  // butterfly order.  The partials are double buffered, so the merge of
  // chunk c-1 runs during chunk c, beside its matrix work.  Every lane of a
  // group also folds the block into a running pair (rm, rs): the largest
  // block maximum so far and the sum of S_J 2^(m_J - rm) over its blocks.
  constexpr int BPW = kChunk / NW;
  static_assert(NW == 4 || NW == 8 || NW == 16, "combine groups");
  int jl = wave * BPW + jj / NW, sw = jj % NW;
  float rm = -INFINITY;
  double rs = 0.0;
  auto combine = [&](int cc) __attribute__((always_inline)) {
    const float pmv = part_m[cc & 1][sw][jl], psv = part_s[cc & 1][sw][jl];
    const float m = group_max<NW>(pmv);
    const float S = group_sum<NW>(psv * __builtin_amdgcn_exp2f(pmv - (m == -INFINITY ? 0.f : m)));
    const int J = cc * kChunk + jl;
    if (J < nJ) {
      const float nm = fmaxf(rm, m);
      const float ref = nm == -INFINITY ? 0.f : nm;
      rs = rs * (double)__builtin_amdgcn_exp2f(rm - ref) +
           (double)S * (double)__builtin_amdgcn_exp2f(m - ref);
      rm = nm;
      if (half == 0 && sw == 0) {
        mJ[J] = m;
        row_out[J] = S;
      }
    }
  };

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) fetch(c + 1);
    if (c > 0) combine(c - 1);
    float pm = -INFINITY, ps = 0.f;
    if (wave_active) {
      sf32x16_t acc[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
      }
      // lo, then hi: the small partial sums first
#pragma unroll
      for (int sp = 1; sp >= 0; --sp) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const sbf16x8_t bop = *reinterpret_cast<const sbf16x8_t*>(
              &kb[buf][sp][jj * LD + ks * 16 + half * 8]);
#pragma unroll
          for (int t = 0; t < RT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t][ks], bop, acc[t], 0, 0, 0);
        }
      }
      // max and sum of exp2(c2 * acc) over the wave's rows of block J; the
      // maximum is taken on the raw products (c2 > 0) and the scale enters
      // the exponent's FMA.  Only the chunk past the last block and the row
      // tile past the last row need masks (a uniform test per wave).
      const int J = c * kChunk + jj;
      float mx = -INFINITY;
      if (row0 + RT * 32 <= R && (c + 1) * kChunk <= nJ) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[t][i]);
        }
      } else {
        // rows r < R of the lane: element i of row tile t is row
        // row0 + 32 t + 8 (i >> 2) + 4 half + (i & 3).  The limit is made
        // opaque here, so the 32 comparisons are not hoisted out of the chunk
        // loop as scalar lane masks.
        int t0 = threadIdx.x;
        asm volatile("" : "+v"(t0));
        const int lim = J < nJ ? R - (t0 >> 6) * (RT * 32) - ((t0 >> 5) & 1) * 4 : 0;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            acc[t][i] = t * 32 + (i >> 2) * 8 + (i & 3) < lim ? acc[t][i] : -INFINITY;
            mx = fmaxf(mx, acc[t][i]);
          }
        }
      }
      mx = pair_max(mx);
      const float nmu = mx == -INFINITY ? 0.f : -mx * c2;
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(fmaf(acc[t][i], c2, nmu));
      }
      pm = mx == -INFINITY ? -INFINITY : mx * c2;
      ps = pair_sum(sum);
    }
    if (half == 0) {
      part_m[buf][wave][jj] = pm;
      part_s[buf][wave][jj] = ps;
    }
    if (c + 1 < nch) store(buf ^ 1);
    __syncthreads();
  }
  // the combine indices again, from an opaque copy of the thread index: the
  // values from before the loop would otherwise stay live through it
  {
    int t1 = threadIdx.x;
    asm volatile("" : "+v"(t1));
    jl = (t1 >> 6) * BPW + (t1 & 31) / NW;
    sw = (t1 & 31) % NW;
  }
  combine(nch - 1);
  // M_I and the total sum_J S_J 2^(m_J - M_I) from the 32 running pairs (one
  // per combine group, merged by every thread in the same order), then every
  // score.  The barrier also makes the S_J stores visible.
  if (half == 0 && sw == 0) {
    red_m[jl] = rm;
    red_s[jl] = rs;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kChunk; ++k) M = fmaxf(M, red_m[k]);
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kChunk; ++k) {
    const float mk = red_m[k];
    if (mk != -INFINITY) tot += red_s[k] * (double)__builtin_amdgcn_exp2f(mk - M);
  }
  const float inv = (float)(1.0 / tot);
  for (int J = tid; J < nJ; J += NT)
    row_out[J] = row_out[J] * __builtin_amdgcn_exp2f(mJ[J] - M) * inv;
}

// Ping-pong form for tiles of 513 to 1024 packed rows: 16 waves in two
// groups of 8 (waves 0-7 hold the first 256 RT rows, waves 8-15 the rest,
// two waves of each group per SIMD), group 1 one phase behind group 0.  In
// every phase one group issues the MFMAs of its chunk while the other
// reduces the chunk it multiplied in the previous phase, so a SIMD's matrix
// and vector work come from different waves.  (With one 16-wave workgroup
// per CU and a barrier per chunk, the plain form has every SIMD's four waves
// in the same phase.  Tiles of up to 512 rows keep the plain form: two of
// its 8-wave workgroups share a CU and overlap on their own.)
// Phase p (a barrier after each):
//   group 0: p = 2c: MFMAs of chunk c; p = 2c + 1: reduce chunk c, then merge
//            the partials of chunk c - 1 (all 16 waves have written them);
//   group 1: p = 2c + 1: MFMAs of chunk c, then the global loads of chunk
//            c + 2; p = 2c + 2: reduce chunk c, then store chunk c + 2 into
//            the LDS buffer chunk c occupied (group 1 was its last reader).
// Rows, scores and their accuracy are those of scores_mfma_kernel.
template <int DT, int D, int RT>
__global__ __launch_bounds__(1024, 1) void scores_pp_kernel(Plan p,
                                                            const typename Elem<DT>::T* __restrict__ q,
                                                            const float* __restrict__ kbar, float c2,
                                                            float* __restrict__ scores) {
  if (p.dscale) c2 *= p.dscale[0];  // fp8 q scale kept on the device
  c2 = __builtin_bit_cast(float, sc_uni(__builtin_bit_cast(int, c2)));  // uniform: a scalar register
  constexpr int NW = 16;                // waves; groups of GW
  constexpr int GW = 8;
  constexpr int GT = GW * 64;           // threads per group
  constexpr int KS = D / 16;            // k-steps of 16 dims
  constexpr int LD = D + 8;             // padded LDS row (bf16), 16-byte multiple
  constexpr int F4 = kChunk * D / 4;    // float4 per kbar chunk
  constexpr int PF = (F4 + GT - 1) / GT;
  __shared__ __attribute__((aligned(16))) uint16_t kb[2][2][kChunk * LD];
  __shared__ float part_m[2][NW][kChunk];
  __shared__ float part_s[2][NW][kChunk];
  __shared__ float red_m[kChunk];
  __shared__ double red_s[kChunk];
  extern __shared__ float dyn[];  // m_J[nch * 32]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave / GW;            // uniform per wave
  const int gt = tid - grp * GT;        // thread index within the group
  const int half = lane >> 5;
  const int jj = lane & 31;
  const int64_t seg = p.num_segments - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int b = seq_of_segment(p, seg);
  const SeqInfo s = p.seq[b];
  int h, I;
  segment_tile(s, (int)(seg - s.seg_base), h, I);
  const int q0 = tile_q0(s, I, p.B);
  const int R = p.g * tile_nq(s, I, p.B);
  const int nJ = I + 1;
  const int nch = (nJ + kChunk - 1) / kChunk;
  float* mJ = dyn;
  float* row_out = scores + score_offset(s, h, I);
  const float* kb_head = kbar + ((int64_t)s.pool_base * p.hkv + h) * D;
  const int64_t kb_stride = (int64_t)p.hkv * D;  // floats between pooled rows

  // ---- this wave's query rows (A operands), zero beyond R
  const int row0 = wave * RT * 32;
  const bool wave_active = row0 < R;
  sbf16x8_t qa[RT][KS];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int r = row0 + t * 32 + jj;
    const bool ok = r < R;
    const int pos = q0 + (ok ? r / p.g : 0);
    const int hq = h * p.g + (ok ? r % p.g : 0);
    const int64_t qoff = (q_row(s, pos) * p.hq + hq) * D;
    if constexpr (DT == kFP8) {
      uint2 cw[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        cw[ks] = *reinterpret_cast<const uint2*>(q + qoff + ks * 16 + half * 8);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 u = widen_e4m3x8(cw[ks]);
        if (!ok) u = make_uint4(0, 0, 0, 0);
        qa[t][ks] = __builtin_bit_cast(sbf16x8_t, u);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (ok) u = *reinterpret_cast<const uint4*>(q + qoff + ks * 16 + half * 8);
        qa[t][ks] = __builtin_bit_cast(sbf16x8_t, u);
      }
    }
  }

  // ---- kbar chunk staging by one group: raw buffer loads from one scalar
  // descriptor per chunk (rows past the chunk's last block read zero), then
  // the two-term split into LDS
  float4 pf[PF];
  auto fetch = [&](int c) __attribute__((always_inline)) {
    const int last = min(kChunk, nJ - c * kChunk) - 1;
    const float* base = kb_head + (int64_t)c * kChunk * kb_stride;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)sc_uniform_ptr(base), (short)0, sc_uni((last * (int)kb_stride + D) * 4), kScRsrcWord3);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int f = gt + i * GT;
      const uint32_t off = (F4 % GT == 0 || f < F4)
          ? (uint32_t)(f / (D / 4)) * (uint32_t)kb_stride * 4u + (uint32_t)(f % (D / 4)) * 16u
          : 0x80000000u;  // past every descriptor: reads zero, never stored
      pf[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int f = gt + i * GT;
      if (F4 % GT != 0 && f >= F4) break;
      const int j = f / (D / 4);
      const int d0 = (f % (D / 4)) * 4;
      const uint2 p01 = split2_pair(pf[i].x, pf[i].y), p23 = split2_pair(pf[i].z, pf[i].w);
      const int o = j * LD + d0;
      *reinterpret_cast<uint2*>(&kb[buf][0][o]) = make_uint2(p01.x, p23.x);
      *reinterpret_cast<uint2*>(&kb[buf][1][o]) = make_uint2(p01.y, p23.y);
    }
  };

  // group 0 stages chunk 0, group 1 chunk 1
  if (grp == 0 || nch > 1) {
    fetch(grp);
    store(grp);
  }
  if (tid < kChunk) {
    red_m[tid] = -INFINITY;
    red_s[tid] = 0.0;
  }
  __syncthreads();

  // merge of chunk cc's partials by group 0: wave gw takes blocks 4 gw ..
  // 4 gw + 3 of the chunk, a lane the partial of wave sw (of 16) for block
  // jl, and groups of 16 lanes reduce in a fixed butterfly order.  The lane
  // group also folds the block into its running pair (rm, rs), kept in LDS
  // by the group's first lane: the largest block maximum so far and the
  // float64 sum of S_J 2^(m_J - rm) over its blocks.
  auto combine = [&](int cc) __attribute__((always_inline)) {
    const int jl = (tid >> 4) & 31, sw = tid & 15;
    const float pmv = part_m[cc & 1][sw][jl], psv = part_s[cc & 1][sw][jl];
    const float m = group_max<16>(pmv);
    const float S = group_sum<16>(psv * __builtin_amdgcn_exp2f(pmv - (m == -INFINITY ? 0.f : m)));
    const int J = cc * kChunk + jl;
    if (J < nJ && sw == 0) {
      const float rm = red_m[jl];
      const float nm = fmaxf(rm, m);
      const float ref = nm == -INFINITY ? 0.f : nm;
      red_s[jl] = red_s[jl] * (double)__builtin_amdgcn_exp2f(rm - ref) +
                  (double)S * (double)__builtin_amdgcn_exp2f(m - ref);
      red_m[jl] = nm;
      mJ[J] = m;
      row_out[J] = S;
    }
  };

  sf32x16_t acc[RT];
  auto mfma = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    }
    // lo, then hi: the small partial sums first
#pragma unroll
    for (int sp = 1; sp >= 0; --sp) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const sbf16x8_t bop = *reinterpret_cast<const sbf16x8_t*>(
            &kb[c & 1][sp][jj * LD + ks * 16 + half * 8]);
#pragma unroll
        for (int t = 0; t < RT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t][ks], bop, acc[t], 0, 0, 0);
      }
    }
  };
  // max and sum of exp2(c2 * acc) over the wave's rows of block J; the
  // maximum is taken on the raw products (c2 > 0) and the scale enters the
  // exponent's FMA.  Only the chunk past the last block and the row tile
  // past the last row need masks (a uniform test per wave).
  auto reduce = [&](int c) __attribute__((always_inline)) {
    float pm = -INFINITY, ps = 0.f;
    if (wave_active) {
      const int J = c * kChunk + jj;
      float mx = -INFINITY;
      if (row0 + RT * 32 <= R && (c + 1) * kChunk <= nJ) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[t][i]);
        }
      } else {
        // element i of row tile t is row row0 + 32 t + 8 (i >> 2) + 4 half + (i & 3)
        int t0 = threadIdx.x;
        asm volatile("" : "+v"(t0));
        const int lim = J < nJ ? R - (t0 >> 6) * (RT * 32) - ((t0 >> 5) & 1) * 4 : 0;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            acc[t][i] = t * 32 + (i >> 2) * 8 + (i & 3) < lim ? acc[t][i] : -INFINITY;
            mx = fmaxf(mx, acc[t][i]);
          }
        }
      }
      mx = pair_max(mx);
      const float nmu = mx == -INFINITY ? 0.f : -mx * c2;
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(fmaf(acc[t][i], c2, nmu));
      }
      pm = mx == -INFINITY ? -INFINITY : mx * c2;
      ps = pair_sum(sum);
    }
    if (half == 0) {
      part_m[c & 1][wave][jj] = pm;
      part_s[c & 1][wave][jj] = ps;
    }
  };

  // Both groups pass 2 nch + 1 barriers; each group's loop keeps a chunk's
  // accumulators within one iteration.
  if (grp == 0) {
    for (int c = 0; c < nch; ++c) {
      if (wave_active) mfma(c);  // phase 2c
      __syncthreads();
      reduce(c);  // phase 2c + 1
      if (c > 0) combine(c - 1);
      __syncthreads();
    }
    __syncthreads();  // phase 2 nch: group 1 reduces the last chunk
  } else {
    __syncthreads();  // phase 0
    for (int c = 0; c < nch; ++c) {
      if (wave_active) mfma(c);  // phase 2c + 1
      if (c + 2 < nch) fetch(c + 2);
      __syncthreads();
      reduce(c);  // phase 2c + 2
      if (c + 2 < nch) store(c & 1);
      __syncthreads();
    }
  }
  if (grp == 0) combine(nch - 1);
  __syncthreads();
  // M_I and the total sum_J S_J 2^(m_J - M_I) from the 32 running pairs
  // (merged by every thread in the same order), then every score
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kChunk; ++k) M = fmaxf(M, red_m[k]);
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kChunk; ++k) {
    const float mk = red_m[k];
    if (mk != -INFINITY) tot += red_s[k] * (double)__builtin_amdgcn_exp2f(mk - M);
  }
  const float inv = (float)(1.0 / tot);
  for (int J = tid; J < nJ; J += 1024)
    row_out[J] = row_out[J] * __builtin_amdgcn_exp2f(mJ[J] - M) * inv;
}

template <int DT, int D, int RT>
static hipError_t launch_scores_pp(const Plan& p, const void* q, const float* kbar, float c2,
                                   float* scores, hipStream_t st) {
  const int nch = (p.max_nblk + kChunk - 1) / kChunk;
  const size_t lds = sizeof(float) * nch * kChunk;
  hipLaunchKernelGGL((scores_pp_kernel<DT, D, RT>), dim3((unsigned)p.num_segments), dim3(1024),
                     lds, st, p, (const typename Elem<DT>::T*)q, kbar, c2, scores);
  return hipGetLastError();
}

template <int DT, int D, int RT, int NW>
static hipError_t launch_scores_t(const Plan& p, const void* q, const float* kbar, float c2,
                                  float* scores, hipStream_t st) {
  const int nch = (p.max_nblk + kChunk - 1) / kChunk;
  const size_t lds = sizeof(float) * nch * kChunk;
  hipLaunchKernelGGL((scores_mfma_kernel<DT, D, RT, NW>), dim3((unsigned)p.num_segments),
                     dim3(NW * 64), lds, st, p, (const typename Elem<DT>::T*)q, kbar, c2, scores);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_scores_d(const Plan& p, const void* q, const float* kbar, float c2,
                                  float* scores, hipStream_t st) {
  const int rmax = p.g * p.B;
  if (rmax <= 128) return launch_scores_t<DT, D, 1, 4>(p, q, kbar, c2, scores, st);
  if (rmax <= 256) return launch_scores_t<DT, D, 2, 4>(p, q, kbar, c2, scores, st);
  if (rmax <= 512) return launch_scores_t<DT, D, 2, 8>(p, q, kbar, c2, scores, st);
  return launch_scores_pp<DT, D, 2>(p, q, kbar, c2, scores, st);
}

bool scores_mfma_supported(const Plan& p, int dtype) {
  return (dtype == kBF16 || dtype == kFP8) && p.g * p.B <= 1024;
}

hipError_t launch_scores_mfma(const Plan& p, int dtype, const void* q, const float* kbar,
                              float c2, float* scores, hipStream_t st) {
  if (p.num_segments == 0) return hipSuccess;
  if (dtype == kBF16)
    return p.d == 128 ? launch_scores_d<kBF16, 128>(p, q, kbar, c2, scores, st)
                      : launch_scores_d<kBF16, 64>(p, q, kbar, c2, scores, st);
  return p.d == 128 ? launch_scores_d<kFP8, 128>(p, q, kbar, c2, scores, st)
                    : launch_scores_d<kFP8, 64>(p, q, kbar, c2, scores, st);
}

}  // namespace bslp
