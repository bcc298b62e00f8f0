// Stage 3 for fp8 (e4m3) inputs on the fp8 matrix cores: block-sparse causal
// online-softmax attention with mean correction and PackGQA rows, in the FP8
// arithmetic of "FlashPrefill V2" (FP8 paragraph; CSR, tile, PackGQA and
// paged-KV paragraphs; Sec. 3.2 / Fig. 3 correction path; Tab. 8 paragraph
// for the quantised pooled statistics).  Written for gfx950 wave64 MFMA.
//
// Arithmetic.  With per-tensor scales c_q, c_k, c_v and x = s * c the logit
// of the codes in log2 units (c = softmax_scale c_q c_k log2 e):
//   m     the exact running row maximum, raised at every 64-key step whose
//         maximum exceeds it (the accumulated numerator and l are rescaled);
//   P~    = e4m3(2^8 * 2^(x - m)), rounded to nearest even by the conversion
//         instruction, so P~ lies in [0, 256];
//   O^T  += V~^T P~^T and l += 1^T P~^T on v_mfma_f32_32x32x64_f8f6f4 (the
//         ones operand makes l the sum of exactly the rounded P~);
//   O     = c_v O^T / l, LSE = m ln 2 + ln l - 8 ln 2.
// Correction steps use the pooled means rounded to e4m3 on the same
// per-tensor scales (the exact mean of a block's codes, rounded to nearest
// even, written once per call into the workspace from K and V themselves),
// with the score shifted by log2 |B_J|.
//
// Work unit and step sequence as in the bf16 kernel (attn_common.hpp): one
// workgroup of NW waves x 32 PackGQA rows of one tile; the selected blocks
// walked backwards in descending 64-key tiles, then the correction chunks.
//
// MFMA layout.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = 32 key rows x
// 16 dims from LDS, B = the lane's query row, both e4m3 codes widened exactly
// to bf16.  (The fp8 MFMA sums its 64 products with about 13 bits relative
// to the largest product - 1.8e-5 of the logit on these workloads, against
// 1e-7 for the bf16 MFMA - which would flip the e4m3 rounding of P~ for
// keys near a rounding midpoint.)  In the 32x32
// accumulator lane half h holds accumulator rows 8a + 4h + r of each 32-row
// tile; K rows are stored in LDS so that those rows are keys 32h + 16kt + 4a
// + r, i.e. lane half h holds keys 32h .. 32h+31 in the order of its bytes.
// P~ then feeds O^T += V~^T P~^T straight from registers as the B operand,
// and V~^T is stored in LDS with its keys in natural order: [d][64 keys],
// rows padded to 80 bytes, the four 16-byte chunks of a row XOR-swizzled by
// (d >> 4) & 3 so the transposing writes spread over the banks.
//
// V layouts.  Row-major V ([tokens, Hkv, d], like K) is transposed while it
// is staged (4 keys x 4 dims per thread, eight byte permutes).  Column-major
// V ([Hkv, d, kv tokens], or [pages, Hkv, d, page] when paged) is staged by
// plain 16-byte copies (the V-layout bullets of the FP8 paragraph).
#include <algorithm>
#include <atomic>
#include <cstddef>

#include "attn_common.hpp"
#include "launch.hpp"

namespace bslp {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr float kOffsetLog2 = 8.f;  // P~ = e4m3(2^8 p)

// LDS row of key `key` (0..63) of a step: key 32h + 16kt + 4a + r goes to
// accumulator row 32kt + 8a + 4h + r.
__device__ __forceinline__ int krow_of(int key) {
  return 32 * ((key >> 4) & 1) + 8 * ((key >> 2) & 3) + 4 * (key >> 5) + (key & 3);
}

// 16-byte chunk swizzle of V^T row d
__device__ __forceinline__ int vswz(int d) { return (d >> 4) & 3; }

template <int D, int NW>
struct F8Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = NW * 32;        // packed rows per unit
  static constexpr int KS = D / 16;           // k-steps of Q K^T (bf16 MFMA)
  static constexpr int DT = D / 32;           // 32-dim tiles of O^T
  static constexpr int KROW = 2 * D + 16;     // LDS bytes per K row (widened to bf16)
  static constexpr int VROW = kKeys + 16;     // LDS bytes per V^T row (e4m3)
  static constexpr int NK = kKeys * D / 8;    // 8-code K pieces per step
  static constexpr int KL = (NK + NT - 1) / NT;
  static constexpr int NP = kKeys * D / 16;   // V blocks (4 keys x 4 dims) or V^T chunks per step
  static constexpr int PL = (NP + NT - 1) / NT;
};

template <int D, int NW>
struct F8Prefetch {
  uint2 k[F8Cfg<D, NW>::KL];    // 8 e4m3 codes of one key
  u32x4_t v[F8Cfg<D, NW>::PL];  // row-major: 4 keys' 4 bytes; d-major: 20 bytes from a
  uint32_t vx[F8Cfg<D, NW>::PL];  //   4-byte boundary (v, vx) holding 16 keys at byte vs
  uint32_t vs[F8Cfg<D, NW>::PL];
};

// Global -> registers for one step.  Exact steps read tokens key0.. of the
// request, correction steps the e4m3 pooled rows pool_base + 64c.. of the
// workspace.  When the step's rows are consecutive in memory the loads are
// raw buffer loads from one scalar descriptor whose range ends after the
// step's last valid row, so rows past it read as zero (their keys are
// masked).  Pages below 64 tokens resolve every key's row on its own.
template <int D, int NW, bool VCOL>
__device__ __forceinline__ void f8_fetch(F8Prefetch<D, NW>& pf, const Step& st, const UnitCtx& u,
                                         const KVDesc& kv, int hkv, int64_t kv_tokens,
                                         const uint8_t* k, const uint8_t* v, const uint8_t* kq,
                                         const uint8_t* vq) {
  using C = F8Cfg<D, NW>;
  const int tid = threadIdx.x;
  const bool exact = st.kind == kExact;
  const int key0 = exact ? st.J * u.B + st.hf * kKeys : kCorrRows * st.c;
  const int last = exact ? min(kKeys, u.len - key0) - 1 : min(kCorrRows, u.I - key0) - 1;
  const bool paged = exact && kv.page_table != nullptr;
  const uint32_t stride = (uint32_t)hkv * D;  // bytes between token rows
  if (!paged || kv.page_shift >= 6) {
    int64_t row0;
    int phys = 0;
    if (!exact) {
      row0 = (int64_t)u.pool_base + key0;
    } else if (paged) {
      phys = uni(kv.page_table[(int64_t)u.b * kv.max_pages + (key0 >> kv.page_shift)]);
      row0 = ((int64_t)phys << kv.page_shift) | (int64_t)(key0 & ((1 << kv.page_shift) - 1));
    } else {
      row0 = (int64_t)u.kv_start + key0;
    }
    const int nrec = (int)(last * stride + D);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr((exact ? k : kq) + row0 * stride + (int64_t)u.h * D), (short)0,
        uni(nrec), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < C::KL; ++i) {
      const int f = min(tid + i * C::NT, C::NK - 1);
      const int key = f / (D / 8), piece = f % (D / 8);
      const auto w =
          __builtin_amdgcn_raw_buffer_load_b64(rk, (int)(key * stride + piece * 8), 0, 0);
      pf.k[i] = make_uint2(w[0], w[1]);
    }
    if (VCOL && exact) {
      // V^T rows of d: [Hkv, d, kv tokens], or [pages, Hkv, d, page].  The
      // token stride need not be a multiple of 4, and the buffer range is
      // checked a 4-byte word at a time, so the loads start from the 4-byte
      // boundary below key0 (sh0 bytes before it) and each 16-key piece is
      // read as 20 bytes from the boundary below it, realigned when stored.
      // The range ends at the word holding the last valid key of row D-1,
      // inside the V array (whose end is a 4-byte boundary).
      int64_t base;
      int64_t dstride;
      if (paged) {
        dstride = (int64_t)1 << kv.page_shift;
        base = ((int64_t)phys * hkv + u.h) * D * dstride + (key0 & ((1 << kv.page_shift) - 1));
      } else {
        dstride = kv_tokens;
        base = (int64_t)u.h * D * dstride + row0;
      }
      const int sh0 = (int)(base & 3);
      const int span = sh0 + (int)((D - 1) * dstride) + last + 1;
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)uniform_ptr(v + (base - sh0)), (short)0, uni((span + 3) & ~3), kRsrcWord3);
#pragma unroll
      for (int i = 0; i < C::PL; ++i) {
        const int f = min(tid + i * C::NT, C::NP - 1);
        const int pos = sh0 + (int)((f >> 2) * dstride) + (f & 3) * 16;
        pf.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, pos & ~3, 0, 0);
        pf.vx[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, (pos & ~3) + 16, 0, 0);
        pf.vs[i] = (uint32_t)(pos & 3);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)uniform_ptr((exact ? v : vq) + row0 * stride + (int64_t)u.h * D), (short)0,
          uni(nrec), kRsrcWord3);
#pragma unroll
      for (int i = 0; i < C::PL; ++i) {
        const int f = min(tid + i * C::NT, C::NP - 1);
        const int u4 = f % (D / 4), q = f / (D / 4);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          pf.v[i][kk] =
              __builtin_amdgcn_raw_buffer_load_b32(rv, (int)((4 * q + kk) * stride + 4 * u4), 0, 0);
      }
    }
    return;
  }
  // paged with pages below 64 tokens (row-major V only): keys past the last
  // valid one re-read it
  const int64_t hoff = (int64_t)u.h * D;
#pragma unroll
  for (int i = 0; i < C::KL; ++i) {
    const int f = min(tid + i * C::NT, C::NK - 1);
    const int key = min(f / (D / 8), last), piece = f % (D / 8);
    const int64_t row = kv.row(u.b, u.kv_start, key0 + key);
    pf.k[i] = *reinterpret_cast<const uint2*>(k + row * stride + hoff + piece * 8);
  }
#pragma unroll
  for (int i = 0; i < C::PL; ++i) {
    const int f = min(tid + i * C::NT, C::NP - 1);
    const int u4 = f % (D / 4), q = f / (D / 4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int64_t row = kv.row(u.b, u.kv_start, key0 + min(4 * q + kk, last));
      pf.v[i][kk] = *reinterpret_cast<const uint32_t*>(v + row * stride + hoff + 4 * u4);
    }
  }
}

// Last valid key (0 .. 63) of an exact step: keys past the request end are
// masked; 63 for every other step.
__device__ __forceinline__ int step_last_key(const Step& st, const UnitCtx& u) {
  if (st.kind != kExact) return kKeys - 1;
  return min(kKeys, u.len - (st.J * u.B + st.hf * kKeys)) - 1;
}

// Eight e4m3 codes widened to eight bf16, exactly (an e4m3 value has 4
// significant bits; its float32 bits end in 16 zeros).
__device__ __forceinline__ u32x4_t widen8(uint2 w) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
  constexpr uint32_t hi16 = 0x07060302u;  // upper halves of src1, then src0
  return u32x4_t{__builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), hi16),
                 __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), hi16),
                 __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), hi16),
                 __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), hi16)};
}

// Registers -> LDS: K rows widened to bf16 at their permuted rows, V^T
// [d][keys] (swizzled 16-byte chunks), transposed here from row-major pieces.
template <int D, int NW>
__device__ __forceinline__ void f8_store(const F8Prefetch<D, NW>& pf, bool vcol, int vlast,
                                         uint8_t* Ks, uint8_t* Vt) {
  using C = F8Cfg<D, NW>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KL; ++i) {
    const int f = tid + i * C::NT;
    if (C::NK % C::NT != 0 && f >= C::NK) break;
    const int key = f / (D / 8), piece = f % (D / 8);
    *reinterpret_cast<u32x4_t*>(Ks + krow_of(key) * C::KROW + piece * 16) = widen8(pf.k[i]);
  }
  if (vcol) {
#pragma unroll
    for (int i = 0; i < C::PL; ++i) {
      const int f = tid + i * C::NT;
      if (C::NP % C::NT != 0 && f >= C::NP) break;
      const int d = f >> 2, ch = f & 3;
      const u32x4_t r = pf.v[i];
      const uint32_t sb = pf.vs[i];  // the piece starts sb bytes into the 20 loaded
      u32x4_t x = {__builtin_amdgcn_alignbyte(r[1], r[0], sb),
                   __builtin_amdgcn_alignbyte(r[2], r[1], sb),
                   __builtin_amdgcn_alignbyte(r[3], r[2], sb),
                   __builtin_amdgcn_alignbyte(pf.vx[i], r[3], sb)};
      // keys past the request's last one hold other tokens (or unwritten page
      // bytes, possibly the NaN code): zero, so that 0 x V stays 0
      if (ch * 16 + 15 > vlast) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int keep = vlast - (ch * 16 + 4 * w) + 1;  // bytes of this word to keep
          x[w] &= keep <= 0 ? 0u : keep >= 4 ? ~0u : (1u << (8 * keep)) - 1u;
        }
      }
      *reinterpret_cast<u32x4_t*>(Vt + d * C::VROW + ((ch ^ vswz(d)) << 4)) = x;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::PL; ++i) {
    const int f = tid + i * C::NT;
    if (C::NP % C::NT != 0 && f >= C::NP) break;
    const int u4 = f % (D / 4), q = f / (D / 4);
    const u32x4_t w = pf.v[i];  // w[kk]: key 4q+kk, dims 4u4 .. 4u4+3
    const uint32_t x01lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
    const uint32_t x01hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
    const uint32_t x23lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t x23hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    const uint32_t o[4] = {__builtin_amdgcn_perm(x23lo, x01lo, 0x05040100u),
                           __builtin_amdgcn_perm(x23lo, x01lo, 0x07060302u),
                           __builtin_amdgcn_perm(x23hi, x01hi, 0x05040100u),
                           __builtin_amdgcn_perm(x23hi, x01hi, 0x07060302u)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 4 * u4 + j;
      *reinterpret_cast<uint32_t*>(Vt + d * C::VROW + (((q >> 2) ^ vswz(d)) << 4) + 4 * (q & 3)) =
          o[j];
    }
  }
}

// 32 bytes from two 16-byte LDS pieces
__device__ __forceinline__ i32x8_t load32(const uint8_t* p0, const uint8_t* p1) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p0);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p1);
  return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                 (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x16_t mfma8(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  // e4m3 x e4m3 (format 0 for both operands), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// kF8CorrAll: a correction chunk of 64 valid pooled blocks, none selected
// (nothing to mask)
enum F8Mode : int { kF8Plain = 0, kF8Diag = 1, kF8Corr = 2, kF8CorrAll = 3 };

// One 64-key step of one wave: S^T = K Q^T on the bf16 matrix cores (codes
// widened exactly, so the logits carry only float32 rounding), exact running
// maximum, P~ = e4m3(2^8 2^(x - m)), O^T += V~^T P~^T and l += 1^T P~^T on
// the fp8 matrix cores.
template <int D, int NW>
__device__ __forceinline__ void f8_step(const uint8_t* Ks, const uint8_t* Vt,
                                        const bf16x8_t (&qf)[D / 16], f32x16_t (&oacc)[D / 32],
                                        f32x16_t& lacc, float& m_run, float c, int mode, int key0,
                                        int qpos, uint64_t todo, float bias) {
  using C = F8Cfg<D, NW>;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 31, half = lane >> 5;
  const f32x16_t zero = {};
  f32x16_t sacc[2];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Ks + (rl + 32 * kt) * C::KROW +
                                                           32 * ks + 16 * half);
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? zero : sacc[kt], 0,
                                                         0, 0);
    }
  }
  // the lane's value e of tile kt is key key0 + 32 half + 16 kt + e
  if (mode == kF8Diag || mode == kF8Corr) {
    uint32_t bits;
    int lim;
    if (mode == kF8Diag) {
      bits = ~0u;
      lim = qpos - key0 - 32 * half;  // keys after the row are masked
    } else {
      bits = (uint32_t)(todo >> (32 * half));
      lim = 31;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int p = 16 * kt + e;
        const bool keep = ((bits >> p) & 1u) && p <= lim;
        sacc[kt][e] = keep ? sacc[kt][e] : -INFINITY;
      }
    }
  }
  const float cb = mode >= kF8Corr ? bias : 0.f;
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kt][e]);
  }
  mx = fmaf(halves_max(mx), c, cb);  // c > 0: the maximum commutes with the scale
  const float m_new = fmaxf(m_run, mx);
  // exact running maximum: rescale whenever it rises (m_run = -inf: nothing
  // accumulated yet, the factor is 0)
  const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
  }
  lacc[0] *= alpha;
  m_run = m_new;
  const float moff = cb + kOffsetLog2 - (m_new == -INFINITY ? 0.f : m_new);
  i32x8_t pb;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int kt = w >> 2, e0 = 4 * (w & 3);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][e0], c, moff));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][e0 + 1], c, moff));
    const float p2 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][e0 + 2], c, moff));
    const float p3 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][e0 + 3], c, moff));
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
    pb[w] = word;
  }
  const i32x8_t ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    const int d = 32 * dt + rl;
    const uint8_t* row = Vt + d * C::VROW;
    oacc[dt] = mfma8(load32(row + (((2 * half) ^ vswz(d)) << 4),
                            row + (((2 * half + 1) ^ vswz(d)) << 4)),
                     pb, oacc[dt]);
  }
  lacc = mfma8(ones, pb, lacc);
}

}  // namespace

// The kernel's parameters as one struct, member for member (the layout of
// the kernel-argument segment; checked below against the kernel's
// signature).  The host packs a launch into it, and persistent unsplit
// launches read their arguments from the segment through opaque_kernargs.
struct F8KernArgs {
  Plan p;
  KVDesc kv;
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* kq;
  const uint8_t* vq;
  const int32_t* cu;
  const int32_t* idx;
  float c, out_scale;
  int correction, dense, units_per_seg, splits;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_ml;
  const int32_t* items;
  int* queue;
};

// PERSIST: workgroups take units from the work list until it is empty.
// OPQ (persistent unsplit launches): the arguments are read through
// opaque_kernargs and units come from per-XCD queues; split launches keep
// plain arguments and one shared queue.
template <int D, int NW, bool PERSIST, bool CORR, bool VCOL, bool OPQ = false>
__global__ __launch_bounds__(NW * 64) void attn_fp8_kernel(
    Plan p, KVDesc kv_a, const uint8_t* __restrict__ q_a, const uint8_t* __restrict__ k_a,
    const uint8_t* __restrict__ v_a, const uint8_t* __restrict__ kq_a,
    const uint8_t* __restrict__ vq_a, const int32_t* __restrict__ cu_a,
    const int32_t* __restrict__ idx_a, float c_a, float out_scale_a, int correction_a,
    int dense_a, int units_per_seg, int splits_a, uint16_t* __restrict__ out_a,
    float* __restrict__ lse_a, float* __restrict__ part_o_a, float* __restrict__ part_ml_a,
    const int32_t* __restrict__ items_a, int* __restrict__ queue_a) {
  using C = F8Cfg<D, NW>;
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][kKeys * C::KROW];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[2][D * C::VROW];
  __shared__ uint32_t selbits[kMaxBlocksPerSeq / 32];
  __shared__ int next_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;

  const Plan& p_outer = p;
  auto run_unit = [&](int b, int I, int h, int mt, int sp) __attribute__((always_inline)) {
  // the arguments, from the segment afresh for every unit when OPQ
  const F8KernArgs* ka = OPQ ? opaque_kernargs<F8KernArgs>() : nullptr;
  const Plan& p = OPQ ? ka->p : p_outer;
  const KVDesc& kv = OPQ ? ka->kv : kv_a;
  const uint8_t* q = OPQ ? ka->q : q_a;
  const uint8_t* k = OPQ ? ka->k : k_a;
  const uint8_t* v = OPQ ? ka->v : v_a;
  const uint8_t* kq = OPQ ? ka->kq : kq_a;
  const uint8_t* vq = OPQ ? ka->vq : vq_a;
  const int32_t* cu = OPQ ? ka->cu : cu_a;
  const int32_t* idx = OPQ ? ka->idx : idx_a;
  float c = OPQ ? ka->c : c_a, out_scale = OPQ ? ka->out_scale : out_scale_a;
  if (p.dscale) {  // scales kept on the device
    c *= p.dscale[0] * p.dscale[1];
    out_scale = p.dscale[2];
  }
  // none when compiled without correction steps
  const int correction = CORR ? (OPQ ? ka->correction : correction_a) : 0;
  const int dense = OPQ ? ka->dense : dense_a;
  const int splits = OPQ ? ka->splits : splits_a;
  uint16_t* out = OPQ ? ka->out : out_a;
  float* lse = OPQ ? ka->lse : lse_a;
  float* part_o = OPQ ? ka->part_o : part_o_a;
  float* part_ml = OPQ ? ka->part_ml : part_ml_a;
  const SeqInfo s = p.seq[b];
  const int64_t seg = (int64_t)s.seg_base + (int64_t)h * ntile(s) + (I - s.i0);
  const int q0 = tile_q0(s, I, p.B);
  const int R = p.g * tile_nq(s, I, p.B);
  const int beg0 = dense ? 0 : cu[seg], n_sel = (dense ? I + 1 : cu[seg + 1]) - beg0;
  const int ns = splits == 1 ? 1 : segment_splits(n_sel, I, p.B, correction, splits);
  const int qmax = q0 + max(min(R, (mt + 1) * C::ROWS) - 1, 0) / p.g;
  UnitCtx u{b, h, I, s.len, s.kv_start, s.pool_base, p.B,
            beg0 + (int)((int64_t)sp * n_sel / ns),
            beg0 + (int)((int64_t)(sp + 1) * n_sel / ns), dense, sp, ns,
            min(s.len, qmax + 1)};

  // ---- this lane's query row (B operand of Q K^T): e4m3 codes widened to
  // bf16, dims 16 ks + 8 half .. +7
  const int r = mt * C::ROWS + wave * 32 + (lane & 31);
  const bool valid = r < R;
  const bool wave_active = mt * C::ROWS + wave * 32 < R;
  const int qpos = q0 + (valid ? r / p.g : 0);
  const int hq = h * p.g + (valid ? r % p.g : 0);
  bf16x8_t qf[C::KS];
  {
    // every lane loads (a padding row reads the tile's first row), then the
    // padding rows are zeroed
    const uint8_t* qp = q + (q_row(s, qpos) * p.hq + hq) * D + 8 * half;
    uint2 cw[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) cw[ks] = *reinterpret_cast<const uint2*>(qp + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4_t w = widen8(cw[ks]);
      if (!valid) w = u32x4_t{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // ---- selected-block bitmap for the correction chunks
  if (correction && I > 0) {
    const int nwords = (I + 31) >> 5;
    for (int w = tid; w < nwords; w += C::NT) selbits[w] = 0u;
    __syncthreads();
    for (int t = beg0 + tid; t < beg0 + n_sel; t += C::NT) {
      const int J = block_at(idx, t, u);
      if (J < I) atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
  }

  f32x16_t oacc[C::DT];
  f32x16_t lacc = {};
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -INFINITY;
  const float bias = __log2f((float)p.B);  // corrected blocks are full blocks

  F8Prefetch<D, NW> pf;
  Step cur = first_step(u, idx, selbits, correction);
  if (cur.kind != kDone) {
    f8_fetch<D, NW, VCOL>(pf, cur, u, kv, p.hkv, p.kv_tokens, k, v, kq, vq);
    f8_store<D, NW>(pf, VCOL && cur.kind == kExact, step_last_key(cur, u), Ks[0], Vt[0]);
  }
  uniform(cur);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): query rows and the first step
  Step nxt = cur;
  if (cur.kind != kDone) advance(nxt, u, idx, selbits, correction);
  uniform(nxt);
  if (nxt.kind != kDone) f8_fetch<D, NW, VCOL>(pf, nxt, u, kv, p.hkv, p.kv_tokens, k, v, kq, vq);
  int buf = 0;
  // Per step: barrier (step n is in LDS, the other buffer is free), write the
  // prefetched step n+1 to the other buffer, issue the loads of step n+2,
  // multiply step n.
  while (cur.kind != kDone) {
    __syncthreads();
    Step nn = nxt;
    if (nn.kind != kDone) {
      advance(nn, u, idx, selbits, correction);
      uniform(nn);
    }
    if (nxt.kind != kDone)
      f8_store<D, NW>(pf, VCOL && nxt.kind == kExact, step_last_key(nxt, u), Ks[buf ^ 1],
                      Vt[buf ^ 1]);
    if (nn.kind != kDone) f8_fetch<D, NW, VCOL>(pf, nn, u, kv, p.hkv, p.kv_tokens, k, v, kq, vq);
    if (wave_active) {
      int mode, key0 = 0;
      uint64_t todo = 0;
      if (cur.kind == kExact) {
        key0 = cur.J * p.B + cur.hf * kKeys;
        mode = cur.J == I ? kF8Diag : kF8Plain;
      } else {
        key0 = kCorrRows * cur.c;
        todo = chunk_todo(selbits, cur.c, I);
        mode = todo == ~0ull ? kF8CorrAll : kF8Corr;
      }
      f8_step<D, NW>(Ks[buf], Vt[buf], qf, oacc, lacc, m_run, c, mode, key0, qpos, todo, bias);
    }
    cur = nxt;
    nxt = nn;
    buf ^= 1;
  }

  // ---- epilogue: l = sum of the rounded probabilities (both lane halves
  // hold it); a split unit leaves its partial result for the merge kernel
  if (!valid) return;
  const float l_tot = lacc[0];
  const float inv = l_tot > 0.f ? out_scale / l_tot : 0.f;
  const int64_t orow = q_row(s, qpos) * p.hq + hq;
  if (ns > 1) {
    const int64_t prow = (int64_t)sp * p.total_tokens * p.hq + orow;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + half * 4;
        *reinterpret_cast<float4*>(part_o + prow * D + d) =
            make_float4(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv,
                        oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
      }
    }
    if (half == 0)
      *reinterpret_cast<float2*>(part_ml + 2 * prow) =
          make_float2(l_tot > 0.f ? m_run : -INFINITY, l_tot);
    return;
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = dt * 32 + g4 * 8 + half * 4;
      const uint32_t lo = pack_bf16x2(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv);
      const uint32_t hi = pack_bf16x2(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv);
      *reinterpret_cast<uint2*>(out + orow * D + d) = make_uint2(lo, hi);
    }
  }
  if (lse && half == 0)
    lse[(int64_t)hq * p.total_tokens + q_row(s, qpos)] =
        l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) - kOffsetLog2 * kLn2 : -INFINITY;
  };

  if constexpr (!PERSIST) {
    // one workgroup per unit, enumerated heaviest first: longest request
    // first, tiles in descending I, then row block, KV head innermost.  (The
    // bf16 kernel turns the head every kHeadTurn groups; here that made no
    // difference to the time and raised the HBM reads, so each XCD keeps one
    // head.)
    const int64_t unit = blockIdx.x;
    int pos = 0;
    while (pos + 1 < p.num_seqs && p.seq[p.order[pos + 1]].unit_base <= unit) ++pos;
    const int b = p.order[pos];
    const int64_t local = unit - p.seq[b].unit_base;
    const int per_I = p.hkv * units_per_seg;
    const int rem = (int)(local % per_I);
    run_unit(b, p.seq[b].nblk - 1 - (int)(local / per_I), rem % p.hkv, rem / p.hkv, 0);
  } else if constexpr (OPQ) {
    // unsplit: item k in queue k mod 8 (the XCD a one-workgroup-per-unit
    // launch would run it on); the own XCD's queue first, then the others
    __shared__ int q_cur[2];  // queue being drained, queues found empty
    if (tid == 0) {
      q_cur[0] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;  // XCC_ID
      q_cur[1] = 0;
    }
    for (;;) {
      if (tid == 0) {
        const F8KernArgs* kg = opaque_kernargs<F8KernArgs>();
        const int n_items = kg->queue[1];
        int qx = q_cur[0], tried = q_cur[1], code = -1;
        while (tried < 8) {
          const int kk = qx + 8 * atomicAdd(&kg->queue[2 + qx], 1);
          if (kk < n_items) {
            code = kg->items[kk];
            break;
          }
          qx = (qx + 1) & 7;
          ++tried;
        }
        q_cur[0] = qx;
        q_cur[1] = tried;
        next_item = code;
      }
      __syncthreads();
      const int code = next_item;
      __syncthreads();  // every wave has read it (and left the last unit's LDS)
      if (code < 0) break;
      const Plan& pd = opaque_kernargs<F8KernArgs>()->p;
      const int64_t seg = code >> 8;
      int b = 0;
      while (b + 1 < pd.num_seqs && pd.seq[b + 1].seg_base <= seg) ++b;
      int h, I;
      segment_tile(pd.seq[b], (int)(seg - pd.seq[b].seg_base), h, I);
      run_unit(b, I, h, (code >> 4) & 15, code & 15);
    }
  } else {
    // split launch: persistent workgroups take items from the work list
    const int n_items = queue_a[1];
    for (;;) {
      if (tid == 0) next_item = atomicAdd(&queue_a[0], 1);
      __syncthreads();
      const int it = next_item;
      __syncthreads();  // every wave has read it (and left the last unit's LDS)
      if (it >= n_items) break;
      const int code = items_a[it];
      const int64_t seg = code >> 8;
      int b = 0;
      while (b + 1 < p.num_seqs && p.seq[b + 1].seg_base <= seg) ++b;
      int h, I;
      segment_tile(p.seq[b], (int)(seg - p.seq[b].seg_base), h, I);
      run_unit(b, I, h, (code >> 4) & 15, code & 15);
    }
  }
}

// e4m3 code nearest to num / 2^sh (num an integer, |num / 2^sh| <= 448),
// ties to the even code: the value is exact in float64, and scaling by a
// power of two keeps it exact, so rint (round half to even) decides exactly.
__device__ __forceinline__ uint32_t e4m3_of_ratio(int64_t num, int sh) {
  if (num == 0) return 0u;
  const uint32_t sign = num < 0 ? 0x80u : 0u;
  const double a = ldexp((double)(num < 0 ? -num : num), -sh);
  int E;
  frexp(a, &E);        // a = f 2^E, f in [0.5, 1)
  int e = E - 1;       // a in [2^e, 2^(e+1))
  if (e < -6) e = -6;  // subnormals share the step of the smallest binade
  double q = rint(ldexp(a, 3 - e));  // mantissa steps of 2^(e-3)
  if (q >= 16.0) {     // rounded up into the next binade
    q = 8.0;
    ++e;
  }
  uint32_t code;
  if (q < 8.0)
    code = (uint32_t)q;  // subnormal (e = -6): field 0, mantissa q
  else
    code = ((uint32_t)(e + 7) << 3) | ((uint32_t)q - 8u);
  if (code > 0x7eu) code = 0x7eu;  // saturate at 448
  return sign | code;
}

// e4m3 code of the mean of a block's cnt codes, from their exact integer sum
// acc = sum code x 2^9: a power-of-two count scales exactly; any other count
// (a short last block, never corrected) is rounded once, from float64.
__device__ __forceinline__ uint32_t pooled_code(int acc, int cnt) {
  int sh = 9;  // code x 2^9 is an integer; the mean divides by cnt
  while ((1 << (sh - 9)) < cnt) ++sh;
  if ((1 << (sh - 9)) == cnt) return e4m3_of_ratio(acc, sh);
  const double m = (double)acc / (512.0 * cnt);
  return e4m3_of_ratio((int64_t)rint(ldexp(m, 20)), 20);
}

// Pooled statistics of the fp8 correction steps, quantised as in FP8 mode:
// kq = e4m3(mean of the block's K codes), vq likewise for V, both [pooled
// row, Hkv, d] bytes.  The codes of a block are summed exactly as integers
// (code x 2^9 is an integer of at most 18 bits), so the rounding is decided
// on the exact mean - block means of e4m3 codes often sit exactly on an
// e4m3 midpoint, where a float32 round trip through kbar / c_k would break
// the tie either way.  One workgroup per (pooled row, K or V); each thread
// sums 8 columns over the block's rows.  A d-major V takes
// pool_v_dmajor_kernel instead (the grid then covers K only).
__global__ __launch_bounds__(256) void pooled_e4m3_kernel(Plan p, KVDesc kv,
                                                          const uint8_t* __restrict__ k,
                                                          const uint8_t* __restrict__ v,
                                                          uint8_t* __restrict__ kq,
                                                          uint8_t* __restrict__ vq) {
  const int prow = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  int b = 0;
  while (b + 1 < p.num_seqs && p.seq[b + 1].pool_base <= prow) ++b;
  const SeqInfo s = p.seq[b];
  const int j0 = (prow - s.pool_base) * p.B;
  const int cnt = min(p.B, s.len - j0);
  const uint8_t* x = is_v ? v : k;
  uint8_t* out = (is_v ? vq : kq) + (int64_t)prow * p.hkv * p.d;
  const int ncol8 = p.hkv * p.d / 8;
  for (int c8 = threadIdx.x; c8 < ncol8; c8 += 256) {
    int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = 0; r < cnt; ++r) {
      const int64_t row = kv.row(b, s.kv_start, j0 + r);
      const uint2 w = *reinterpret_cast<const uint2*>(x + row * p.hkv * p.d + c8 * 8);
      const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false);
      const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
      const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false);
      const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
      const float f[8] = {f0[0], f0[1], f1[0], f1[1], f2[0], f2[1], f3[0], f3[1]};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (int)(f[e] * 512.f);  // exact
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = pooled_code(acc[e], cnt);
      if (e < 4)
        lo |= c << (8 * e);
      else
        hi |= c << (8 * (e - 4));
    }
    *reinterpret_cast<uint2*>(out + c8 * 8) = make_uint2(lo, hi);
  }
}

// Pooled means of a d-major fp8 V ([Hkv, d, kv tokens], or [pages, Hkv, d,
// page] with pages of at least 64 tokens).  Eight lanes per (pooled row,
// head, dim): lane e reads tokens 16e .. 16e + 15 of the block (one 16-byte
// piece, inside one page), the codes are summed exactly as integers (code x
// 2^9 is an integer) and the eight lanes' sums are added.  With vq the e4m3
// code of each mean is written (the quantised pooled values of the fp8
// correction), else vbar = the float32 mean times the V scale, formed as the
// row-major pooling forms it (sum / count * scale).
__global__ __launch_bounds__(256) void pool_v_dmajor_kernel(Plan p, KVDesc kv,
                                                            const uint8_t* __restrict__ v,
                                                            float v_scale,
                                                            float* __restrict__ vbar,
                                                            uint8_t* __restrict__ vq) {
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const int e = threadIdx.x & 7;
  const int hd_n = p.hkv * p.d;
  const bool in = item < (int64_t)p.pooled_rows * hd_n;  // every lane stays for the shuffles
  int acc = 0, cnt = 1;
  int64_t o = 0;
  if (in) {
    const int prow = (int)(item / hd_n);
    const int hd = (int)(item % hd_n);  // h * d + dim
    o = item;
    int b = 0;
    while (b + 1 < p.num_seqs && p.seq[b + 1].pool_base <= prow) ++b;
    const SeqInfo s = p.seq[b];
    const int j0 = (prow - s.pool_base) * p.B;
    cnt = min(p.B, s.len - j0);
    const int r0 = 16 * e;
    if (r0 < cnt) {
      const int j = j0 + r0;
      int64_t off;
      if (kv.page_table != nullptr) {
        const int64_t phys = kv.page_table[(int64_t)b * kv.max_pages + (j >> kv.page_shift)];
        off = ((phys * hd_n + hd) << kv.page_shift) + (j & ((1 << kv.page_shift) - 1));
      } else {
        off = (int64_t)hd * p.kv_tokens + s.kv_start + j;
      }
      const int m = min(16, cnt - r0);
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (m == 16 && (off & 15) == 0) {
        const uint4 u = *reinterpret_cast<const uint4*>(v + off);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
      } else {
        for (int t = 0; t < m; ++t) w[t >> 2] |= (uint32_t)v[off + t] << (8 * (t & 3));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
        const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
        acc += (int)(f0[0] * 512.f) + (int)(f0[1] * 512.f) + (int)(f1[0] * 512.f) +
               (int)(f1[1] * 512.f);  // exact; a zero code adds nothing
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (!in || e != 0) return;
  if (vq) {
    vq[o] = (uint8_t)pooled_code(acc, cnt);
  } else {
    const float sc = p.dscale ? p.dscale[2] : v_scale;
    const float t = (float)acc * (1.f / 512.f);
    vbar[o] = t / (float)cnt * sc;
  }
}

hipError_t launch_pool_v_dmajor(const Plan& p, const KVDesc& kv, const void* v, float v_scale,
                                float* vbar, uint8_t* vq, hipStream_t st) {
  const int64_t lanes = (int64_t)p.pooled_rows * p.hkv * p.d * 8;
  if (lanes == 0) return hipSuccess;
  hipLaunchKernelGGL(pool_v_dmajor_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st,
                     p, kv, static_cast<const uint8_t*>(v), v_scale, vbar, vq);
  return hipGetLastError();
}

namespace {

// F8KernArgs must be laid out as the kernel's parameter list.
using F8Params = KernelParams<decltype(attn_fp8_kernel<128, 8, true, true, false, true>)>;
static_assert(F8Params::count == 21, "F8KernArgs mirrors 21 kernel parameters");
#define BSLP_ARG_AT(i, m) \
  static_assert(F8Params::offset(i) == offsetof(F8KernArgs, m), "F8KernArgs." #m);
BSLP_ARG_AT(0, p) BSLP_ARG_AT(1, kv) BSLP_ARG_AT(2, q) BSLP_ARG_AT(3, k) BSLP_ARG_AT(4, v)
BSLP_ARG_AT(5, kq) BSLP_ARG_AT(6, vq) BSLP_ARG_AT(7, cu) BSLP_ARG_AT(8, idx)
BSLP_ARG_AT(9, c) BSLP_ARG_AT(10, out_scale) BSLP_ARG_AT(11, correction) BSLP_ARG_AT(12, dense)
BSLP_ARG_AT(13, units_per_seg) BSLP_ARG_AT(14, splits) BSLP_ARG_AT(15, out) BSLP_ARG_AT(16, lse)
BSLP_ARG_AT(17, part_o) BSLP_ARG_AT(18, part_ml) BSLP_ARG_AT(19, items) BSLP_ARG_AT(20, queue)
#undef BSLP_ARG_AT

// A persistent launch of `kernel`: as many workgroups as stay resident at
// once (asked once per process and instantiation), at most one per item.
template <void (*kernel)(Plan, KVDesc, const uint8_t*, const uint8_t*, const uint8_t*,
                         const uint8_t*, const uint8_t*, const int32_t*, const int32_t*, float,
                         float, int, int, int, int, uint16_t*, float*, float*, float*,
                         const int32_t*, int*)>
hipError_t launch_persistent_f8(const Plan& p, int splits, int threads, const F8KernArgs& ka,
                                hipStream_t st) {
  static std::atomic<int> occupancy{0};
  int per_cu = occupancy.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(kernel), threads, 0);
    if (e != hipSuccess) return e;
    occupancy.store(per_cu, std::memory_order_relaxed);
  }
  int64_t grid = 0;
  const hipError_t e = persistent_grid(p, splits, per_cu, &grid);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, st, ka.p, ka.kv, ka.q, ka.k,
                     ka.v, ka.kq, ka.vq, ka.cu, ka.idx, ka.c, ka.out_scale, ka.correction,
                     ka.dense, ka.units_per_seg, ka.splits, ka.out, ka.lse, ka.part_o, ka.part_ml,
                     ka.items, ka.queue);
  return hipGetLastError();
}

template <int D, int NW, bool CORR, bool VCOL>
hipError_t launch_fp8_t(const Plan& p, const KVDesc& kv, const AttnArgs& a, hipStream_t st) {
  const int rows = F8Cfg<D, NW>::ROWS;
  const int units_per_seg = (p.g * p.B + rows - 1) / rows;
  Plan pl = p;
  int64_t base = 0;
  for (int i = 0; i < pl.num_seqs; ++i) {
    const int b = pl.order[i];
    pl.seq[b].unit_base = (int32_t)base;
    base += (int64_t)ntile(pl.seq[b]) * pl.hkv * units_per_seg;
  }
  if (base == 0) return hipSuccess;
  const size_t n = (size_t)p.pooled_rows * p.hkv * p.d;
  uint8_t* kq = reinterpret_cast<uint8_t*>(a.workspace);
  uint8_t* vq = kq + n;
  const int corr = a.correction && !a.dense;
  if (n > 0 && corr) {
    hipLaunchKernelGGL(pooled_e4m3_kernel, dim3((unsigned)p.pooled_rows, VCOL ? 1 : 2), dim3(256),
                       0, st, p, kv, static_cast<const uint8_t*>(a.k),
                       static_cast<const uint8_t*>(a.v), kq, vq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (VCOL) {
      e = launch_pool_v_dmajor(p, kv, a.v, a.v_scale, nullptr, vq, st);
      if (e != hipSuccess) return e;
    }
  }
  // logits of the codes: softmax_scale * q_scale * k_scale, in units of log2
  const float c = (float)((double)a.lscale * (double)a.k_scale * 1.4426950408889634);
  const int splits = a.splits;
  F8KernArgs ka{pl, kv, static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                static_cast<const uint8_t*>(a.v), kq, vq, a.cu, a.idx, c, a.v_scale, corr,
                a.dense, units_per_seg, splits, (uint16_t*)a.out, a.lse, nullptr, nullptr,
                nullptr, nullptr};
  // persistent workgroups as for bf16: split launches, and unsplit sparse
  // ones with enough units per CU; otherwise one workgroup per unit.  With
  // d-major V the unsplit launch stays one workgroup per unit: at 128K the
  // queue made its attention 4.6% slower (4.53 -> 4.74 ms) where it made the
  // row-major one 3.3% faster (4.34 -> 4.20 ms).
  int cus = 0;
  if (!VCOL && splits == 1 && !a.dense && a.workspace && a.cu) {
    const hipError_t e = attn_device_cus(&cus);
    if (e != hipSuccess) return e;
  }
  if (!(splits > 1 || (cus > 0 && base >= kPersistUnitsPerCU * cus))) {
    hipLaunchKernelGGL((attn_fp8_kernel<D, NW, false, CORR, VCOL>), dim3((unsigned)base),
                       dim3(NW * 64), 0, st, ka.p, ka.kv, ka.q, ka.k, ka.v, ka.kq, ka.vq, ka.cu,
                       ka.idx, ka.c, ka.out_scale, ka.correction, ka.dense, ka.units_per_seg,
                       ka.splits, ka.out, ka.lse, ka.part_o, ka.part_ml, ka.items, ka.queue);
    return hipGetLastError();
  }
  SplitBufs sb = split_bufs(p, a.workspace, splits);
  hipError_t e = launch_split_items(pl, a.cu, splits, corr, units_per_seg, sb, st);
  if (e != hipSuccess) return e;
  ka.part_o = sb.part_o;
  ka.part_ml = sb.part_ml;
  ka.items = sb.items;
  ka.queue = sb.queue;
  if constexpr (!VCOL) {
    if (splits == 1)
      return launch_persistent_f8<attn_fp8_kernel<D, NW, true, CORR, VCOL, true>>(p, splits,
                                                                                 NW * 64, ka, st);
  }
  e = launch_persistent_f8<attn_fp8_kernel<D, NW, true, CORR, VCOL, false>>(p, splits, NW * 64, ka,
                                                                            st);
  if (e != hipSuccess) return e;
  return launch_split_merge(p, a.cu, sb, splits, corr, 8.f * kLn2, (uint16_t*)a.out, a.lse, st);
}

template <int D, bool VCOL>
hipError_t launch_fp8_d(const Plan& p, const KVDesc& kv, const AttnArgs& a, hipStream_t st) {
  const int rows = p.g * p.B;
  if (a.correction && !a.dense) {
    if (rows >= 256) return launch_fp8_t<D, 8, true, VCOL>(p, kv, a, st);
    if (rows >= 128) return launch_fp8_t<D, 4, true, VCOL>(p, kv, a, st);
    return launch_fp8_t<D, 2, true, VCOL>(p, kv, a, st);
  }
  if (rows >= 256) return launch_fp8_t<D, 8, false, VCOL>(p, kv, a, st);
  if (rows >= 128) return launch_fp8_t<D, 4, false, VCOL>(p, kv, a, st);
  return launch_fp8_t<D, 2, false, VCOL>(p, kv, a, st);
}

}  // namespace

hipError_t launch_attn_fp8(const Plan& p, const KVDesc& kv, const AttnArgs& a, hipStream_t st) {
  if (p.v_dmajor)
    return p.d == 128 ? launch_fp8_d<128, true>(p, kv, a, st)
                      : launch_fp8_d<64, true>(p, kv, a, st);
  return p.d == 128 ? launch_fp8_d<128, false>(p, kv, a, st)
                    : launch_fp8_d<64, false>(p, kv, a, st);
}

}  // namespace bslp
