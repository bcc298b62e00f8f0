// Shared definitions of libbslp: the per-call plan (request table passed to
// every kernel by value, so no host->device copy is needed), paged/contiguous
// K/V row addressing, and element conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bslp {

constexpr int kMaxSeqs = 64;
constexpr int kMaxBlocksPerSeq = 16384;
constexpr int kMaxGroup = 16;
constexpr int kMaxSplits = 16;  // KV splits per attention work unit

enum DType : int32_t { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// One packed request.  All bases are prefix sums over earlier requests.
// Its keys are positions 0 .. len-1; its queries are the last len - q_off of
// them (a chunk of a chunked prefill; q_off = 0 for a whole prompt), and only
// the tiles I >= i0 that hold a query are scored, selected and attended.
struct SeqInfo {
  int32_t tok_start;   // first Q / O row (LSE column) of the request's queries
  int32_t kv_start;    // first K / V row of the request (contiguous K/V)
  int32_t len;         // L_b^kv: keys
  int32_t q_off;       // L_b^kv - L_b^q: position of the first query
  int32_t nblk;        // N_b = ceil(L_b^kv / B): key blocks
  int32_t i0;          // first query tile: q_off / B
  int32_t pool_base;   // first pooled row (kbar / vbar)
  int32_t seg_base;    // first segment: (h, I) is segment h*(N_b - i0) + I - i0
  int32_t unit_base;   // first work unit of the request (kernel specific use)
  int64_t score_base;  // first score element of the request
};

__host__ __device__ __forceinline__ int ntile(const SeqInfo& s) { return s.nblk - s.i0; }

// KV head and tile of the request's local segment index.
__host__ __device__ __forceinline__ void segment_tile(const SeqInfo& s, int local, int& h,
                                                      int& I) {
  h = local / ntile(s);
  I = s.i0 + local % ntile(s);
}

// Query positions of tile I: tile_q0 .. tile_q0 + tile_nq - 1.
__host__ __device__ __forceinline__ int tile_q0(const SeqInfo& s, int I, int B) {
  return I * B > s.q_off ? I * B : s.q_off;
}
__host__ __device__ __forceinline__ int tile_nq(const SeqInfo& s, int I, int B) {
  return ((I + 1) * B < s.len ? (I + 1) * B : s.len) - tile_q0(s, I, B);
}

// Q / O row (and LSE column) of query position pos.
__host__ __device__ __forceinline__ int64_t q_row(const SeqInfo& s, int pos) {
  return (int64_t)s.tok_start + pos - s.q_off;
}

struct Plan {
  int32_t num_seqs;
  int32_t hq, hkv, g, d, B;
  int32_t max_nblk;
  int64_t total_tokens, pooled_rows, score_elems, num_segments;  // total_tokens: query rows
  int64_t kv_tokens;  // key / value rows (contiguous K/V)
  SeqInfo seq[kMaxSeqs];
  int32_t order[kMaxSeqs];  // requests by descending block count (ties: packed order)
  // fp8 scales (q, k, v) in device memory, or nullptr: the host floats apply
  const float* dscale;
  int32_t v_dmajor;  // V as [Hkv, d, kv tokens] (or [pages, Hkv, d, page]), fp8 only
};

// Where key/value token j of request b lives.
struct KVDesc {
  const int32_t* page_table;  // nullptr: contiguous
  int32_t page_shift;         // log2(page_size)
  int32_t max_pages;          // row stride of page_table

  __device__ __forceinline__ int64_t row(int b, int tok_start, int j) const {
    if (page_table == nullptr) return (int64_t)tok_start + j;
    const int32_t phys = page_table[(int64_t)b * max_pages + (j >> page_shift)];
    return ((int64_t)phys << page_shift) | (int64_t)(j & ((1 << page_shift) - 1));
  }
};

struct SelectArgs {
  float alpha;
  int32_t sink, window, recent, correction;
};

// Score row of segment (b, h, I) starts here.
__host__ __device__ __forceinline__ int64_t score_offset(const SeqInfo& s, int h, int I) {
  // rows I = i0 .. N-1 of I+1 scores each, per KV head
  const int64_t first = (int64_t)s.i0 * (s.i0 + 1) / 2;
  return s.score_base + (int64_t)h * ((int64_t)s.nblk * (s.nblk + 1) / 2 - first) +
         (int64_t)I * (I + 1) / 2 - first;
}

// Request owning a segment / unit index (linear scan; at most kMaxSeqs).
__device__ __forceinline__ int seq_of_segment(const Plan& p, int64_t seg) {
  int b = 0;
  while (b + 1 < p.num_seqs && p.seq[b + 1].seg_base <= seg) ++b;
  return b;
}

// ---------------------------------------------------------------- elements

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}

// float -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP e4m3fn code -> float (exact): bias 7, subnormals m/8 * 2^-6, the codes
// with all exponent and mantissa bits set are NaN, no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const uint32_t s = (uint32_t)(c & 0x80) << 24;
  const uint32_t e = (c >> 3) & 0xF;
  const uint32_t m = c & 0x7;
  if (e == 0) {
    const float v = (float)m * 0.001953125f;  // m * 2^-9
    return __uint_as_float(__float_as_uint(v) | s);
  }
  if (e == 0xF && m == 0x7) return __uint_as_float(0x7fc00000u | s);
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

template <int DT> struct Elem;
template <> struct Elem<kF32> {
  using T = float;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
};
template <> struct Elem<kBF16> {
  using T = uint16_t;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return bf16_to_f32(p[i]); }
};
template <> struct Elem<kFP8> {
  using T = uint8_t;
  static __device__ __forceinline__ float load(const T* p, int64_t i) { return e4m3_to_f32(p[i]); }
};

// Eight consecutive elements (16-byte aligned for f32/bf16, 8-byte for fp8)
// widened to float.
template <int DT>
__device__ __forceinline__ void load8(const typename Elem<DT>::T* p, int64_t off, float out[8]) {
  if constexpr (DT == kF32) {
    const float4 a = *reinterpret_cast<const float4*>(p + off);
    const float4 b = *reinterpret_cast<const float4*>(p + off + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else if constexpr (DT == kBF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    // OCP e4m3 codes widened by v_cvt_pk_f32_fp8 (two codes per instruction,
    // exact: every e4m3 value is a float32)
    const uint2 u = *reinterpret_cast<const uint2*>(p + off);
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(u.x, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(u.x, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(u.y, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(u.y, true);
    out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
    out[4] = c[0]; out[5] = c[1]; out[6] = d[0]; out[7] = d[1];
  }
}

}  // namespace bslp
