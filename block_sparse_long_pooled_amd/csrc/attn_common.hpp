// Pieces shared by the matrix-core attention kernels (bf16 and fp8): the
// step sequence of a work unit, which every thread derives alike, and small
// wave-level helpers.  Device code only; each kernel file includes it.
//
// Step sequence of a unit ("FlashPrefill V2", CSR paragraph: the selected
// blocks of a segment are walked backwards, and split u of a segment takes a
// contiguous share of its CSR list, Eq. 18; tile paragraph: 64-key tiles,
// B/64 of them per block; Sec. 3.2 / Fig. 3 paragraph: correction chunks
// with a todo bitmask, skipped when every block is selected):
//   exact steps: CSR positions end-1 down to beg; for each block its 64-key
//     tiles in descending order, starting at the highest tile that begins
//     before the unit's key limit (keys past the unit's last query position
//     are masked for every row, so such a tile is skipped);
//   correction steps: chunks c0, c0 + cstep, ... of 64 pooled blocks that
//     hold a block of todo = valid & ~selected (valid: J <= I-1).
#pragma once

#include <cstddef>

#include "common.hpp"

namespace bslp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16 bytes, kept in registers

namespace {

constexpr int kKeys = 64;      // keys per pipeline step
constexpr int kCorrRows = 64;  // pooled blocks per correction step
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer descriptor, 32-bit data format

enum StepKind : int { kExact = 0, kCorr = 1, kDone = 2 };

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

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)uni((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)uni((int)(uint32_t)(x >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// One step of the unit's sequence.  Every field is the same in all lanes of
// the workgroup; `uniform` moves them to scalar registers, so branches on
// them are scalar and reading the block index needs no vector load (which
// would also make the next step's prefetch wait).
struct Step {
  int kind;  // StepKind
  int t;     // exact: CSR position
  int hf;    // exact: 64-key tile of the block
  int c;     // correction: chunk of 64 pooled blocks
  int J;     // exact: block index idx[t]
  int Jn;    // exact: idx[t-1], loaded one block ahead so no step waits on it
};

__device__ __forceinline__ void uniform(Step& st) {
  st.kind = uni(st.kind);
  st.t = uni(st.t);
  st.hf = uni(st.hf);
  st.c = uni(st.c);
  st.J = uni(st.J);
}

struct UnitCtx {
  int b, h, I, len, kv_start, pool_base, B;  // len: keys of the request
  int beg, end;  // the unit's share of the CSR positions of its segment
  int dense;     // blocks are J = t for t in [0, I]: no index list
  int c0, cstep; // correction chunks c0, c0 + cstep, ... belong to the unit
  int kend;      // keys >= kend are invisible to every row of the unit
};

// KV head of the unit at position `local` of a request's one-workgroup-per-
// unit enumeration (tiles in descending I, then row block, then KV head).
// The dispatcher deals workgroups to the XCDs round robin, so with the head
// innermost every XCD would see one head only, and heads differ in how many
// blocks they select: the XCDs would finish unevenly, and a workgroup waiting
// for a busy XCD holds back the dispatch of those behind it.  The head
// therefore turns by one every kHeadTurn groups of hkv units: each XCD keeps a
// head for 16 consecutive units (their K/V stay warm in its L2) and sees
// every head over the launch.  Within a group the turn is a permutation.
constexpr int kHeadTurn = 16;
__device__ __forceinline__ int unit_head(int64_t local, int hkv) {
  return (int)((local % hkv + local / ((int64_t)kHeadTurn * hkv)) % hkv);
}

// KV splits a segment actually uses, at most `splits`: one per 24 steps of
// estimated work (its selected blocks in 64-key tiles plus an upper bound on
// its correction chunks), so light segments stay whole and write no partial
// result.  The attention and the merge kernel evaluate it alike.
__device__ __forceinline__ int segment_splits(int n_sel, int I, int B, int correction,
                                              int splits) {
  const int steps = n_sel * (B / 64) + (correction && I > 0 ? (I + kCorrRows - 1) / kCorrRows : 0);
  return max(1, min(splits, steps / 24));
}

// Block index at CSR position t (the position itself on the dense path).
__device__ __forceinline__ int block_at(const int32_t* idx, int t, const UnitCtx& u) {
  return u.dense ? t : idx[t];
}

// The highest 64-key tile of block J that starts before the unit's key limit
// (J*B < kend holds for every block a unit walks: J <= I).
__device__ __forceinline__ int top_tile(int J, const UnitCtx& u) {
  return min(u.B / kKeys, (u.kend - J * u.B + kKeys - 1) / kKeys) - 1;
}

// todo bits of correction chunk c (blocks 64c .. 64c+63, valid J <= I-1).
__device__ __forceinline__ uint64_t chunk_todo(const uint32_t* selbits, int c, int I) {
  const int nv = min(max(I - kCorrRows * c, 0), kCorrRows);
  if (nv == 0) return 0;
  const uint64_t m = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
  const uint64_t t = ~((uint64_t)selbits[2 * c] | ((uint64_t)selbits[2 * c + 1] << 32)) & m;
  return (uint64_t)(uint32_t)uni((int)(uint32_t)t) |
         ((uint64_t)(uint32_t)uni((int)(uint32_t)(t >> 32)) << 32);
}

__device__ __forceinline__ void find_chunk(Step& st, const uint32_t* selbits, int I, int cstep) {
  while (kCorrRows * st.c < I && chunk_todo(selbits, st.c, I) == 0) st.c += cstep;
  st.kind = kCorrRows * st.c < I ? kCorr : kDone;
}

// The step after `st`; identical in every thread.  idx[t-1] is loaded when
// the walk enters block t and first used when it leaves it, so no step waits
// for it.
__device__ __forceinline__ void advance(Step& st, const UnitCtx& u, const int32_t* idx,
                                        const uint32_t* selbits, int correction) {
  if (st.kind == kExact) {
    if (st.hf > 0) {
      --st.hf;
      return;
    }
    --st.t;
    if (st.t >= u.beg) {
      st.J = st.Jn;
      st.hf = top_tile(st.J, u);
      st.Jn = block_at(idx, max(st.t - 1, u.beg), u);
      return;
    }
    st.kind = kCorr;
    st.c = u.c0 - u.cstep;
  }
  if (st.kind == kCorr) {
    if (!correction || u.I == 0) {
      st.kind = kDone;
      return;
    }
    st.c += u.cstep;
    find_chunk(st, selbits, u.I, u.cstep);
  }
}

__device__ __forceinline__ Step first_step(const UnitCtx& u, const int32_t* idx,
                                           const uint32_t* selbits, int correction) {
  Step st{kExact, u.end - 1, 0, 0, 0, 0};
  if (u.end > u.beg) {
    st.J = block_at(idx, st.t, u);
    st.hf = top_tile(st.J, u);
    st.Jn = block_at(idx, max(st.t - 1, u.beg), u);
    return st;
  }
  st.kind = kCorr;
  st.c = u.c0 - u.cstep;
  advance(st, u, idx, selbits, correction);
  return st;
}

// A kernel's arguments read from its kernel-argument segment, as the struct
// Args that mirrors its parameter list, through a pointer the compiler cannot
// follow, so each use is a fresh scalar load: in a persistent workgroup
// nothing derived from them is hoisted out of the loop over units and kept
// live through every unit's walk (which left too few registers for the
// walk's LDS operands to be read ahead: in the bf16 kernel 59 of the 64
// MFMAs waited on their own operand read, and each step ran 12-15% slower).
template <class Args>
__device__ __forceinline__ const Args* opaque_kernargs() {
  auto seg = __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(seg));
  return (const Args*)(seg);
}

// KernelParams<decltype(kernel)>::offset(i): where parameter i of a kernel
// lies in its kernel-argument segment (each parameter in order at the next
// offset aligned to its type, as struct members are laid out), for checking
// a struct that mirrors the parameter list member for member.
template <class F>
struct KernelParams;
template <class... A>
struct KernelParams<void(A...)> {
  static constexpr size_t count = sizeof...(A);
  static constexpr size_t offset(size_t i) {
    constexpr size_t size[] = {sizeof(A)...}, align[] = {alignof(A)...};
    size_t off = 0;
    for (size_t j = 0;; ++j) {
      off = (off + align[j] - 1) / align[j] * align[j];
      if (j == i) return off;
      off += size[j];
    }
  }
};

}  // namespace

}  // namespace bslp
