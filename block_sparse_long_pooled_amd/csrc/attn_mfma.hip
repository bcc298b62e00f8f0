// Stage 3 on the matrix cores: block-sparse causal online-softmax attention
// with mean correction and PackGQA rows, bf16 inputs (fp8 inputs take the
// kernel of attn_fp8.hip)
// ("FlashPrefill V2",
// Sec. 3.1 last sentence, Sec. 3.2 / Fig. 3 correction path, PackGQA, CSR
// and paged-KV paragraphs).  Written for gfx950 wave64 MFMA.
//
// Work unit.  (segment (b, h, I), 32*RT*NW consecutive PackGQA rows of tile
// I), one workgroup of NW waves x RT row tiles of 32 rows (RT = 1 keeps a
// wave within 256 VGPRs, so two waves share each SIMD).  Packed row r of the tile is
// position I*B + r / g of query head h*g + r % g, so every staged K/V key
// serves all g heads of the group.  Units are enumerated heaviest first
// (longest request first, tiles in descending I, then row block) with the KV
// head innermost, turned every few groups (unit_head) so that the XCDs,
// which the dispatcher feeds round robin, share the heads evenly while each
// keeps one head for a run of consecutive units.
//
// Pipeline.  The unit's work is a uniform sequence of 64-key steps: the
// selected blocks from the CSR list walked backwards (B/64 steps each), then
// the correction chunks of 64 pooled blocks that hold at least one block of
// todo = valid & ~selected (valid = J <= I-1, fully visible to the tile).
// A correction step's 64 keys are 64 pooled means as bf16 pairs hi + lo
// (the float32 mean to within 2^-18 of itself), hi in the K buffer and lo
// loaded straight into a ring of LDS slots; both products accumulate into
// the same scores, so the pooled logits carry no bf16 rounding.
// Every thread derives the same sequence, so no step needs a vote.  After
// the step's barrier each wave writes the prefetched step n+1 into the other
// LDS buffer, issues the global loads of step n+2 into registers and then
// multiplies step n, so the loads have a whole step to arrive and the LDS
// writes of one wave overlap the matrix work of the others.
//
// MFMA layout.  Per wave S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32
// keys x 16 dims of K from LDS, B = the wave's 32 query rows from
// registers): every lane owns one query row and 16 keys of each 32-key tile,
// the other 16 being in lane ^ 32, so the row max and row sum are in-lane plus
// one v_permlane32_swap.  The probabilities feed O^T += V^T P^T straight from
// registers as the B operand: the 8 values a lane holds for 16 consecutive
// keys are keys {0-3, 8-11} (lanes 0-31) or {4-7, 12-15} (lanes 32-63), so
// V^T is stored in LDS with its key columns permuted the same way and each
// A operand is one 16-byte LDS read.  K and V^T rows are padded by 16 bytes
// so the operand reads of 16 lanes fall in distinct banks.
//
// Softmax.  Scores stay unscaled in the accumulator; with c = scale*log2(e),
// p = exp2(s*c - m) is one FMA and one v_exp_f32.  The running maximum m is
// raised only when a step exceeds it by more than 8 (so p < 2^8), which makes
// the output rescale rare.  Correction terms enter as s*c + log2|B_J| with
// unselected or invisible columns at -inf.
#include <algorithm>
#include <cstddef>
#include <atomic>
#include <type_traits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace bslp {

namespace {

__device__ __forceinline__ int kperm(int key) {  // V^T column of a key
  return (key & ~15) | ((key & 4) << 1) | ((key & 8) >> 1) | (key & 3);
}

}  // namespace

template <int D, int NW, int RT>
struct AttnCfg {
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = NW * RT * 32;  // packed rows per unit
  static constexpr int KS = D / 16;          // k-steps of Q K^T
  static constexpr int DT = D / 32;          // 32-dim tiles of O^T
  static constexpr int KU = D / 8;           // 16-byte units per key row
  static constexpr int KUN = kKeys * KU;     // K units per step
  static constexpr int VPN = kKeys / 2 * KU; // V (key pair x unit) groups per step
  static constexpr int KL = (KUN + NT - 1) / NT;
  static constexpr int VL = (VPN + NT - 1) / NT;
  static constexpr int KLD = D + 8;          // padded K row (bf16)
  // lo rows of a correction step, loaded straight into LDS as [16-byte dim
  // chunk][key]: NCH chunk rows of KCS bytes, CPW of them per wave
  static constexpr int NCH = D / 8;
  static constexpr int KCS = kKeys * 16;
  static constexpr int CPW = NCH / NW;
  static constexpr int VLD = kKeys + 8;      // padded V^T row (bf16)
};

template <int D, int NW, int RT>
struct Prefetch {
  u32x4_t k[AttnCfg<D, NW, RT>::KL];
  u32x4_t v0[AttnCfg<D, NW, RT>::VL];  // key 2a of the pair
  u32x4_t v1[AttnCfg<D, NW, RT>::VL];  // key 2a + 1
};

// Per-thread byte offsets of the 8-element (16-byte) pieces this thread
// fetches, relative to the first row of a step (K/V rows and pooled rows
// share the [row, Hkv, D] layout); fixed for the whole unit.
template <int D, int NW, int RT>
struct FetchOffsets {
  uint32_t k[AttnCfg<D, NW, RT>::KL];
  uint32_t v0[AttnCfg<D, NW, RT>::VL];
  uint32_t v1[AttnCfg<D, NW, RT>::VL];
};

template <int D, int NW, int RT>
__device__ __forceinline__ FetchOffsets<D, NW, RT> fetch_offsets(int hkv) {
  constexpr int esize = 2;  // bf16
  using C = AttnCfg<D, NW, RT>;
  constexpr int PAIRS = kKeys / 2;
  const int tid = threadIdx.x;
  const uint32_t row_bytes = (uint32_t)hkv * D * esize;
  FetchOffsets<D, NW, RT> o;
#pragma unroll
  for (int i = 0; i < C::KL; ++i) {
    const int f = min(tid + i * C::NT, C::KUN - 1);
    o.k[i] = (uint32_t)(f / C::KU) * row_bytes + (uint32_t)(f % C::KU) * 8 * esize;
  }
#pragma unroll
  for (int i = 0; i < C::VL; ++i) {
    const int s = min(tid + i * C::NT, C::VPN - 1);
    const uint32_t unit = (uint32_t)(s / PAIRS) * 8 * esize;
    o.v0[i] = (uint32_t)(2 * (s % PAIRS)) * row_bytes + unit;
    o.v1[i] = (uint32_t)(2 * (s % PAIRS) + 1) * row_bytes + unit;
  }
  return o;
}

// Offsets of the K pieces of a correction step: key r is pooled block r, its
// hi row for the K buffer and its lo row for the second one, from the [pooled
// row, {hi, lo}, Hkv, D] bf16 layout.
template <int D, int NW, int RT>
struct CorrOffsets {
  uint32_t k[AttnCfg<D, NW, RT>::KL];    // hi rows
  uint32_t kl[AttnCfg<D, NW, RT>::CPW];  // lo rows: key = lane, this wave's chunks
};

template <int D, int NW, int RT>
__device__ __forceinline__ CorrOffsets<D, NW, RT> corr_offsets(int hkv) {
  using C = AttnCfg<D, NW, RT>;
  const int tid = threadIdx.x;
  const uint32_t row_bytes = (uint32_t)hkv * D * 2;
  CorrOffsets<D, NW, RT> o;
#pragma unroll
  for (int i = 0; i < C::KL; ++i) {
    const int f = min(tid + i * C::NT, C::KUN - 1);
    const int key = f / C::KU;
    o.k[i] = (uint32_t)(2 * key) * row_bytes + (uint32_t)(f % C::KU) * 16;
  }
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < C::CPW; ++i)
    o.kl[i] = (uint32_t)(2 * lane + 1) * row_bytes + (uint32_t)(wave + i * NW) * 16;
  return o;
}

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// One wave-wide load of 16 bytes per lane from a raw buffer straight into LDS
// at lds_addr + 16*lane (gfx950 buffer_load_dwordx4 ... lds).  Inline
// assembly, so the compiler does not track it: it would otherwise wait for it
// before every LDS access.  Its data has landed once a later load of the same
// wave has (loads complete in order): the kernel issues it before the V loads
// of the same step and stores those V registers before the next barrier.  M0
// holds the LDS address; one wait state separates its write from the load.
__device__ __forceinline__ void lds_load16(i32x4_t rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Global -> registers for one step.  Exact steps read bf16 tokens key0.. of
// the request (through the page table when K/V are paged); correction steps
// read the bf16 hi and lo rows of 64 pooled keys and their 64 pooled values.
// When the step's rows are consecutive in memory (contiguous K/V, pages of at
// least 64 tokens, pooled rows) the loads are raw buffer loads from one
// scalar descriptor plus the fixed per-thread offsets; the descriptor ends
// after the step's last valid row, so rows past it (the short last block, the
// last correction chunk) read as zero.  With smaller pages every key's row is resolved on its own
// and keys past the end re-read the last valid row.  Either way those keys'
// scores are masked.
template <int D, int NW, int RT, bool CORR>
__device__ __forceinline__ void fetch_step(Prefetch<D, NW, RT>& pf,
                                           const FetchOffsets<D, NW, RT>& off16,
                                           const CorrOffsets<D, NW, RT>& offc, const Step& st,
                                           const UnitCtx& u, const KVDesc& kv, int hkv,
                                           const void* k, const void* v,
                                           const uint16_t* kb2, const uint16_t* vb16,
                                           uint16_t* kl_slot) {
  using C = AttnCfg<D, NW, RT>;
  constexpr int PAIRS = kKeys / 2;
  const bool exact = st.kind == kExact;
  const int key0 = exact ? st.J * u.B + st.hf * kKeys : kCorrRows * st.c;
  const int last = exact ? min(kKeys, u.len - key0) - 1 : min(kCorrRows, u.I - key0) - 1;
  const bool paged = exact && kv.page_table != nullptr;
  const int64_t stride = (int64_t)hkv * D;
  const char* ksrc = exact ? static_cast<const char*>(k) : reinterpret_cast<const char*>(kb2);
  const char* vsrc = exact ? static_cast<const char*>(v) : reinterpret_cast<const char*>(vb16);
  if (!paged || kv.page_shift >= 6) {
    int64_t kb0, vb0;
    int nrec_k, nrec_v;
    if (!exact) {
      const int64_t prow = (int64_t)u.pool_base + key0;
      kb0 = (prow * 2 * stride + (int64_t)u.h * D) * 2;
      vb0 = (prow * stride + (int64_t)u.h * D) * 2;
      nrec_k = ((2 * last + 1) * (int)stride + D) * 2;
      nrec_v = (last * (int)stride + D) * 2;
    } else {
      int64_t row0;
      if (paged) {
        const int phys = uni(kv.page_table[(int64_t)u.b * kv.max_pages + (key0 >> kv.page_shift)]);
        row0 = ((int64_t)phys << kv.page_shift) | (int64_t)(key0 & ((1 << kv.page_shift) - 1));
      } else {
        row0 = (int64_t)u.kv_start + key0;
      }
      kb0 = vb0 = (row0 * stride + (int64_t)u.h * D) * 2;
      nrec_k = nrec_v = (last * (int)stride + D) * 2;
    }
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(ksrc + kb0), (short)0, uni(nrec_k), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)uniform_ptr(vsrc + vb0), (short)0, uni(nrec_v), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < C::KL; ++i)
      pf.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(exact ? off16.k[i] : offc.k[i]),
                                                      0, 0);
    if (CORR && !exact) {
      // the lo rows go straight to LDS, [chunk][key], between the K and the
      // V loads of the step
      const uint64_t a = reinterpret_cast<uint64_t>(ksrc + kb0);
      const i32x4_t rw = {uni((int)(uint32_t)a), uni((int)(uint32_t)(a >> 32)), uni(nrec_k),
                          kRsrcWord3};
      const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t)kl_slot;
      const int wave = uni(threadIdx.x >> 6);
#pragma unroll
      for (int i = 0; i < C::CPW; ++i)
        lds_load16(rw, uni((int)(base + (uint32_t)(wave + i * NW) * C::KCS)), offc.kl[i]);
    }
#pragma unroll
    for (int i = 0; i < C::VL; ++i) {
      pf.v0[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off16.v0[i], 0, 0);
      pf.v1[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off16.v1[i], 0, 0);
    }
    return;
  }
  // paged with pages below 64 tokens: exact steps only
  const int tid = threadIdx.x;
  int kkey[C::KL], vkey[C::VL];
#pragma unroll
  for (int i = 0; i < C::KL; ++i) kkey[i] = min(min(tid + i * C::NT, C::KUN - 1) / C::KU, last);
#pragma unroll
  for (int i = 0; i < C::VL; ++i)
    vkey[i] = min(2 * (min(tid + i * C::NT, C::VPN - 1) % PAIRS), last);
  int64_t krow[C::KL], vrow0[C::VL], vrow1[C::VL];
#pragma unroll
  for (int i = 0; i < C::KL; ++i) krow[i] = kv.row(u.b, u.kv_start, key0 + kkey[i]);
#pragma unroll
  for (int i = 0; i < C::VL; ++i) {
    vrow0[i] = kv.row(u.b, u.kv_start, key0 + vkey[i]);
    vrow1[i] = kv.row(u.b, u.kv_start, key0 + min(vkey[i] + 1, last));
  }
  const int64_t hoff = (int64_t)u.h * D;
#pragma unroll
  for (int i = 0; i < C::KL; ++i) {
    const int f = min(tid + i * C::NT, C::KUN - 1);
    const int64_t e = krow[i] * stride + hoff + (f % C::KU) * 8;
    pf.k[i] = *reinterpret_cast<const u32x4_t*>(ksrc + 2 * e);
  }
#pragma unroll
  for (int i = 0; i < C::VL; ++i) {
    const int un = min(tid + i * C::NT, C::VPN - 1) / PAIRS;
    const int64_t e0 = vrow0[i] * stride + hoff + un * 8, e1 = vrow1[i] * stride + hoff + un * 8;
    pf.v0[i] = *reinterpret_cast<const u32x4_t*>(vsrc + 2 * e0);
    pf.v1[i] = *reinterpret_cast<const u32x4_t*>(vsrc + 2 * e1);
  }
}

// Registers -> LDS: K row-major, V transposed with permuted key columns; both
// with padded rows so the 16-byte operand reads of 16 lanes hit distinct banks.
template <int D, int NW, int RT, bool CORR>
__device__ __forceinline__ void store_step(const Prefetch<D, NW, RT>& pf, uint16_t* Ks,
                                           uint16_t* Vt) {
  using C = AttnCfg<D, NW, RT>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KL; ++i) {
    const int f = tid + i * C::NT;
    if (C::KUN % C::NT != 0 && f >= C::KUN) break;
    const int key = f / C::KU, un = f % C::KU;
    *reinterpret_cast<u32x4_t*>(Ks + key * C::KLD + un * 8) = pf.k[i];
  }
#pragma unroll
  for (int i = 0; i < C::VL; ++i) {
    const int s = tid + i * C::NT;
    if (C::VPN % C::NT != 0 && s >= C::VPN) break;
    // key pairs run fastest across lanes: the 4-byte transposing writes of a
    // wave then fall in distinct banks (with 16 dims fastest they collide)
    const int a = s % (kKeys / 2), un = s / (kKeys / 2);
    const int col = kperm(2 * a);  // even; the pair stays adjacent
    const u32x4_t w0 = pf.v0[i], w1 = pf.v1[i];
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t word = __builtin_amdgcn_perm(w1[dd >> 1], w0[dd >> 1], sel);
      *reinterpret_cast<uint32_t*>(Vt + (8 * un + dd) * C::VLD + col) = word;
    }
  }
}

// kCorrAll: a correction chunk of 64 valid pooled blocks, none selected
// (nothing to mask)
enum Mode : int { kPlain = 0, kDiag = 1, kCorrMode = 2, kCorrAll = 3 };

// One 64-key step of one wave over its RT row tiles: S^T = K Q^T, online
// softmax, O^T += V^T P^T.  `mode` is uniform across the workgroup.
template <int D, int NW, int RT, bool CORR>
__device__ __forceinline__ void compute_step(const uint16_t* Ks, const uint16_t* Kl,
                                             const uint16_t* Vt,
                                             const bf16x8_t (&qf)[RT][D / 16],
                                             f32x16_t (&oacc)[RT][D / 32], float (&m_run)[RT],
                                             float (&l_run)[RT], float c, int mode, int key0,
                                             int len, const int (&qpos)[RT], uint64_t todo,
                                             float bias) {
  using C = AttnCfg<D, NW, RT>;
  const int lane = threadIdx.x & 63;
  const int key_l = lane & 31, half = lane >> 5;
  // Each path's first MFMA starts from a zero accumulator operand (an inline
  // constant), so no step spends vector moves clearing the scores.
  f32x16_t sacc[RT][2];
  const f32x16_t zero = {};
  auto qk = [&](const uint16_t* Kb, auto first) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first)::value;
    const uint16_t* kbase = Kb + key_l * C::KLD + half * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(kbase + kt * 32 * C::KLD + ks * 16);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[rt][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, qf[rt][ks], (kFirst && ks == 0) ? zero : sacc[rt][kt], 0, 0, 0);
      }
    }
  };
  // a correction step's pooled logits: the lo rows' products first (the
  // small terms), then the hi rows', into the same accumulators.  The lo rows
  // are [16-byte dim chunk][key]: the operand of key kt*32 + key_l, dims
  // 16 ks + 8 half .. +7, is chunk 2 ks + half.
  if (CORR && mode >= kCorrMode) {
    const char* lb = reinterpret_cast<const char*>(Kl) + half * C::KCS + key_l * 16;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(lb + ks * 2 * C::KCS + kt * 512);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[rt][kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a, qf[rt][ks], ks == 0 ? zero : sacc[rt][kt], 0, 0, 0);
      }
    }
    qk(Ks, std::false_type{});
  } else {
    qk(Ks, std::true_type{});
  }
  // masks: diagonal block (token causality and the request end) or the
  // correction chunk's todo bits; branch-free per element, uniform per step
  if (mode == kDiag || mode == kCorrMode) {
    uint64_t bits;
    if (mode == kDiag) {
      const int nvis = len - key0;  // >= 1
      bits = nvis >= 64 ? ~0ull : ((1ull << nvis) - 1ull);
    } else {
      bits = todo;
    }
    bits >>= 4 * half;  // the lane's keys are kk0 + 4*half
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int lim = (mode == kDiag ? qpos[rt] - key0 : 63) - 4 * half;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk0 = kt * 32 + (r >> 2) * 8 + (r & 3);
          const bool keep = ((bits >> kk0) & 1ull) && kk0 <= lim;
          sacc[rt][kt][r] = keep ? sacc[rt][kt][r] : -INFINITY;
        }
      }
    }
  }
  // online softmax in units of log2 (x = s*c, + log2|B_J| for pooled terms).
  // The running maximum is raised only when the step's maximum exceeds it by
  // more than 8, so probabilities stay below 2^8 and the output rescale is
  // rare; the final normalisation uses the same reference, so it is exact.
  const float cb = mode >= kCorrMode ? bias : 0.f;
  bf16x8_t pb[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rt][kt][r]);
    }
    mx = fmaf(halves_max(mx), c, cb);  // c > 0: the maximum commutes with the scale
    if (mx > m_run[rt] + 8.f) {
      const float alpha = m_run[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rt] - mx);
      l_run[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[rt][dt][r] *= alpha;
      }
      m_run[rt] = mx;
    }
    const float moff = cb - (m_run[rt] == -INFINITY ? 0.f : m_run[rt]);
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[rt][t >> 1][8 * (t & 1) + j], c, moff));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(sacc[rt][t >> 1][8 * (t & 1) + j + 1], c, moff));
        lsum += p0 + p1;
        pb[rt][t][j] = (__bf16)p0;
        pb[rt][t][j + 1] = (__bf16)p1;
      }
    }
    l_run[rt] += lsum;
  }
  const uint16_t* vbase = Vt + key_l * C::VLD + half * 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const bf16x8_t a =
          *reinterpret_cast<const bf16x8_t*>(vbase + dt * 32 * C::VLD + t * 16);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        oacc[rt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rt][t], oacc[rt][dt], 0, 0, 0);
    }
  }
}

// The kernel's parameters as one struct, member for member: the layout of the
// kernel-argument segment (each argument in order at the next offset aligned
// to its type, as for struct members; checked below against the kernel's
// signature).  The host packs a launch into it, and persistent unsplit
// launches read their arguments from the segment through it (opaque_args).
struct AttnKernArgs {
  Plan p;
  KVDesc kv;
  const void* q;
  const void* k;
  const void* v;
  const uint16_t* kb2;
  const uint16_t* vb16;
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

__device__ __forceinline__ const AttnKernArgs* opaque_args() {
  return opaque_kernargs<AttnKernArgs>();
}

// PERSIST: workgroups take units from the work list until it is empty.
// OPQ (persistent unsplit launches): the arguments are read through
// opaque_args() and units come from per-XCD queues.  Split launches, a few
// light items per workgroup, keep plain arguments and one shared queue: the
// OPQ path ran their attention 14% slower.
template <int DT, int D, int NW, int RT, bool PERSIST, bool CORR, bool OPQ = false>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(
    Plan p, KVDesc kv_a, const void* __restrict__ q_a, const void* __restrict__ k_a,
    const void* __restrict__ v_a, const uint16_t* __restrict__ kb2_a,
    const uint16_t* __restrict__ vb16_a, const int32_t* __restrict__ cu_a,
    const int32_t* __restrict__ idx_a, float c_a, float out_scale_a, int correction_a,
    int dense_a, int units_per_seg, int splits_a, uint16_t* __restrict__ out_a,
    float* __restrict__ lse_a, float* __restrict__ part_o_a, float* __restrict__ part_ml_a,
    const int32_t* __restrict__ items_a, int* __restrict__ queue_a) {
  using C = AttnCfg<D, NW, RT>;
  static_assert(DT == kBF16, "bf16 inputs only; fp8 takes attn_fp8_kernel");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKeys * C::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * C::VLD];
  // correction steps: the lo rows of the pooled keys, a ring of three slots
  // (the steps being multiplied, staged and loaded); a stub without them
  __shared__ __attribute__((aligned(16))) uint16_t Kl[3][CORR ? C::NCH * kKeys * 8 : 8];
  __shared__ uint32_t selbits[kMaxBlocksPerSeq / 32];
  __shared__ int next_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;

  // One work unit: (segment (b, h, I), row block mt, KV split sp).
  const Plan& p_outer = p;
  auto run_unit = [&](int b, int I, int h, int mt, int sp) __attribute__((always_inline)) {
  // the arguments: through the opaque pointer for OPQ, else the parameters
  const AttnKernArgs* ka = OPQ ? opaque_args() : nullptr;
  const Plan& p = OPQ ? ka->p : p_outer;
  const KVDesc& kv = OPQ ? ka->kv : kv_a;
  const void* q = OPQ ? ka->q : q_a;
  const void* k = OPQ ? ka->k : k_a;
  const void* v = OPQ ? ka->v : v_a;
  const uint16_t* kb2 = OPQ ? ka->kb2 : kb2_a;
  const uint16_t* vb16 = OPQ ? ka->vb16 : vb16_a;
  const int32_t* cu = OPQ ? ka->cu : cu_a;
  const int32_t* idx = OPQ ? ka->idx : idx_a;
  const float c = OPQ ? ka->c : c_a, out_scale = OPQ ? ka->out_scale : out_scale_a;
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
  // split sp of the segment's ns takes a contiguous share of the CSR
  // positions, balanced by count, and every ns-th correction chunk
  const int beg0 = dense ? 0 : cu[seg], n_sel = (dense ? I + 1 : cu[seg + 1]) - beg0;
  const int ns = splits == 1 ? 1 : segment_splits(n_sel, I, p.B, correction, splits);
  // the unit's last query position bounds the keys it can see: a 64-key
  // half of the diagonal block past it is skipped (all its keys are masked)
  const int qmax = q0 + max(min(R, (mt + 1) * C::ROWS) - 1, 0) / p.g;
  UnitCtx u{b, h, I, s.len, s.kv_start, s.pool_base, p.B,
            beg0 + (int)((int64_t)sp * n_sel / ns),
            beg0 + (int)((int64_t)(sp + 1) * n_sel / ns), dense, sp, ns,
            min(s.len, qmax + 1)};

  // ---- this lane's query rows (B operands of Q K^T), one per row tile
  const int row0 = mt * C::ROWS + wave * RT * 32;
  const bool wave_active = row0 < R;
  int qpos[RT], hqs[RT];
  bool valid[RT];
  bf16x8_t qf[RT][C::KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = row0 + rt * 32 + (lane & 31);
    valid[rt] = r < R;
    qpos[rt] = q0 + (valid[rt] ? r / p.g : 0);
    hqs[rt] = h * p.g + (valid[rt] ? r % p.g : 0);
    const int64_t qoff = (q_row(s, qpos[rt]) * p.hq + hqs[rt]) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (valid[rt])
        w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(q) + qoff + ks * 16 +
                                              half * 8);
      qf[rt][ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // ---- selected-block bitmap for the correction chunks
  if (correction && I > 0) {
    const int nwords = (I + 31) >> 5;
    for (int w = tid; w < nwords; w += C::NT) selbits[w] = 0u;
    __syncthreads();
    // every selected block of the segment, not only this split's share: the
    // others are attended exactly by the other splits
    for (int t = beg0 + tid; t < beg0 + n_sel; t += C::NT) {
      const int J = block_at(idx, t, u);
      if (J < I) atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
  }

  f32x16_t oacc[RT][C::DT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) oacc[rt][dt][rr] = 0.f;
    }
  }
  const float bias = __log2f((float)p.B);  // corrected blocks are full blocks

  const FetchOffsets<D, NW, RT> off16 = fetch_offsets<D, NW, RT>(p.hkv);
  const CorrOffsets<D, NW, RT> offc = corr_offsets<D, NW, RT>(p.hkv);
  Prefetch<D, NW, RT> pf;
  Step cur = first_step(u, idx, selbits, correction);
  if (cur.kind != kDone) {
    fetch_step<D, NW, RT, CORR>(pf, off16, offc, cur, u, kv, p.hkv, k, v, kb2, vb16,
                                    Kl[0]);
    store_step<D, NW, RT, CORR>(pf, Ks[0], Vt[0]);
  }
  uniform(cur);
  // the query rows and the first step have arrived; saying so here keeps the
  // compiler from waiting on every outstanding load at the top of the loop
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  Step nxt = cur;
  if (cur.kind != kDone) advance(nxt, u, idx, selbits, correction);
  uniform(nxt);
  if (nxt.kind != kDone)
    fetch_step<D, NW, RT, CORR>(pf, off16, offc, nxt, u, kv, p.hkv, k, v, kb2, vb16,
                                    Kl[1]);
  int buf = 0;
  int ls = 0;  // Kl slot of step n (n+1 and n+2 follow, modulo 3)
  // Per step: barrier (step n is in LDS, the other buffer is free), write the
  // prefetched step n+1 to the other buffer, issue the loads of step n+2,
  // multiply step n.  A wave that has written its share starts computing
  // while the others still write.
  while (cur.kind != kDone) {
    __syncthreads();
    // advance first: its scalar index loads were issued a block earlier, and
    // no LDS write is in flight yet for their wait to cover
    Step nn = nxt;
    if (nn.kind != kDone) {
      advance(nn, u, idx, selbits, correction);
      uniform(nn);
    }
    if (nxt.kind != kDone)
      store_step<D, NW, RT, CORR>(pf, Ks[buf ^ 1], Vt[buf ^ 1]);
    // slot ls + 2 held step n-1, which every wave finished before the barrier
    if (nn.kind != kDone)
      fetch_step<D, NW, RT, CORR>(pf, off16, offc, nn, u, kv, p.hkv, k, v, kb2, vb16,
                                      Kl[ls == 0 ? 2 : ls - 1]);
    if (wave_active) {
      int mode, key0 = 0;
      uint64_t todo = 0;
      if (cur.kind == kExact) {
        key0 = cur.J * p.B + cur.hf * kKeys;
        mode = cur.J == I ? kDiag : kPlain;
      } else {
        todo = chunk_todo(selbits, cur.c, I);
        mode = todo == ~0ull ? kCorrAll : kCorrMode;
      }
      compute_step<D, NW, RT, CORR>(Ks[buf], Kl[ls], Vt[buf], qf, oacc, m_run, l_run, c, mode,
                                    key0, s.len, qpos, todo, bias);
    }
    cur = nxt;
    nxt = nn;
    buf ^= 1;
    ls = ls == 2 ? 0 : ls + 1;
  }

  // ---- epilogue: l over all keys of the row = both lane halves.  A split
  // unit leaves its partial result (O normalised by its own l, the log2
  // reference m and l) for the merge kernel.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_tot = halves_sum(l_run[rt]);
    if (!valid[rt]) continue;
    const float inv = l_tot > 0.f ? out_scale / l_tot : 0.f;
    const int64_t orow = q_row(s, qpos[rt]) * p.hq + hqs[rt];
    if (ns > 1) {
      const int64_t prow = (int64_t)sp * p.total_tokens * p.hq + orow;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = dt * 32 + g4 * 8 + half * 4;
          *reinterpret_cast<float4*>(part_o + prow * D + d) =
              make_float4(oacc[rt][dt][4 * g4] * inv, oacc[rt][dt][4 * g4 + 1] * inv,
                          oacc[rt][dt][4 * g4 + 2] * inv, oacc[rt][dt][4 * g4 + 3] * inv);
        }
      }
      if (half == 0)
        *reinterpret_cast<float2*>(part_ml + 2 * prow) =
            make_float2(l_tot > 0.f ? m_run[rt] : -INFINITY, l_tot);
      continue;
    }
    const int64_t ooff = orow * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + half * 4;
        const uint32_t lo =
            pack_bf16x2(oacc[rt][dt][4 * g4] * inv, oacc[rt][dt][4 * g4 + 1] * inv);
        const uint32_t hi =
            pack_bf16x2(oacc[rt][dt][4 * g4 + 2] * inv, oacc[rt][dt][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(out + ooff + d) = make_uint2(lo, hi);
      }
    }
    if (lse && half == 0)
      lse[(int64_t)hqs[rt] * p.total_tokens + q_row(s, qpos[rt])] =
          l_tot > 0.f ? m_run[rt] * kLn2 + __logf(l_tot) : -INFINITY;
  }
  };

  if constexpr (!PERSIST) {
    // one workgroup per unit, enumerated heaviest first: longest request
    // first, tiles in descending I, then row block, KV head innermost (turned
    // every kHeadTurn groups, unit_head)
    const int64_t unit = blockIdx.x;
    int pos = 0;
    while (pos + 1 < p.num_seqs && p.seq[p.order[pos + 1]].unit_base <= unit) ++pos;
    const int b = p.order[pos];
    const int64_t local = unit - p.seq[b].unit_base;
    const int per_I = p.hkv * units_per_seg;
    const int rem = (int)(local % per_I);
    run_unit(b, p.seq[b].nblk - 1 - (int)(local / per_I), unit_head(local, p.hkv), rem / p.hkv, 0);
  } else {
  if constexpr (OPQ) {
  // unsplit: persistent workgroups take items from the list the preparation
  // kernel wrote (heaviest first).  Item k belongs to queue k mod 8, the XCD
  // a one-workgroup-per-item launch would run it on (the dispatcher deals
  // workgroups to the XCDs round robin); a workgroup drains its own XCD's
  // queue, then what is left of the others in turn.  Thread 0 keeps the
  // cursor in LDS and hands each item's code to the workgroup there, and the
  // decode reads the plan through the opaque pointer, so no value of one unit
  // stays live into the next.
  __shared__ int q_cur[2];  // queue being drained, queues found empty
  if (tid == 0) {
    q_cur[0] = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7;  // XCC_ID
    q_cur[1] = 0;
  }
  for (;;) {
    if (tid == 0) {
      const AttnKernArgs* kq = opaque_args();
      const int n_items = kq->queue[1];
      int qx = q_cur[0], tried = q_cur[1], code = -1;
      while (tried < 8) {
        const int kk = qx + 8 * atomicAdd(&kq->queue[2 + qx], 1);
        if (kk < n_items) {
          code = kq->items[kk];
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
    const Plan& pd = opaque_args()->p;
    const int64_t seg = code >> 8;
    int b = 0;
    while (b + 1 < pd.num_seqs && pd.seq[b + 1].seg_base <= seg) ++b;
    int h, I;
    segment_tile(pd.seq[b], (int)(seg - pd.seq[b].seg_base), h, I);
    run_unit(b, I, h, (code >> 4) & 15, code & 15);
  }
  } else {
  // split launch: persistent workgroups take items from one shared queue
  // (heaviest segments first) until it is empty
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
}

// AttnKernArgs must be laid out as the kernel's parameter list.
using AttnParams = KernelParams<decltype(attn_mfma_kernel<kBF16, 128, 8, 1, true, true, true>)>;
static_assert(AttnParams::count == 21, "AttnKernArgs mirrors 21 kernel parameters");
#define BSLP_ARG_AT(i, m) \
  static_assert(AttnParams::offset(i) == offsetof(AttnKernArgs, m), "AttnKernArgs." #m);
BSLP_ARG_AT(0, p) BSLP_ARG_AT(1, kv) BSLP_ARG_AT(2, q) BSLP_ARG_AT(3, k) BSLP_ARG_AT(4, v)
BSLP_ARG_AT(5, kb2) BSLP_ARG_AT(6, vb16) BSLP_ARG_AT(7, cu) BSLP_ARG_AT(8, idx)
BSLP_ARG_AT(9, c) BSLP_ARG_AT(10, out_scale) BSLP_ARG_AT(11, correction) BSLP_ARG_AT(12, dense)
BSLP_ARG_AT(13, units_per_seg) BSLP_ARG_AT(14, splits) BSLP_ARG_AT(15, out) BSLP_ARG_AT(16, lse)
BSLP_ARG_AT(17, part_o) BSLP_ARG_AT(18, part_ml) BSLP_ARG_AT(19, items) BSLP_ARG_AT(20, queue)
#undef BSLP_ARG_AT

// Merge of the KV splits of the rows of every split segment: with M =
// max_u m_u and weights w_u = l_u 2^(m_u - M), O = sum_u w_u O_u / sum_u w_u
// and LSE = M ln 2 + ln sum_u w_u - lse_off (lse_off = 8 ln 2 when the l_u
// sum probabilities scaled by 2^8, as in the fp8 kernel) (the KV splits of "FlashPrefill V2", CSR
// paragraph, Eq. 18; the combine is the online-softmax merge of the PRR review
// page, Sec. 4.3 Eq. 6).  One workgroup per segment (b, h, I); segments that
// were not split wrote their rows directly and are skipped.
template <int D>
__global__ __launch_bounds__(256) void merge_splits_kernel(Plan p, const int32_t* __restrict__ cu,
                                                           const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int splits, int correction,
                                                           float lse_off,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int64_t seg = blockIdx.x;
  const int b = seq_of_segment(p, seg);
  const SeqInfo s = p.seq[b];
  int h, I;
  segment_tile(s, (int)(seg - s.seg_base), h, I);
  const int ns = segment_splits(cu[seg + 1] - cu[seg], I, p.B, correction, splits);
  if (ns == 1) return;
  const int q0 = tile_q0(s, I, p.B), nq = tile_nq(s, I, p.B);
  const int64_t prows = p.total_tokens * p.hq;  // rows of one split's partials
  for (int i = threadIdx.x; i < p.g * nq * (D / 4); i += 256) {
    const int r = i / (D / 4), d = (i % (D / 4)) * 4;
    const int64_t tok = q_row(s, q0 + r / p.g);
    const int hq = h * p.g + r % p.g;
    const int64_t row = tok * p.hq + hq;
    float M = -INFINITY;
    for (int u = 0; u < ns; ++u) M = fmaxf(M, part_ml[2 * (u * prows + row)]);
    float L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    if (M != -INFINITY) {
      for (int u = 0; u < ns; ++u) {
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + 2 * (u * prows + row));
        if (ml.x == -INFINITY) continue;
        const float w = ml.y * __builtin_amdgcn_exp2f(ml.x - M);
        const float4 o = *reinterpret_cast<const float4*>(part_o + (u * prows + row) * D + d);
        L += w;
        o0 = fmaf(w, o.x, o0);
        o1 = fmaf(w, o.y, o1);
        o2 = fmaf(w, o.z, o2);
        o3 = fmaf(w, o.w, o3);
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<uint2*>(out + row * D + d) =
        make_uint2(pack_bf16x2(o0 * inv, o1 * inv), pack_bf16x2(o2 * inv, o3 * inv));
    if (lse && d == 0)
      lse[(int64_t)hq * p.total_tokens + tok] =
          L > 0.f ? M * kLn2 + __logf(L) - lse_off : -INFINITY;
  }
}

// Work list of a persistent launch ("FlashPrefill V2", CSR paragraph, Eq. 18,
// and the scheduling paragraph after it: splits balanced by selected count,
// heaviest work first): one workgroup walks the segments in the order of the
// one-workgroup-per-unit launch (longest request first, tiles in descending
// I, KV head innermost), gives each its split count from its selected count
// and writes one item (segment << 8 | row block << 4 | split) per (row
// block, split), with a block-wide prefix sum for the offsets.  Unsplit
// (splits = 1: every segment has units_per_seg items) the items go in that
// launch's exact unit order, row block outside the KV head, so item k is the
// unit it would have run on XCD k mod 8.  queue[0]: next item of one shared
// queue (split launches); queue[1]: the number of items; queue[2 + x]: next
// item of XCD x's queue (items x, x + 8, ...; unsplit bf16 launches).
__global__ __launch_bounds__(1024) void split_items_kernel(Plan p, const int32_t* __restrict__ cu,
                                                           int splits, int correction,
                                                           int units_per_seg,
                                                           int32_t* __restrict__ items,
                                                           int* __restrict__ queue) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < p.num_segments; base += 1024) {
    const int64_t q = base + tid;
    int n = 0, seg = 0, I = 0;
    if (q < p.num_segments) {
      // q-th segment in launch order
      int i = 0;
      int64_t qb = 0;
      while (qb + (int64_t)ntile(p.seq[p.order[i]]) * p.hkv <= q) {
        qb += (int64_t)ntile(p.seq[p.order[i]]) * p.hkv;
        ++i;
      }
      const SeqInfo& si = p.seq[p.order[i]];
      const int local = (int)(q - qb);
      I = si.nblk - 1 - local / p.hkv;
      seg = si.seg_base + (local % p.hkv) * ntile(si) + (I - si.i0);
      n = segment_splits(cu[seg + 1] - cu[seg], I, p.B, correction, splits) * units_per_seg;
    }
    // block-wide exclusive prefix sum of n
    int x = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int off = before + x - n;
    if (n > 0) {
      const int ns = n / units_per_seg;
      if (splits == 1) {
        const int hh = (int)(q % p.hkv);  // q - hh is a multiple of hkv
        for (int t = 0; t < n; ++t)
          items[(q - hh) * units_per_seg + t * p.hkv + hh] = (seg << 8) | (t << 4);
      } else {
        for (int t = 0; t < n; ++t)
          items[off + t] = (seg << 8) | ((t / ns) << 4) | (t % ns);
      }
    }
    __syncthreads();
    if (tid == 1023) carry_s = off + n;
    __syncthreads();
  }
  if (tid < 10) queue[tid] = tid == 1 ? carry_s : 0;
}

// float32 pooled means -> bf16 for the correction steps.  Keys become the pair
// hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in float32, so hi + lo is
// x to within 2^-18 |x|), stored as [pooled row, {hi, lo}, Hkv, D]; values are
// rounded once, [pooled row, Hkv, D].  n8 = 8-element groups per tensor,
// row8 = groups per pooled row.
__global__ __launch_bounds__(256) void pooled_to_bf16_kernel(const float* __restrict__ kbar,
                                                            const float* __restrict__ vbar,
                                                            int64_t n8, int row8,
                                                            uint16_t* __restrict__ kb2,
                                                            uint16_t* __restrict__ vb16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n8) return;
  const bool is_v = i >= n8;
  const int64_t j = is_v ? i - n8 : i;
  const float* src = (is_v ? vbar : kbar) + 8 * j;
  float x[8];
  const float4 a = *reinterpret_cast<const float4*>(src);
  const float4 bq = *reinterpret_cast<const float4*>(src + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = bq.x; x[5] = bq.y; x[6] = bq.z; x[7] = bq.w;
  u32x4_t hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    const float h0 = __uint_as_float(hi[e] << 16), h1 = __uint_as_float(hi[e] & 0xffff0000u);
    lo[e] = pack_bf16x2(x[2 * e] - h0, x[2 * e + 1] - h1);
  }
  if (is_v) {
    *reinterpret_cast<u32x4_t*>(vb16 + 8 * j) = hi;
  } else {
    const int64_t row = j / row8, col = j % row8;
    *reinterpret_cast<u32x4_t*>(kb2 + 8 * (row * 2 * row8 + col)) = hi;
    *reinterpret_cast<u32x4_t*>(kb2 + 8 * (row * 2 * row8 + row8 + col)) = lo;
  }
}

int attn_rows_per_unit(const Plan& p) {
  const int rows = p.g * p.B;
  return rows >= 256 ? 256 : rows >= 128 ? 128 : 64;  // the launch table below
}

int attn_splits(const Plan& p, int dtype, int requested) {
  // work items carry the segment in 23 bits
  if (dtype == kF32 || requested == 1 || p.num_segments >= (1 << 23)) return 1;
  if (requested >= 2) return requested;
  // automatic: when the launch holds fewer than about two workgroups per CU
  // and some tile can select enough blocks to be worth cutting, split until
  // it does (at most 4 ways)
  int64_t units = 0;
  const int ups = (p.g * p.B + attn_rows_per_unit(p) - 1) / attn_rows_per_unit(p);
  for (int i = 0; i < p.num_seqs; ++i) units += (int64_t)ntile(p.seq[i]) * p.hkv * ups;
  constexpr int64_t kTarget = 512;  // 2 x 256 CUs
  if (units == 0 || units >= kTarget || p.max_nblk < 16) return 1;
  return (int)std::min<int64_t>(4, (kTarget + units - 1) / units);
}

// pooled keys as hi/lo bf16 pairs and pooled values as bf16, then (split
// launches) the per-split partial O (float32 [splits, T * Hq, d]) and (m, l)
// pairs (float32 [splits, T * Hq, 2])
size_t attn_pooled_bytes(const Plan& p) {
  const size_t n = (size_t)p.pooled_rows * p.hkv * p.d;  // elements per pooled tensor
  return (3 * n * sizeof(uint16_t) + 255) / 256 * 256;
}

// counters after the work list: queue[0 .. 9] (see split_items_kernel) + 2
constexpr size_t kQueueWords = 12;

size_t attn_split_items(const Plan& p, int splits) {
  const int ups = (p.g * p.B + attn_rows_per_unit(p) - 1) / attn_rows_per_unit(p);
  return (size_t)p.num_segments * ups * splits;
}

size_t attn_workspace_bytes(const Plan& p, int splits) {
  size_t bytes = attn_pooled_bytes(p);
  if (splits > 1) bytes += (size_t)splits * p.total_tokens * p.hq * (p.d + 2) * sizeof(float);
  // the work list and its queue counters (persistent launches)
  return bytes + (attn_split_items(p, splits) + kQueueWords) * sizeof(int32_t);
}

SplitBufs split_bufs(const Plan& p, void* workspace, int splits) {
  SplitBufs b;
  const size_t parts = splits > 1 ? (size_t)splits * p.total_tokens * p.hq : 0;  // partial rows
  b.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + attn_pooled_bytes(p));
  b.part_ml = b.part_o + parts * p.d;
  b.items = reinterpret_cast<int32_t*>(b.part_ml + parts * 2);
  b.queue = b.items + attn_split_items(p, splits);
  return b;
}

hipError_t launch_split_items(const Plan& pl, const int32_t* cu, int splits, int corr,
                              int units_per_seg, const SplitBufs& b, hipStream_t st) {
  hipLaunchKernelGGL(split_items_kernel, dim3(1), dim3(1024), 0, st, pl, cu, splits, corr,
                     units_per_seg, b.items, b.queue);
  return hipGetLastError();
}

// Asked once per device: a launch of a few tens of microseconds would
// otherwise carry the query.
hipError_t attn_device_cus(int* cus) {
  static std::atomic<int> known[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && (*cus = known[dev].load(std::memory_order_relaxed)) > 0)
    return hipSuccess;
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < 64) known[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

hipError_t persistent_grid(const Plan& p, int splits, int per_cu, int64_t* grid) {
  int cus = 0;
  const hipError_t e = attn_device_cus(&cus);
  if (e != hipSuccess) return e;
  *grid = std::min<int64_t>(attn_split_items(p, splits), (int64_t)cus * std::max(1, per_cu));
  return hipSuccess;
}

hipError_t launch_split_merge(const Plan& p, const int32_t* cu, const SplitBufs& b, int splits,
                              int corr, float lse_off, uint16_t* out, float* lse,
                              hipStream_t st) {
  if (p.d == 128)
    hipLaunchKernelGGL((merge_splits_kernel<128>), dim3((unsigned)p.num_segments), dim3(256), 0,
                       st, p, cu, b.part_o, b.part_ml, splits, corr, lse_off, out, lse);
  else
    hipLaunchKernelGGL((merge_splits_kernel<64>), dim3((unsigned)p.num_segments), dim3(256), 0,
                       st, p, cu, b.part_o, b.part_ml, splits, corr, lse_off, out, lse);
  return hipGetLastError();
}

// A persistent launch of `kernel`: as many workgroups as stay resident at
// once (the occupancy of a compiled kernel does not change, so it is asked
// once per process), at most one per work item.
template <void (*kernel)(Plan, KVDesc, const void*, const void*, const void*, const uint16_t*,
                         const uint16_t*, const int32_t*, const int32_t*, float, float, int, int,
                         int, int, uint16_t*, float*, float*, float*, const int32_t*, int*)>
static hipError_t launch_persistent(const Plan& p, int splits, int threads, const AttnKernArgs& ka,
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
                     ka.v, ka.kb2, ka.vb16, ka.cu, ka.idx, ka.c, ka.out_scale, ka.correction,
                     ka.dense, ka.units_per_seg, ka.splits, ka.out, ka.lse, ka.part_o, ka.part_ml,
                     ka.items, ka.queue);
  return hipGetLastError();
}

// CORR: the instantiation with correction steps.  Launches without them (the
// dense path, correction off) use one compiled without, whose plain steps keep
// no registers for the pooled keys' lo rows.
template <int DT, int D, int NW, int RT, bool CORR>
static hipError_t launch_mfma_t(const Plan& p, const KVDesc& kv, const AttnArgs& a,
                                hipStream_t st) {
  const int rows = AttnCfg<D, NW, RT>::ROWS;
  const int units_per_seg = (p.g * p.B + rows - 1) / rows;
  // enumerate units: longest request first, tiles in descending I, then row
  // block, KV head innermost
  Plan pl = p;
  int64_t base = 0;
  for (int i = 0; i < pl.num_seqs; ++i) {
    const int b = pl.order[i];
    pl.seq[b].unit_base = (int32_t)base;
    base += (int64_t)ntile(pl.seq[b]) * pl.hkv * units_per_seg;
  }
  if (base == 0) return hipSuccess;
  const size_t n = (size_t)p.pooled_rows * p.hkv * p.d;
  uint16_t* kb2 = reinterpret_cast<uint16_t*>(a.workspace);
  uint16_t* vb16 = kb2 + 2 * n;
  if (n > 0 && a.correction && !a.dense) {
    const int64_t n8 = (int64_t)(n / 8);
    hipLaunchKernelGGL(pooled_to_bf16_kernel, dim3((unsigned)((2 * n8 + 255) / 256)), dim3(256),
                       0, st, a.kbar, a.vbar, n8, p.hkv * p.d / 8, kb2, vb16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // logits in units of log2
  const float c = (float)((double)a.lscale * 1.4426950408889634);
  const int splits = a.splits;
  const int corr = a.correction && !a.dense;
  AttnKernArgs ka{pl, kv, a.q, a.k, a.v, kb2, vb16, a.cu, a.idx, c, a.v_scale, corr, a.dense,
                  units_per_seg, splits, (uint16_t*)a.out, a.lse, nullptr, nullptr, nullptr,
                  nullptr};
  // Persistent workgroups over a work list for split launches, and for
  // unsplit sparse ones with enough units per CU that the queue's cost (a
  // list-building launch, an atomic per unit) is repaid by the idle time
  // between one-workgroup-per-unit dispatches it removes; otherwise one
  // workgroup per unit.
  int cus = 0;
  if (splits == 1 && !a.dense && a.workspace && a.cu) {
    const hipError_t e = attn_device_cus(&cus);
    if (e != hipSuccess) return e;
  }
  const bool persist =
      splits > 1 || (cus > 0 && base >= (int64_t)kPersistUnitsPerCU * cus);
  if (!persist) {
    hipLaunchKernelGGL((attn_mfma_kernel<DT, D, NW, RT, false, CORR>), dim3((unsigned)base),
                       dim3(NW * 64), 0, st, ka.p, ka.kv, ka.q, ka.k, ka.v, ka.kb2, ka.vb16,
                       ka.cu, ka.idx, ka.c, ka.out_scale, ka.correction, ka.dense,
                       ka.units_per_seg, ka.splits, ka.out, ka.lse, ka.part_o, ka.part_ml,
                       ka.items, ka.queue);
    return hipGetLastError();
  }
  SplitBufs sb = split_bufs(p, a.workspace, splits);
  hipError_t e = launch_split_items(pl, a.cu, splits, corr, units_per_seg, sb, st);
  if (e != hipSuccess) return e;
  ka.part_o = sb.part_o;
  ka.part_ml = sb.part_ml;
  ka.items = sb.items;
  ka.queue = sb.queue;
  if (splits == 1)
    return launch_persistent<attn_mfma_kernel<DT, D, NW, RT, true, CORR, true>>(p, splits, NW * 64,
                                                                                  ka, st);
  e = launch_persistent<attn_mfma_kernel<DT, D, NW, RT, true, CORR, false>>(p, splits, NW * 64, ka,
                                                                              st);
  if (e != hipSuccess) return e;
  return launch_split_merge(p, a.cu, sb, splits, corr, 0.f, (uint16_t*)a.out, a.lse, st);
}

template <int DT, int D>
static hipError_t launch_mfma_d(const Plan& p, const KVDesc& kv, const AttnArgs& a,
                                hipStream_t st) {
  const int rows = p.g * p.B;
  if (a.correction && !a.dense) {
    if (rows >= 256) return launch_mfma_t<DT, D, 8, 1, true>(p, kv, a, st);
    if (rows >= 128) return launch_mfma_t<DT, D, 4, 1, true>(p, kv, a, st);
    return launch_mfma_t<DT, D, 2, 1, true>(p, kv, a, st);
  }
  if (rows >= 256) return launch_mfma_t<DT, D, 8, 1, false>(p, kv, a, st);
  if (rows >= 128) return launch_mfma_t<DT, D, 4, 1, false>(p, kv, a, st);
  return launch_mfma_t<DT, D, 2, 1, false>(p, kv, a, st);
}

hipError_t launch_attn_mfma(const Plan& p, const KVDesc& kv, int dtype, const AttnArgs& a,
                            hipStream_t st) {
  if (dtype != kBF16) return hipErrorInvalidValue;  // fp8 runs in attn_fp8.hip
  return p.d == 128 ? launch_mfma_d<kBF16, 128>(p, kv, a, st)
                    : launch_mfma_d<kBF16, 64>(p, kv, a, st);
}

}  // namespace bslp
