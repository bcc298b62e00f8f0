// Internal launchers of libbslp (host side).  Each enqueues its kernels on the
// given stream and returns the first HIP error, if any.
#pragma once

#include "common.hpp"

namespace bslp {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* kbar;
  const float* vbar;
  const int32_t* cu;
  const int32_t* idx;
  void* out;
  float* lse;
  void* workspace;  // attn_workspace_bytes(plan) bytes, device
  float lscale;   // softmax_scale * q_scale
  float k_scale;  // 1 unless fp8
  float v_scale;
  int correction;
  int dense;   // walk every causal block J <= I (cu, idx, kbar, vbar unused)
  int splits;  // KV splits per work unit (1: none), from attn_splits
};

// Stage 1: pooling (kStagePool) and / or block scores (kStageScores).
constexpr int kStagePool = 1;
constexpr int kStageScores = 2;
hipError_t launch_stage1(const Plan& p, const KVDesc& kv, int dtype, const void* q, const void* k,
                         const void* v, float q_scale, float k_scale, float v_scale,
                         float softmax_scale, float* kbar, float* vbar, float* scores,
                         int parts, hipStream_t st);

// Block scores on the matrix cores (bf16 / fp8 inputs, g*B <= 1024 rows per
// tile); c2 = softmax_scale * q_scale * log2(e).
bool scores_mfma_supported(const Plan& p, int dtype);
hipError_t launch_scores_mfma(const Plan& p, int dtype, const void* q, const float* kbar,
                              float c2, float* scores, hipStream_t st);

// Selection; q, kbar and lscale = softmax_scale * q_scale serve the exact
// float64 re-decision of blocks near the threshold.  The scores of the
// re-decided blocks that are dropped are negated by the first pass and
// restored by the last.
hipError_t launch_select(const Plan& p, const SelectArgs& a, const void* q, const float* kbar,
                         int dtype, float lscale, float* scores, int32_t* counts, int32_t* cu,
                         int32_t* idx, hipStream_t st);

hipError_t launch_attn_valu(const Plan& p, const KVDesc& kv, int dtype, const AttnArgs& a,
                            hipStream_t st);

// KV splits per attention work unit for a requested count (0: automatic, 1:
// none, 2..kMaxSplits: that many); 1 for the float32 path.
int attn_splits(const Plan& p, int dtype, int requested);

// Device scratch the attention launch needs: bf16 copies of the pooled means
// and, for split launches, the per-split partial results.
size_t attn_pooled_bytes(const Plan& p);
size_t attn_workspace_bytes(const Plan& p, int splits);

// Online per-tensor e4m3 quantisation: scale (device, one float) and codes.
hipError_t launch_quantize_e4m3(int src_dtype, const void* x, int64_t n, uint8_t* codes,
                                float* scale, hipStream_t st);

// KV-split machinery shared by the matrix-core attention launchers: rows per
// work unit, work-list length, the workspace regions of the partial results,
// the work-list and merge launches, and the persistent grid size.
int attn_rows_per_unit(const Plan& p);
size_t attn_split_items(const Plan& p, int splits);
struct SplitBufs {
  float* part_o;   // [splits, T * Hq, d]
  float* part_ml;  // [splits, T * Hq, 2]: (m in log2 units, l)
  int32_t* items;  // work list
  int* queue;      // [0] next item, [1] item count
};
SplitBufs split_bufs(const Plan& p, void* workspace, int splits);
hipError_t launch_split_items(const Plan& pl, const int32_t* cu, int splits, int corr,
                              int units_per_seg, const SplitBufs& b, hipStream_t st);
hipError_t launch_split_merge(const Plan& p, const int32_t* cu, const SplitBufs& b, int splits,
                              int corr, float lse_off, uint16_t* out, float* lse, hipStream_t st);
hipError_t persistent_grid(const Plan& p, int splits, int per_cu, int64_t* grid);
// Compute units of the current device (asked of the runtime once per device).
hipError_t attn_device_cus(int* cus);
// Unsplit sparse launches with at least this many work units per CU run
// persistent over per-XCD queues (bf16 64K: 32 per CU, 5% faster than one
// workgroup per unit; 16K: 8 per CU, 4% slower; fp8 128K: 32 per CU, 3%
// faster).
constexpr int64_t kPersistUnitsPerCU = 16;

// fp8 inputs on the fp8 matrix cores (e4m3 probabilities, FlashPrefill V2 FP8
// arithmetic); with p.v_dmajor, V is [Hkv, d, kv tokens] (contiguous) or
// [pages, Hkv, d, page_size] (paged).
hipError_t launch_attn_fp8(const Plan& p, const KVDesc& kv, const AttnArgs& a, hipStream_t st);

// Pooled means of a d-major fp8 V: vbar (float32, times the V scale) or,
// with codes, the e4m3 code of each mean (the quantised pooled values).
hipError_t launch_pool_v_dmajor(const Plan& p, const KVDesc& kv, const void* v, float v_scale,
                                float* vbar, uint8_t* vq, hipStream_t st);

// Size of the device array that serves as the attention workspace of the
// entry point that allocates nothing, and its address on the current device
// (taken once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** out);

// bf16 inputs on the matrix cores (fp8 inputs take launch_attn_fp8).
hipError_t launch_attn_mfma(const Plan& p, const KVDesc& kv, int dtype, const AttnArgs& a,
                            hipStream_t st);

}  // namespace bslp
