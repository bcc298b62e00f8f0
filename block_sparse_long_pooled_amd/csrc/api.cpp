// extern "C" entry points of libbslp: argument validation on the host, the
// per-call plan (request table), then kernel launches on the caller's stream.
// Nothing here allocates device memory, synchronises, or reads device memory.
#include <cmath>
#include <string>

#include "bslp.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

bslp_status fail(bslp_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }

// The q / k / v scale the host formulas use: 1 when the scales live in
// device memory (the kernels apply those themselves).
float host_scale(const bslp_problem* pr, int which) {
  if (pr->scales_dev) return 1.f;
  return which == 0 ? pr->q_scale : which == 1 ? pr->k_scale : pr->v_scale;
}

bslp_status build_plan(const bslp_problem* pr, bslp::Plan* plan, bslp::KVDesc* kv) {
  if (!pr) return fail(BSLP_ERR_INVALID_ARG, "problem is NULL");
  if (pr->dtype < BSLP_F32 || pr->dtype > BSLP_FP8_E4M3)
    return fail(BSLP_ERR_INVALID_ARG, "unknown dtype " + std::to_string(pr->dtype));
  if (pr->num_heads_q < 1 || pr->num_heads_kv < 1)
    return fail(BSLP_ERR_INVALID_ARG, "head counts must be >= 1");
  if (pr->num_heads_q % pr->num_heads_kv)
    return fail(BSLP_ERR_INVALID_ARG, "num_heads_q must be a multiple of num_heads_kv");
  const int g = pr->num_heads_q / pr->num_heads_kv;
  if (g > bslp::kMaxGroup)
    return fail(BSLP_ERR_UNSUPPORTED, "group size Hq/Hkv above 16 is not built");
  if (pr->head_dim != 64 && pr->head_dim != 128)
    return fail(BSLP_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (pr->block_size != 64 && pr->block_size != 128)
    return fail(BSLP_ERR_UNSUPPORTED, "block_size must be 64 or 128");
  if (!finite_pos(pr->softmax_scale))
    return fail(BSLP_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!finite_pos(pr->q_scale) || !finite_pos(pr->k_scale) || !finite_pos(pr->v_scale))
    return fail(BSLP_ERR_INVALID_ARG, "q/k/v scales must be finite and > 0");
  if (pr->dtype != BSLP_FP8_E4M3 &&
      (pr->q_scale != 1.f || pr->k_scale != 1.f || pr->v_scale != 1.f))
    return fail(BSLP_ERR_INVALID_ARG, "q/k/v scales must be 1 unless dtype is fp8");
  if (pr->num_seqs < 1) return fail(BSLP_ERR_INVALID_ARG, "num_seqs must be >= 1");
  if (pr->num_seqs > bslp::kMaxSeqs)
    return fail(BSLP_ERR_UNSUPPORTED, "more than 64 packed requests per call");
  if (!pr->seqlens) return fail(BSLP_ERR_INVALID_ARG, "seqlens is NULL");
  int page_shift = 0;
  if (pr->page_table) {
    const int ps = pr->page_size;
    if (ps < 1 || ps > (1 << 20) || (ps & (ps - 1)))
      return fail(BSLP_ERR_INVALID_ARG, "page_size must be a power of two in [1, 2^20]");
    while ((1 << page_shift) < ps) ++page_shift;
    if (pr->max_pages_per_seq < 1)
      return fail(BSLP_ERR_INVALID_ARG, "max_pages_per_seq must be >= 1");
  }
  if (pr->kv_splits < 0 || pr->kv_splits > bslp::kMaxSplits)
    return fail(BSLP_ERR_INVALID_ARG, "kv_splits must be in 0 .. 16");
  if (pr->scales_dev && pr->dtype != BSLP_FP8_E4M3)
    return fail(BSLP_ERR_INVALID_ARG, "scales_dev is for fp8 inputs only");
  if (reinterpret_cast<uintptr_t>(pr->scales_dev) % 4)
    return fail(BSLP_ERR_INVALID_ARG, "scales_dev must be 4-byte aligned");
  if (pr->v_layout != BSLP_V_ROWS && pr->v_layout != BSLP_V_DMAJOR)
    return fail(BSLP_ERR_INVALID_ARG, "v_layout must be BSLP_V_ROWS or BSLP_V_DMAJOR");
  if (pr->v_layout == BSLP_V_DMAJOR && pr->dtype != BSLP_FP8_E4M3)
    return fail(BSLP_ERR_UNSUPPORTED, "d-major V is built for fp8 inputs only");
  if (pr->v_layout == BSLP_V_DMAJOR && pr->page_table && pr->page_size < 64)
    return fail(BSLP_ERR_UNSUPPORTED, "d-major V needs pages of at least 64 tokens");

  *plan = bslp::Plan{};
  plan->num_seqs = pr->num_seqs;
  plan->hq = pr->num_heads_q;
  plan->hkv = pr->num_heads_kv;
  plan->dscale = pr->scales_dev;
  plan->v_dmajor = pr->v_layout == BSLP_V_DMAJOR;
  plan->g = g;
  plan->d = pr->head_dim;
  plan->B = pr->block_size;
  int64_t tok = 0, kvtok = 0, pool = 0, seg = 0, score = 0;
  int max_nblk = 0;
  for (int b = 0; b < pr->num_seqs; ++b) {
    const int64_t Lq = pr->seqlens[b];
    const int64_t L = pr->kv_seqlens ? pr->kv_seqlens[b] : Lq;
    if (Lq < 0 || L < 0) return fail(BSLP_ERR_INVALID_ARG, "negative sequence length");
    if (Lq > L)
      return fail(BSLP_ERR_INVALID_ARG, "a request has more queries than keys (seqlens > kv_seqlens)");
    const int64_t N = (L + plan->B - 1) / plan->B;
    const int64_t i0 = Lq > 0 ? (L - Lq) / plan->B : N;  // no query: no tile
    if (N > bslp::kMaxBlocksPerSeq)
      return fail(BSLP_ERR_UNSUPPORTED, "more than 16384 blocks in one request");
    if (pr->page_table && (L + pr->page_size - 1) / pr->page_size > pr->max_pages_per_seq)
      return fail(BSLP_ERR_INVALID_ARG, "request longer than max_pages_per_seq pages");
    bslp::SeqInfo& s = plan->seq[b];
    s.tok_start = (int32_t)tok;
    s.kv_start = (int32_t)kvtok;
    s.len = (int32_t)L;
    s.q_off = (int32_t)(L - Lq);
    s.nblk = (int32_t)N;
    s.i0 = (int32_t)i0;
    s.pool_base = (int32_t)pool;
    s.seg_base = (int32_t)seg;
    s.unit_base = 0;
    s.score_base = score;
    tok += Lq;
    kvtok += L;
    pool += N;
    seg += (int64_t)plan->hkv * (N - i0);
    score += (int64_t)plan->hkv * (N * (N + 1) / 2 - i0 * (i0 + 1) / 2);
    if (N > max_nblk) max_nblk = (int)N;
    if (kvtok >= (int64_t(1) << 31) || score >= (int64_t(1) << 31))
      return fail(BSLP_ERR_UNSUPPORTED, "problem exceeds 2^31 tokens or index entries");
  }
  if (plan->v_dmajor && !pr->page_table && (int64_t)plan->d * kvtok >= (int64_t(1) << 31))
    return fail(BSLP_ERR_UNSUPPORTED, "d-major V beyond 2^31 bytes needs paged K/V");
  plan->max_nblk = max_nblk;
  // heaviest requests first (stable insertion sort, at most 64 entries)
  for (int i = 0; i < pr->num_seqs; ++i) {
    int j = i;
    while (j > 0 && plan->seq[plan->order[j - 1]].nblk < plan->seq[i].nblk) {
      plan->order[j] = plan->order[j - 1];
      --j;
    }
    plan->order[j] = i;
  }
  plan->total_tokens = tok;
  plan->kv_tokens = kvtok;
  plan->pooled_rows = pool;
  plan->num_segments = seg;
  plan->score_elems = score;
  kv->page_table = pr->page_table;
  kv->page_shift = page_shift;
  kv->max_pages = pr->page_table ? pr->max_pages_per_seq : 0;
  return BSLP_OK;
}

bslp_status check_params(const bslp_select_params* a, bslp::SelectArgs* out) {
  if (!a) return fail(BSLP_ERR_INVALID_ARG, "params is NULL");
  if (!std::isfinite(a->alpha) || a->alpha < 0.f)
    return fail(BSLP_ERR_INVALID_ARG, "alpha must be finite and >= 0");
  if (a->sink_blocks < 0 || a->window_blocks < 0 || a->recent_blocks < 0)
    return fail(BSLP_ERR_INVALID_ARG, "sink/window/recent block counts must be >= 0");
  if (a->mean_correction != 0 && a->mean_correction != 1)
    return fail(BSLP_ERR_INVALID_ARG, "mean_correction must be 0 or 1");
  out->alpha = a->alpha;
  out->sink = a->sink_blocks;
  out->window = a->window_blocks;
  out->recent = a->recent_blocks;
  out->correction = a->mean_correction;
  return BSLP_OK;
}

bslp_status hip_result(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSLP_OK;
  return fail(BSLP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// float32 keeps exact fp32 arithmetic on the vector ALUs; bf16 runs on the
// bf16 matrix cores; fp8 on the fp8 matrix cores with e4m3 probabilities.
hipError_t launch_attn(const bslp::Plan& plan, const bslp::KVDesc& kv, int dtype,
                       const bslp::AttnArgs& a, hipStream_t stream) {
  if (dtype == BSLP_F32) return bslp::launch_attn_valu(plan, kv, dtype, a, stream);
  if (dtype == BSLP_FP8_E4M3) return bslp::launch_attn_fp8(plan, kv, a, stream);
  return bslp::launch_attn_mfma(plan, kv, dtype, a, stream);
}

static_assert(BSLP_NOALLOC_SCRATCH_BYTES == bslp::kNoAllocScratchBytes,
              "the header states the device scratch size of the no-allocation entry point");

// Stage 3 with a caller workspace, or (noalloc) with the library's device
// scratch array in its place.
bslp_status sparse_attn(const bslp_problem* problem, const bslp_select_params* params,
                        const void* q, const void* k, const void* v, const float* kbar,
                        const float* vbar, const int32_t* cu, const int32_t* idx, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream,
                        bool noalloc) {
  const char* what = noalloc ? "bslp_sparse_prefill_attn_noalloc" : "bslp_sparse_prefill_attn";
  bslp::Plan plan;
  bslp::KVDesc kv;
  bslp::SelectArgs sa;
  bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  st = check_params(params, &sa);
  if (st != BSLP_OK) return st;
  if (plan.total_tokens == 0) return BSLP_OK;
  if (!q || !k || !v || !kbar || !vbar || !cu || !idx || !out)
    return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  int splits = bslp::attn_splits(plan, problem->dtype, problem->kv_splits);
  size_t need = bslp::attn_workspace_bytes(plan, splits);
  if (noalloc) {
    // an automatic split count falls back to no split when its partial
    // results do not fit the scratch array; a requested count does not
    if (need > bslp::kNoAllocScratchBytes && problem->kv_splits == 0 && splits > 1) {
      splits = 1;
      need = bslp::attn_workspace_bytes(plan, splits);
    }
    if (need > bslp::kNoAllocScratchBytes)
      return fail(BSLP_ERR_UNSUPPORTED,
                  std::string(what) + " needs " + std::to_string(need) +
                      " bytes of scratch, above its fixed " +
                      std::to_string(bslp::kNoAllocScratchBytes) +
                      " (pass kv_splits = 1, or use bslp_sparse_prefill_attn with a workspace)");
    const hipError_t e = bslp::noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_result(e, what);
  } else {
    if (workspace_bytes < need)
      return fail(BSLP_ERR_WORKSPACE, "workspace_bytes " + std::to_string(workspace_bytes) +
                                            " is below the " + std::to_string(need) +
                                            " bytes bslp_get_sizes reports");
    if (need > 0 && !workspace) return fail(BSLP_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 16)
      return fail(BSLP_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  bslp::AttnArgs a{q, k, v, kbar, vbar, cu, idx, out, lse, workspace,
                   problem->softmax_scale * host_scale(problem, 0), host_scale(problem, 1),
                   host_scale(problem, 2), sa.correction, 0, splits};
  return hip_result(launch_attn(plan, kv, problem->dtype, a, (hipStream_t)stream), what);
}

}  // namespace

extern "C" {

bslp_status bslp_get_sizes(const bslp_problem* problem, bslp_sizes* out) {
  bslp::Plan plan;
  bslp::KVDesc kv;
  if (!out) return fail(BSLP_ERR_INVALID_ARG, "sizes output is NULL");
  const bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  out->total_tokens = plan.total_tokens;
  out->kv_tokens = plan.kv_tokens;
  out->pooled_rows = plan.pooled_rows;
  out->score_elems = plan.score_elems;
  out->num_segments = plan.num_segments;
  out->workspace_bytes = (int64_t)bslp::attn_workspace_bytes(
      plan, bslp::attn_splits(plan, problem->dtype, problem->kv_splits));
  return BSLP_OK;
}

size_t bslp_workspace_bytes(const bslp_problem* problem) {
  bslp_sizes sz;
  if (bslp_get_sizes(problem, &sz) != BSLP_OK) return 0;
  return (size_t)sz.workspace_bytes;
}

bslp_status bslp_block_scores(const bslp_problem* problem, const void* q, const void* k,
                              const void* v, float* kbar, float* vbar, float* scores,
                              void* stream) {
  bslp::Plan plan;
  bslp::KVDesc kv;
  bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  if (plan.total_tokens == 0) return BSLP_OK;
  if (!q || !k || !v || !kbar || !vbar || !scores)
    return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  return hip_result(bslp::launch_stage1(plan, kv, problem->dtype, q, k, v, host_scale(problem, 0),
                                        host_scale(problem, 1), host_scale(problem, 2),
                                        problem->softmax_scale, kbar, vbar, scores,
                                        bslp::kStagePool | bslp::kStageScores,
                                        (hipStream_t)stream),
                    "bslp_block_scores");
}

bslp_status bslp_pool_kv(const bslp_problem* problem, const void* k, const void* v, float* kbar,
                         float* vbar, void* stream) {
  bslp::Plan plan;
  bslp::KVDesc kv;
  bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  if (plan.pooled_rows == 0) return BSLP_OK;
  if (!k || !v || !kbar || !vbar) return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  return hip_result(bslp::launch_stage1(plan, kv, problem->dtype, nullptr, k, v,
                                        host_scale(problem, 0), host_scale(problem, 1),
                                        host_scale(problem, 2), problem->softmax_scale, kbar, vbar,
                                        nullptr, bslp::kStagePool, (hipStream_t)stream),
                    "bslp_pool_kv");
}

bslp_status bslp_score_blocks(const bslp_problem* problem, const void* q, const float* kbar,
                              float* scores, void* stream) {
  bslp::Plan plan;
  bslp::KVDesc kv;
  bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  if (plan.total_tokens == 0) return BSLP_OK;
  if (!q || !kbar || !scores) return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  return hip_result(bslp::launch_stage1(plan, kv, problem->dtype, q, nullptr, nullptr,
                                        host_scale(problem, 0), host_scale(problem, 1),
                                        host_scale(problem, 2), problem->softmax_scale,
                                        const_cast<float*>(kbar), nullptr, scores,
                                        bslp::kStageScores, (hipStream_t)stream),
                    "bslp_score_blocks");
}

bslp_status bslp_select_blocks(const bslp_problem* problem, const bslp_select_params* params,
                               const void* q, const float* kbar, float* scores,
                               int32_t* counts, int32_t* cu, int32_t* idx, void* stream) {
  bslp::Plan plan;
  bslp::KVDesc kv;
  bslp::SelectArgs a;
  bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  st = check_params(params, &a);
  if (st != BSLP_OK) return st;
  if (!cu) return fail(BSLP_ERR_INVALID_ARG, "cu is NULL");
  if (plan.num_segments > 0 && (!q || !kbar || !scores || !counts || !idx))
    return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  return hip_result(bslp::launch_select(plan, a, q, kbar, problem->dtype,
                                        problem->softmax_scale * host_scale(problem, 0), scores,
                                        counts, cu, idx, (hipStream_t)stream),
                    "bslp_select_blocks");
}

bslp_status bslp_sparse_prefill_attn(const bslp_problem* problem,
                                     const bslp_select_params* params, const void* q,
                                     const void* k, const void* v, const float* kbar,
                                     const float* vbar, const int32_t* cu, const int32_t* idx,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return sparse_attn(problem, params, q, k, v, kbar, vbar, cu, idx, out, lse, workspace,
                     workspace_bytes, stream, false);
}

bslp_status bslp_sparse_prefill_attn_noalloc(const bslp_problem* problem,
                                             const bslp_select_params* params, const void* q,
                                             const void* k, const void* v, const float* kbar,
                                             const float* vbar, const int32_t* cu,
                                             const int32_t* idx, void* out, float* lse,
                                             void* stream) {
  return sparse_attn(problem, params, q, k, v, kbar, vbar, cu, idx, out, lse, nullptr, 0, stream,
                     true);
}

bslp_status bslp_dense_prefill_attn(const bslp_problem* problem, const void* q, const void* k,
                                    const void* v, void* out, float* lse, void* stream) {
  bslp::Plan plan;
  bslp::KVDesc kv;
  bslp_status st = build_plan(problem, &plan, &kv);
  if (st != BSLP_OK) return st;
  if (plan.total_tokens == 0) return BSLP_OK;
  if (!q || !k || !v || !out) return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  bslp::AttnArgs a{q, k, v, nullptr, nullptr, nullptr, nullptr, out, lse, nullptr,
                   problem->softmax_scale * host_scale(problem, 0), host_scale(problem, 1),
                   host_scale(problem, 2), 0, 1, 1};
  return hip_result(launch_attn(plan, kv, problem->dtype, a, (hipStream_t)stream),
                    "bslp_dense_prefill_attn");
}

bslp_status bslp_quantize_e4m3(int32_t src_dtype, const void* x, int64_t n, uint8_t* codes,
                               float* scale, void* stream) {
  if (src_dtype != BSLP_BF16 && src_dtype != BSLP_F32)
    return fail(BSLP_ERR_INVALID_ARG, "src_dtype must be BSLP_BF16 or BSLP_F32");
  if (n < 0) return fail(BSLP_ERR_INVALID_ARG, "n must be >= 0");
  if (!scale || (n > 0 && (!x || !codes)))
    return fail(BSLP_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codes) % 8 ||
      reinterpret_cast<uintptr_t>(scale) % 4)
    return fail(BSLP_ERR_INVALID_ARG, "x must be 16-byte, codes 8-byte, scale 4-byte aligned");
  return hip_result(bslp::launch_quantize_e4m3(src_dtype, x, n, codes, scale, (hipStream_t)stream),
                    "bslp_quantize_e4m3");
}

const char* bslp_status_string(bslp_status status) {
  switch (status) {
    case BSLP_OK: return "ok";
    case BSLP_ERR_INVALID_ARG: return "invalid argument";
    case BSLP_ERR_UNSUPPORTED: return "unsupported";
    case BSLP_ERR_HIP: return "HIP error";
    case BSLP_ERR_WORKSPACE: return "workspace";
  }
  return "unknown status";
}

const char* bslp_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
