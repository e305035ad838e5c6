// C ABI entry points: host-side validation, workspace sizing and dispatch to
// the HIP kernels.  Nothing here allocates device memory or synchronizes.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "egs_launch.h"

using egs::DecodeDims;
using egs::PrefillDims;

namespace {

thread_local std::string g_last_error;

egs_status fail(egs_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

egs_status ok() {
  return EGS_OK;
}

egs_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return EGS_OK;
  return fail(EGS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

constexpr size_t kWsAlign = 256;
size_t round_up(size_t x, size_t a) {
  return (x + a - 1) / a * a;
}

bool supported_head_dim(int d) {
  return d == 16 || d == 32 || d == 64 || d == 128;
}

egs_status check_prefill(const egs_prefill_shape* s, PrefillDims* p) {
  if (s == nullptr) return fail(EGS_EINVAL, "prefill shape is NULL");
  if (s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 || s->seq_len <= 0 ||
      s->block_size <= 0 || s->segment_size <= 0 || s->probe_len <= 0)
    return fail(EGS_EINVAL, "prefill shape has a non-positive field");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(EGS_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->seq_len % s->segment_size != 0)
    return fail(EGS_EINVAL, "seq_len (%d) is not a multiple of segment_size (%d)", s->seq_len,
                s->segment_size);
  if (s->segment_size % s->block_size != 0)
    return fail(EGS_EINVAL, "segment_size (%d) is not a multiple of block_size (%d)",
                s->segment_size, s->block_size);
  if (s->probe_len > s->segment_size)
    return fail(EGS_EINVAL, "probe_len (%d) exceeds segment_size (%d)", s->probe_len,
                s->segment_size);
  if (s->dtype != EGS_BF16 && s->dtype != EGS_F32)
    return fail(EGS_EINVAL, "unknown dtype %d", s->dtype);
  if (!(std::isfinite(s->sm_scale) && s->sm_scale >= 0.f))
    return fail(EGS_EINVAL, "sm_scale must be finite and >= 0");
  if (!supported_head_dim(s->head_dim))
    return fail(EGS_ENOTSUP, "head_dim %d not supported (16, 32, 64, 128)", s->head_dim);
  if (s->block_size % 16 != 0 || s->block_size > 256)
    return fail(EGS_ENOTSUP, "block_size %d not supported (multiple of 16, <= 256)",
                s->block_size);
  const long long CB = s->seq_len / s->block_size;
  if (CB > 16384) return fail(EGS_ENOTSUP, "more than 16384 key blocks (%lld)", CB);
  const long long elems = (long long)s->n_q_heads * s->seq_len * s->head_dim;
  if (elems > (1LL << 40)) return fail(EGS_ENOTSUP, "tensor too large");
  p->Hq = s->n_q_heads;
  p->Hkv = s->n_kv_heads;
  p->r = s->n_q_heads / s->n_kv_heads;
  p->D = s->head_dim;
  p->N = s->seq_len;
  p->LB = s->block_size;
  p->LS = s->segment_size;
  p->P = s->probe_len;
  p->CS = s->seq_len / s->segment_size;
  p->CB = (int)CB;
  p->dtype = s->dtype;
  p->sm_scale = s->sm_scale > 0.f ? s->sm_scale : 1.0f / std::sqrt((float)s->head_dim);
  return EGS_OK;
}

egs_status need(const void* ptr, const char* name, size_t align) {
  if (ptr == nullptr) return fail(EGS_EINVAL, "%s is NULL", name);
  if (!aligned(ptr, align)) return fail(EGS_EINVAL, "%s is not %zu-byte aligned", name, align);
  return EGS_OK;
}

egs_status check_decode(const egs_decode_shape* s, DecodeDims* p) {
  if (s == nullptr) return fail(EGS_EINVAL, "decode shape is NULL");
  if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 ||
      s->cache_len <= 0 || s->n_obs <= 0)
    return fail(EGS_EINVAL, "decode shape has a non-positive field");
  if (s->n_sink < 0 || s->n_recent < 0 || s->n_keep < 0)
    return fail(EGS_EINVAL, "n_sink, n_recent and n_keep must be >= 0");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(EGS_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->n_obs > s->cache_len)
    return fail(EGS_EINVAL, "n_obs (%d) exceeds cache_len (%d)", s->n_obs, s->cache_len);
  if (!(std::isfinite(s->sm_scale) && s->sm_scale >= 0.f))
    return fail(EGS_EINVAL, "sm_scale must be finite and >= 0");
  if (s->dtype != EGS_BF16 && s->dtype != EGS_F32)
    return fail(EGS_EINVAL, "unknown dtype %d", s->dtype);
  if (s->dtype != EGS_BF16) return fail(EGS_ENOTSUP, "decode retention supports bf16 only");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(EGS_ENOTSUP, "decode head_dim %d not supported (64, 128)", s->head_dim);
  if (s->cache_len > (1 << 26)) return fail(EGS_ENOTSUP, "cache_len above 2^26");
  if (s->n_q_heads / s->n_kv_heads > 16)
    return fail(EGS_ENOTSUP, "more than 16 query heads per KV head");
  if (s->n_obs > 128) return fail(EGS_ENOTSUP, "n_obs above 128 is not supported");
  p->B = s->batch;
  p->Hq = s->n_q_heads;
  p->Hkv = s->n_kv_heads;
  p->r = s->n_q_heads / s->n_kv_heads;
  p->D = s->head_dim;
  p->L = s->cache_len;
  p->W = s->n_obs;
  p->n_sink = s->n_sink;
  p->n_recent = s->n_recent;
  p->n_keep = s->n_keep;
  const long long tot = (long long)s->n_sink + s->n_recent + s->n_keep;
  p->n_total = tot >= s->cache_len ? s->cache_len : (int)tot;
  p->Lk = p->L;
  p->dtype = s->dtype;
  p->sm_scale = s->sm_scale > 0.f ? s->sm_scale : 1.0f / std::sqrt((float)s->head_dim);
  return EGS_OK;
}

}  // namespace

extern "C" {

int32_t egs_abi_version(void) {
  return EGS_ABI_VERSION;
}

const char* egs_status_string(egs_status st) {
  switch (st) {
    case EGS_OK: return "EGS_OK";
    case EGS_EINVAL: return "EGS_EINVAL: invalid argument";
    case EGS_ENOTSUP: return "EGS_ENOTSUP: unsupported shape or mode";
    case EGS_EWORKSPACE: return "EGS_EWORKSPACE: workspace too small";
    case EGS_EHIP: return "EGS_EHIP: HIP launch failure";
  }
  return "unknown egs_status";
}

const char* egs_last_error(void) {
  return g_last_error.c_str();
}

size_t egs_entropy_score_workspace(const egs_prefill_shape* shape) {
  PrefillDims p;
  if (check_prefill(shape, &p) != EGS_OK) return 0;
  return egs::score_workspace_bytes(p);
}

// argument checks shared by egs_entropy_score and its static-scratch form;
// a Renyi order of 1 is Shannon
static egs_status check_score(const egs_prefill_shape* shape, int32_t pool_kind,
                              int32_t entropy_kind, float renyi_alpha, const void* q,
                              const void* k, const float* block_scores, const float* entropy,
                              PrefillDims* p, int* kind) {
  egs_status st = check_prefill(shape, p);
  if (st != EGS_OK) return st;
  if (pool_kind != EGS_POOL_MEAN_PROBE && pool_kind != EGS_POOL_MAXMIN)
    return fail(EGS_EINVAL, "unknown pool_kind %d", pool_kind);
  *kind = entropy_kind;
  if (*kind != EGS_SHANNON && *kind != EGS_RENYI)
    return fail(EGS_EINVAL, "unknown entropy_kind %d", entropy_kind);
  if (*kind == EGS_RENYI) {
    if (!(std::isfinite(renyi_alpha) && renyi_alpha > 0.f))
      return fail(EGS_EINVAL, "renyi_alpha must be finite and > 0");
    if (renyi_alpha == 1.0f) *kind = EGS_SHANNON;
  }
  if ((st = need(q, "q", 16)) != EGS_OK) return st;
  if ((st = need(k, "k", 16)) != EGS_OK) return st;
  if ((st = need(block_scores, "block_scores", 4)) != EGS_OK) return st;
  return need(entropy, "entropy", 4);
}

egs_status egs_entropy_score(const egs_prefill_shape* shape, int32_t pool_kind,
                             int32_t entropy_kind, float renyi_alpha, const void* q,
                             const void* k, float* block_scores, float* entropy,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  PrefillDims p;
  int kind;
  egs_status st = check_score(shape, pool_kind, entropy_kind, renyi_alpha, q, k, block_scores,
                              entropy, &p, &kind);
  if (st != EGS_OK) return st;
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::score_workspace_bytes(p);
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  if (pool_kind == EGS_POOL_MAXMIN)
    return hip_status(egs::launch_entropy_score_maxmin(p, q, k, kind, renyi_alpha, block_scores,
                                                       entropy, workspace, stream),
                      "entropy_score (max/min) launch");
  return hip_status(egs::launch_entropy_score(p, q, k, kind, renyi_alpha, block_scores, entropy,
                                              workspace, stream),
                    "entropy_score launch");
}

egs_status egs_entropy_score_static(const egs_prefill_shape* shape, int32_t pool_kind,
                                    int32_t entropy_kind, float renyi_alpha, const void* q,
                                    const void* k, float* block_scores, float* entropy,
                                    hipStream_t stream) {
  PrefillDims p;
  int kind;
  egs_status st = check_score(shape, pool_kind, entropy_kind, renyi_alpha, q, k, block_scores,
                              entropy, &p, &kind);
  if (st != EGS_OK) return st;
  const size_t wsb = egs::score_workspace_bytes(p);
  if (wsb > EGS_STATIC_SCRATCH_BYTES)
    return fail(EGS_EWORKSPACE, "the shape needs %zu bytes of scratch, above the static %zu",
                wsb, (size_t)EGS_STATIC_SCRATCH_BYTES);
  return hip_status(egs::launch_entropy_score_static(p, pool_kind == EGS_POOL_MAXMIN, q, k,
                                                     kind, renyi_alpha, block_scores, entropy,
                                                     stream),
                    "entropy_score (static scratch) launch");
}

// budget policy checks shared by egs_allocate_budget and egs_score_select
static egs_status check_policy(const egs_budget_policy* policy) {
  if (policy == nullptr) return fail(EGS_EINVAL, "policy is NULL");
  const egs_budget_policy& pol = *policy;
  if (pol.mode < EGS_BUDGET_FIXED || pol.mode > EGS_BUDGET_ALG3)
    return fail(EGS_EINVAL, "unknown budget mode %d", pol.mode);
  if (!std::isfinite(pol.entropy_threshold))
    return fail(EGS_EINVAL, "entropy_threshold must be finite");
  switch (pol.mode) {
    case EGS_BUDGET_FIXED:
      if (!(std::isfinite(pol.frac) && pol.frac >= 0.0)) return fail(EGS_EINVAL, "frac must be >= 0");
      break;
    case EGS_BUDGET_TWO_LEVEL:
      if (!(std::isfinite(pol.frac_rigid) && pol.frac_rigid >= 0.0 &&
            std::isfinite(pol.frac_dynamic) && pol.frac_dynamic >= 0.0))
        return fail(EGS_EINVAL, "frac_rigid and frac_dynamic must be >= 0");
      break;
    case EGS_BUDGET_PROPORTIONAL:
      if (!(std::isfinite(pol.frac_min) && std::isfinite(pol.frac_max) && pol.frac_min >= 0.0 &&
            pol.frac_max >= pol.frac_min))
        return fail(EGS_EINVAL, "need 0 <= frac_min <= frac_max");
      break;
    case EGS_BUDGET_ALG3:
      if (!(std::isfinite(pol.base_tokens) && pol.base_tokens > 0.0 &&
            std::isfinite(pol.alg3_alpha) && std::isfinite(pol.alg3_delta_t) &&
            pol.entropy_threshold > 0.0))
        return fail(EGS_EINVAL, "ALG3 needs base_tokens > 0, finite alpha / delta_t, e_t > 0");
      break;
  }
  return EGS_OK;
}

egs_status egs_allocate_budget(const egs_prefill_shape* shape, const egs_budget_policy* policy,
                               const float* entropy, int8_t* head_is_rigid, int32_t* budget,
                               hipStream_t stream) {
  PrefillDims p;
  egs_status st = check_prefill(shape, &p);
  if (st != EGS_OK) return st;
  if ((st = check_policy(policy)) != EGS_OK) return st;
  if ((st = need(entropy, "entropy", 4)) != EGS_OK) return st;
  if ((st = need(head_is_rigid, "head_is_rigid", 1)) != EGS_OK) return st;
  if ((st = need(budget, "budget", 4)) != EGS_OK) return st;
  return hip_status(egs::launch_budget(p, *policy, entropy, head_is_rigid, budget, stream),
                    "budget launch");
}

egs_status egs_score_select(const egs_prefill_shape* shape, int32_t pool_kind,
                            int32_t entropy_kind, float renyi_alpha,
                            const egs_budget_policy* policy, const void* q, const void* k,
                            int32_t k_max, float* block_scores, float* entropy,
                            int8_t* head_is_rigid, int32_t* budget, int32_t* block_idx,
                            int32_t* block_cnt, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  PrefillDims p;
  int kind;
  egs_status st = check_score(shape, pool_kind, entropy_kind, renyi_alpha, q, k, block_scores,
                              entropy, &p, &kind);
  if (st != EGS_OK) return st;
  if ((st = check_policy(policy)) != EGS_OK) return st;
  if (k_max < 1 || k_max > p.CB)
    return fail(EGS_EINVAL, "k_max (%d) must be in [1, C_B = %d]", k_max, p.CB);
  if ((st = need(head_is_rigid, "head_is_rigid", 1)) != EGS_OK) return st;
  if ((st = need(budget, "budget", 4)) != EGS_OK) return st;
  if ((st = need(block_idx, "block_idx", 4)) != EGS_OK) return st;
  if ((st = need(block_cnt, "block_cnt", 4)) != EGS_OK) return st;
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::score_workspace_bytes(p);
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  hipError_t e;
  egs::EntropyParts parts{nullptr, 0, 1};
  if (pool_kind == EGS_POOL_MAXMIN) {
    e = egs::launch_entropy_score_maxmin(p, q, k, kind, renyi_alpha, block_scores, entropy,
                                         workspace, stream);
  } else {
    e = egs::launch_entropy_score(p, q, k, kind, renyi_alpha, block_scores, nullptr, workspace,
                                  stream);
    parts = egs::entropy_parts(p, workspace);
  }
  if (e != hipSuccess) return hip_status(e, "score_select scoring launch");
  return hip_status(egs::launch_budget_select(p, *policy, parts, kind, renyi_alpha, entropy,
                                              block_scores, k_max, head_is_rigid, budget,
                                              block_idx, block_cnt, stream),
                    "score_select budget / select launch");
}

egs_status egs_select_blocks(const egs_prefill_shape* shape, const float* block_scores,
                             const int32_t* budget, int32_t k_max, int32_t* block_idx,
                             int32_t* block_cnt, hipStream_t stream) {
  PrefillDims p;
  egs_status st = check_prefill(shape, &p);
  if (st != EGS_OK) return st;
  if (k_max < 1 || k_max > p.CB)
    return fail(EGS_EINVAL, "k_max (%d) must be in [1, C_B = %d]", k_max, p.CB);
  if ((st = need(block_scores, "block_scores", 4)) != EGS_OK) return st;
  if ((st = need(budget, "budget", 4)) != EGS_OK) return st;
  if ((st = need(block_idx, "block_idx", 4)) != EGS_OK) return st;
  if ((st = need(block_cnt, "block_cnt", 4)) != EGS_OK) return st;
  return hip_status(egs::launch_select(p, block_scores, budget, k_max, block_idx, block_cnt,
                                       stream),
                    "select launch");
}

size_t egs_sparse_prefill_attn_workspace(const egs_prefill_shape* shape) {
  PrefillDims p;
  if (check_prefill(shape, &p) != EGS_OK) return 0;
  return round_up(egs::sparse_attn_workspace_bytes(p), kWsAlign);
}

egs_status egs_sparse_prefill_attn(const egs_prefill_shape* shape, const void* q, const void* k,
                                   const void* v, const int32_t* block_idx,
                                   const int32_t* block_cnt, int32_t k_max, void* out,
                                   float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  PrefillDims p;
  egs_status st = check_prefill(shape, &p);
  if (st != EGS_OK) return st;
  if (k_max < 1 || k_max > p.CB)
    return fail(EGS_EINVAL, "k_max (%d) must be in [1, C_B = %d]", k_max, p.CB);
  if ((st = need(q, "q", 16)) != EGS_OK) return st;
  if ((st = need(k, "k", 16)) != EGS_OK) return st;
  if ((st = need(v, "v", 16)) != EGS_OK) return st;
  if ((st = need(out, "out", 16)) != EGS_OK) return st;
  if ((st = need(block_idx, "block_idx", 4)) != EGS_OK) return st;
  if ((st = need(block_cnt, "block_cnt", 4)) != EGS_OK) return st;
  if (lse != nullptr && !aligned(lse, 4)) return fail(EGS_EINVAL, "lse is not 4-byte aligned");
  if (out == q || out == k || out == v) return fail(EGS_EINVAL, "out aliases an input");
  const size_t wsb = egs::sparse_attn_workspace_bytes(p);
  if (wsb > 0) {
    if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
    if (workspace_bytes < wsb)
      return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                  workspace_bytes, wsb);
  }
  return hip_status(egs::launch_sparse_attn(p, q, k, v, block_idx, block_cnt, k_max, out, lse,
                                            workspace, stream),
                    "sparse_attn launch");
}

int32_t egs_kv_retain_total(const egs_decode_shape* shape) {
  DecodeDims p;
  if (check_decode(shape, &p) != EGS_OK) return -1;
  return p.n_total;
}

size_t egs_kv_retain_workspace(const egs_decode_shape* shape) {
  DecodeDims p;
  if (check_decode(shape, &p) != EGS_OK) return 0;
  return egs::retain_workspace_bytes(p);
}

// retention parameters, normalised (Renyi order 1 is Shannon)
static egs_status check_retain_params(const egs_retain_params* params, egs_retain_params* out) {
  if (params == nullptr) return fail(EGS_EINVAL, "params is NULL");
  egs_retain_params prm = *params;
  if (prm.raw_logit_mode != 0 && prm.raw_logit_mode != 1)
    return fail(EGS_EINVAL, "raw_logit_mode must be 0 or 1");
  if (!prm.raw_logit_mode) {
    if (prm.entropy_kind != EGS_SHANNON && prm.entropy_kind != EGS_RENYI)
      return fail(EGS_EINVAL, "unknown entropy_kind %d", prm.entropy_kind);
    if (prm.entropy_kind == EGS_RENYI) {
      if (!(std::isfinite(prm.renyi_alpha) && prm.renyi_alpha > 0.f))
        return fail(EGS_EINVAL, "renyi_alpha must be finite and > 0");
      if (prm.renyi_alpha == 1.0f) prm.entropy_kind = EGS_SHANNON;
    }
    if (!(prm.zeta > 0.0 && prm.zeta <= 1.0)) return fail(EGS_EINVAL, "zeta must be in (0, 1]");
    if (!(std::isfinite(prm.tau) && prm.tau > 0.0)) return fail(EGS_EINVAL, "tau must be > 0");
    if (!(prm.info_alpha >= 0.0 && prm.info_alpha <= 1.0))
      return fail(EGS_EINVAL, "info_alpha must be in [0, 1]");
  }
  *out = prm;
  return EGS_OK;
}

egs_status egs_kv_retain(const egs_decode_shape* shape, const egs_retain_params* params,
                         const void* q_obs, const void* k_cache, const void* v_cache,
                         const float* token_entropy, int32_t* keep_idx, void* k_out,
                         void* v_out, float* head_entropy, float* scores, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  DecodeDims p;
  egs_status st = check_decode(shape, &p);
  if (st != EGS_OK) return st;
  egs_retain_params prm;
  if ((st = check_retain_params(params, &prm)) != EGS_OK) return st;
  if ((st = need(q_obs, "q_obs", 16)) != EGS_OK) return st;
  if ((st = need(k_cache, "k_cache", 16)) != EGS_OK) return st;
  if ((st = need(keep_idx, "keep_idx", 4)) != EGS_OK) return st;
  if ((k_out == nullptr) != (v_out == nullptr))
    return fail(EGS_EINVAL, "k_out and v_out must both be given or both be NULL");
  if (k_out != nullptr) {
    if ((st = need(v_cache, "v_cache", 16)) != EGS_OK) return st;
    if ((st = need(k_out, "k_out", 16)) != EGS_OK) return st;
    if ((st = need(v_out, "v_out", 16)) != EGS_OK) return st;
  }
  if (token_entropy != nullptr && !aligned(token_entropy, 4))
    return fail(EGS_EINVAL, "token_entropy is not 4-byte aligned");
  if (head_entropy != nullptr && !aligned(head_entropy, 4))
    return fail(EGS_EINVAL, "head_entropy is not 4-byte aligned");
  if (scores != nullptr && !aligned(scores, 4))
    return fail(EGS_EINVAL, "scores is not 4-byte aligned");
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::retain_workspace_bytes(p);
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  return hip_status(egs::launch_kv_retain(p, prm, q_obs, k_cache, v_cache, token_entropy,
                                          keep_idx, k_out, v_out, head_entropy, scores,
                                          workspace, stream),
                    "kv_retain launch");
}

size_t egs_sparse_decode_attn_workspace(const egs_decode_shape* shape, int32_t n_total) {
  DecodeDims p;
  if (check_decode(shape, &p) != EGS_OK || n_total < 1) return 0;
  return egs::decode_attn_workspace_bytes(p, n_total);
}

egs_status egs_sparse_decode_attn(const egs_decode_shape* shape, const void* q_new,
                                  const void* k_kept, const void* v_kept, int32_t n_total,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  DecodeDims p;
  egs_status st = check_decode(shape, &p);
  if (st != EGS_OK) return st;
  if (n_total < 1 || n_total > p.L)
    return fail(EGS_EINVAL, "n_total (%d) must be in [1, cache_len = %d]", n_total, p.L);
  if ((st = need(q_new, "q_new", 16)) != EGS_OK) return st;
  if ((st = need(k_kept, "k_kept", 16)) != EGS_OK) return st;
  if ((st = need(v_kept, "v_kept", 16)) != EGS_OK) return st;
  if ((st = need(out, "out", 16)) != EGS_OK) return st;
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::decode_attn_workspace_bytes(p, n_total);
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  return hip_status(egs::launch_decode_attn(p, q_new, k_kept, v_kept, n_total, n_total, out,
                                            workspace, stream),
                    "decode_attn launch");
}

static egs_status check_prune(const egs_decode_shape* shape, int32_t n_chunks, DecodeDims* p) {
  egs_status st = check_decode(shape, p);
  if (st != EGS_OK) return st;
  if (p->B != 1) return fail(EGS_EINVAL, "chunk pruning takes one prompt (batch 1)");
  if (n_chunks < 1 || n_chunks > egs::kMaxPruneChunks)
    return fail(EGS_EINVAL, "n_chunks must be in [1, %d]", egs::kMaxPruneChunks);
  if (p->Hq * p->W > egs::kMaxPruneRows)
    return fail(EGS_ENOTSUP, "more than %d observer rows", egs::kMaxPruneRows);
  return EGS_OK;
}

size_t egs_chunk_prune_workspace(const egs_decode_shape* shape, int32_t n_chunks) {
  DecodeDims p;
  if (check_prune(shape, n_chunks, &p) != EGS_OK) return 0;
  return egs::prune_layout(p, n_chunks).total;
}

egs_status egs_chunk_prune(const egs_decode_shape* shape, const egs_prune_params* params,
                           const void* q_obs, const void* k, const int32_t* chunk_bounds,
                           int32_t n_chunks, int8_t* removed, int32_t* removed_tokens,
                           float* priority, float* row_mass, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  DecodeDims p;
  egs_status st = check_prune(shape, n_chunks, &p);
  if (st != EGS_OK) return st;
  if (params == nullptr) return fail(EGS_EINVAL, "params is NULL");
  const egs_prune_params& q = *params;
  if (!(std::isfinite(q.eps_s) && q.eps_s > 0.0)) return fail(EGS_EINVAL, "eps_s must be > 0");
  if (!(std::isfinite(q.lambda) && q.lambda >= 0.0))
    return fail(EGS_EINVAL, "lambda must be >= 0");
  if (!(std::isfinite(q.eps) && q.eps >= 0.0)) return fail(EGS_EINVAL, "eps must be >= 0");
  if (q.m0 < 0 || q.target < 0) return fail(EGS_EINVAL, "m0 and target must be >= 0");
  if (!(q.zeta > 0.0 && q.zeta <= 1.0)) return fail(EGS_EINVAL, "zeta must be in (0, 1]");
  if (!(std::isfinite(q.tau) && q.tau > 0.0)) return fail(EGS_EINVAL, "tau must be > 0");
  if ((st = need(chunk_bounds, "chunk_bounds", 4)) != EGS_OK) return st;
  if ((st = need(q_obs, "q_obs", 16)) != EGS_OK) return st;
  if ((st = need(k, "k", 16)) != EGS_OK) return st;
  if ((st = need(removed, "removed", 1)) != EGS_OK) return st;
  if ((st = need(removed_tokens, "removed_tokens", 4)) != EGS_OK) return st;
  if ((st = need(priority, "priority", 4)) != EGS_OK) return st;
  if (row_mass != nullptr && !aligned(row_mass, 4))
    return fail(EGS_EINVAL, "row_mass is not 4-byte aligned");
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::prune_layout(p, n_chunks).total;
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  egs::PruneArgs a;
  a.k = n_chunks;
  a.zeta = q.zeta;
  a.tau = q.tau;
  a.eps_s = (float)q.eps_s;
  a.lam = (float)q.lambda;
  a.eps = (float)q.eps;
  a.m0 = q.m0;
  a.target = q.target;
  return hip_status(egs::launch_chunk_prune(p, a, q_obs, k, chunk_bounds, removed,
                                            removed_tokens, priority, row_mass, workspace,
                                            stream),
                    "chunk_prune launch");
}

size_t egs_prune_certificate_workspace(int32_t n_chunks) {
  if (n_chunks < 1 || n_chunks > egs::kMaxPruneChunks) return 0;
  return egs::certificate_workspace_bytes(n_chunks);
}

egs_status egs_prune_certificate(const int32_t* chunk_bounds, int32_t n_chunks, int32_t n_rows,
                                 const float* row_mass, const float* row_price, double eps,
                                 int32_t m0, double t, double* certificate, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (n_chunks < 1 || n_chunks > egs::kMaxPruneChunks)
    return fail(EGS_EINVAL, "n_chunks must be in [1, %d]", egs::kMaxPruneChunks);
  if (n_rows < 1 || n_rows > egs::kMaxPruneRows)
    return fail(EGS_EINVAL, "n_rows must be in [1, %d]", egs::kMaxPruneRows);
  if (!(std::isfinite(eps) && eps >= 0.0)) return fail(EGS_EINVAL, "eps must be >= 0");
  if (!(std::isfinite(t) && t >= 0.0)) return fail(EGS_EINVAL, "t must be >= 0");
  if (m0 < 0) return fail(EGS_EINVAL, "m0 must be >= 0");
  egs_status st;
  if ((st = need(chunk_bounds, "chunk_bounds", 4)) != EGS_OK) return st;
  if ((st = need(row_mass, "row_mass", 4)) != EGS_OK) return st;
  if ((st = need(row_price, "row_price", 4)) != EGS_OK) return st;
  if ((st = need(certificate, "certificate", 8)) != EGS_OK) return st;
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::certificate_workspace_bytes(n_chunks);
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  return hip_status(egs::launch_prune_certificate(chunk_bounds, n_chunks, n_rows, row_mass,
                                                  row_price, eps, m0, t, certificate, workspace,
                                                  stream),
                    "prune_certificate launch");
}

size_t egs_latent_decode_workspace(const egs_decode_shape* shape) {
  DecodeDims p;
  if (check_decode(shape, &p) != EGS_OK) return 0;
  return egs::latent_layout(p).total;
}

egs_status egs_latent_decode_step(const egs_decode_shape* shape, const egs_retain_params* params,
                                  egs_latent_state* state, const void* q_new, const void* k_new,
                                  const void* v_new, void* q_window, void* k_cache,
                                  void* v_cache, void* out, int32_t* keep_idx, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  DecodeDims p;   // p.L = the capacity of the cache rows
  egs_status st = check_decode(shape, &p);
  if (st != EGS_OK) return st;
  egs_retain_params prm;
  if ((st = check_retain_params(params, &prm)) != EGS_OK) return st;
  if (state == nullptr) return fail(EGS_EINVAL, "state is NULL");
  const int cap = p.L, len = state->length;
  if (len < p.W || len + 1 > cap)
    return fail(EGS_EINVAL, "length (%d) must be in [n_obs = %d, capacity - 1 = %d]", len, p.W,
                cap - 1);
  if (state->generated < 0 || state->n_delay < 0)
    return fail(EGS_EINVAL, "generated and n_delay must be >= 0");
  if (state->interval < 0 || (state->interval > 0 && state->interval < p.W))
    return fail(EGS_EINVAL, "interval must be 0 or >= n_obs (%d)", p.W);
  if ((st = need(q_new, "q_new", 16)) != EGS_OK) return st;
  if ((st = need(k_new, "k_new", 16)) != EGS_OK) return st;
  if ((st = need(v_new, "v_new", 16)) != EGS_OK) return st;
  if ((st = need(q_window, "q_window", 16)) != EGS_OK) return st;
  if ((st = need(k_cache, "k_cache", 16)) != EGS_OK) return st;
  if ((st = need(v_cache, "v_cache", 16)) != EGS_OK) return st;
  if ((st = need(out, "out", 16)) != EGS_OK) return st;
  if (keep_idx != nullptr && !aligned(keep_idx, 4))
    return fail(EGS_EINVAL, "keep_idx is not 4-byte aligned");
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const egs::LatentLayout ly = egs::latent_layout(p);
  if (workspace_bytes < ly.total)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, ly.total);
  char* w = static_cast<char*>(workspace);
  hipError_t e = egs::launch_latent_append(p, q_new, k_new, v_new, q_window, k_cache, v_cache,
                                           len, cap, stream);
  if (e != hipSuccess) return hip_status(e, "latent append launch");
  const int n = len + 1;
  if (egs::decode_attn_workspace_bytes(p, n) > ly.retain - ly.attn)
    return fail(EGS_EWORKSPACE, "internal: decode partials for %d entries exceed their region", n);
  e = egs::launch_decode_attn(p, q_new, k_cache, v_cache, n, cap, out, w + ly.attn, stream);
  if (e != hipSuccess) return hip_status(e, "latent decode attention launch");
  const int gen = state->generated + 1;
  const bool due = gen == state->n_delay ||
                   (state->interval > 0 && gen > state->n_delay &&
                    (gen - state->n_delay) % state->interval == 0);
  state->generated = gen;
  state->length = n;
  state->compressed = 0;
  if (due) {
    DecodeDims pr = p;
    pr.L = n;
    pr.Lk = cap;
    const long long tot = (long long)p.n_sink + p.n_recent + p.n_keep;
    pr.n_total = tot >= n ? n : (int)tot;
    int32_t* keep = keep_idx != nullptr ? keep_idx : reinterpret_cast<int32_t*>(w + ly.keep);
    e = egs::launch_kv_retain(pr, prm, q_window, k_cache, v_cache, nullptr, keep, w + ly.ks,
                              w + ly.vs, nullptr, nullptr, w + ly.retain, stream);
    if (e != hipSuccess) return hip_status(e, "latent retention launch");
    e = egs::launch_copy_rows(pr, w + ly.ks, w + ly.vs, pr.n_total, cap, k_cache, v_cache,
                              stream);
    if (e != hipSuccess) return hip_status(e, "latent compaction launch");
    state->length = pr.n_total;
    state->compressed = 1;
  }
  return EGS_OK;
}

// page-level retention: shape checks shared by the queries and the call
static egs_status check_pages(const egs_decode_shape* shape, int32_t page_size,
                              int32_t n_keep_pages, int32_t mode, DecodeDims* p,
                              egs::PageDims* q) {
  egs_status st = check_decode(shape, p);
  if (st != EGS_OK) return st;
  if (page_size < 1) return fail(EGS_EINVAL, "page_size must be >= 1");
  if (n_keep_pages < 0) return fail(EGS_EINVAL, "n_keep_pages must be >= 0");
  if (mode != EGS_PAGE_GROUP && mode != EGS_PAGE_LAYER_UNION && mode != EGS_PAGE_HEAD_UNION)
    return fail(EGS_EINVAL, "unknown page mode %d", mode);
  if ((p->L + (long long)page_size - 1) / page_size > egs::kMaxPages)
    return fail(EGS_ENOTSUP, "more than %d pages", egs::kMaxPages);
  *q = egs::page_dims(*p, page_size, n_keep_pages, mode);
  return EGS_OK;
}

int32_t egs_page_retain_capacity(const egs_decode_shape* shape, int32_t page_size,
                                 int32_t n_keep_pages, int32_t mode) {
  DecodeDims p;
  egs::PageDims q;
  if (check_pages(shape, page_size, n_keep_pages, mode, &p, &q) != EGS_OK) return -1;
  return q.cap;
}

size_t egs_page_retain_workspace(const egs_decode_shape* shape, int32_t page_size,
                                 int32_t n_keep_pages, int32_t mode) {
  DecodeDims p;
  egs::PageDims q;
  if (check_pages(shape, page_size, n_keep_pages, mode, &p, &q) != EGS_OK) return 0;
  return egs::page_retain_workspace_bytes(p, q);
}

egs_status egs_page_retain(const egs_decode_shape* shape, int32_t page_size,
                           int32_t n_keep_pages, int32_t mode, const float* token_scores,
                           int32_t* page_idx, int32_t* page_cnt, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  DecodeDims p;
  egs::PageDims q;
  egs_status st = check_pages(shape, page_size, n_keep_pages, mode, &p, &q);
  if (st != EGS_OK) return st;
  if ((st = need(token_scores, "token_scores", 4)) != EGS_OK) return st;
  if ((st = need(page_idx, "page_idx", 4)) != EGS_OK) return st;
  if ((st = need(page_cnt, "page_cnt", 4)) != EGS_OK) return st;
  if ((st = need(workspace, "workspace", kWsAlign)) != EGS_OK) return st;
  const size_t wsb = egs::page_retain_workspace_bytes(p, q);
  if (workspace_bytes < wsb)
    return fail(EGS_EWORKSPACE, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, wsb);
  return hip_status(egs::launch_page_retain(p, q, token_scores, page_idx, page_cnt, workspace,
                                            stream),
                    "page_retain launch");
}

}  // extern "C"
