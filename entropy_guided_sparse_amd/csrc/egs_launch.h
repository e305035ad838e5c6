// Host-side launcher interface between the C ABI (egs_api.cpp) and the HIP
// kernels.  Shapes reaching these functions have already been validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/egs.h"

namespace egs {

struct PrefillDims {
  int Hq, Hkv, r, D, N, LB, LS, P, CS, CB;
  int dtype;         // egs_dtype
  float sm_scale;    // resolved (never 0)
};

struct DecodeDims {
  int B, Hq, Hkv, r, D, L, W, n_sink, n_recent, n_keep, n_total;
  int Lk;   // cache row stride in entries between (batch, KV group) rows (>= L)
  int dtype;
  float sm_scale;
};

// Page-level retention (retain.hip): NP pages of S tokens, X members (KV
// groups or query heads), Y output sets of m members each; ps sink pages
// [0, ps) and recent pages [pr, NP) are forced; ntl pages per member, at most
// cap per output set.
struct PageDims {
  int S, K, mode, NP, X, Y, m, ps, pr, ntl, cap;
};
PageDims page_dims(const DecodeDims& p, int S, int K, int mode);
size_t page_retain_workspace_bytes(const DecodeDims& p, const PageDims& q);
hipError_t launch_page_retain(const DecodeDims& p, const PageDims& q, const float* scores,
                              int32_t* page_idx, int32_t* page_cnt, void* ws, hipStream_t st);
constexpr int kMaxPages = 262144;

// Chunk pruning (retain.hip) of one prompt: p.L = T, p.W observers.
struct PruneArgs {
  int k;            // chunks
  double zeta, tau;
  float eps_s, lam, eps;
  int m0, target;
};
struct PruneLayout {
  size_t retain, cid, bounds, bounds_ok, segb, stats, mtab, seg_v, seg_m, total;
};
constexpr int kMaxPruneChunks = 4096;
constexpr int kMaxPruneRows = 8192;
PruneLayout prune_layout(const DecodeDims& p, int k);
size_t certificate_workspace_bytes(int k);
hipError_t launch_prune_certificate(const int32_t* bounds, int k, int R, const float* m,
                                    const float* y, double eps, int m0, double t, double* out,
                                    void* workspace, hipStream_t st);
hipError_t launch_chunk_prune(const DecodeDims& p, const PruneArgs& a, const void* q_obs,
                              const void* k, const int32_t* bounds, int8_t* removed,
                              int32_t* removed_tokens, float* prio, float* row_mass, void* workspace,
                              hipStream_t st);

// Latent decoding (retain.hip): workspace of one step for a cache of p.L
// entries (attention, retention, keep list, gathered K / V), the append of a
// generated token and the copy of kept rows back into the cache.
struct LatentLayout {
  size_t attn, retain, keep, ks, vs, total;
  int ntot_max;
};
LatentLayout latent_layout(const DecodeDims& p);
size_t retain_workspace_bytes(const DecodeDims& p);
hipError_t launch_latent_append(const DecodeDims& p, const void* q_new, const void* k_new,
                                const void* v_new, void* q_win, void* k_cache, void* v_cache,
                                int pos, int ldk, hipStream_t st);
hipError_t launch_copy_rows(const DecodeDims& p, const void* sk, const void* sv, int n, int ldk,
                            void* dk, void* dv, hipStream_t st);

// K1 + K2: key-block means (a bf16 hi/lo pair), probe observation rows and
// per-(head, segment) entropy.  Workspace layout is owned by score.hip.
size_t score_workspace_bytes(const PrefillDims& p);
hipError_t launch_entropy_score(const PrefillDims& p, const void* q, const void* k, int kind,
                                float alpha, float* scores, float* entropy, void* ws,
                                hipStream_t st);
// egs_entropy_score on the library's static device scratch
// (EGS_STATIC_SCRATCH_BYTES per GPU; the caller has checked the size)
hipError_t launch_entropy_score_static(const PrefillDims& p, bool maxmin, const void* q,
                                       const void* k, int kind, float alpha, float* scores,
                                       float* entropy, hipStream_t st);
// With entropy == nullptr, launch_entropy_score stops after the mass pass;
// the per-(head, segment, piece) entropy partial sums are then in the
// workspace at entropy_parts(p, ws).part, [Hq, C_S, npc] floats, piece c of
// segment s covering blocks c * pc .. (the first ceil(C_B(s) / pc) count).
struct EntropyParts {
  const float* part;
  int npc, pc;
};
EntropyParts entropy_parts(const PrefillDims& p, const void* ws);
// The same outputs from the max / min representatives (maxmin.hip); its
// workspace need is included in score_workspace_bytes.
size_t maxmin_workspace_bytes(const PrefillDims& p);
hipError_t launch_entropy_score_maxmin(const PrefillDims& p, const void* q, const void* k,
                                       int kind, float alpha, float* scores, float* entropy,
                                       void* ws, hipStream_t st);
// K3: head classes and budgets (float64 arithmetic).
hipError_t launch_budget(const PrefillDims& p, const egs_budget_policy& pol,
                         const float* entropy, int8_t* rigid, int32_t* budget,
                         hipStream_t st);
// K4: top-k block lists.
hipError_t launch_select(const PrefillDims& p, const float* scores,
                         const int32_t* budget, int k_max, int32_t* idx,
                         int32_t* cnt, hipStream_t st);
// K3 + K4 in one launch, after the scoring kernels: every (head, segment)
// workgroup forms its head's entropies (from the partials when parts.part is
// set, writing `entropy`; else reading `entropy`), class and budgets with the
// arithmetic of launch_budget, then selects as launch_select.
hipError_t launch_budget_select(const PrefillDims& p, const egs_budget_policy& pol,
                                EntropyParts parts, int kind, float alpha, float* entropy,
                                const float* scores, int k_max, int8_t* rigid,
                                int32_t* budget, int32_t* idx, int32_t* cnt, hipStream_t st);
// K5: block-sparse causal GQA attention (workspace: the packed V^T tiles).
size_t sparse_attn_workspace_bytes(const PrefillDims& p);
hipError_t launch_sparse_attn(const PrefillDims& p, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* cnt,
                              int k_max, void* out, float* lse, void* ws, hipStream_t st);

// K6/K7: decode retention.  Workspace layout is owned by retain.hip.
size_t retain_workspace_bytes(const DecodeDims& p);
hipError_t launch_kv_retain(const DecodeDims& p, const egs_retain_params& prm,
                            const void* q_obs, const void* k, const void* v,
                            const float* token_entropy, int32_t* keep_idx,
                            void* k_out, void* v_out, float* head_entropy,
                            float* scores, void* ws, hipStream_t st);
// K8: decode attention over the first n_total entries of every (batch, KV
// group) row of k / v, rows ldk entries apart (split over the kept range).
size_t decode_attn_workspace_bytes(const DecodeDims& p, int n_total);
size_t decode_attn_workspace_bytes_upto(const DecodeDims& p, int cap);
hipError_t launch_decode_attn(const DecodeDims& p, const void* q_new, const void* k,
                              const void* v, int n_total, int ldk, void* out, void* ws,
                              hipStream_t st);

}  // namespace egs
