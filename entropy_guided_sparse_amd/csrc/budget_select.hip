// K3 head classification + budget allocation and K4 top-k block selection.
//
// Method: EntropyInfer (arXiv 2606.09508) Sec. 4.2, Alg. 3 classifies a head
// as rigid when its largest segment entropy stays under a threshold and gives
// dynamic heads a budget that follows the entropy fluctuation between
// adjacent segments, clamped to [B_h, 3 B_h]; Sec. 1 states the two-level
// principle (fixed minimal budget for rigid heads, more for dynamic ones).
// App. A eq. (2) keeps the top-k blocks of every segment.
//
// gfx950 design:
//  * K3: one wavefront per head; budgets are computed in float64 with
//    contraction disabled so integer budgets are reproducible bit for bit.
//  * K4: one workgroup per (head, segment).  The scores are staged in LDS as
//    order-preserving integers; an 8-bit radix select (4 passes, LDS
//    histogram, one wavefront scan over 256 digits) finds the k-th largest
//    key; two block scans then emit the selected indices in ascending order,
//    taking tied keys by lower index.
#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

__device__ __forceinline__ int kclamp_dev(double x, int cb) {
#pragma clang fp contract(off)
  const double c = ceil(x - 1e-9);
  return (int)fmin((double)cb, fmax(1.0, c));
}

// One step of the [EI] Alg. 3 recurrence (reading: clamp to [B_h, 3 B_h],
// divisor max(e_{i-1}, e_t)): the budget of a segment from the previous one.
__device__ __forceinline__ double alg3_next(double Bs, float prev_e, float cur_e,
                                            const egs_budget_policy& pol) {
#pragma clang fp contract(off)
  const double prev = (double)prev_e;
  const double fluct = fabs((double)cur_e - prev) / fmax(prev, pol.entropy_threshold);
  const double step = pol.alg3_alpha * pol.base_tokens;
  Bs = Bs + step * (fluct - pol.alg3_delta_t);
  return fmin(fmax(Bs, pol.base_tokens), 3.0 * pol.base_tokens);
}

// Budget of a segment with cb causal blocks and entropy e_s under the FIXED,
// TWO_LEVEL and PROPORTIONAL policies.
__device__ __forceinline__ int frac_budget(float e_s, int cb, bool rig,
                                           const egs_budget_policy& pol) {
#pragma clang fp contract(off)
  double f;
  if (pol.mode == EGS_BUDGET_FIXED) {
    f = pol.frac;
  } else if (pol.mode == EGS_BUDGET_TWO_LEVEL) {
    f = rig ? pol.frac_rigid : pol.frac_dynamic;
  } else {
    const double ehat = cb > 1 ? (double)e_s / log((double)cb) : 0.0;
    const double prod = pol.frac_max * ehat;
    f = fmin(pol.frac_max, fmax(pol.frac_min, prod));
  }
  const double x = f * (double)cb;
  return kclamp_dev(x, cb);
}

__global__ __launch_bounds__(64) void budget_kernel(const float* __restrict__ E, int CS,
                                                    int bps, int LB, egs_budget_policy pol,
                                                    int8_t* __restrict__ rigid,
                                                    int32_t* __restrict__ budget) {
#pragma clang fp contract(off)
  const int h = blockIdx.x, lane = threadIdx.x;
  const float* e = E + (size_t)h * CS;
  int32_t* out = budget + (size_t)h * CS;
  double mx = -INFINITY;
  for (int s = lane; s < CS; s += 64) mx = fmax(mx, (double)e[s]);
  mx = wave_max_d(mx);
  const bool rig = mx < pol.entropy_threshold;
  if (lane == 0) rigid[h] = rig ? 1 : 0;
  if (pol.mode == EGS_BUDGET_ALG3) {
    if (lane == 0) {
      double Bs = pol.base_tokens;
      for (int s = 0; s < CS; ++s) {
        if (s > 0 && !rig) Bs = alg3_next(Bs, e[s - 1], e[s], pol);
        out[s] = kclamp_dev(Bs / (double)LB, (s + 1) * bps);
      }
    }
    return;
  }
  for (int s = lane; s < CS; s += 64) out[s] = frac_budget(e[s], (s + 1) * bps, rig, pol);
}

hipError_t launch_budget(const PrefillDims& p, const egs_budget_policy& pol,
                         const float* entropy, int8_t* rigid, int32_t* budget,
                         hipStream_t st) {
  budget_kernel<<<p.Hq, 64, 0, st>>>(entropy, p.CS, p.LS / p.LB, p.LB, pol, rigid, budget);
  return hipGetLastError();
}

// Exclusive scan of one int per thread over a 256-thread workgroup.
__device__ __forceinline__ int block_excl_scan256(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int base = 0;
  for (int q = 0; q < w; ++q) base += wtot[q];
  __syncthreads();
  return base + incl - v;
}

// Selection state shared by the workgroup (LDS).
struct SelShared {
  int hist[256];
  int wtot[4];
  int digit, above;
};

// The k largest of row[0 .. cb) (k clamped to [0, min(cb, k_max)]) in
// ascending order into out[0 .. k), -1 up to k_max, and k into *cnt_out;
// keys: cb words of LDS.  One 256-thread workgroup.
__device__ void select_row(const float* __restrict__ row, int cb, int k, int k_max,
                           int32_t* __restrict__ out, int32_t* __restrict__ cnt_out,
                           uint32_t* keys, SelShared& sh) {
  const int tid = threadIdx.x;
  k = max(0, min(k, min(cb, k_max)));
  // four loads per thread per round, issued together (index clamped)
  for (int j0 = 0; j0 < cb; j0 += 1024) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = row[min(j0 + u * 256 + tid, cb - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + u * 256 + tid < cb) keys[j0 + u * 256 + tid] = orderable(v[u]);
  }
  __syncthreads();

  uint32_t prefix = 0, mask = 0;
  int kr = k;
  const bool partial = (k > 0 && k < cb);
  if (partial) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      sh.hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < cb; j += 256) {
        const uint32_t kk = keys[j];
        if ((kk & mask) == prefix) atomicAdd(&sh.hist[(kk >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        const int d0 = 255 - 4 * tid;   // this lane's digits, descending
        const int c0 = sh.hist[d0], c1 = sh.hist[d0 - 1], c2 = sh.hist[d0 - 2],
                  c3 = sh.hist[d0 - 3];
        const int tot = c0 + c1 + c2 + c3;
        const int incl = wave_incl_scan(tot);
        const int excl = incl - tot;
        if (excl < kr && kr <= incl) {
          int run = excl, d;
          if (run + c0 >= kr) {
            d = d0;
          } else if (run + c0 + c1 >= kr) {
            run += c0;
            d = d0 - 1;
          } else if (run + c0 + c1 + c2 >= kr) {
            run += c0 + c1;
            d = d0 - 2;
          } else {
            run += c0 + c1 + c2;
            d = d0 - 3;
          }
          sh.digit = d;
          sh.above = run;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh.digit << shift;
      mask |= 0xFFu << shift;
      kr -= sh.above;
    }
  }
  const uint32_t T = prefix;

  // ascending compaction: contiguous chunk per thread
  const int E = (cb + 255) / 256;
  const int j0 = min(cb, tid * E), j1 = min(cb, j0 + E);
  int n_eq = 0;
  if (partial)
    for (int j = j0; j < j1; ++j) n_eq += (keys[j] == T);
  int eq_seen = block_excl_scan256(n_eq, sh.wtot);
  int n_sel = 0;
  if (k == cb) {
    n_sel = j1 - j0;
  } else if (partial) {
    int es = eq_seen;
    for (int j = j0; j < j1; ++j) {
      const uint32_t kk = keys[j];
      if (kk > T) {
        ++n_sel;
      } else if (kk == T) {
        n_sel += (es < kr);
        ++es;
      }
    }
  }
  const int pos0 = block_excl_scan256(n_sel, sh.wtot);
  int pos = pos0;
  if (k == cb) {
    for (int j = j0; j < j1; ++j) out[pos++] = j;
  } else if (partial) {
    int es = eq_seen;
    for (int j = j0; j < j1; ++j) {
      const uint32_t kk = keys[j];
      bool take = false;
      if (kk > T) {
        take = true;
      } else if (kk == T) {
        take = es < kr;
        ++es;
      }
      if (take) out[pos++] = j;
    }
  }
  for (int p = k + tid; p < k_max; p += 256) out[p] = -1;
  if (tid == 0) *cnt_out = k;
}

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores,
                                                     const int32_t* __restrict__ budget,
                                                     int CS, int CB, int bps, int k_max,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ cnt) {
  extern __shared__ uint32_t keys[];
  __shared__ SelShared sh;
  const int hs = blockIdx.x, s = hs % CS;
  select_row(scores + (size_t)hs * CB, (s + 1) * bps, budget[hs], k_max,
             idx + (size_t)hs * k_max, cnt + hs, keys, sh);
}

// K3 + K4 fused: one workgroup per (head, segment).  The head's entropies
// are summed from the scoring pass's per-piece partials in piece order (the
// arithmetic of probe_entropy_kernel; the segment-0 workgroup stores them),
// or read when already final; the class and this segment's budget follow
// with the arithmetic of budget_kernel; then the selection.
__global__ __launch_bounds__(256) void budget_select_kernel(
    EntropyParts parts, int kind, float alpha, float* __restrict__ entropy,
    const float* __restrict__ scores, int CS, int CB, int bps, int LB, egs_budget_policy pol,
    int k_max, int8_t* __restrict__ rigid, int32_t* __restrict__ budget,
    int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
#pragma clang fp contract(off)
  // CB words of LDS: first the head's CS <= C_B entropies, then (once the
  // budget is fixed, past a barrier) the selection keys
  extern __shared__ uint32_t dyn[];
  uint32_t* keys = dyn;
  float* Es = reinterpret_cast<float*>(dyn);
  __shared__ SelShared sh;
  __shared__ int sh_k;
  const int hs = blockIdx.x, h = hs / CS, s = hs % CS, tid = threadIdx.x;
  for (int t = tid; t < CS; t += 256) {
    float E;
    if (parts.part != nullptr) {
      const int np = ((t + 1) * bps + parts.pc - 1) / parts.pc;
      const float* e = parts.part + ((size_t)h * CS + t) * parts.npc;
      float tot = 0.f;
      for (int c = 0; c < np; ++c) tot += e[c];
      E = (kind == EGS_SHANNON) ? tot : logf(tot) / (1.0f - alpha);
      if (s == 0) entropy[(size_t)h * CS + t] = E;
    } else {
      E = entropy[(size_t)h * CS + t];
    }
    Es[t] = E;
  }
  __syncthreads();
  if (tid == 0) {
    double mx = -INFINITY;
    for (int t = 0; t < CS; ++t) mx = fmax(mx, (double)Es[t]);
    const bool rig = mx < pol.entropy_threshold;
    if (s == 0) rigid[h] = rig ? 1 : 0;
    int kb;
    if (pol.mode == EGS_BUDGET_ALG3) {
      double Bs = pol.base_tokens;
      for (int t = 1; t <= s; ++t)
        if (!rig) Bs = alg3_next(Bs, Es[t - 1], Es[t], pol);
      kb = kclamp_dev(Bs / (double)LB, (s + 1) * bps);
    } else {
      kb = frac_budget(Es[s], (s + 1) * bps, rig, pol);
    }
    budget[hs] = kb;
    sh_k = kb;
  }
  __syncthreads();
  select_row(scores + (size_t)hs * CB, (s + 1) * bps, sh_k, k_max, idx + (size_t)hs * k_max,
             cnt + hs, keys, sh);
}

hipError_t launch_select(const PrefillDims& p, const float* scores, const int32_t* budget,
                         int k_max, int32_t* idx, int32_t* cnt, hipStream_t st) {
  const size_t lds = (size_t)p.CB * sizeof(uint32_t);
  select_kernel<<<p.Hq * p.CS, 256, lds, st>>>(scores, budget, p.CS, p.CB, p.LS / p.LB,
                                               k_max, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_budget_select(const PrefillDims& p, const egs_budget_policy& pol,
                                EntropyParts parts, int kind, float alpha, float* entropy,
                                const float* scores, int k_max, int8_t* rigid,
                                int32_t* budget, int32_t* idx, int32_t* cnt, hipStream_t st) {
  const size_t lds = (size_t)p.CB * sizeof(uint32_t);
  budget_select_kernel<<<p.Hq * p.CS, 256, lds, st>>>(parts, kind, alpha, entropy, scores,
                                                      p.CS, p.CB, p.LS / p.LB, p.LB, pol, k_max,
                                                      rigid, budget, idx, cnt);
  return hipGetLastError();
}

}  // namespace egs
