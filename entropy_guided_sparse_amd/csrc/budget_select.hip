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
        if (s > 0 && !rig) {
          const double prev = (double)e[s - 1];
          const double fluct = fabs((double)e[s] - prev) / fmax(prev, pol.entropy_threshold);
          const double step = pol.alg3_alpha * pol.base_tokens;
          Bs = Bs + step * (fluct - pol.alg3_delta_t);
          Bs = fmin(fmax(Bs, pol.base_tokens), 3.0 * pol.base_tokens);
        }
        out[s] = kclamp_dev(Bs / (double)LB, (s + 1) * bps);
      }
    }
    return;
  }
  for (int s = lane; s < CS; s += 64) {
    const int cb = (s + 1) * bps;
    double f;
    if (pol.mode == EGS_BUDGET_FIXED) {
      f = pol.frac;
    } else if (pol.mode == EGS_BUDGET_TWO_LEVEL) {
      f = rig ? pol.frac_rigid : pol.frac_dynamic;
    } else {
      const double ehat = cb > 1 ? (double)e[s] / log((double)cb) : 0.0;
      const double prod = pol.frac_max * ehat;
      f = fmin(pol.frac_max, fmax(pol.frac_min, prod));
    }
    const double x = f * (double)cb;
    out[s] = kclamp_dev(x, cb);
  }
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

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores,
                                                     const int32_t* __restrict__ budget,
                                                     int CS, int CB, int bps, int k_max,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ cnt) {
  extern __shared__ uint32_t keys[];
  __shared__ int hist[256];
  __shared__ int wtot[4];
  __shared__ int sh_digit, sh_above;
  const int hs = blockIdx.x;
  const int s = hs % CS;
  const int tid = threadIdx.x;
  const int cb = (s + 1) * bps;
  int k = budget[hs];
  k = max(0, min(k, min(cb, k_max)));
  const float* row = scores + (size_t)hs * CB;
  int32_t* out = idx + (size_t)hs * k_max;
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
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < cb; j += 256) {
        const uint32_t kk = keys[j];
        if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        const int d0 = 255 - 4 * tid;   // this lane's digits, descending
        const int c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
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
          sh_digit = d;
          sh_above = run;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      mask |= 0xFFu << shift;
      kr -= sh_above;
    }
  }
  const uint32_t T = prefix;

  // ascending compaction: contiguous chunk per thread
  const int E = (cb + 255) / 256;
  const int j0 = min(cb, tid * E), j1 = min(cb, j0 + E);
  int n_eq = 0;
  if (partial)
    for (int j = j0; j < j1; ++j) n_eq += (keys[j] == T);
  int eq_seen = block_excl_scan256(n_eq, wtot);
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
  const int pos0 = block_excl_scan256(n_sel, wtot);
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
  if (tid == 0) cnt[hs] = k;
}

hipError_t launch_select(const PrefillDims& p, const float* scores, const int32_t* budget,
                         int k_max, int32_t* idx, int32_t* cnt, hipStream_t st) {
  const size_t lds = (size_t)p.CB * sizeof(uint32_t);
  select_kernel<<<p.Hq * p.CS, 256, lds, st>>>(scores, budget, p.CS, p.CB, p.LS / p.LB,
                                               k_max, idx, cnt);
  return hipGetLastError();
}

}  // namespace egs
