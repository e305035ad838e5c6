// K6 / K7: decode-time KV retention, and K8: decode attention over the kept
// entries.
//
// Method: EntropyInfer (arXiv 2606.09508) Sec. 4.3 and App. B Alg. 4 score
// every cache entry with a window of the most recent queries, keep the B_d
// best and gather the kept K/V rows.  The score used here is the
// entropy-weighted window attention mass: per head, the window mean of the
// causal attention rows (InfoKV eq. 4; EntroPrefill Sec. 2.1), mixed over the
// GQA group with the regularized weights w_h = zeta/r + (1-zeta) softmax(-H/tau)
// of the sink-isolated head entropies (EntroPrefill Sec. 3.1); optionally fused
// with softmax(token entropy) (InfoKV eq. 8).  Raw mode keeps Alg. 4's literal
// score, the sum of the window's raw logits.  Sinks and the recent window are
// always kept; compaction preserves token order (EntroPrefill Sec. 8.1).
//
// gfx950 design:
//  * Pass 1 (obs_stats): one workgroup per (1024-key chunk, batch x KV group,
//    4-head group).  128-key K stages are staged in LDS and shared by the four
//    wavefronts (one query head each); S^T = K Q^T on v_mfma_f32_32x32x16_bf16
//    gives every lane one observer row: running max / sum in registers.
//  * A combine kernel folds the per-chunk statistics into each row's final
//    max and 1/sum.
//  * Pass 2 (obs_mass) recomputes the logits with keys as the N dimension, so
//    a lane owns one key and the window mean is a register sum; it writes the
//    per-head mass and the per-chunk sink-isolated entropy partial sums.
//  * head_weight turns the partial sums into H_h and w_h; retain_select forms
//    mu_t, runs an exact 12/12/8-bit radix select over the candidates in LDS
//    and compacts the kept indices in ascending order; gather copies K/V rows.
//  * Decode attention splits the kept range in 512-key chunks (one wavefront
//    per query head, lane-per-key dot products, LDS-broadcast probabilities)
//    and combines the chunks with their log-sum-exp.
#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

constexpr int RT_CK = 1024;   // keys per chunk (pass 1 / pass 2 work unit)
constexpr int RT_KS = 128;    // keys per LDS stage
constexpr int SEL_T = 1024;   // threads of the select kernel
constexpr int DA_SPL = 512;   // keys per decode-attention split

struct RetainLayout {
  size_t stat_m, stat_l, row_m, row_inv, mass, ent, weight, mu, qsum, total;
  int nch;
};

static size_t align_up(size_t x) {
  return (x + 255) / 256 * 256;
}

static RetainLayout retain_layout(const DecodeDims& p) {
  RetainLayout o;
  o.nch = (p.L + RT_CK - 1) / RT_CK;
  const size_t rows = (size_t)p.B * p.Hq * p.W;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  o.stat_m = take(rows * o.nch * 4);
  o.stat_l = take(rows * o.nch * 4);
  o.row_m = take(rows * 4);
  o.row_inv = take(rows * 4);
  o.mass = take((size_t)p.B * p.Hq * p.L * 4);
  o.ent = take((size_t)p.B * p.Hq * o.nch * 2 * 4);
  o.weight = take((size_t)p.B * p.Hq * 4);
  o.mu = take((size_t)p.B * p.Hkv * p.L * 4);
  o.qsum = take((size_t)p.B * p.Hkv * p.D * 4);
  o.total = off;
  return o;
}

size_t retain_workspace_bytes(const DecodeDims& p) {
  return retain_layout(p).total;
}

// ---------------------------------------------------------------------------
// shared pieces of pass 1 / pass 2
// ---------------------------------------------------------------------------
template <int D>
struct KStage {
  static constexpr int KPAD = D + 8;
  static constexpr int CH = RT_KS * D / 8;   // 16-byte chunks per stage
  // cooperative copy of keys [t0, t0 + RT_KS) (zero past t_end) into LDS
  __device__ static void load(bf16* Ks, const bf16* Kg, int t0, int t_end) {
    for (int q = threadIdx.x; q < CH; q += 256) {
      const int row = q / (D / 8), c8 = q % (D / 8);
      const int t = t0 + row;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < t_end) v = *reinterpret_cast<const u32x4*>(Kg + (size_t)t * D + c8 * 8);
      *reinterpret_cast<u32x4*>(Ks + row * KPAD + c8 * 8) = v;
    }
  }
};

template <int D, int RT>
__device__ __forceinline__ void load_obs_q(bf16x8 (&qf)[RT][D / 16], const bf16* Qo, int b,
                                           int h, int Hq, int W, bool hvalid, int lane) {
  const int l32 = lane & 31, hg = lane >> 5;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int u = rt * 32 + l32;
    const bool ok = hvalid && u < W;
    const bf16* src = Qo + (((size_t)b * Hq + h) * W + (ok ? u : 0)) * D + 8 * hg;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (ok) {
        qf[rt][c] = load8(src + 16 * c);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[rt][c][e] = (bf16)0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// pass 1: per-chunk running max / sum of every observer row
// ---------------------------------------------------------------------------
template <int D, int RT>
__global__ __launch_bounds__(256) void obs_stats_kernel(
    const bf16* __restrict__ Qo, const bf16* __restrict__ K, int Hq, int Hkv, int r, int L,
    int W, int nch, float sl2, float* __restrict__ stat_m, float* __restrict__ stat_l) {
  constexpr int NC = D / 16;
  constexpr int KPAD = KStage<D>::KPAD;
  __shared__ __attribute__((aligned(16))) bf16 Ks[RT_KS * KPAD];
  const int chunk = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const int hl = blockIdx.z * 4 + w;
  const bool hvalid = hl < r;
  const int h = g * r + (hvalid ? hl : 0);
  bf16x8 qf[RT][NC];
  load_obs_q<D, RT>(qf, Qo, b, h, Hq, W, hvalid, lane);
  float m[RT], l[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegBig;
    l[rt] = 0.f;
  }
  const int t_begin = chunk * RT_CK, t_end = min(L, t_begin + RT_CK);
  const bf16* Kg = K + (size_t)bg * L * D;
  const int pos0 = L - W;   // observer u sits at pos0 + u
  for (int t0 = t_begin; t0 < t_end; t0 += RT_KS) {
    __syncthreads();
    KStage<D>::load(Ks, Kg, t0, t_end);
    __syncthreads();
    if (!hvalid) continue;
    for (int kt = 0; kt < RT_KS / 32; ++kt) {
      const int tk = t0 + kt * 32;
      if (tk >= t_end) break;
      floatx16 st[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[rt][i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = load8(Ks + (kt * 32 + l32) * KPAD + 16 * c + 8 * hg);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) st[rt] = mfma32(a, qf[rt][c], st[rt]);
      }
      const bool edge = (tk + 31 >= t_end) || (tk + 31 > pos0);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int u = rt * 32 + l32;
        float tmax = kNegBig;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float v = st[rt][i] * sl2;
          if (edge) {
            const int t = tk + acc_row(i, lane);
            if (t >= t_end || t > pos0 + u) v = -INFINITY;
          }
          st[rt][i] = v;
          tmax = fmaxf(tmax, v);
        }
        const float mn = fmaxf(m[rt], tmax);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(st[rt][i] - mn);
        l[rt] = l[rt] * fast_exp2(m[rt] - mn) + sum;
        m[rt] = mn;
      }
    }
  }
  if (!hvalid) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float m2 = __shfl_xor(m[rt], 32), l2 = __shfl_xor(l[rt], 32);
    const float M = fmaxf(m[rt], m2);
    const float Lr = l[rt] * fast_exp2(m[rt] - M) + l2 * fast_exp2(m2 - M);
    const int u = rt * 32 + l32;
    if (hg == 0 && u < W) {
      const size_t o = (((size_t)b * Hq + h) * nch + chunk) * W + u;
      stat_m[o] = M;
      stat_l[o] = Lr;
    }
  }
}

__global__ __launch_bounds__(256) void obs_combine_kernel(const float* __restrict__ stat_m,
                                                          const float* __restrict__ stat_l,
                                                          int rows, int nch, int W,
                                                          float* __restrict__ row_m,
                                                          float* __restrict__ row_inv) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  const int bh = i / W, u = i % W;
  float M = kNegBig;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, stat_m[((size_t)bh * nch + c) * W + u]);
  float Lr = 0.f;
  for (int c = 0; c < nch; ++c) {
    const size_t o = ((size_t)bh * nch + c) * W + u;
    Lr += stat_l[o] * fast_exp2(stat_m[o] - M);
  }
  row_m[i] = M;
  row_inv[i] = Lr > 0.f ? 1.0f / Lr : 0.f;
}

// ---------------------------------------------------------------------------
// pass 2: per-head window-mean mass and sink-isolated entropy partial sums
// ---------------------------------------------------------------------------
template <int D, int RT>
__global__ __launch_bounds__(256) void obs_mass_kernel(
    const bf16* __restrict__ Qo, const bf16* __restrict__ K, int Hq, int Hkv, int r, int L,
    int W, int nch, float sl2, const float* __restrict__ row_m,
    const float* __restrict__ row_inv, int n_sink, int kind, float alpha,
    float* __restrict__ mass, float* __restrict__ ent) {
  constexpr int NC = D / 16;
  constexpr int KPAD = KStage<D>::KPAD;
  __shared__ __attribute__((aligned(16))) bf16 Ks[RT_KS * KPAD];
  const int chunk = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const int hl = blockIdx.z * 4 + w;
  const bool hvalid = hl < r;
  const int h = g * r + (hvalid ? hl : 0);
  bf16x8 qf[RT][NC];
  load_obs_q<D, RT>(qf, Qo, b, h, Hq, W, hvalid, lane);
  float rm[RT][16], ri[RT][16];
  const size_t rbase = ((size_t)b * Hq + h) * W;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = rt * 32 + acc_row(i, lane);
      const bool ok = hvalid && u < W;
      rm[rt][i] = ok ? row_m[rbase + u] : 0.f;
      ri[rt][i] = ok ? row_inv[rbase + u] : 0.f;
    }
  const float invW = 1.0f / (float)W;
  float s1 = 0.f, s2 = 0.f;
  const int t_begin = chunk * RT_CK, t_end = min(L, t_begin + RT_CK);
  const bf16* Kg = K + (size_t)bg * L * D;
  float* mrow = mass + ((size_t)b * Hq + h) * L;
  const int pos0 = L - W;
  for (int t0 = t_begin; t0 < t_end; t0 += RT_KS) {
    __syncthreads();
    KStage<D>::load(Ks, Kg, t0, t_end);
    __syncthreads();
    if (!hvalid) continue;
    for (int kt = 0; kt < RT_KS / 32; ++kt) {
      const int tk = t0 + kt * 32;
      if (tk >= t_end) break;
      floatx16 z[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[rt][i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 bk = load8(Ks + (kt * 32 + l32) * KPAD + 16 * c + 8 * hg);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) z[rt] = mfma32(qf[rt][c], bk, z[rt]);
      }
      const int t = tk + l32;            // this lane's key
      const bool edge = tk + 31 > pos0;  // causal mask only near the end
      float colsum = 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(z[rt][i] * sl2 - rm[rt][i]) * ri[rt][i];
          if (edge && t > pos0 + rt * 32 + acc_row(i, lane)) pv = 0.f;
          colsum += pv;
        }
      colsum += __shfl_xor(colsum, 32);
      if (hg == 0 && t < t_end) {
        const float a = colsum * invW;
        mrow[t] = a;
        if (t >= n_sink && a > 0.f) {
          s1 += a;
          s2 += (kind == EGS_SHANNON) ? a * logf(a) : powf(a, alpha);
        }
      }
    }
  }
  if (!hvalid) return;
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) {
    float* e = ent + (((size_t)b * Hq + h) * nch + chunk) * 2;
    e[0] = s1;
    e[1] = s2;
  }
}

// ---------------------------------------------------------------------------
// head entropies and weights; one wavefront per (batch, KV group)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void head_weight_kernel(const float* __restrict__ ent, int Hq,
                                                         int Hkv, int r, int nch, int kind,
                                                         float alpha, double zeta, double tau,
                                                         float* __restrict__ weight,
                                                         float* __restrict__ head_entropy) {
  const int bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
  const int lane = threadIdx.x;
  const bool on = lane < r;
  const int h = g * r + (on ? lane : 0);
  double H = 0.0;
  if (on) {
    float s1 = 0.f, s2 = 0.f;
    const float* e = ent + ((size_t)b * Hq + h) * nch * 2;
    for (int c = 0; c < nch; ++c) {
      s1 += e[2 * c];
      s2 += e[2 * c + 1];
    }
    if (s1 > 0.f) {
      if (kind == EGS_SHANNON)
        H = log((double)s1) - (double)s2 / (double)s1;
      else
        H = (log((double)s2) - (double)alpha * log((double)s1)) / (1.0 - (double)alpha);
    }
  }
  const double x = on ? -H / tau : -INFINITY;
  const double mx = wave_max_d(x);
  double ex = on ? exp(x - mx) : 0.0;
  double sum = ex;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (on) {
    const double wv = zeta / (double)r + (1.0 - zeta) * (ex / sum);
    weight[(size_t)b * Hq + h] = (float)wv;
    if (head_entropy != nullptr) head_entropy[(size_t)b * Hq + h] = (float)H;
  }
}

// ---------------------------------------------------------------------------
// raw mode ([EI] Alg. 4 literal): mu_t = k_t . (sigma * sum_{h in g, u} q_{h,u})
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void raw_qsum_kernel(const bf16* __restrict__ Qo, int Hq,
                                                       int Hkv, int r, int W, int D, float sc,
                                                       float* __restrict__ qsum) {
  const int bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
  for (int d = threadIdx.x; d < D; d += 256) {
    float acc = 0.f;
    for (int hl = 0; hl < r; ++hl) {
      const bf16* q = Qo + (((size_t)b * Hq + g * r + hl) * W) * D + d;
      for (int u = 0; u < W; ++u) acc += bf2f(q[(size_t)u * D]);
    }
    qsum[(size_t)bg * D + d] = acc * sc;
  }
}

template <int D>
__global__ __launch_bounds__(256) void raw_score_kernel(const bf16* __restrict__ K,
                                                        const float* __restrict__ qsum, int L,
                                                        float* __restrict__ mu) {
  __shared__ float qs[D];
  const int bg = blockIdx.y;
  for (int d = threadIdx.x; d < D; d += 256) qs[d] = qsum[(size_t)bg * D + d];
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  const bf16* k = K + ((size_t)bg * L + t) * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    float x[8];
    load8f(k + 8 * c, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[e] * qs[8 * c + e];
  }
  mu[(size_t)bg * L + t] = acc;
}

// ---------------------------------------------------------------------------
// group score, exact top-n_keep and ascending compaction; one workgroup per
// (batch, KV group)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int block_sum_1024(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum_i(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int q = 0; q < SEL_T / 64; ++q) t += red[q];
  __syncthreads();
  return t;
}
__device__ __forceinline__ float block_max_1024f(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int q = 1; q < SEL_T / 64; ++q) t = fmaxf(t, red[q]);
  __syncthreads();
  return t;
}
__device__ __forceinline__ float block_sum_1024f(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int q = 0; q < SEL_T / 64; ++q) t += red[q];
  __syncthreads();
  return t;
}
__device__ __forceinline__ int block_excl_scan_1024(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) red[w] = incl;
  __syncthreads();
  int base = 0;
  for (int q = 0; q < w; ++q) base += red[q];
  __syncthreads();
  return base + incl - v;
}

__global__ __launch_bounds__(SEL_T) void retain_select_kernel(
    const float* __restrict__ mass, const float* __restrict__ weight,
    const float* __restrict__ token_entropy, int raw, float info_alpha, int Hq, int Hkv, int r,
    int L, int n_sink, int n_recent, int n_keep, int n_total, float* __restrict__ mu,
    float* __restrict__ scores, int32_t* __restrict__ keep_idx) {
  __shared__ int hist[4096];
  __shared__ int ired[SEL_T / 64];
  __shared__ float fred[SEL_T / 64];
  __shared__ int sh_digit, sh_above;
  const int bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x;
  float* mu_row = mu + (size_t)bg * L;

  // ---- mu_t ----
  if (!raw) {
    __shared__ float wv[16];
    if (tid < r) wv[tid] = weight[(size_t)b * Hq + g * r + tid];
    __syncthreads();
    const float* mrow = mass + ((size_t)b * Hq + g * r) * L;
    for (int t = tid; t < L; t += SEL_T) {
      float acc = 0.f;
      for (int hl = 0; hl < r; ++hl) acc += wv[hl] * mrow[(size_t)hl * L + t];
      mu_row[t] = acc;
    }
    if (token_entropy != nullptr && info_alpha < 1.0f) {
      const float* E = token_entropy + (size_t)b * L;
      float mx = -INFINITY;
      for (int t = tid; t < L; t += SEL_T) mx = fmaxf(mx, E[t]);
      mx = block_max_1024f(mx, fred);
      float se = 0.f;
      for (int t = tid; t < L; t += SEL_T) se += expf(E[t] - mx);
      se = block_sum_1024f(se, fred);
      const float inv = 1.0f / se;
      for (int t = tid; t < L; t += SEL_T)
        mu_row[t] = info_alpha * mu_row[t] + (1.0f - info_alpha) * (expf(E[t] - mx) * inv);
    }
  }
  __syncthreads();
  if (scores != nullptr)
    for (int t = tid; t < L; t += SEL_T) scores[(size_t)bg * L + t] = mu_row[t];

  const bool keep_all = (long long)n_sink + n_recent + n_keep >= L;
  const int c_lo = n_sink, c_hi = L - n_recent;   // candidates [c_lo, c_hi)
  uint32_t prefix = 0, mask = 0;
  int kr = n_keep;
  const bool partial = !keep_all && n_keep > 0;
  if (partial) {
    // 12 / 12 / 8-bit radix select of the n_keep-th largest key
    const int shifts[3] = {20, 8, 0};
    const int bits[3] = {12, 12, 8};
    for (int ps = 0; ps < 3; ++ps) {
      const int sh = shifts[ps], nb = 1 << bits[ps];
      for (int i = tid; i < 4096; i += SEL_T) hist[i] = 0;
      __syncthreads();
      for (int t = c_lo + tid; t < c_hi; t += SEL_T) {
        const uint32_t key = orderable(mu_row[t]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> sh) & (uint32_t)(nb - 1)], 1);
      }
      __syncthreads();
      // thread tid owns digits nb-1-4*tid .. nb-4-4*tid (descending)
      const int d0 = nb - 1 - 4 * tid;
      const bool own = d0 >= 3;
      const int c0 = own ? hist[d0] : 0, c1 = own ? hist[d0 - 1] : 0;
      const int c2 = own ? hist[d0 - 2] : 0, c3 = own ? hist[d0 - 3] : 0;
      const int tot = c0 + c1 + c2 + c3;
      const int excl = block_excl_scan_1024(tot, ired);
      if (own && excl < kr && kr <= excl + tot) {
        int run = excl, dd;
        if (run + c0 >= kr) {
          dd = d0;
        } else if (run + c0 + c1 >= kr) {
          run += c0;
          dd = d0 - 1;
        } else if (run + c0 + c1 + c2 >= kr) {
          run += c0 + c1;
          dd = d0 - 2;
        } else {
          run += c0 + c1 + c2;
          dd = d0 - 3;
        }
        sh_digit = dd;
        sh_above = run;
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << sh;
      mask |= (uint32_t)(nb - 1) << sh;
      kr -= sh_above;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;

  // ---- ascending compaction over [0, L): contiguous chunk per thread ----
  const int E = (L + SEL_T - 1) / SEL_T;
  const int j0 = min(L, tid * E), j1 = min(L, j0 + E);
  int n_eq = 0;
  if (partial)
    for (int t = max(j0, c_lo); t < min(j1, c_hi); ++t) n_eq += (orderable(mu_row[t]) == T);
  const int eq0 = block_excl_scan_1024(n_eq, ired);
  auto take = [&](int t, int& es) -> bool {
    if (keep_all || t < c_lo || t >= c_hi) return true;
    if (!partial) return false;
    const uint32_t key = orderable(mu_row[t]);
    if (key > T) return true;
    if (key == T) return (es++) < kr;
    return false;
  };
  int n_sel = 0;
  {
    int es = eq0;
    for (int t = j0; t < j1; ++t) n_sel += take(t, es) ? 1 : 0;
  }
  int pos = block_excl_scan_1024(n_sel, ired);
  int32_t* out = keep_idx + (size_t)bg * n_total;
  {
    int es = eq0;
    for (int t = j0; t < j1; ++t)
      if (take(t, es) && pos < n_total) out[pos++] = t;
  }
}

// copy the kept K / V rows: one thread per 16 bytes
template <int D>
__global__ __launch_bounds__(256) void gather_kv_kernel(const bf16* __restrict__ K,
                                                        const bf16* __restrict__ V,
                                                        const int32_t* __restrict__ keep, int L,
                                                        int n_total, long long units,
                                                        bf16* __restrict__ Ko,
                                                        bf16* __restrict__ Vo) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= units) return;
  constexpr int CPR = D / 8;
  const long long row = i / CPR;
  const int c8 = (int)(i % CPR);
  const long long bg = row / n_total;
  int t = keep[row];
  t = min(max(t, 0), L - 1);
  const size_t src = ((size_t)bg * L + t) * D + c8 * 8;
  const size_t dst = (size_t)row * D + c8 * 8;
  *reinterpret_cast<u32x4*>(Ko + dst) = *reinterpret_cast<const u32x4*>(K + src);
  *reinterpret_cast<u32x4*>(Vo + dst) = *reinterpret_cast<const u32x4*>(V + src);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int D, int RT>
static hipError_t retain_passes(const DecodeDims& p, const RetainLayout& lay, char* ws,
                                const void* q_obs, const void* k, int kind, float alpha,
                                hipStream_t st) {
  const float sl2 = p.sm_scale * kLog2e;
  dim3 grid(lay.nch, p.B * p.Hkv, (p.r + 3) / 4);
  const bf16* Qo = static_cast<const bf16*>(q_obs);
  const bf16* K = static_cast<const bf16*>(k);
  float* stat_m = reinterpret_cast<float*>(ws + lay.stat_m);
  float* stat_l = reinterpret_cast<float*>(ws + lay.stat_l);
  float* row_m = reinterpret_cast<float*>(ws + lay.row_m);
  float* row_inv = reinterpret_cast<float*>(ws + lay.row_inv);
  obs_stats_kernel<D, RT><<<grid, 256, 0, st>>>(Qo, K, p.Hq, p.Hkv, p.r, p.L, p.W, lay.nch, sl2,
                                                stat_m, stat_l);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.Hq * p.W;
  obs_combine_kernel<<<(rows + 255) / 256, 256, 0, st>>>(stat_m, stat_l, rows, lay.nch, p.W,
                                                         row_m, row_inv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  obs_mass_kernel<D, RT><<<grid, 256, 0, st>>>(
      Qo, K, p.Hq, p.Hkv, p.r, p.L, p.W, lay.nch, sl2, row_m, row_inv, p.n_sink, kind, alpha,
      reinterpret_cast<float*>(ws + lay.mass), reinterpret_cast<float*>(ws + lay.ent));
  return hipGetLastError();
}

hipError_t launch_kv_retain(const DecodeDims& p, const egs_retain_params& prm, const void* q_obs,
                            const void* k, const void* v, const float* token_entropy,
                            int32_t* keep_idx, void* k_out, void* v_out, float* head_entropy,
                            float* scores, void* workspace, hipStream_t st) {
  const RetainLayout lay = retain_layout(p);
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  const int raw = prm.raw_logit_mode ? 1 : 0;
  if (!raw) {
    const int kind = prm.entropy_kind;
    const float alpha = prm.renyi_alpha;
    const int RT = (p.W + 31) / 32;
#define EGS_RP(DD, RR) e = retain_passes<DD, RR>(p, lay, ws, q_obs, k, kind, alpha, st)
    if (p.D == 128) {
      if (RT == 1) EGS_RP(128, 1);
      else if (RT == 2) EGS_RP(128, 2);
      else if (RT == 3) EGS_RP(128, 3);
      else EGS_RP(128, 4);
    } else {
      if (RT == 1) EGS_RP(64, 1);
      else if (RT == 2) EGS_RP(64, 2);
      else if (RT == 3) EGS_RP(64, 3);
      else EGS_RP(64, 4);
    }
#undef EGS_RP
    if (e != hipSuccess) return e;
    head_weight_kernel<<<p.B * p.Hkv, 64, 0, st>>>(
        reinterpret_cast<const float*>(ws + lay.ent), p.Hq, p.Hkv, p.r, lay.nch, kind, alpha,
        prm.zeta, prm.tau, reinterpret_cast<float*>(ws + lay.weight), head_entropy);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    float* qsum = reinterpret_cast<float*>(ws + lay.qsum);
    raw_qsum_kernel<<<p.B * p.Hkv, 256, 0, st>>>(static_cast<const bf16*>(q_obs), p.Hq, p.Hkv,
                                                 p.r, p.W, p.D, p.sm_scale, qsum);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 grid((p.L + 255) / 256, p.B * p.Hkv);
    float* mu = reinterpret_cast<float*>(ws + lay.mu);
    if (p.D == 128)
      raw_score_kernel<128><<<grid, 256, 0, st>>>(static_cast<const bf16*>(k), qsum, p.L, mu);
    else
      raw_score_kernel<64><<<grid, 256, 0, st>>>(static_cast<const bf16*>(k), qsum, p.L, mu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (head_entropy != nullptr) {
      const int n = p.B * p.Hq;
      fill_zero_kernel<<<(n + 255) / 256, 256, 0, st>>>(head_entropy, n);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  retain_select_kernel<<<p.B * p.Hkv, SEL_T, 0, st>>>(
      reinterpret_cast<const float*>(ws + lay.mass), reinterpret_cast<const float*>(ws + lay.weight),
      raw ? nullptr : token_entropy, raw, (float)prm.info_alpha, p.Hq, p.Hkv, p.r, p.L, p.n_sink,
      p.n_recent, p.n_keep, p.n_total, reinterpret_cast<float*>(ws + lay.mu), scores, keep_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (k_out != nullptr) {
    const long long units = (long long)p.B * p.Hkv * p.n_total * (p.D / 8);
    const unsigned blocks = (unsigned)((units + 255) / 256);
    if (p.D == 128)
      gather_kv_kernel<128><<<blocks, 256, 0, st>>>(
          static_cast<const bf16*>(k), static_cast<const bf16*>(v), keep_idx, p.L, p.n_total,
          units, static_cast<bf16*>(k_out), static_cast<bf16*>(v_out));
    else
      gather_kv_kernel<64><<<blocks, 256, 0, st>>>(
          static_cast<const bf16*>(k), static_cast<const bf16*>(v), keep_idx, p.L, p.n_total,
          units, static_cast<bf16*>(k_out), static_cast<bf16*>(v_out));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// K8: decode attention over the kept entries
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_attn_split_kernel(
    const bf16* __restrict__ Qn, const bf16* __restrict__ K, const bf16* __restrict__ V,
    int Hq, int Hkv, int r, int n, int nsplit, float sl2, float* __restrict__ part) {
  constexpr int DPL = D / 64;    // output dims per lane
  __shared__ float pbuf[4][DA_SPL];
  const int sp = blockIdx.x, bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t_begin = sp * DA_SPL, t_end = min(n, t_begin + DA_SPL);
  const bf16* Kg = K + (size_t)bg * n * D;
  const bf16* Vg = V + (size_t)bg * n * D;
  for (int hl = w; hl < r; hl += 4) {
    const int h = g * r + hl;
    const bf16* q = Qn + ((size_t)b * Hq + h) * D;
    float qv[D];
#pragma unroll
    for (int c = 0; c < D / 8; ++c) load8f(q + 8 * c, qv + 8 * c);
    // logits: lane owns keys t_begin + lane + 64 j
    float mx = kNegBig;
    for (int t = t_begin + lane; t < t_end; t += 64) {
      const bf16* kr = Kg + (size_t)t * D;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        float x[8];
        load8f(kr + 8 * c, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += qv[8 * c + e] * x[e];
      }
      const float s = acc * sl2;
      pbuf[w][t - t_begin] = s;
      mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int t = t_begin + lane; t < t_end; t += 64) {
      const float pv = fast_exp2(pbuf[w][t - t_begin] - mx);
      pbuf[w][t - t_begin] = pv;
      sum += pv;
    }
    sum = wave_sum(sum);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    float o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
    for (int t = t_begin; t < t_end; ++t) {
      const float pv = pbuf[w][t - t_begin];
      const bf16* vr = Vg + (size_t)t * D + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] += pv * bf2f(vr[e]);
    }
    float* pp = part + (((size_t)b * Hq + h) * nsplit + sp) * (D + 2);
#pragma unroll
    for (int e = 0; e < DPL; ++e) pp[lane * DPL + e] = o[e];
    if (lane == 0) {
      pp[D] = mx;
      pp[D + 1] = sum;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int D>
__global__ __launch_bounds__(64) void decode_attn_combine_kernel(const float* __restrict__ part,
                                                                 int nsplit, bf16* __restrict__ out) {
  constexpr int DPL = D / 64;
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* pp = part + (size_t)bh * nsplit * (D + 2);
  float M = kNegBig;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pp[(size_t)s * (D + 2) + D]);
  float Lr = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* q = pp + (size_t)s * (D + 2);
    const float f = fast_exp2(q[D] - M);
    Lr += q[D + 1] * f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] += q[lane * DPL + e] * f;
  }
  const float inv = 1.0f / Lr;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[(size_t)bh * D + lane * DPL + e] = f2bf(o[e] * inv);
}

size_t decode_attn_workspace_bytes(const DecodeDims& p, int n_total) {
  const int nsplit = (n_total + DA_SPL - 1) / DA_SPL;
  return align_up((size_t)p.B * p.Hq * nsplit * (p.D + 2) * 4);
}

hipError_t launch_decode_attn(const DecodeDims& p, const void* q_new, const void* k,
                              const void* v, int n_total, void* out, void* ws, hipStream_t st) {
  const int nsplit = (n_total + DA_SPL - 1) / DA_SPL;
  const float sl2 = p.sm_scale * kLog2e;
  float* part = static_cast<float*>(ws);
  dim3 grid(nsplit, p.B * p.Hkv);
  const bf16* Qn = static_cast<const bf16*>(q_new);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  if (p.D == 128)
    decode_attn_split_kernel<128><<<grid, 256, 0, st>>>(Qn, K, V, p.Hq, p.Hkv, p.r, n_total,
                                                        nsplit, sl2, part);
  else
    decode_attn_split_kernel<64><<<grid, 256, 0, st>>>(Qn, K, V, p.Hq, p.Hkv, p.r, n_total,
                                                       nsplit, sl2, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 128)
    decode_attn_combine_kernel<128><<<p.B * p.Hq, 64, 0, st>>>(part, nsplit,
                                                               static_cast<bf16*>(out));
  else
    decode_attn_combine_kernel<64><<<p.B * p.Hq, 64, 0, st>>>(part, nsplit,
                                                              static_cast<bf16*>(out));
  return hipGetLastError();
}

}  // namespace egs
