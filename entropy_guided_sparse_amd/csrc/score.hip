// K1 key-block mean pooling and K2 probe observation rows + entropy.
//
// Method: EntropyInfer (arXiv 2606.09508) Sec. 4.2 builds a small
// "observation attention matrix" over key blocks and takes the entropy of
// each of its rows; App. A eq. (1) sizes it C_S x C_B.  Here a key block is
// represented by the mean of its keys and a segment by its last P queries;
// each probe query's softmax over the causal blocks is averaged over the
// probe (InfoKV window-mean score, eq. 4; EntroPrefill Sec. 2.1 observer
// pool) and the Shannon or Renyi entropy of that row is reported
// (EntroPrefill Sec. 3.1).  The softmax statistics use the online max / sum
// recurrence of EntroPrefill Sec. 8.1.
//
// gfx950 design:
//  * K1 streams K once from HBM (16-byte loads along d, fp32 sums) and writes
//    the block means as a bf16 hi/lo pair, so the probe logits can run on
//    bf16 MFMA with ~2^-17 relative error (two MFMAs per product).
//  * K2 splits the causal blocks of every (segment, KV group) into chunks of
//    64 blocks; a workgroup stages one chunk's hi/lo block means in LDS once
//    and scores the probe rows of all r heads of the group against it on
//    v_mfma_f32_32x32x16_bf16.  Four kernels, no logits stored:
//      probe_stats   blocks as M: a lane owns a probe row; the chunk's row
//                    maximum and sum of exponentials;
//      probe_combine the chunks' (max, sum) pairs folded into each row's
//                    maximum and 1/sum;
//      probe_mass    blocks as N: a lane owns a block; the probe-averaged mass
//                    is a register sum, written as the block's score, with
//                    the chunk's entropy partial sum;
//      probe_entropy the partial sums of every (head, segment) added in chunk
//                    order.
//    Work items run on a 1-D grid with every chunk of a (segment, group) on
//    one XCD, so its probe queries and block means are fetched into one L2.
#include <algorithm>

#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

// ---------------------------------------------------------------------------
// K1: kbar[g, j, :] = mean of keys j*LB .. (j+1)*LB-1 of KV head g.
// One workgroup per (block, KV head); thread = (row phase, 8-wide d chunk).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_keys_kernel(const T* __restrict__ K, int N,
                                                        int LB, int CB,
                                                        bf16* __restrict__ kb_hi,
                                                        bf16* __restrict__ kb_lo) {
  constexpr int CH = D / 8;        // 8-element chunks per key row
  constexpr int RP = 256 / CH;     // key rows covered per pass
  __shared__ float red[RP][D];
  const int j = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, c = tid % CH, ro = tid / CH;
  const T* base = K + ((size_t)g * N + (size_t)j * LB) * D + c * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // four rows in flight per step
  for (int r0 = ro; r0 < LB; r0 += 4 * RP) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u * RP;
      if (r < LB) {
        load8f(base + (size_t)r * D, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[u][e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[ro][c * 8 + e] = acc[e];
  __syncthreads();
  for (int col = tid; col < D; col += 256) {
    float s = 0.f;
    for (int q = 0; q < RP; ++q) s += red[q][col];
    const float mean = s / (float)LB;
    const bf16 hi = f2bf(mean);
    const bf16 lo = f2bf(mean - bf2f(hi));
    const size_t o = ((size_t)g * CB + j) * D + col;
    kb_hi[o] = hi;
    kb_lo[o] = lo;
  }
}

// ---------------------------------------------------------------------------
// K2: probe observation rows and entropy, in 64-block chunks.
//
// Work item (chunk of SC_CK key blocks, segment s, KV group g); the r query
// heads of the group share the chunk's pooled keys, staged once in LDS.
//   probe_stats:   per probe row, the maximum and the sum of exp of its logits
//                  over the chunk's causal blocks (online softmax statistics).
//   probe_combine: one thread per (head, segment, probe row) folds the chunk
//                  statistics into the row's maximum and 1/sum.
//   probe_mass:    recomputes the chunk's logits with blocks as the MFMA N
//                  dimension (a lane owns a block) and sums the normalised
//                  probabilities over the probe rows: a_bar for the chunk's
//                  blocks, plus the chunk's partial entropy sum.  Chunks past
//                  the segment's causal range write the -1 sentinels.
//   probe_entropy: one thread per (head, segment) adds the partial sums, in
//                  chunk order, into E.
// Every workgroup issues its global loads before it waits on any of them.
// ---------------------------------------------------------------------------
constexpr int SC_CK = 64;     // key blocks per chunk
constexpr int SC_RT = 2;      // probe row tiles (32 rows) in registers at once (stats)
constexpr int SC_RTM = 1;     // the same for the mass pass

struct ScoreLayout {
  size_t kb_hi, kb_lo, stat_m, stat_l, row_m, row_inv, ent, total;
  int nch;
};

static size_t sc_align(size_t x) {
  return (x + 255) / 256 * 256;
}

static ScoreLayout score_layout(const PrefillDims& p) {
  ScoreLayout o;
  o.nch = (p.CB + SC_CK - 1) / SC_CK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += sc_align(bytes);
    return at;
  };
  o.kb_hi = take((size_t)p.Hkv * p.CB * p.D * sizeof(bf16));
  o.kb_lo = take((size_t)p.Hkv * p.CB * p.D * sizeof(bf16));
  const size_t rows = (size_t)p.Hq * p.CS * p.P;
  o.stat_m = take(rows * o.nch * sizeof(float));
  o.stat_l = take(rows * o.nch * sizeof(float));
  o.row_m = take(rows * sizeof(float));
  o.row_inv = take(rows * sizeof(float));
  o.ent = take((size_t)p.Hq * p.CS * o.nch * sizeof(float));
  o.total = off;
  return o;
}

size_t score_workspace_bytes(const PrefillDims& p) {
  return std::max(score_layout(p).total, maxmin_workspace_bytes(p));
}

template <typename TQ>
struct QFrag;

template <>
struct QFrag<bf16> {
  static constexpr bool kSplit = false;
  typedef bf16x8 raw_t;
  __device__ static raw_t load(const bf16* p, bool valid) {
    raw_t v;
    if (valid) {
      v = load8(p);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
    }
    return v;
  }
  __device__ static void split(const raw_t& v, bf16x8& hi, bf16x8& lo) {
    hi = v;
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = (bf16)0.f;
  }
};

template <>
struct QFrag<float> {
  static constexpr bool kSplit = true;
  struct raw_t {
    float x[8];
  };
  __device__ static raw_t load(const float* p, bool valid) {
    raw_t v;
    if (valid) {
      load8f(p, v.x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v.x[e] = 0.f;
    }
    return v;
  }
  __device__ static void split(const raw_t& v, bf16x8& hi, bf16x8& lo) { split8(v.x, hi, lo); }
};

// XOR swizzle of the 16-byte chunks of a D-wide bf16 row in LDS
template <int D>
__device__ __forceinline__ int kbar_swz(int row) {
  return lds_swz<D * 2>(row);
}

// Stage the hi / lo pooled keys of blocks c0 .. c0 + nb - 1 (zero beyond) in
// LDS, 16-byte chunks XOR-swizzled by row; all loads are issued first.
template <int D>
__device__ __forceinline__ void stage_kbar(bf16* kh, bf16* kl, const bf16* KH, const bf16* KL,
                                           int c0, int nb) {
  constexpr int KCH = D / 8;
  constexpr int PER = (SC_CK * KCH + 255) / 256;
  u32x4 vh[PER], vl[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int row = q / KCH, c8 = q % KCH;
    vh[i] = u32x4{0u, 0u, 0u, 0u};
    vl[i] = u32x4{0u, 0u, 0u, 0u};
    if (q < SC_CK * KCH && row < nb) {
      const size_t o = (size_t)(c0 + row) * D + c8 * 8;
      vh[i] = *reinterpret_cast<const u32x4*>(KH + o);
      vl[i] = *reinterpret_cast<const u32x4*>(KL + o);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = threadIdx.x + 256 * i;
    if (q < SC_CK * KCH) {
      const int row = q / KCH, c8 = q % KCH;
      const int at = row * D + ((c8 ^ kbar_swz<D>(row)) * 8);
      *reinterpret_cast<u32x4*>(kh + at) = vh[i];
      *reinterpret_cast<u32x4*>(kl + at) = vl[i];
    }
  }
}

// 1-D grid -> (chunk, segment, KV group) with every chunk of one (segment,
// group) pair on the same XCD (workgroup id mod 8), so the pair's probe
// queries and pooled keys are fetched into one L2 only.  Within every run of
// eight pairs XCD x takes pair 8m + ((x - m) mod 8), so the pairs rotate over
// the XCDs and the causal segments' unequal work spreads evenly.  Returns
// false for the padding ids of the last, partial group of eight pairs.
__device__ __forceinline__ bool probe_item(int bid, int nch, int CS, int Hkv, int& ch, int& s,
                                           int& g) {
  const int xcd = bid & 7, k = bid >> 3;
  ch = k % nch;
  const int m = k / nch;
  const int pair = 8 * m + ((xcd - m) & 7);
  if (pair >= CS * Hkv) return false;
  g = pair / CS;
  s = pair % CS;
  return true;
}

// 16 bf16 of pooled-key row `row`, d chunk (2c + hg), from the swizzled stage
template <int D>
__device__ __forceinline__ bf16x8 kbar_frag(const bf16* k, int row, int c, int hg) {
  return load8(k + row * D + (((2 * c + hg) ^ kbar_swz<D>(row)) * 8));
}

template <typename TQ, int D>
__global__ __launch_bounds__(256) void probe_stats_kernel(
    const TQ* __restrict__ Q, const bf16* __restrict__ kb_hi, const bf16* __restrict__ kb_lo,
    int Hq, int r, int N, int LS, int LB, int P, int CS, int CB, int nch, float scale_log2,
    float* __restrict__ stat_m, float* __restrict__ stat_l) {
  constexpr int NC = D / 16;
  typedef typename QFrag<TQ>::raw_t raw_t;
  __shared__ __attribute__((aligned(16))) bf16 kh[SC_CK * D];
  __shared__ __attribute__((aligned(16))) bf16 kl[SC_CK * D];
  int ch, s, g;
  if (!probe_item(blockIdx.x, nch, CS, Hq / r, ch, s, g)) return;
  const int cb = (s + 1) * (LS / LB);
  const int c0 = ch * SC_CK;
  if (c0 >= cb) return;
  const int nb = min(SC_CK, cb - c0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const size_t u_begin = (size_t)(s + 1) * LS - P;
  const int nrt = (P + 31) / 32;
  // (head, row tile) work items of this wave, SC_RT row tiles per round
  for (int it0 = w * SC_RT; it0 < r * nrt; it0 += 4 * SC_RT) {
    raw_t qr[SC_RT][NC];
#pragma unroll
    for (int t = 0; t < SC_RT; ++t) {
      const int it = it0 + t;
      const int hl = it / nrt, rt = it % nrt;
      const int urow = rt * 32 + l32;
      const bool ok = it < r * nrt && urow < P;
      const TQ* qp = Q + ((size_t)(g * r + (ok ? hl : 0)) * N + u_begin + (ok ? urow : 0)) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) qr[t][c] = QFrag<TQ>::load(qp + 16 * c + 8 * hg, ok);
    }
    if (it0 == w * SC_RT) {
      stage_kbar<D>(kh, kl, kb_hi + (size_t)g * CB * D, kb_lo + (size_t)g * CB * D, c0, nb);
      __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < SC_RT; ++t) {
      const int it = it0 + t;
      if (it >= r * nrt) break;
      const int hl = it / nrt, rt = it % nrt;
      const int urow = rt * 32 + l32;
      bf16x8 qh[NC], ql[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) QFrag<TQ>::split(qr[t][c], qh[c], ql[c]);
      float m = kNegBig, l = 0.f;
      for (int bt = 0; bt * 32 < nb; ++bt) {
        floatx16 zt;
#pragma unroll
        for (int i = 0; i < 16; ++i) zt[i] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 ah = kbar_frag<D>(kh, bt * 32 + l32, c, hg);
          const bf16x8 al = kbar_frag<D>(kl, bt * 32 + l32, c, hg);
          zt = mfma32(ah, qh[c], zt);
          zt = mfma32(al, qh[c], zt);
          if (QFrag<TQ>::kSplit) zt = mfma32(ah, ql[c], zt);
        }
        float tmax = kNegBig;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = (bt * 32 + acc_row(i, lane) < nb) ? zt[i] * scale_log2 : -INFINITY;
          zt[i] = v;
          tmax = fmaxf(tmax, v);
        }
        const float mn = fmaxf(m, tmax);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += fast_exp2(zt[i] - mn);
        l = l * fast_exp2(m - mn) + sum;
        m = mn;
      }
      const float M = xhalf_max(m);
      const float Lr = xhalf_sum(l * fast_exp2(m - M));
      if (hg == 0 && urow < P) {
        const size_t o = (((size_t)(g * r + hl) * CS + s) * nch + ch) * P + urow;
        stat_m[o] = M;
        stat_l[o] = Lr;
      }
    }
  }
  // waves without work items still take part in the staging barrier
  if (w * SC_RT >= r * nrt) {
    stage_kbar<D>(kh, kl, kb_hi + (size_t)g * CB * D, kb_lo + (size_t)g * CB * D, c0, nb);
    __syncthreads();
  }
}

// one thread per (head, segment, probe row): the row's maximum and 1/sum
__global__ __launch_bounds__(256) void probe_combine_kernel(
    const float* __restrict__ stat_m, const float* __restrict__ stat_l, int CS, int P, int nch,
    int bps, int total, float* __restrict__ row_m, float* __restrict__ row_inv) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int u = i % P, hs = i / P, s = hs % CS;
  const int nch_s = ((s + 1) * bps + SC_CK - 1) / SC_CK;
  const float* sm = stat_m + (size_t)hs * nch * P + u;
  const float* sl = stat_l + (size_t)hs * nch * P + u;
  // chunks in rounds of eight, loads issued together (index clamped), the
  // running maximum raised per round
  float M = kNegBig, L = 0.f;
  for (int c0 = 0; c0 < nch_s; c0 += 8) {
    float m8[8], l8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t c = (size_t)min(c0 + j, nch_s - 1) * P;
      m8[j] = sm[c];
      l8[j] = sl[c];
    }
    float bm = M;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nch_s) bm = fmaxf(bm, m8[j]);
    L *= fast_exp2(M - bm);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nch_s) L += l8[j] * fast_exp2(m8[j] - bm);
    M = bm;
  }
  row_m[i] = M;
  row_inv[i] = L > 0.f ? 1.0f / L : 0.f;
}

template <typename TQ, int D>
__global__ __launch_bounds__(256) void probe_mass_kernel(
    const TQ* __restrict__ Q, const bf16* __restrict__ kb_hi, const bf16* __restrict__ kb_lo,
    int Hq, int r, int N, int LS, int LB, int P, int CS, int CB, int nch, float scale_log2,
    int kind, float alpha, const float* __restrict__ row_m, const float* __restrict__ row_inv,
    float* __restrict__ ent, float* __restrict__ scores) {
  constexpr int NC = D / 16;
  constexpr int BT = SC_CK / 32;
  typedef typename QFrag<TQ>::raw_t raw_t;
  __shared__ __attribute__((aligned(16))) bf16 kh[SC_CK * D];
  __shared__ __attribute__((aligned(16))) bf16 kl[SC_CK * D];
  int ch, s, g;
  if (!probe_item(blockIdx.x, nch, CS, Hq / r, ch, s, g)) return;
  const int cb = (s + 1) * (LS / LB);
  const int c0 = ch * SC_CK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const int cend = min(CB, c0 + SC_CK);
  if (c0 >= cb) {   // beyond the causal range: sentinels only
    for (int hl = 0; hl < r; ++hl) {
      float* out = scores + ((size_t)(g * r + hl) * CS + s) * CB;
      for (int j = c0 + tid; j < cend; j += 256) out[j] = -1.0f;
    }
    return;
  }
  const int nb = min(SC_CK, cb - c0);
  const size_t u_begin = (size_t)(s + 1) * LS - P;
  const float invP = 1.0f / (float)P;
  const int nrt = (P + 31) / 32;
  bool staged = false;
  // one head per wave at a time; its row tiles SC_RT at a time
  for (int hl = w; hl < r; hl += 4) {
    const int h = g * r + hl;
    const size_t rbase = ((size_t)h * CS + s) * P;
    float acc[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) acc[bt] = 0.f;
    for (int rt0 = 0; rt0 < nrt; rt0 += SC_RTM) {
      raw_t qr[SC_RTM][NC];
      float mown[SC_RTM], iown[SC_RTM];
#pragma unroll
      for (int t = 0; t < SC_RTM; ++t) {
        const int urow = (rt0 + t) * 32 + l32;
        const bool ok = rt0 + t < nrt && urow < P;
        const TQ* qp = Q + ((size_t)h * N + u_begin + (ok ? urow : 0)) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) qr[t][c] = QFrag<TQ>::load(qp + 16 * c + 8 * hg, ok);
        // rows past the probe keep M = 0 and 1/L = 0: their zero logits add nothing
        mown[t] = ok ? row_m[rbase + urow] : 0.f;
        iown[t] = ok ? row_inv[rbase + urow] : 0.f;
      }
      if (!staged) {
        stage_kbar<D>(kh, kl, kb_hi + (size_t)g * CB * D, kb_lo + (size_t)g * CB * D, c0, nb);
        __syncthreads();
        staged = true;
      }
#pragma unroll
      for (int t = 0; t < SC_RTM; ++t) {
        if (rt0 + t >= nrt) break;
        // registers of the mass pass hold rows acc_row(i, lane): fetch their stats
        float rm[16], ri[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          rm[i] = __shfl(mown[t], acc_row(i, lane));
          ri[i] = __shfl(iown[t], acc_row(i, lane));
        }
        bf16x8 qh[NC], ql[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) QFrag<TQ>::split(qr[t][c], qh[c], ql[c]);
#pragma unroll
        for (int bt = 0; bt < BT; ++bt) {
          if (bt * 32 >= nb) break;
          floatx16 z;
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const bf16x8 bh = kbar_frag<D>(kh, bt * 32 + l32, c, hg);
            const bf16x8 bl = kbar_frag<D>(kl, bt * 32 + l32, c, hg);
            z = mfma32(qh[c], bh, z);
            z = mfma32(qh[c], bl, z);
            if (QFrag<TQ>::kSplit) z = mfma32(ql[c], bh, z);
          }
          float colsum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            colsum += fast_exp2(__builtin_fmaf(z[i], scale_log2, -rm[i])) * ri[i];
          acc[bt] += xhalf_sum(colsum);
        }
      }
    }
    float* out = scores + ((size_t)h * CS + s) * CB;
    float epart = 0.f;
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) {
      const int jl = bt * 32 + l32;
      if (hg == 0 && jl < nb) {
        const float a = acc[bt] * invP;
        out[c0 + jl] = a;
        if (a > 0.f) epart += (kind == EGS_SHANNON) ? -a * logf(a) : powf(a, alpha);
      }
    }
    for (int j = c0 + nb + lane; j < cend; j += 64) out[j] = -1.0f;
    epart = wave_sum(epart);
    if (lane == 0) ent[((size_t)h * CS + s) * nch + ch] = epart;
  }
  // waves without a head still take part in the staging barrier
  if (!staged) {
    stage_kbar<D>(kh, kl, kb_hi + (size_t)g * CB * D, kb_lo + (size_t)g * CB * D, c0, nb);
    __syncthreads();
  }
}

// one thread per (head, segment): E from the chunks' partial sums, in order
__global__ __launch_bounds__(256) void probe_entropy_kernel(const float* __restrict__ ent,
                                                            int Hq, int CS, int nch, int bps,
                                                            int kind, float alpha,
                                                            float* __restrict__ entropy) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= Hq * CS) return;
  const int s = i % CS;
  const int nch_s = ((s + 1) * bps + SC_CK - 1) / SC_CK;
  const float* e = ent + (size_t)i * nch;
  float tot = 0.f;
  for (int c = 0; c < nch_s; ++c) tot += e[c];
  entropy[i] = (kind == EGS_SHANNON) ? tot : logf(tot) / (1.0f - alpha);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t pool_dispatch(const PrefillDims& p, const void* k, bf16* hi, bf16* lo,
                                hipStream_t st) {
  dim3 grid(p.CB, p.Hkv);
  const T* K = static_cast<const T*>(k);
#define EGS_POOL(DD) pool_keys_kernel<T, DD><<<grid, 256, 0, st>>>(K, p.N, p.LB, p.CB, hi, lo)
  switch (p.D) {
    case 16: EGS_POOL(16); break;
    case 32: EGS_POOL(32); break;
    case 64: EGS_POOL(64); break;
    case 128: EGS_POOL(128); break;
    default: return hipErrorInvalidValue;
  }
#undef EGS_POOL
  return hipGetLastError();
}

template <typename TQ>
static hipError_t probe_dispatch(const PrefillDims& p, const ScoreLayout& ly, const void* q,
                                 char* ws, int kind, float alpha, float* scores,
                                 float* entropy, hipStream_t st) {
  const int grid = ((p.CS * p.Hkv + 7) / 8) * ly.nch * 8;
  const float sl2 = p.sm_scale * kLog2e;
  const int bps = p.LS / p.LB;
  const TQ* Q = static_cast<const TQ*>(q);
  const bf16* H = reinterpret_cast<const bf16*>(ws + ly.kb_hi);
  const bf16* L = reinterpret_cast<const bf16*>(ws + ly.kb_lo);
  float* sm = reinterpret_cast<float*>(ws + ly.stat_m);
  float* sl = reinterpret_cast<float*>(ws + ly.stat_l);
  float* rm = reinterpret_cast<float*>(ws + ly.row_m);
  float* ri = reinterpret_cast<float*>(ws + ly.row_inv);
  float* en = reinterpret_cast<float*>(ws + ly.ent);
  const int rows = p.Hq * p.CS * p.P;
  hipError_t e;
#define EGS_STATS(DD)                                                                      \
  probe_stats_kernel<TQ, DD><<<grid, 256, 0, st>>>(Q, H, L, p.Hq, p.r, p.N, p.LS, p.LB,   \
                                                    p.P, p.CS, p.CB, ly.nch, sl2, sm, sl)
#define EGS_MASS(DD)                                                                      \
  probe_mass_kernel<TQ, DD><<<grid, 256, 0, st>>>(Q, H, L, p.Hq, p.r, p.N, p.LS, p.LB,   \
                                                   p.P, p.CS, p.CB, ly.nch, sl2, kind,     \
                                                   alpha, rm, ri, en, scores)
  switch (p.D) {
    case 16: EGS_STATS(16); break;
    case 32: EGS_STATS(32); break;
    case 64: EGS_STATS(64); break;
    case 128: EGS_STATS(128); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  probe_combine_kernel<<<(rows + 255) / 256, 256, 0, st>>>(sm, sl, p.CS, p.P, ly.nch, bps, rows,
                                                           rm, ri);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (p.D) {
    case 16: EGS_MASS(16); break;
    case 32: EGS_MASS(32); break;
    case 64: EGS_MASS(64); break;
    case 128: EGS_MASS(128); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
#undef EGS_STATS
#undef EGS_MASS
  probe_entropy_kernel<<<(p.Hq * p.CS + 255) / 256, 256, 0, st>>>(en, p.Hq, p.CS, ly.nch, bps,
                                                                  kind, alpha, entropy);
  return hipGetLastError();
}

hipError_t launch_entropy_score(const PrefillDims& p, const void* q, const void* k, int kind,
                                float alpha, float* scores, float* entropy, void* ws,
                                hipStream_t st) {
  const ScoreLayout ly = score_layout(p);
  char* w = static_cast<char*>(ws);
  bf16* hi = reinterpret_cast<bf16*>(w + ly.kb_hi);
  bf16* lo = reinterpret_cast<bf16*>(w + ly.kb_lo);
  hipError_t e = p.dtype == EGS_F32 ? pool_dispatch<float>(p, k, hi, lo, st)
                                    : pool_dispatch<bf16>(p, k, hi, lo, st);
  if (e != hipSuccess) return e;
  return p.dtype == EGS_F32
             ? probe_dispatch<float>(p, ly, q, w, kind, alpha, scores, entropy, st)
             : probe_dispatch<bf16>(p, ly, q, w, kind, alpha, scores, entropy, st);
}

}  // namespace egs
