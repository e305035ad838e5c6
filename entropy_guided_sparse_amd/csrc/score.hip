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
//  * K2 runs one workgroup per (head, segment), heaviest segments first.  Each
//    32-row probe tile is scored against 32-block tiles with
//    v_mfma_f32_32x32x16_bf16 twice: pass 1 with blocks as the M dimension
//    (a lane owns a probe row: running max / sum in registers), pass 2 with
//    blocks as the N dimension (a lane owns a block: the probe average is a
//    register sum).  No logits are stored.
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
// K2: probe observation rows and entropy.
// ---------------------------------------------------------------------------
template <typename TQ>
struct QFrag;

template <>
struct QFrag<bf16> {
  static constexpr bool kSplit = false;
  __device__ static void load(const bf16* p, bool valid, bf16x8& hi, bf16x8& lo) {
    if (valid) {
      hi = load8(p);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hi[e] = (bf16)0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = (bf16)0.f;
  }
};

template <>
struct QFrag<float> {
  static constexpr bool kSplit = true;
  __device__ static void load(const float* p, bool valid, bf16x8& hi, bf16x8& lo) {
    float x[8];
    if (valid) {
      load8f(p, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    split8(x, hi, lo);
  }
};

template <typename TQ, int D>
__global__ __launch_bounds__(256) void probe_score_kernel(
    const TQ* __restrict__ Q, const bf16* __restrict__ kb_hi,
    const bf16* __restrict__ kb_lo, int Hq, int r, int N, int LS, int LB, int P,
    int CS, int CB, float scale_log2, int kind, float alpha,
    float* __restrict__ scores, float* __restrict__ entropy) {
  constexpr int NC = D / 16;
  extern __shared__ float acc[];          // probe-summed block mass, per block
  __shared__ float st_m[4][32], st_l[4][32];
  __shared__ float rowM[32], rowInvL[32];
  __shared__ float red[4];

  const int wid = blockIdx.x;
  const int s = CS - 1 - wid / Hq;        // heaviest segments first
  const int h = wid % Hq, g = h / r;
  const int cb = (s + 1) * (LS / LB);
  const int NT = (cb + 31) / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;

  for (int j = tid; j < NT * 32; j += 256) acc[j] = 0.f;

  const size_t u_begin = (size_t)(s + 1) * LS - P;
  const TQ* Qh = Q + (size_t)h * N * D;
  const bf16* KH = kb_hi + (size_t)g * CB * D;
  const bf16* KL = kb_lo + (size_t)g * CB * D;
  bf16x8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = (bf16)0.f;

  for (int rt = 0; rt * 32 < P; ++rt) {
    const int urow = rt * 32 + l32;
    const bool rvalid = urow < P;
    bf16x8 qh[NC], ql[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      QFrag<TQ>::load(Qh + (u_begin + urow) * D + 16 * c + 8 * hg, rvalid, qh[c], ql[c]);

    // ---- pass 1: running max / sum per probe row (lane owns a row) ----
    float m = kNegBig, l = 0.f;
    for (int t = w; t < NT; t += 4) {
      const int blk = t * 32 + l32;
      const bool bvalid = blk < cb;
      floatx16 zt;
#pragma unroll
      for (int i = 0; i < 16; ++i) zt[i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const size_t off = (size_t)blk * D + 16 * c + 8 * hg;
        const bf16x8 ah = bvalid ? load8(KH + off) : zero8;
        const bf16x8 al = bvalid ? load8(KL + off) : zero8;
        zt = mfma32(ah, qh[c], zt);
        zt = mfma32(al, qh[c], zt);
        if (QFrag<TQ>::kSplit) zt = mfma32(ah, ql[c], zt);
      }
      float tmax = kNegBig;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int bi = t * 32 + acc_row(i, lane);
        const float v = (bi < cb) ? zt[i] * scale_log2 : -INFINITY;
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
    {
      const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
      const float M = fmaxf(m, m2);
      const float Lr = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
      if (hg == 0) {
        st_m[w][l32] = M;
        st_l[w][l32] = Lr;
      }
    }
    __syncthreads();
    if (tid < 32) {
      float M = st_m[0][tid];
#pragma unroll
      for (int q = 1; q < 4; ++q) M = fmaxf(M, st_m[q][tid]);
      float Lr = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) Lr += st_l[q][tid] * fast_exp2(st_m[q][tid] - M);
      rowM[tid] = M;
      rowInvL[tid] = (rt * 32 + tid < P && Lr > 0.f) ? 1.0f / Lr : 0.f;
    }
    __syncthreads();

    // ---- pass 2: probe-summed softmax mass per block (lane owns a block) ----
    float rm[16], ril[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      rm[i] = rowM[acc_row(i, lane)];
      ril[i] = rowInvL[acc_row(i, lane)];
    }
    for (int t = w; t < NT; t += 4) {
      const int blk = t * 32 + l32;
      const bool bvalid = blk < cb;
      floatx16 z;
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const size_t off = (size_t)blk * D + 16 * c + 8 * hg;
        const bf16x8 bh = bvalid ? load8(KH + off) : zero8;
        const bf16x8 bl = bvalid ? load8(KL + off) : zero8;
        z = mfma32(qh[c], bh, z);
        z = mfma32(qh[c], bl, z);
        if (QFrag<TQ>::kSplit) z = mfma32(ql[c], bh, z);
      }
      float colsum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) colsum += fast_exp2(z[i] * scale_log2 - rm[i]) * ril[i];
      colsum += __shfl_xor(colsum, 32);
      if (hg == 0 && bvalid) acc[blk] += colsum;
    }
    __syncthreads();
  }

  // ---- finalize: a_bar = mass / P, sentinel -1 beyond C_B(s), entropy ----
  float epart = 0.f;
  float* out = scores + ((size_t)h * CS + s) * CB;
  const float fP = (float)P;
  for (int j = tid; j < CB; j += 256) {
    if (j < cb) {
      const float a = acc[j] / fP;
      out[j] = a;
      if (a > 0.f) epart += (kind == EGS_SHANNON) ? -a * logf(a) : powf(a, alpha);
    } else {
      out[j] = -1.0f;
    }
  }
  epart = wave_sum(epart);
  if (lane == 0) red[w] = epart;
  __syncthreads();
  if (tid == 0) {
    const float tot = red[0] + red[1] + red[2] + red[3];
    entropy[(size_t)h * CS + s] = (kind == EGS_SHANNON) ? tot : logf(tot) / (1.0f - alpha);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t pool_dispatch(const PrefillDims& p, const void* k, void* hi, void* lo,
                                hipStream_t st) {
  dim3 grid(p.CB, p.Hkv);
  const T* K = static_cast<const T*>(k);
  bf16* H = static_cast<bf16*>(hi);
  bf16* L = static_cast<bf16*>(lo);
  switch (p.D) {
    case 16: pool_keys_kernel<T, 16><<<grid, 256, 0, st>>>(K, p.N, p.LB, p.CB, H, L); break;
    case 32: pool_keys_kernel<T, 32><<<grid, 256, 0, st>>>(K, p.N, p.LB, p.CB, H, L); break;
    case 64: pool_keys_kernel<T, 64><<<grid, 256, 0, st>>>(K, p.N, p.LB, p.CB, H, L); break;
    case 128: pool_keys_kernel<T, 128><<<grid, 256, 0, st>>>(K, p.N, p.LB, p.CB, H, L); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pool_keys(const PrefillDims& p, const void* k, void* kb_hi, void* kb_lo,
                            hipStream_t st) {
  return p.dtype == EGS_F32 ? pool_dispatch<float>(p, k, kb_hi, kb_lo, st)
                            : pool_dispatch<bf16>(p, k, kb_hi, kb_lo, st);
}

template <typename TQ>
static hipError_t probe_dispatch(const PrefillDims& p, const void* q, const void* hi,
                                 const void* lo, int kind, float alpha, float* scores,
                                 float* entropy, hipStream_t st) {
  const int grid = p.CS * p.Hq;
  const size_t lds = (size_t)((p.CB + 31) / 32) * 32 * sizeof(float);
  const float sl2 = p.sm_scale * kLog2e;
  const TQ* Q = static_cast<const TQ*>(q);
  const bf16* H = static_cast<const bf16*>(hi);
  const bf16* L = static_cast<const bf16*>(lo);
#define EGS_PROBE(DD)                                                                    \
  probe_score_kernel<TQ, DD><<<grid, 256, lds, st>>>(Q, H, L, p.Hq, p.r, p.N, p.LS, p.LB, \
                                                     p.P, p.CS, p.CB, sl2, kind, alpha,  \
                                                     scores, entropy)
  switch (p.D) {
    case 16: EGS_PROBE(16); break;
    case 32: EGS_PROBE(32); break;
    case 64: EGS_PROBE(64); break;
    case 128: EGS_PROBE(128); break;
    default: return hipErrorInvalidValue;
  }
#undef EGS_PROBE
  return hipGetLastError();
}

hipError_t launch_probe_score(const PrefillDims& p, const void* q, const void* kb_hi,
                              const void* kb_lo, int kind, float alpha, float* scores,
                              float* entropy, hipStream_t st) {
  return p.dtype == EGS_F32
             ? probe_dispatch<float>(p, q, kb_hi, kb_lo, kind, alpha, scores, entropy, st)
             : probe_dispatch<bf16>(p, q, kb_hi, kb_lo, kind, alpha, scores, entropy, st);
}

}  // namespace egs
