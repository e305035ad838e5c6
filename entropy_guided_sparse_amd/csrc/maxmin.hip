// K1b / K2b: the paper-literal observation rows from max / min representatives.
//
// Method: EntropyInfer (arXiv 2606.09508) Sec. 4.2, Alg. 1 represents every
// segment by the element-wise maximum and minimum of its queries over the
// segment's tokens (Q_Max, Q_Min) and forms key representatives the same way
// (taken per key block: K_Max, K_Min).  Alg. 2 scores the four pairings of
// query and key representatives, takes a softmax over the causal blocks for
// each, averages the two pairings that share a query representative and keeps
// the element-wise maximum of the two averages.  Readings: the 1/sqrt(d)
// scale is applied (Alg. 2 leaves it out) and the max-combined row, which does
// not sum to one, is renormalised before its entropy is taken.
//
// gfx950 design:
//  * pool_maxmin: one workgroup per (chunk of rows, head); 16-byte loads along
//    d, running max / min in registers, an LDS reduction over the row phases.
//    The max and min of stored values are stored values, so the
//    representatives are exact in the input type.  Queries are pooled in
//    chunks of up to 1024 rows (the score kernel folds the chunks of a
//    segment), keys per block.  One pass over Q and one over K: HBM-bound.
//  * maxmin_score: one workgroup per (head, segment), latest segment first; a
//    thread per causal block computes the four dot products against the two
//    query representatives held in LDS, in fp64: representatives of planted
//    or outlying tokens give logits of 1e4 and more, where an fp32 sum would
//    move the softmax visibly (the work is tiny, 4 d FMAs per block).  The
//    logits wait in the workspace while block-wide reductions give the four
//    maxima (fp64), the four sums, the normaliser of the max-combined row and
//    its entropy (fp32, on the differences to the maxima).
#include <algorithm>

#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

constexpr int MM_QCH_MAX = 1024;   // query rows pooled per chunk, at most

struct MaxMinLayout {
  size_t kmx, kmn, qmx, qmn, z, total;
  int qch;   // query rows per pooled chunk (divides L_S, a multiple of L_B)
};

static MaxMinLayout mm_layout(const PrefillDims& p) {
  MaxMinLayout o;
  const int ratio = p.LS / p.LB;
  int f = std::min(ratio, std::max(1, MM_QCH_MAX / p.LB));
  while (ratio % f) --f;
  o.qch = p.LB * f;
  const size_t elt = p.dtype == EGS_F32 ? 4 : 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  const size_t nk = (size_t)p.Hkv * p.CB * p.D * elt;
  const size_t nq = (size_t)p.Hq * (p.N / o.qch) * p.D * elt;
  o.kmx = take(nk);
  o.kmn = take(nk);
  o.qmx = take(nq);
  o.qmn = take(nq);
  o.z = take((size_t)p.Hq * p.CS * 4 * p.CB * sizeof(double));
  o.total = off;
  return o;
}

size_t maxmin_workspace_bytes(const PrefillDims& p) {
  return mm_layout(p).total;
}

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  typedef float __attribute__((ext_vector_type(4))) type;
};

// ---------------------------------------------------------------------------
// pool_maxmin: mx[h, c, :] / mn[h, c, :] = element-wise max / min of rows
// c*Lc .. (c+1)*Lc-1 of X[h].  Workgroup = (chunk c, head h); thread = (row
// phase, 16-byte vector along d).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_maxmin_kernel(const T* __restrict__ X, int N, int Lc,
                                                          int nchunk, T* __restrict__ mx,
                                                          T* __restrict__ mn) {
  typedef typename Vec16<T>::type vec_t;
  constexpr int EPV = Vec16<T>::N;   // elements per 16-byte vector
  constexpr int NV = D / EPV;        // vectors per row
  constexpr int PH = 256 / NV;       // row phases
  __shared__ float smx[PH * D];
  __shared__ float smn[PH * D];
  const int c = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, v = tid % NV, ph = tid / NV;
  const T* src = X + ((size_t)h * N + (size_t)c * Lc) * D + v * EPV;
  float a[EPV], b[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    a[e] = -INFINITY;
    b[e] = INFINITY;
  }
  int row = ph;
  // eight loads in flight per thread, then the remainder
  for (; row + 7 * PH < Lc; row += 8 * PH) {
    vec_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = *reinterpret_cast<const vec_t*>(src + (size_t)(row + u * PH) * D);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float t = (float)x[u][e];
        a[e] = fmaxf(a[e], t);
        b[e] = fminf(b[e], t);
      }
  }
  for (; row < Lc; row += PH) {
    const vec_t x = *reinterpret_cast<const vec_t*>(src + (size_t)row * D);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float t = (float)x[e];
      a[e] = fmaxf(a[e], t);
      b[e] = fminf(b[e], t);
    }
  }
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    smx[ph * D + v * EPV + e] = a[e];
    smn[ph * D + v * EPV + e] = b[e];
  }
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float m = smx[d], n = smn[d];
    for (int q = 1; q < PH; ++q) {
      m = fmaxf(m, smx[q * D + d]);
      n = fminf(n, smn[q * D + d]);
    }
    // m and n are input values, so the conversion back is exact
    mx[((size_t)h * nchunk + c) * D + d] = (T)m;
    mn[((size_t)h * nchunk + c) * D + d] = (T)n;
  }
}

// block-wide reductions over 256 threads (four wavefronts); every thread gets
// the result
template <typename F, int K, bool MAX>
__device__ __forceinline__ void block_reduce(F (&v)[K], F (*red)[4]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    F x = v[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const F y = __shfl_xor(x, o, 64);
      x = MAX ? (x > y ? x : y) : x + y;
    }
    if (lane == 0) red[i][w] = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < K; ++i)
    if (MAX) {
      const F a = red[i][0] > red[i][1] ? red[i][0] : red[i][1];
      const F b = red[i][2] > red[i][3] ? red[i][2] : red[i][3];
      v[i] = a > b ? a : b;
    } else {
      v[i] = (red[i][0] + red[i][1]) + (red[i][2] + red[i][3]);
    }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// maxmin_score: block scores and entropy of one (head, segment).
//   z1..z4[j] = sigma log2(e) * (Qmax.Kmax_j, Qmax.Kmin_j, Qmin.Kmax_j, Qmin.Kmin_j)
//               (fp64)
//   S_i = softmax_j(z_i) (base 2),  A_j = max((S1+S2)/2, (S3+S4)/2)
//   a_j = A_j / sum_j A_j,  entropy of a (Shannon or Renyi)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void maxmin_score_kernel(
    const T* __restrict__ qmx, const T* __restrict__ qmn, const T* __restrict__ kmx,
    const T* __restrict__ kmn, int Hq, int r, int CS, int CB, int bps, int nqc, int qtot,
    double sl2, int kind, float alpha, double* __restrict__ z, float* __restrict__ scores,
    float* __restrict__ entropy) {
  typedef typename Vec16<T>::type vec_t;
  constexpr int EPV = Vec16<T>::N;
  __shared__ float qr[2][D];
  __shared__ float red[4][4];
  __shared__ double redd[4][4];
  const int s = CS - 1 - (int)blockIdx.x / Hq, h = (int)blockIdx.x % Hq;
  const int g = h / r;
  const int tid = threadIdx.x;
  // fold the segment's pooled query chunks
  for (int d = tid; d < D; d += 256) {
    float a = -INFINITY, b = INFINITY;
#pragma unroll 8
    for (int c = 0; c < nqc; ++c) {
      const size_t o = ((size_t)h * qtot + (size_t)s * nqc + c) * D + d;
      a = fmaxf(a, (float)qmx[o]);
      b = fminf(b, (float)qmn[o]);
    }
    qr[0][d] = a;
    qr[1][d] = b;
  }
  __syncthreads();
  const int cb = (s + 1) * bps;
  double* zz = z + ((size_t)h * CS + s) * 4 * CB;
  float* row = scores + ((size_t)h * CS + s) * CB;

  // pass 1: the four logits of every causal block, and their maxima
  double m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int j = tid; j < cb; j += 256) {
    const vec_t* kx = reinterpret_cast<const vec_t*>(kmx + ((size_t)g * CB + j) * D);
    const vec_t* kn = reinterpret_cast<const vec_t*>(kmn + ((size_t)g * CB + j) * D);
    double dot[4] = {0.0, 0.0, 0.0, 0.0};
    // the loads of half a row are issued together, before its products (a
    // whole row at once spills registers)
    constexpr int NV = D / EPV, HV = NV >= 8 ? NV / 2 : NV;
#pragma unroll 1
    for (int c0 = 0; c0 < NV; c0 += HV) {
      vec_t xs[HV], ns[HV];
#pragma unroll
      for (int c = 0; c < HV; ++c) {
        xs[c] = kx[c0 + c];
        ns[c] = kn[c0 + c];
      }
#pragma unroll
      for (int cc = 0; cc < HV; ++cc) {
        const int c = c0 + cc;
        const vec_t x = xs[cc], n = ns[cc];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const double qa = qr[0][c * EPV + e], qb = qr[1][c * EPV + e];
          const double fx = (float)x[e], fn = (float)n[e];
          dot[0] = __builtin_fma(qa, fx, dot[0]);
          dot[1] = __builtin_fma(qa, fn, dot[1]);
          dot[2] = __builtin_fma(qb, fx, dot[2]);
          dot[3] = __builtin_fma(qb, fn, dot[3]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double zi = dot[i] * sl2;
      zz[(size_t)i * CB + j] = zi;
      m4[i] = zi > m4[i] ? zi : m4[i];
    }
  }
  block_reduce<double, 4, true>(m4, redd);

  // pass 2: the four normalisers
  float l4[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = tid; j < cb; j += 256)
#pragma unroll
    for (int i = 0; i < 4; ++i) l4[i] += exp2f((float)(zz[(size_t)i * CB + j] - m4[i]));
  block_reduce<float, 4, false>(l4, red);
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv[i] = 1.0f / l4[i];

  // pass 3: the max-combined row and its total
  float tot[1] = {0.f};
  for (int j = tid; j < cb; j += 256) {
    float sp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[i] = exp2f((float)(zz[(size_t)i * CB + j] - m4[i])) * inv[i];
    const float A = fmaxf(0.5f * (sp[0] + sp[1]), 0.5f * (sp[2] + sp[3]));
    row[j] = A;
    tot[0] += A;
  }
  block_reduce<float, 1, false>(tot, red);

  // pass 4: renormalise, entropy terms, sentinels past the causal range
  const float it = 1.0f / tot[0];
  float ent[1] = {0.f};
  for (int j = tid; j < cb; j += 256) {
    const float a = row[j] * it;
    row[j] = a;
    if (kind == EGS_SHANNON)
      ent[0] += a > 0.f ? -a * logf(a) : 0.f;
    else
      ent[0] += powf(a, alpha);
  }
  for (int j = cb + tid; j < CB; j += 256) row[j] = -1.0f;
  block_reduce<float, 1, false>(ent, red);
  if (tid == 0)
    entropy[(size_t)h * CS + s] = kind == EGS_SHANNON ? ent[0] : logf(ent[0]) / (1.0f - alpha);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t maxmin_run(const PrefillDims& p, const MaxMinLayout& ly, const void* q,
                             const void* k, int kind, float alpha, float* scores,
                             float* entropy, char* ws, hipStream_t st) {
  T* kmx = reinterpret_cast<T*>(ws + ly.kmx);
  T* kmn = reinterpret_cast<T*>(ws + ly.kmn);
  T* qmx = reinterpret_cast<T*>(ws + ly.qmx);
  T* qmn = reinterpret_cast<T*>(ws + ly.qmn);
  double* z = reinterpret_cast<double*>(ws + ly.z);
  const int qtot = p.N / ly.qch;
  pool_maxmin_kernel<T, D><<<dim3(p.CB, p.Hkv), 256, 0, st>>>(static_cast<const T*>(k), p.N,
                                                               p.LB, p.CB, kmx, kmn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pool_maxmin_kernel<T, D><<<dim3(qtot, p.Hq), 256, 0, st>>>(static_cast<const T*>(q), p.N,
                                                              ly.qch, qtot, qmx, qmn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  maxmin_score_kernel<T, D><<<p.Hq * p.CS, 256, 0, st>>>(
      qmx, qmn, kmx, kmn, p.Hq, p.r, p.CS, p.CB, p.LS / p.LB, p.LS / ly.qch, qtot,
      (double)p.sm_scale * 1.4426950408889634, kind, alpha, z, scores, entropy);
  return hipGetLastError();
}

template <typename T>
static hipError_t maxmin_dispatch(const PrefillDims& p, const MaxMinLayout& ly, const void* q,
                                  const void* k, int kind, float alpha, float* scores,
                                  float* entropy, char* ws, hipStream_t st) {
  switch (p.D) {
    case 16: return maxmin_run<T, 16>(p, ly, q, k, kind, alpha, scores, entropy, ws, st);
    case 32: return maxmin_run<T, 32>(p, ly, q, k, kind, alpha, scores, entropy, ws, st);
    case 64: return maxmin_run<T, 64>(p, ly, q, k, kind, alpha, scores, entropy, ws, st);
    case 128: return maxmin_run<T, 128>(p, ly, q, k, kind, alpha, scores, entropy, ws, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_entropy_score_maxmin(const PrefillDims& p, const void* q, const void* k,
                                       int kind, float alpha, float* scores, float* entropy,
                                       void* ws, hipStream_t st) {
  const MaxMinLayout ly = mm_layout(p);
  char* w = static_cast<char*>(ws);
  return p.dtype == EGS_F32
             ? maxmin_dispatch<float>(p, ly, q, k, kind, alpha, scores, entropy, w, st)
             : maxmin_dispatch<bf16>(p, ly, q, k, kind, alpha, scores, entropy, w, st);
}

}  // namespace egs
