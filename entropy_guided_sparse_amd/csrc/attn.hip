// K5: block-sparse causal GQA attention over per-(head, segment) block lists.
//
// Method: EntropyInfer (arXiv 2606.09508) App. A eq. (3) computes attention of
// every segment only over its selected key blocks; the causal GQA softmax is
// the one of EntroPrefill Sec. 2.1 (query head h reads KV head g(h)).  Query
// block b of segment s attends { j in Sel(h, s) : j < b } plus its own block b
// under the causal mask, so a full budget reproduces dense causal attention.
//
// gfx950 design (bf16, head_dim 64/128, block 64/128):
//  * One workgroup per (head, query block), L_B/32 wavefronts of 32 query rows.
//    Workgroups are ordered heaviest (latest) query block first, and the r
//    heads of one KV group for the same query block are dispatched to the same
//    XCD so their shared K/V blocks meet in that XCD's L2.
//  * The "transposed" flash formulation keeps every operand in the layout the
//    next MFMA wants, with no cross-lane shuffles:
//        S^T = K Q^T     (A = K tile from LDS, B = Q^T held in registers)
//        P^T  = exp2(S^T - m)   (a lane owns one query row -> row statistics
//                                are lane-local plus one xor-32 exchange)
//        O^T += V^T P^T  (A = V^T tile from LDS, B = P^T straight from the
//                         accumulator registers)
//    using v_mfma_f32_32x32x16_bf16, fp32 accumulation and online softmax.
//  * K/V sub-tiles of 64 keys are double-buffered in LDS; the next sub-tile's
//    global loads are issued before the current one is computed.  V is stored
//    transposed (d-major) so the A operand of O^T is two 8-byte LDS reads.
//
// Generic path: a VALU kernel (one thread per query row, fp32 math) serves
// fp32 inputs and shapes outside the MFMA kernel's range.
#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
template <int D, int LB>
__global__ __launch_bounds__(LB * 2) void sparse_attn_mfma_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int k_max,
    bf16* __restrict__ O, float* __restrict__ lse, int Hkv, int r, int N, int LS, int CS,
    int CB, float scale_log2, int xcd_remap) {
  constexpr int NW = LB / 32;
  constexpr int NT = NW * 64;
  constexpr int KT = 64;              // keys per LDS sub-tile
  constexpr int SUB = LB / KT;
  constexpr int KPAD = D + 8;         // K row pitch (bf16 elements)
  constexpr int VPAD = KT + 4;        // V^T row pitch (bf16 elements)
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int KCT = KT * D / 8;     // 16-byte K chunks per sub-tile
  constexpr int KI = (KCT + NT - 1) / NT;
  constexpr int VUT = (KT / 4) * (D / 8);   // (4 keys x 8 d) V units per sub-tile
  constexpr int VI = (VUT + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][KT * KPAD];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][D * VPAD];

  // ---- work item: (KV group, query block) pair, head within group ----
  const int bid = blockIdx.x;
  int grp, hl;
  if (xcd_remap) {
    const int xcd = bid & 7, slot = bid >> 3;
    grp = 8 * (slot / r) + xcd;
    hl = slot % r;
  } else {
    grp = bid / r;
    hl = bid % r;
  }
  const int g = grp % Hkv;
  const int b = CB - 1 - grp / Hkv;
  const int h = g * r + hl;
  const int s = (b * LB) / LS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const size_t qrow0 = (size_t)b * LB + w * 32;

  bf16x8 qf[NC];
  {
    const bf16* qp = Q + ((size_t)h * N + qrow0 + l32) * D + 8 * hg;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = load8(qp + 16 * c);
  }
  floatx16 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  const int32_t* sel = idx + ((size_t)h * CS + s) * k_max;
  const int n = min(max(cnt[(size_t)h * CS + s], 0), k_max);
  int p = 0;
  auto next_sel = [&]() -> int {
    while (p < n) {
      const int j = sel[p++];
      if (j >= 0 && j < b) return j;
    }
    return -1;
  };

  const bf16* Kg = K + (size_t)g * N * D;
  const bf16* Vg = V + (size_t)g * N * D;
  u32x4 kreg[KI];
  u32x4 vreg[VI][4];

  auto gload = [&](int blk, int sub) {
    const size_t key0 = (size_t)blk * LB + sub * KT;
#pragma unroll
    for (int ii = 0; ii < KI; ++ii) {
      const int q = tid + ii * NT;
      if (q < KCT) {
        const int row = q / (D / 8), c8 = q % (D / 8);
        kreg[ii] = *reinterpret_cast<const u32x4*>(Kg + (key0 + row) * D + c8 * 8);
      }
    }
#pragma unroll
    for (int ii = 0; ii < VI; ++ii) {
      const int u = tid + ii * NT;
      if (u < VUT) {
        const int k4 = u / (D / 8), c8 = u % (D / 8);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          vreg[ii][kk] =
              *reinterpret_cast<const u32x4*>(Vg + (key0 + 4 * k4 + kk) * D + c8 * 8);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int ii = 0; ii < KI; ++ii) {
      const int q = tid + ii * NT;
      if (q < KCT) {
        const int row = q / (D / 8), c8 = q % (D / 8);
        *reinterpret_cast<u32x4*>(&Ks[buf][row * KPAD + c8 * 8]) = kreg[ii];
      }
    }
#pragma unroll
    for (int ii = 0; ii < VI; ++ii) {
      const int u = tid + ii * NT;
      if (u < VUT) {
        const int k4 = u / (D / 8), c8 = u % (D / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int wd = e >> 1, sh = 16 * (e & 1);
          const uint32_t a0 = (vreg[ii][0][wd] >> sh) & 0xFFFFu;
          const uint32_t a1 = (vreg[ii][1][wd] >> sh) & 0xFFFFu;
          const uint32_t a2 = (vreg[ii][2][wd] >> sh) & 0xFFFFu;
          const uint32_t a3 = (vreg[ii][3][wd] >> sh) & 0xFFFFu;
          u32x2 pk;
          pk[0] = a0 | (a1 << 16);
          pk[1] = a2 | (a3 << 16);
          *reinterpret_cast<u32x2*>(&Vt[buf][(c8 * 8 + e) * VPAD + 4 * k4]) = pk;
        }
      }
    }
  };

  auto compute = [&](int buf, bool diag, int sub) {
    if (diag && sub * KT > w * 32 + 31) return;   // wave-uniform: all keys in the future
    const bf16* ks = Ks[buf];
    const bf16* vt = Vt[buf];
    floatx16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a = load8(ks + (kt * 32 + l32) * KPAD + 16 * c + 8 * hg);
        st[kt] = mfma32(a, qf[c], st[kt]);
      }
    }
    const bool need_mask = diag && (sub * KT + KT - 1 > w * 32);
    const int row_local = w * 32 + l32;
    float mx = m_run;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = st[kt][i] * scale_log2;
        if (need_mask) {
          const int key_local = sub * KT + kt * 32 + acc_row(i, lane);
          if (key_local > row_local) v = -INFINITY;
        }
        st[kt][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float alpha = exp2f(m_run - mx);
    m_run = mx;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    bf16x8 pb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2f(st[kt][i] - mx);
        l_run += pv;
        pb[kt * 2 + (i >> 3)][i & 7] = f2bf(pv);
      }
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const int base = (ch >> 1) * 32 + 16 * (ch & 1);
        const bf16* vrow = vt + (dt * 32 + l32) * VPAD + base + 4 * hg;
        const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vrow + 8);
        const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = mfma32(a, pb[ch], o[dt]);
      }
    }
  };

  int cur = next_sel();
  bool cur_diag = false;
  if (cur < 0) {
    cur = b;
    cur_diag = true;
  }
  int sub = 0, buf = 0;
  gload(cur, 0);
  lstore(0);
  __syncthreads();
  while (true) {
    int nblk = cur, nsub = sub + 1;
    bool ndiag = cur_diag, has_next = true;
    if (nsub == SUB) {
      nsub = 0;
      if (cur_diag) {
        has_next = false;
      } else {
        nblk = next_sel();
        ndiag = nblk < 0;
        if (ndiag) nblk = b;
      }
    }
    if (has_next) gload(nblk, nsub);
    compute(buf, cur_diag, sub);
    if (!has_next) break;
    lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    cur = nblk;
    sub = nsub;
    cur_diag = ndiag;
  }

  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / lt;
  bf16* op = O + ((size_t)h * N + qrow0 + l32) * D;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = f2bf(o[dt][4 * i4 + t] * inv);
      *reinterpret_cast<bf16x4*>(op + dt * 32 + 8 * i4 + 4 * hg) = v;
    }
  }
  if (lse != nullptr && hg == 0) lse[(size_t)h * N + qrow0 + l32] = m_run * kLn2 + logf(lt);
}

// ---------------------------------------------------------------------------
// Generic VALU kernel: one thread per query row, fp32 math, 32-key LDS tiles.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void sparse_attn_generic_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int k_max,
    T* __restrict__ O, float* __restrict__ lse, int Hq, int r, int N, int LS, int LB,
    int CS, int CB, float scale_log2) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  const int b = CB - 1 - blockIdx.x / Hq;
  const int h = blockIdx.x % Hq, g = h / r;
  const int s = (b * LB) / LS;
  const int tid = threadIdx.x;
  const bool active = tid < LB;
  const int row = b * LB + (active ? tid : 0);
  float q[D], o[D];
  {
    const T* qp = Q + ((size_t)h * N + row) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      q[d] = active ? (float)qp[d] : 0.f;
      o[d] = 0.f;
    }
  }
  float m = kNegBig, l = 0.f;
  const int32_t* sel = idx + ((size_t)h * CS + s) * k_max;
  const int n = min(max(cnt[(size_t)h * CS + s], 0), k_max);
  const T* Kg = K + (size_t)g * N * D;
  const T* Vg = V + (size_t)g * N * D;
  for (int pp = 0; pp <= n; ++pp) {
    int j = b;
    if (pp < n) {
      j = sel[pp];
      if (j < 0 || j >= b) continue;
    }
    for (int k0 = 0; k0 < LB; k0 += KT) {
      __syncthreads();
      for (int e = tid; e < KT * D; e += blockDim.x) {
        const int kk = e / D, dd = e % D;
        if (k0 + kk < LB) {
          const size_t t = (size_t)j * LB + k0 + kk;
          Ks[kk][dd] = (float)Kg[t * D + dd];
          Vs[kk][dd] = (float)Vg[t * D + dd];
        }
      }
      __syncthreads();
      if (active) {
        float sc[KT];
        float mx = m;
#pragma unroll 4
        for (int kk = 0; kk < KT; ++kk) {
          const int t = j * LB + k0 + kk;
          float v = -INFINITY;
          if (k0 + kk < LB && t <= row) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot += q[d] * Ks[kk][d];
            v = dot * scale_log2;
          }
          sc[kk] = v;
          mx = fmaxf(mx, v);
        }
        const float alpha = exp2f(m - mx);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        m = mx;
        for (int kk = 0; kk < KT; ++kk) {
          const float pv = exp2f(sc[kk] - mx);
          l += pv;
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] += pv * Vs[kk][d];
        }
      }
    }
  }
  if (active) {
    const float inv = 1.0f / l;
    T* op = O + ((size_t)h * N + row) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = (T)(o[d] * inv);
    if (lse != nullptr) lse[(size_t)h * N + row] = m * kLn2 + logf(l);
  }
}

template <typename T>
static hipError_t generic_dispatch(const PrefillDims& p, const void* q, const void* k,
                                   const void* v, const int32_t* idx, const int32_t* cnt,
                                   int k_max, void* out, float* lse, hipStream_t st) {
  const int threads = ((p.LB + 63) / 64) * 64;
  const int grid = p.Hq * p.CB;
  const float sl2 = p.sm_scale * kLog2e;
  const T* Q = static_cast<const T*>(q);
  const T* K = static_cast<const T*>(k);
  const T* V = static_cast<const T*>(v);
  T* O = static_cast<T*>(out);
#define EGS_GEN(DD)                                                                       \
  sparse_attn_generic_kernel<T, DD><<<grid, threads, 0, st>>>(                            \
      Q, K, V, idx, cnt, k_max, O, lse, p.Hq, p.r, p.N, p.LS, p.LB, p.CS, p.CB, sl2)
  switch (p.D) {
    case 16: EGS_GEN(16); break;
    case 32: EGS_GEN(32); break;
    case 64: EGS_GEN(64); break;
    case 128: EGS_GEN(128); break;
    default: return hipErrorInvalidValue;
  }
#undef EGS_GEN
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const PrefillDims& p, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* cnt,
                              int k_max, void* out, float* lse, hipStream_t st) {
  if (p.dtype == EGS_F32) return generic_dispatch<float>(p, q, k, v, idx, cnt, k_max, out, lse, st);
  const bool mfma_ok = (p.D == 64 || p.D == 128) && (p.LB == 64 || p.LB == 128);
  if (!mfma_ok) return generic_dispatch<bf16>(p, q, k, v, idx, cnt, k_max, out, lse, st);
  const int grid = p.Hq * p.CB;
  const int remap = ((p.Hkv * p.CB) % 8 == 0) ? 1 : 0;
  const float sl2 = p.sm_scale * kLog2e;
  const bf16* Q = static_cast<const bf16*>(q);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  bf16* O = static_cast<bf16*>(out);
#define EGS_MF(DD, BB)                                                                    \
  sparse_attn_mfma_kernel<DD, BB><<<grid, BB * 2, 0, st>>>(                               \
      Q, K, V, idx, cnt, k_max, O, lse, p.Hkv, p.r, p.N, p.LS, p.CS, p.CB, sl2, remap)
  if (p.D == 128 && p.LB == 128) EGS_MF(128, 128);
  else if (p.D == 128 && p.LB == 64) EGS_MF(128, 64);
  else if (p.D == 64 && p.LB == 128) EGS_MF(64, 128);
  else EGS_MF(64, 64);
#undef EGS_MF
  return hipGetLastError();
}

}  // namespace egs
