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
//  * Both passes run obs_pass_kernel: one workgroup per (2048-key span,
//    batch x KV group, 4-head group).  64-key K stages are copied straight
//    into LDS, four deep, and shared by the four wavefronts (one query head
//    each); the logits of a stage take v_mfma_f32_32x32x16_bf16.
//    Pass 1 (keys as M: a lane owns an observer row) keeps the span's
//    running max / sum of every row; a combine kernel folds the spans into
//    each row's final max and 1/sum.  Pass 2 recomputes the logits with keys
//    as N, so a lane owns one key and the window mean is a register sum; it
//    writes the per-head mass and the span's sink-isolated entropy partial
//    sums.
//  * head_weight turns the partial sums into H_h and w_h; retain_mu forms
//    mu_t; retain_select runs an exact 12/12/8-bit radix select over the
//    candidates and compacts the kept indices in ascending order through LDS;
//    gather copies the kept K/V rows.
//  * Page-level retention (EntroPrefill Sec. 7) keeps whole pages: page maxima
//    of the token scores, the same select over page scores, and unions over
//    the heads of a group or the groups of a layer through an LDS bitmap.
//  * Decode attention splits the kept range into 192- to 1024-entry splits
//    (chosen per call so the last round of workgroups fills the CUs); the GQA
//    group's heads share each 64-entry K / V stage in LDS (lane-per-entry dot
//    products, lane-per-dim PV) and a combine kernel merges the splits with
//    their log-sum-exp.
//  * Chunk pruning (EntroPrefill Sec. 3.1-3.2, 4.2) runs both passes on one
//    prompt; pass 1 also splits each row's sums by candidate chunk (a
//    "chunk" below is always one of the prompt's candidate documents, a
//    "span" the passes' 2048-key work unit).  The pooled measure is formed
//    per position, one workgroup orders the chunks by priority and scans
//    them greedily with block votes, and two small kernels evaluate the
//    Sec. 4.2 optimality-gap certificate for caller prices.
#include <algorithm>
#include <type_traits>

#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// All-reduces over the 64 lanes of a wave without the LDS path: DPP within
// each 16-lane row (lane ^ 1, lane ^ 2, then the mirrored half and the
// mirrored row, which pair lanes whose earlier steps already agree), then
// the row and half swaps of v_permlane16_swap / v_permlane32_swap.
__device__ __forceinline__ float dpp_row_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
}
__device__ __forceinline__ float dpp_row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}
__device__ __forceinline__ float xrow_sum(float v) {   // lanes l and l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max_v(float v) {
  v = dpp_row_max(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return xhalf_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float wave_sum_v(float v) { return xhalf_sum(xrow_sum(dpp_row_sum(v))); }

// The compiler schedules nothing across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// Keeps the computation of x before this point: an empty volatile asm that
// reads and writes x is ordered against the scheduling fences, so work that
// only feeds a later sum cannot drift past the next fence.
__device__ __forceinline__ void pin_vgpr(float& x) { asm volatile("" : "+v"(x)); }

constexpr int RT_CK = 2048;   // keys per span (the pass 1 / pass 2 work unit)
constexpr int RT_KT = 64;     // keys per LDS stage
constexpr int SEL_T = 1024;   // threads of the select kernel
constexpr int SEL_CH = 16384; // keys per chunk of the split top-k
constexpr int DA_SPL_MIN = 192;   // kept entries per decode-attention split: the
constexpr int DA_SPL_MAX = 1024;   // range the launcher chooses from (multiples of 64)

struct RetainLayout {
  size_t stat_m, stat_l, row_m, row_inv, mass, ent, weight, mu, qsum, tstats;
  size_t sel_hist, sel_state, sel_cnt, total;
  int nch;    // 2048-key spans of the cache
  int nsel;   // key chunks of the split top-k (histogram and compaction)
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
  o.tstats = take((size_t)p.B * 2 * 4);
  o.nsel = (p.L + SEL_CH - 1) / SEL_CH;
  const size_t slices = (size_t)p.B * p.Hkv;
  o.sel_hist = take(slices * o.nsel * 4096 * 4);
  o.sel_state = take(slices * 4 * 4);
  o.sel_cnt = take(slices * o.nsel * 2 * 4);
  o.total = off;
  return o;
}

size_t retain_workspace_bytes(const DecodeDims& p) {
  return retain_layout(p).total;
}

// ---------------------------------------------------------------------------
// shared pieces of pass 1 / pass 2
// ---------------------------------------------------------------------------
// 64-key K stages copied straight into LDS (global_load_lds_dwordx4) by the
// four wavefronts, 16-byte pieces XOR-swizzled by row; rows past the span's
// last key repeat that key (in bounds) and are masked by the consumer.
template <int D>
struct KPipe {
  static constexpr int PIECES = RT_KT * D * 2 / 1024;   // 1-KB wave copies per stage
  static constexpr int PER_W = PIECES / 4;
  static constexpr int KROWS = 1024 / (D * 2);          // K rows per piece
  static constexpr int KCH = D / 8;
  static_assert(PIECES % 4 == 0, "stage copies must split evenly over four waves");
  __device__ static void copy(bf16* kbuf, const bf16* Kg, int t0, int t_last, int w,
                              int lane) {
    const bf16* src = Kg + (size_t)t0 * D;
#pragma unroll
    for (int ii = 0; ii < PER_W; ++ii) {
      const int pc = w * PER_W + ii;
      const int row = pc * KROWS + lane / KCH;
      const int c = (lane % KCH) ^ lds_swz<D * 2>(row);
      const int t = min(t0 + row, t_last);
      copy16_to_lds(src, (uint32_t)(((t - t0) * D + c * 8) * sizeof(bf16)), kbuf + pc * 512);
    }
  }
  // the 8 bf16 of key row `row` (0..63 in the stage), d chunk (2c + hg)
  __device__ static bf16x8 frag(const bf16* kbuf, int row, int c, int hg) {
    return load8(kbuf + row * D + (((2 * c + hg) ^ lds_swz<D * 2>(row)) * 8));
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
// pass 1 (MASS = false): per span and observer row, a reference m (at most
// 64 below the row's maximum in log2 units) and the sum of exp2(z - m).
// pass 2 (MASS = true): per-head window-mean mass of every key and the
// span's sink-isolated entropy partial sums.
// Workgroup = (2048-key span, batch x KV group, 4-head group); the four
// wavefronts (one query head each) share every K stage.  Stages are copied
// RT_DEPTH - 1 ahead of the one being computed (four LDS buffers), so each
// workgroup keeps three 16-KB copies in flight against HBM latency.  Pass 2
// stores the masses of every stage as it goes; those stores share the vector
// memory counter with the copies, and the wait before a stage counts them.
// SEG (pass 1 of chunk pruning, one sequence): the same tile sums are also
// split by candidate chunk.  A row's sum over the keys of chunk c in this
// span, taken against the row's reference, is written with that reference as
// segment seg_base[c] + span - first span of c, row h * W + u, of
// (seg_v, seg_m); after the combine, chunk_norm_kernel turns the segments
// into probabilities.  Tiles inside one chunk cost one add; tiles where a
// chunk starts or ends split the sum by the chunk ids of their keys.
// ---------------------------------------------------------------------------
constexpr int RT_DEPTH = 4;

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

template <int D, int RT, bool MASS, bool SEG = false>
__global__ __launch_bounds__(256) void obs_pass_kernel(
    const bf16* __restrict__ Qo, const bf16* __restrict__ K, int Hq, int Hkv, int r, int L,
    int ldk, int W, int nch, float sl2, float* __restrict__ stat_m, float* __restrict__ stat_l,
    const float* __restrict__ row_m, const float* __restrict__ row_inv, int n_sink, int kind,
    float alpha, float* __restrict__ mass, float* __restrict__ ent,
    const int32_t* __restrict__ cid = nullptr, const int32_t* __restrict__ bounds = nullptr,
    const int32_t* __restrict__ seg_base = nullptr, float* __restrict__ seg_v = nullptr,
    float* __restrict__ seg_m = nullptr) {
  static_assert(!SEG || !MASS, "chunk segments ride on pass 1");
  constexpr int NC = D / 16;
  constexpr int PW = KPipe<D>::PER_W;
  __shared__ __attribute__((aligned(1024))) bf16 Ks[RT_DEPTH][RT_KT * D];
  __shared__ int cs[SEG ? RT_CK : 1];
  // The hardware hands a grid's workgroups to the CUs in a fixed rotation
  // (workgroup i to CU i mod 256 when each CU holds the same count), so with
  // the span index fastest every CU would always get the same span position
  // and the few CUs that get the edge spans (observer window, sinks; the
  // slower masked path) would set the pass length.  The linear workgroup id
  // therefore runs over (batch x group) fastest, and the edge spans - the
  // last, then the first - come first.
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int bg = lin % gridDim.y, srank = lin / gridDim.y;
  const int span = srank == 0 ? (int)gridDim.x - 1 : srank - 1;
  const int b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const int hl = blockIdx.z * 4 + w;
  const bool hvalid = hl < r;
  const int h = g * r + (hvalid ? hl : 0);
  const int t_begin = span * RT_CK, t_end = min(L, t_begin + RT_CK);
  const int nst = (t_end - t_begin + RT_KT - 1) / RT_KT;
  const bf16* Kg = K + (size_t)bg * ldk * D;
  const int pos0 = L - W;   // observer u sits at pos0 + u

  bf16x8 qf[RT][NC];
  load_obs_q<D, RT>(qf, Qo, b, h, Hq, W, hvalid, lane);
  float m[RT], l[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegBig;
    l[rt] = 0.f;
  }
  // pass 2: the final statistics of the rows this lane's registers hold
  float rm[RT][16];
  float s1 = 0.f, s2 = 0.f;
  const float invW = 1.0f / (float)W;
  if (MASS) {
    // every load is issued before the first result is used (row indices
    // clamped into the window; h is a valid head even for an idle wave), so
    // the wave waits out one memory latency here, not one per row
    const size_t rbase = ((size_t)b * Hq + h) * W;
    float inv[RT][16];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const size_t at = rbase + min(rt * 32 + acc_row(i, lane), W - 1);
        inv[rt][i] = row_inv[at];
        rm[rt][i] = row_m[at];
      }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int u = rt * 32 + acc_row(i, lane);
        // exp2(z sl2 - M) / L = exp2(z sl2 - (M + log2 L)); rows past the
        // window get an infinite offset, i.e. probability 0
        const bool ok = hvalid && u < W && inv[rt][i] > 0.f;
        rm[rt][i] = ok ? rm[rt][i] - __log2f(inv[rt][i]) : INFINITY;
      }
  }
  // chunk segments: the chunk id of every key of the span (-1 outside the
  // chunks and past the end), read after the first barrier of the loop; the
  // open chunk and its sums against m
  float cacc[RT];
  int curc = -1;
  if constexpr (SEG) {
    for (int j = tid; j < RT_CK; j += 256) cs[j] = t_begin + j < t_end ? cid[t_begin + j] : -1;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) cacc[rt] = 0.f;
  }
  // closes the open chunk c: both halves of the row to one reference
  auto flush = [&](int c) {
    if (c < 0) return;
    const int seg = seg_base[c] + span - bounds[2 * c] / RT_CK;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float M = xhalf_max(m[rt]);
      const float v = xhalf_sum(cacc[rt] * fast_exp2(m[rt] - M));
      const int u = rt * 32 + l32;
      if (hg == 0 && u < W) {
        const size_t o = (size_t)seg * Hq * W + (size_t)h * W + u;
        seg_v[o] = v;
        seg_m[o] = M;
      }
      cacc[rt] = 0.f;
    }
  };
  wait_vmem();   // only the copies below are in flight from here on
#pragma unroll
  for (int d = 0; d < RT_DEPTH - 1; ++d)
    if (d < nst) KPipe<D>::copy(Ks[d], Kg, t_begin + d * RT_KT, t_end - 1, w, lane);

  // EDGE: the stage holds keys past the span or after an observer position
  auto compute = [&](const bf16* ks, int t0, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
#pragma unroll
    for (int kt = 0; kt < RT_KT / 32; ++kt) {
      const int tk = t0 + kt * 32;
      if (tk >= t_end) break;
      const bool edge = EDGE && ((tk + 31 >= t_end) || (tk + 31 > pos0));
      floatx16 z[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) z[rt][i] = 0.f;
      if (!MASS) {
        // S^T: lane owns observer row (rt*32 + l32), registers hold keys
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 a = KPipe<D>::frag(ks, kt * 32 + l32, c, hg);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) z[rt] = mfma32(a, qf[rt][c], z[rt]);
        }
        // chunk ids rise with the position: keys tk and tk + 31 in one chunk
        // means the whole tile is in it
        int tc = -1;
        if constexpr (SEG) {
          const int cf = __builtin_amdgcn_readfirstlane(cs[tk - t_begin]);
          const int cb = __builtin_amdgcn_readfirstlane(cs[tk + 31 - t_begin]);
          tc = (cf == cb && cf >= 0) ? cf : -2;
          if (tc >= 0 && tc != curc) {
            flush(curc);
            curc = tc;
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int u = rt * 32 + l32;
          if (edge) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int t = tk + acc_row(i, lane);
              if (t >= t_end || t > pos0 + u) z[rt][i] = -INFINITY;
            }
          }
          // The terms are taken against the running reference m (log2
          // units), which is raised only when this tile would overflow
          // against it (a term above 2^64, or the first tile, m = kNegBig).
          // Otherwise m may sit below the true maximum: l then holds the sum
          // relative to m, which is all the combine needs (it rescales every
          // span's (m, l) to a common reference), and fp32 keeps the ratios.
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(z[rt][i], sl2, -m[rt]));
          if (!(sum <= 0x1p64f)) {
            float tmax = z[rt][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, z[rt][i]);
            // sl2 > 0 commutes with max
            const float mn = fmaxf(m[rt], tmax * sl2);
            sum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(z[rt][i], sl2, -mn));
            const float sc = fast_exp2(m[rt] - mn);
            l[rt] *= sc;
            if constexpr (SEG) cacc[rt] *= sc;
            m[rt] = mn;
          }
          l[rt] += sum;
          if constexpr (SEG) {
            if (tc >= 0) cacc[rt] += sum;
          }
        }
        if constexpr (SEG) {
          if (tc == -2) {
            // a chunk starts or ends in this tile (or none is in it): the
            // ids of the lane's keys, the range lo..hi over the wave, and
            // the sums split by id
            int ci[16];
            int lo = 0x7fffffff, hi = -1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              ci[i] = cs[tk - t_begin + acc_row(i, lane)];
              if (ci[i] >= 0) lo = min(lo, ci[i]);
              hi = max(hi, ci[i]);
            }
            lo = __builtin_amdgcn_readfirstlane(wave_min_i(lo));
            hi = __builtin_amdgcn_readfirstlane(wave_max_i(hi));
            for (int cc = lo; cc <= hi; ++cc) {
              if (cc != curc) {
                flush(curc);
                curc = cc;
              }
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) {
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                  if (ci[i] == cc) part += fast_exp2(__builtin_fmaf(z[rt][i], sl2, -m[rt]));
                cacc[rt] += part;
              }
            }
          }
        }
      } else {
        // Z: lane owns key (tk + l32), registers hold observer rows
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 bk = KPipe<D>::frag(ks, kt * 32 + l32, c, hg);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) z[rt] = mfma32(qf[rt][c], bk, z[rt]);
        }
        const int t = tk + l32;
        // summed in the order of the pipelined interior path (runs of 16 / NC
        // terms, a tree over the runs, then the row tiles), so that equal
        // masses come out bit-equal in every span
        constexpr int EPS = 16 / NC;
        float part[RT][NC];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < EPS; ++q) {
              const int i = c * EPS + q;
              float pv = fast_exp2(__builtin_fmaf(z[rt][i], sl2, -rm[rt][i]));
              if (edge && t > pos0 + rt * 32 + acc_row(i, lane)) pv = 0.f;
              acc += pv;
            }
            part[rt][c] = acc;
          }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int n = NC; n > 1; n >>= 1)
#pragma unroll
            for (int i = 0; i < n / 2; ++i) part[rt][i] += part[rt][i + n / 2];
        float colsum = part[0][0];
#pragma unroll
        for (int rt = 1; rt < RT; ++rt) colsum += part[rt][0];
        colsum = xhalf_sum(colsum);
        if (hg == 0 && t < t_end) {
          const float a = colsum * invW;
          mass[((size_t)b * Hq + h) * L + t] = a;
          if (t >= n_sink && a > 0.f) {
            s1 += a;
            // one v_log_f32: a ln a, or a^alpha = 2^(alpha log2 a)
            const float lg = __log2f(a);
            s2 += (kind == EGS_SHANNON) ? a * lg * kLn2 : fast_exp2(alpha * lg);
          }
        }
      }
    }
  };
  // Stage st sits in buffer st % RT_DEPTH.  At the top of stage st a wave
  // waits for its copies of stage st (the copies of the stages after it stay
  // in flight), meets the others at the barrier and copies stage
  // st + RT_DEPTH - 1 into the buffer stage st - 1 used.  stores = the vector
  // stores the wave is known to have issued after those copies: the
  // pipelined pass-2 loop below stores once per stage, so from its stage 4 on
  // the three stores of stages st - 4 .. st - 2 may stay in flight too.
  // Counting fewer stores than were issued only makes the wait longer.
  auto stage_top = [&](int st, int stores) {
    const int ahead = min(RT_DEPTH - 2, nst - 1 - st);   // copies issued after stage st's
    if (ahead >= 2) {
      if (stores >= 3) wait_vmem_upto<2 * PW + 3>();
      else wait_vmem_upto<2 * PW>();
    } else if (ahead == 1) {
      wait_vmem_upto<PW>();
    } else {
      wait_vmem();
    }
    __syncthreads();
    if (st + RT_DEPTH - 1 < nst)
      KPipe<D>::copy(Ks[(st + RT_DEPTH - 1) % RT_DEPTH], Kg, t_begin + (st + RT_DEPTH - 1) * RT_KT,
                     t_end - 1, w, lane);
  };
  // Interior spans: every key of a whole span precedes the first observer
  // (and, in pass 2, the sinks), so no tile needs a mask.  There the tile
  // loop is software-pipelined: the MFMAs of tile j + 1 issue in between the
  // VALU work of tile j (its exponentials and sums), which otherwise waits
  // for them and then runs alone.
  constexpr bool kPipe = !SEG && RT <= 2;
  const bool interior = kPipe && t_end - t_begin == RT_CK && t_end - 1 <= pos0 &&
                        (!MASS || t_begin >= n_sink);
  if (interior) {
    constexpr int NST = RT_CK / RT_KT;
    // One region: the logits of tile kt of a stage (keys as M in pass 1, as
    // N in pass 2) into zn, and the exponentials of the previous tile zc.
    // The region runs in NC slices split by scheduling fences: slice c
    // issues the MFMAs of d chunk c and then 16 / NC exponentials of every
    // row tile of zc, so the VALU works while the MFMAs of the slice run.
    // Pass 1 returns the tile's row sums against the running reference in
    // sm; pass 2 the lane's column sum of probabilities in sm[0].
    constexpr int EPS = 16 / NC;   // exponentials per row tile and slice
    auto region = [&](const bf16* ks, int kt, floatx16 (&zn)[RT], const floatx16 (&zc)[RT],
                      float (&sm)[RT]) {
      bf16x8 fr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) fr[c] = KPipe<D>::frag(ks, kt * 32 + l32, c, hg);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) zn[rt][i] = 0.f;
      float part[RT][NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          zn[rt] = MASS ? mfma32(qf[rt][c], fr[c], zn[rt]) : mfma32(fr[c], qf[rt][c], zn[rt]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // the run's terms are positive, so starting from the first term
          // gives the same sum as starting from zero
          float acc = fast_exp2(__builtin_fmaf(zc[rt][c * EPS], sl2,
                                               MASS ? -rm[rt][c * EPS] : -m[rt]));
#pragma unroll
          for (int q = 1; q < EPS; ++q) {
            const int i = c * EPS + q;
            acc += fast_exp2(__builtin_fmaf(zc[rt][i], sl2, MASS ? -rm[rt][i] : -m[rt]));
          }
          part[rt][c] = acc;
          pin_vgpr(part[rt][c]);
        }
        sched_fence();
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int n = NC; n > 1; n >>= 1)
#pragma unroll
          for (int i = 0; i < n / 2; ++i) part[rt][i] += part[rt][i + n / 2];
      }
      if constexpr (MASS) {
        float t = part[0][0];
#pragma unroll
        for (int rt = 1; rt < RT; ++rt) t += part[rt][0];
        sm[0] = t;
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sm[rt] = part[rt][0];
      }
    };
    // the same exponentials, summed in the same order, with no MFMAs beside
    // them (the span's last tile)
    auto tail = [&](const floatx16 (&zc)[RT], float (&sm)[RT]) {
      float part[RT][NC];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float acc = fast_exp2(__builtin_fmaf(zc[rt][c * EPS], sl2,
                                               MASS ? -rm[rt][c * EPS] : -m[rt]));
#pragma unroll
          for (int q = 1; q < EPS; ++q) {
            const int i = c * EPS + q;
            acc += fast_exp2(__builtin_fmaf(zc[rt][i], sl2, MASS ? -rm[rt][i] : -m[rt]));
          }
          part[rt][c] = acc;
        }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int n = NC; n > 1; n >>= 1)
#pragma unroll
          for (int i = 0; i < n / 2; ++i) part[rt][i] += part[rt][i + n / 2];
      if constexpr (MASS) {
        float t = part[0][0];
#pragma unroll
        for (int rt = 1; rt < RT; ++rt) t += part[rt][0];
        sm[0] = t;
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sm[rt] = part[rt][0];
      }
    };
    // the first tile of the span: its logits alone
    auto first = [&](const bf16* ks, floatx16 (&zn)[RT]) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) zn[rt][i] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = KPipe<D>::frag(ks, l32, c, hg);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          zn[rt] = MASS ? mfma32(qf[rt][c], a, zn[rt]) : mfma32(a, qf[rt][c], zn[rt]);
      }
    };
    // pass 1: fold a tile's row sums into (m, l); a sum above 2^64 (rare)
    // raises the reference first
    auto fold1 = [&](const floatx16 (&z)[RT], float (&sm)[RT]) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (!(sm[rt] <= 0x1p64f)) {
          float tmax = z[rt][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, z[rt][i]);
          const float mn = fmaxf(m[rt], tmax * sl2);
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(z[rt][i], sl2, -mn));
          l[rt] *= fast_exp2(m[rt] - mn);
          m[rt] = mn;
          sm[rt] = sum;
        }
        l[rt] += sm[rt];
      }
    };
    // pass 2: the window-mean mass of the lane's key (both halves of the
    // wave hold it) and its sink-isolated entropy terms, counted by the low half
    auto mass2 = [&](float colsum) -> float {
      const float a = xhalf_sum(colsum) * invW;
      const float lg = __log2f(a);
      const float term = kind == EGS_SHANNON ? a * lg * kLn2 : fast_exp2(alpha * lg);
      const bool on = hg == 0 && a > 0.f;
      s1 += on ? a : 0.f;
      s2 += on ? term : 0.f;
      return a;
    };
    float* mrow = MASS ? mass + ((size_t)b * Hq + h) * L : nullptr;
    floatx16 za[RT], zb[RT];
    stage_top(0, 0);
    if (hvalid) first(Ks[0], za);
    for (int st = 0; st < NST; ++st) {
      float a0 = 0.f, a1 = 0.f;
      if (hvalid) {
        // tile 1 of stage st on the MFMA unit, tile 0 on the VALU
        float sm[RT];
        region(Ks[st % RT_DEPTH], 1, zb, za, sm);
        if constexpr (MASS) a0 = mass2(sm[0]);
        else fold1(za, sm);
      }
      if (st + 1 < NST) {
        stage_top(st + 1, MASS && hvalid && st + 1 >= 4 ? 3 : 0);
        if (hvalid) {
          // tile 0 of stage st + 1 on the MFMA unit, tile 1 of stage st on the VALU
          float sm[RT];
          region(Ks[(st + 1) % RT_DEPTH], 0, za, zb, sm);
          if constexpr (MASS) a1 = mass2(sm[0]);
          else fold1(zb, sm);
        }
      } else if (hvalid) {
        float sm[RT];
        tail(zb, sm);
        if constexpr (MASS) a1 = mass2(sm[0]);
        else fold1(zb, sm);
      }
      // one store per stage: the low half of the wave writes tile 0's keys,
      // the high half tile 1's
      if (MASS && hvalid) mrow[t_begin + st * RT_KT + hg * 32 + l32] = hg ? a1 : a0;
    }
  } else {
    for (int st = 0; st < nst; ++st) {
      stage_top(st, 0);
      if (hvalid) {
        const int t0 = t_begin + st * RT_KT;
        if (t0 + RT_KT - 1 >= t_end || t0 + RT_KT - 1 > pos0)
          compute(Ks[st % RT_DEPTH], t0, std::true_type{});
        else
          compute(Ks[st % RT_DEPTH], t0, std::false_type{});
      }
    }
  }
  if (!hvalid) return;
  if constexpr (SEG) flush(curc);
  if (!MASS) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float M = xhalf_max(m[rt]);
      const float Lr = xhalf_sum(l[rt] * fast_exp2(m[rt] - M));
      const int u = rt * 32 + l32;
      if (hg == 0 && u < W) {
        const size_t o = (((size_t)b * Hq + h) * nch + span) * W + u;
        stat_m[o] = M;
        stat_l[o] = Lr;
      }
    }
  } else {
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    if (lane == 0) {
      float* e = ent + (((size_t)b * Hq + h) * nch + span) * 2;
      e[0] = s1;
      e[1] = s2;
    }
  }
}

// the rows' common reference (the largest span reference) and 1/sum: one
// workgroup per (batch, head); the W rows of the head each get 256 / W
// threads that split the spans
__global__ __launch_bounds__(256) void obs_combine_kernel(const float* __restrict__ stat_m,
                                                          const float* __restrict__ stat_l,
                                                          int nch, int W,
                                                          float* __restrict__ row_m,
                                                          float* __restrict__ row_inv) {
  __shared__ float pm[256], pl[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int parts = max(1, 256 / W);
  const int u = tid % W, part = tid / W;
  const bool on = tid < parts * W;
  float M = kNegBig, Lr = 0.f;
  if (on) {
    const float* sm = stat_m + (size_t)bh * nch * W + u;
    const float* sl = stat_l + (size_t)bh * nch * W + u;
    // eight spans per round: their loads are issued together (indices
    // clamped into range, the extra ones ignored), then folded in order
    constexpr int NB = 8;
    for (int c0 = part; c0 < nch; c0 += parts * NB) {
      float mc[NB], lc[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const size_t c = (size_t)min(c0 + i * parts, nch - 1);
        mc[i] = sm[c * W];
        lc[i] = sl[c * W];
      }
      float bm = M;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (c0 + i * parts < nch) bm = fmaxf(bm, mc[i]);
      float acc = Lr * fast_exp2(M - bm);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (c0 + i * parts < nch) acc += lc[i] * fast_exp2(mc[i] - bm);
      M = bm;
      Lr = acc;
    }
  }
  pm[tid] = M;
  pl[tid] = Lr;
  __syncthreads();
  if (tid < W) {
    float Mt = kNegBig;
    for (int q = 0; q < parts; ++q) Mt = fmaxf(Mt, pm[q * W + tid]);
    float Lt = 0.f;
    for (int q = 0; q < parts; ++q) Lt += pl[q * W + tid] * fast_exp2(pm[q * W + tid] - Mt);
    row_m[(size_t)bh * W + tid] = Mt;
    row_inv[(size_t)bh * W + tid] = Lt > 0.f ? 1.0f / Lt : 0.f;
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
  // the span partial sums: LPH lanes per head, four loads in flight each
  int rp = 1;
  while (rp < r) rp <<= 1;   // r <= 16
  const int LPH = 64 / rp;
  const int hs = lane / LPH, ph = lane % LPH;
  float p1 = 0.f, p2 = 0.f;
  if (hs < r) {
    const float* e = ent + ((size_t)b * Hq + g * r + hs) * nch * 2;
    for (int c0 = ph; c0 < nch; c0 += 4 * LPH) {
      float2 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = *reinterpret_cast<const float2*>(e + 2 * min(c0 + j * LPH, nch - 1));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + j * LPH < nch) {
          p1 += v[j].x;
          p2 += v[j].y;
        }
    }
  }
  for (int o = LPH / 2; o > 0; o >>= 1) {
    p1 += __shfl_xor(p1, o);
    p2 += __shfl_xor(p2, o);
  }
  const float s1 = __shfl(p1, (on ? lane : 0) * LPH), s2 = __shfl(p2, (on ? lane : 0) * LPH);
  double H = 0.0;
  if (on) {
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
                                                        int ldk, float* __restrict__ mu,
                                                        float* __restrict__ scores) {
  __shared__ float qs[D];
  const int bg = blockIdx.y;
  for (int d = threadIdx.x; d < D; d += 256) qs[d] = qsum[(size_t)bg * D + d];
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  const bf16* k = K + ((size_t)bg * ldk + t) * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    float x[8];
    load8f(k + 8 * c, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[e] * qs[8 * c + e];
  }
  mu[(size_t)bg * L + t] = acc;
  if (scores != nullptr) scores[(size_t)bg * L + t] = acc;
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

// InfoKV fusion input: per batch, the maximum of the token entropies and the
// sum of exp(E - max) over the cache (one workgroup per batch)
__global__ __launch_bounds__(SEL_T) void token_softmax_stats_kernel(const float* __restrict__ E,
                                                                    int L,
                                                                    float* __restrict__ stats) {
  __shared__ float fred[SEL_T / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* e = E + (size_t)b * L;
  float mx = -INFINITY;
  for (int t = tid; t < L; t += SEL_T) mx = fmaxf(mx, e[t]);
  mx = block_max_1024f(mx, fred);
  float se = 0.f;
  for (int t = tid; t < L; t += SEL_T) se += expf(e[t] - mx);
  se = block_sum_1024f(se, fred);
  if (tid == 0) {
    stats[2 * b] = mx;
    stats[2 * b + 1] = 1.0f / se;
  }
}

// group score mu_t = sum_{h in g} w_h a^h_t, optionally fused with the
// softmax of the token entropies; one thread per (batch x KV group, key)
__global__ __launch_bounds__(256) void retain_mu_kernel(
    const float* __restrict__ mass, const float* __restrict__ weight,
    const float* __restrict__ token_entropy, const float* __restrict__ tstats,
    float info_alpha, int Hq, int Hkv, int r, int L, float* __restrict__ mu,
    float* __restrict__ scores) {
  const int bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  const float* mrow = mass + ((size_t)b * Hq + g * r) * L + t;
  const float* wv = weight + (size_t)b * Hq + g * r;
  // the group's head masses in rounds of four loads issued together (index
  // clamped; the sum keeps head order)
  float acc = 0.f;
  for (int h0 = 0; h0 < r; h0 += 4) {
    float mv[4], wh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hl = min(h0 + j, r - 1);
      mv[j] = mrow[(size_t)hl * L];
      wh[j] = wv[hl];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (h0 + j < r) acc += wh[j] * mv[j];
  }
  if (token_entropy != nullptr) {
    const float sm = expf(token_entropy[(size_t)b * L + t] - tstats[2 * b]) * tstats[2 * b + 1];
    acc = info_alpha * acc + (1.0f - info_alpha) * sm;
  }
  mu[(size_t)bg * L + t] = acc;
  if (scores != nullptr) scores[(size_t)bg * L + t] = acc;
}

// exact top-n_keep of mu over the candidates and ascending compaction of the
// keep set; one workgroup per (batch, KV group).
//   radix select: 12 / 12 / 8-bit digits of the order-preserving key, each
//     pass a coalesced sweep over the candidates (eight loads in flight per
//     thread) into an LDS histogram, then a scan that fixes the digit;
//   compaction: rounds of SEL_R consecutive keys staged in LDS with coalesced
//     loads; each thread takes SEL_R / SEL_T consecutive keys, one block scan
//     of (selected, tied) counts places them, ties to T taken by lower index.
constexpr int SEL_R = 16384;
constexpr int SEL_U = 8;

__global__ __launch_bounds__(SEL_T) void retain_select_kernel(
    const float* __restrict__ mu, int L, int n_sink, int n_recent, int n_keep, int n_total,
    int32_t* __restrict__ keep_idx) {
  __shared__ int hist[4096];
  // the round's keys, one pad word after every 16: a thread scans 16
  // consecutive keys, so the lanes of a wave read 17 words apart (distinct
  // banks) instead of 16 (a few banks, many-way conflicts)
  __shared__ uint32_t keys[SEL_R + SEL_R / 16];
  auto kslot = [](int j) { return j + (j >> 4); };
  __shared__ int ired[SEL_T / 64];
  __shared__ int sh_digit, sh_above, tot_sel, tot_eq;
  const int bg = blockIdx.x;
  const int tid = threadIdx.x;
  const float* mu_row = mu + (size_t)bg * L;

  const bool keep_all = (long long)n_sink + n_recent + n_keep >= L;
  const int c_lo = n_sink, c_hi = L - n_recent;   // candidates [c_lo, c_hi)
  uint32_t prefix = 0, mask = 0;
  int kr = n_keep;
  const bool partial = !keep_all && n_keep > 0;
  if (partial) {
    const int shifts[3] = {20, 8, 0};
    const int bits[3] = {12, 12, 8};
    for (int ps = 0; ps < 3; ++ps) {
      const int sh = shifts[ps], nb = 1 << bits[ps];
      for (int i = tid; i < 4096; i += SEL_T) hist[i] = 0;
      __syncthreads();
      for (int t0 = c_lo; t0 < c_hi; t0 += SEL_T * SEL_U) {
        uint32_t kv[SEL_U];
        // unconditional loads (index clamped into the candidates, which are
        // not empty here) so that all SEL_U are in flight before the first use
#pragma unroll
        for (int u = 0; u < SEL_U; ++u) kv[u] = orderable(mu_row[min(t0 + u * SEL_T + tid, c_hi - 1)]);
#pragma unroll
        for (int u = 0; u < SEL_U; ++u) {
          const int t = t0 + u * SEL_T + tid;
          if (t < c_hi && (kv[u] & mask) == prefix)
            atomicAdd(&hist[(kv[u] >> sh) & (uint32_t)(nb - 1)], 1);
        }
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
  const uint32_t T = prefix;   // key of the n_keep-th candidate; kr ties to T are kept

  // ---- ascending compaction over [0, L) ----
  constexpr int PER = SEL_R / SEL_T;
  int32_t* out = keep_idx + (size_t)bg * n_total;
  int base_sel = 0, base_eq = 0;   // kept and tied entries before this round
  for (int r0 = 0; r0 < L; r0 += SEL_R) {
    const int rn = min(SEL_R, L - r0);
    __syncthreads();   // the previous round's keys are consumed
    {
      // SEL_R / SEL_T loads per thread, issued together (clamped index)
      uint32_t kk[SEL_R / SEL_T];
#pragma unroll
      for (int e = 0; e < SEL_R / SEL_T; ++e) kk[e] = orderable(mu_row[r0 + min(e * SEL_T + tid, rn - 1)]);
#pragma unroll
      for (int e = 0; e < SEL_R / SEL_T; ++e)
        if (e * SEL_T + tid < rn) keys[kslot(e * SEL_T + tid)] = kk[e];
    }
    __syncthreads();
    const int j0 = tid * PER;
    int n_sel = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int j = j0 + e, t = r0 + j;
      if (j < rn) {
        const bool cand = t >= c_lo && t < c_hi;
        if (!cand || keep_all) {
          ++n_sel;
        } else if (partial) {
          const uint32_t kj = keys[kslot(j)];
          n_sel += kj > T;
          n_eq += kj == T;
        }
      }
    }
    // one scan of both counts (each below 2^16 per round); the ties kept
    // before this thread are the first kr ties in index order
    const int packed = block_excl_scan_1024((n_sel << 16) | n_eq, ired);
    int es = base_eq + (packed & 0xFFFF);
    int pos = base_sel + (packed >> 16) + min(es, kr);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int j = j0 + e, t = r0 + j;
      if (j < rn) {
        const bool cand = t >= c_lo && t < c_hi;
        bool take;
        if (!cand || keep_all) {
          take = true;
        } else if (!partial) {
          take = false;
        } else if (keys[kslot(j)] > T) {
          take = true;
        } else if (keys[kslot(j)] == T) {
          take = es < kr;
          ++es;
        } else {
          take = false;
        }
        if (take) {
          if (pos < n_total) out[pos] = t;
          ++pos;
        }
      }
    }
    // round totals: the last thread's exclusive prefix plus its own counts
    if (tid == SEL_T - 1) {
      tot_sel = (packed >> 16) + n_sel;
      tot_eq = (packed & 0xFFFF) + n_eq;
    }
    __syncthreads();
    base_sel += tot_sel;
    base_eq += tot_eq;
  }
}

// ---------------------------------------------------------------------------
// The same top-n_keep and compaction split over many workgroups (the kv_retain
// rows are long: one workgroup per row leaves most of the chip idle).  Per
// row, state = {prefix, mask, kr, flags}.  Three radix passes of 12 / 12 / 8
// bits: rsel_hist counts one digit over a chunk of the candidates into its
// own 4096-bin histogram in global memory (no atomics across workgroups),
// rsel_digit sums the chunks' histograms and fixes the digit; then
// rsel_count counts the kept and tied entries of every chunk of [0, L) and
// rsel_write places the chunk's entries after the earlier chunks' counts.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rsel_pass_bits(int pass, int& sh, int& nb) {
  sh = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
  nb = pass == 2 ? 256 : 4096;
}

__global__ __launch_bounds__(SEL_T) void rsel_hist_kernel(const float* __restrict__ mu, int L,
                                                          int c_lo, int c_hi, int nsel,
                                                          int pass,
                                                          const int32_t* __restrict__ state,
                                                          int32_t* __restrict__ gh) {
  __shared__ int hist[4096];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  int sh, nb;
  rsel_pass_bits(pass, sh, nb);
  uint32_t prefix = 0, mask = 0;
  if (pass > 0) {
    prefix = (uint32_t)state[row * 4];
    mask = (uint32_t)state[row * 4 + 1];
  }
  for (int i = tid; i < 4096; i += SEL_T) hist[i] = 0;
  __syncthreads();
  const int per = (c_hi - c_lo + nsel - 1) / nsel;
  const int t_lo = c_lo + c * per, t_hi = min(c_hi, t_lo + per);
  const float* m = mu + (size_t)row * L;
  for (int t0 = t_lo; t0 < t_hi; t0 += SEL_T * SEL_U) {
    uint32_t kv[SEL_U];
    // unconditional clamped loads, all in flight before the first use
#pragma unroll
    for (int u = 0; u < SEL_U; ++u) kv[u] = orderable(m[min(t0 + u * SEL_T + tid, t_hi - 1)]);
#pragma unroll
    for (int u = 0; u < SEL_U; ++u)
      if (t0 + u * SEL_T + tid < t_hi && (kv[u] & mask) == prefix)
        atomicAdd(&hist[(kv[u] >> sh) & (uint32_t)(nb - 1)], 1);
  }
  __syncthreads();
  int32_t* out = gh + ((size_t)row * nsel + c) * 4096;
  for (int i = tid; i < nb; i += SEL_T) out[i] = hist[i];
}

__global__ __launch_bounds__(SEL_T) void rsel_digit_kernel(int nsel, int n_keep, int pass,
                                                           const int32_t* __restrict__ gh,
                                                           int32_t* __restrict__ state) {
  __shared__ int ired[SEL_T / 64];
  __shared__ int sh_digit, sh_above;
  const int row = blockIdx.x, tid = threadIdx.x;
  int sh, nb;
  rsel_pass_bits(pass, sh, nb);
  uint32_t prefix = 0, mask = 0;
  int kr = n_keep;
  if (pass > 0) {
    prefix = (uint32_t)state[row * 4];
    mask = (uint32_t)state[row * 4 + 1];
    kr = state[row * 4 + 2];
  }
  // thread tid owns digits nb-1-4*tid .. nb-4-4*tid (descending), summed over the chunks
  const int d0 = nb - 1 - 4 * tid;
  const bool own = d0 >= 3;
  int cnt4[4] = {0, 0, 0, 0};
  if (own) {
    const int32_t* h = gh + (size_t)row * nsel * 4096;
    for (int c = 0; c < nsel; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) cnt4[q] += h[(size_t)c * 4096 + d0 - q];
  }
  const int tot = cnt4[0] + cnt4[1] + cnt4[2] + cnt4[3];
  const int excl = block_excl_scan_1024(tot, ired);
  if (own && excl < kr && kr <= excl + tot) {
    int run = excl, dd = d0 - 3;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (run + cnt4[q] >= kr) {
        dd = d0 - q;
        break;
      }
      run += cnt4[q];
    }
    sh_digit = dd;
    sh_above = run;
  }
  __syncthreads();
  if (tid == 0) {
    state[row * 4] = (int32_t)(prefix | ((uint32_t)sh_digit << sh));
    state[row * 4 + 1] = (int32_t)(mask | ((uint32_t)(nb - 1) << sh));
    state[row * 4 + 2] = kr - sh_above;
  }
}

// per chunk of [0, L): entries kept for sure (non-candidates when partial,
// every entry when keep_all, keys above T) and keys equal to T
__global__ __launch_bounds__(SEL_T) void rsel_count_kernel(const float* __restrict__ mu, int L,
                                                           int c_lo, int c_hi, int keep_all,
                                                           int partial,
                                                           const int32_t* __restrict__ state,
                                                           int32_t* __restrict__ cnt) {
  __shared__ int ired[SEL_T / 64];
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, nsel = gridDim.x;
  const uint32_t T = partial ? (uint32_t)state[row * 4] : 0u;
  const int r0 = c * SEL_CH, rn = min(SEL_CH, L - r0);
  const float* m = mu + (size_t)row * L + r0;
  int n_sel = 0, n_eq = 0;
  constexpr int PER = SEL_CH / SEL_T;
  uint32_t kk[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) kk[e] = orderable(m[min(e * SEL_T + tid, rn - 1)]);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = e * SEL_T + tid, t = r0 + j;
    if (j < rn) {
      const bool cand = t >= c_lo && t < c_hi;
      if (!cand || keep_all) {
        ++n_sel;
      } else if (partial) {
        n_sel += kk[e] > T;
        n_eq += kk[e] == T;
      }
    }
  }
  const int packed = block_sum_1024((n_sel << 16) | n_eq, ired);
  if (tid == 0) {
    cnt[((size_t)row * nsel + c) * 2] = packed >> 16;
    cnt[((size_t)row * nsel + c) * 2 + 1] = packed & 0xFFFF;
  }
}

__global__ __launch_bounds__(SEL_T) void rsel_write_kernel(const float* __restrict__ mu, int L,
                                                           int c_lo, int c_hi, int keep_all,
                                                           int partial, int n_total,
                                                           const int32_t* __restrict__ state,
                                                           const int32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ keep_idx) {
  __shared__ uint32_t keys[SEL_CH + SEL_CH / 16];
  auto kslot = [](int j) { return j + (j >> 4); };
  __shared__ int ired[SEL_T / 64];
  __shared__ int sh_base_sel, sh_base_eq;
  const int c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, nsel = gridDim.x;
  const uint32_t T = partial ? (uint32_t)state[row * 4] : 0u;
  const int kr = partial ? state[row * 4 + 2] : 0;
  if (tid == 0) {
    int bs = 0, be = 0;
    for (int q = 0; q < c; ++q) {
      bs += cnt[((size_t)row * nsel + q) * 2];
      be += cnt[((size_t)row * nsel + q) * 2 + 1];
    }
    sh_base_sel = bs;
    sh_base_eq = be;
  }
  const int r0 = c * SEL_CH, rn = min(SEL_CH, L - r0);
  const float* m = mu + (size_t)row * L + r0;
  {
    uint32_t kk[SEL_CH / SEL_T];
#pragma unroll
    for (int e = 0; e < SEL_CH / SEL_T; ++e) kk[e] = orderable(m[min(e * SEL_T + tid, rn - 1)]);
#pragma unroll
    for (int e = 0; e < SEL_CH / SEL_T; ++e)
      if (e * SEL_T + tid < rn) keys[kslot(e * SEL_T + tid)] = kk[e];
  }
  __syncthreads();
  constexpr int PER = SEL_CH / SEL_T;
  const int j0 = tid * PER;
  int n_sel = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = j0 + e, t = r0 + j;
    if (j < rn) {
      const bool cand = t >= c_lo && t < c_hi;
      if (!cand || keep_all) {
        ++n_sel;
      } else if (partial) {
        const uint32_t kj = keys[kslot(j)];
        n_sel += kj > T;
        n_eq += kj == T;
      }
    }
  }
  const int packed = block_excl_scan_1024((n_sel << 16) | n_eq, ired);
  int es = sh_base_eq + (packed & 0xFFFF);
  int pos = sh_base_sel + (packed >> 16) + min(es, kr);
  int32_t* out = keep_idx + (size_t)row * n_total;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = j0 + e, t = r0 + j;
    if (j < rn) {
      const bool cand = t >= c_lo && t < c_hi;
      bool take;
      if (!cand || keep_all) {
        take = true;
      } else if (!partial) {
        take = false;
      } else if (keys[kslot(j)] > T) {
        take = true;
      } else if (keys[kslot(j)] == T) {
        take = es < kr;
        ++es;
      } else {
        take = false;
      }
      if (take) {
        if (pos < n_total) out[pos] = t;
        ++pos;
      }
    }
  }
}

// the kv_retain top-k: the split kernels for long rows, the one-workgroup
// kernel otherwise
static hipError_t launch_retain_topk(const DecodeDims& p, const RetainLayout& lay, char* ws,
                                     const float* mu, int32_t* keep_idx, hipStream_t st) {
  const int rows = p.B * p.Hkv;
  if (p.L < 4 * SEL_CH) {
    retain_select_kernel<<<rows, SEL_T, 0, st>>>(mu, p.L, p.n_sink, p.n_recent, p.n_keep,
                                                 p.n_total, keep_idx);
    return hipGetLastError();
  }
  int32_t* gh = reinterpret_cast<int32_t*>(ws + lay.sel_hist);
  int32_t* state = reinterpret_cast<int32_t*>(ws + lay.sel_state);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + lay.sel_cnt);
  const int c_lo = p.n_sink, c_hi = p.L - p.n_recent;
  const bool keep_all = (long long)p.n_sink + p.n_recent + p.n_keep >= p.L;
  const bool partial = !keep_all && p.n_keep > 0;
  hipError_t e;
  if (partial) {
    for (int pass = 0; pass < 3; ++pass) {
      rsel_hist_kernel<<<dim3(lay.nsel, rows), SEL_T, 0, st>>>(mu, p.L, c_lo, c_hi, lay.nsel,
                                                               pass, state, gh);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      rsel_digit_kernel<<<rows, SEL_T, 0, st>>>(lay.nsel, p.n_keep, pass, gh, state);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  rsel_count_kernel<<<dim3(lay.nsel, rows), SEL_T, 0, st>>>(mu, p.L, c_lo, c_hi, keep_all ? 1 : 0,
                                                            partial ? 1 : 0, state, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  rsel_write_kernel<<<dim3(lay.nsel, rows), SEL_T, 0, st>>>(mu, p.L, c_lo, c_hi,
                                                            keep_all ? 1 : 0, partial ? 1 : 0,
                                                            p.n_total, state, cnt, keep_idx);
  return hipGetLastError();
}

// copy the kept K / V rows: one thread per 16 bytes
template <int D>
__global__ __launch_bounds__(256) void gather_kv_kernel(const bf16* __restrict__ K,
                                                        const bf16* __restrict__ V,
                                                        const int32_t* __restrict__ keep, int L,
                                                        int ldk, int n_total, long long units,
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
  const size_t src = ((size_t)bg * ldk + t) * D + c8 * 8;
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
// With sg (chunk pruning, batch 1), pass 1 also writes the chunk segments.
struct SegArgs {
  const int32_t* cid;
  const int32_t* bounds;
  const int32_t* seg_base;
  float* seg_v;
  float* seg_m;
};

template <int D, int RT>
static hipError_t retain_passes(const DecodeDims& p, const RetainLayout& lay, char* ws,
                                const void* q_obs, const void* k, int kind, float alpha,
                                hipStream_t st, const SegArgs* sg = nullptr) {
  const float sl2 = p.sm_scale * kLog2e;
  dim3 grid(lay.nch, p.B * p.Hkv, (p.r + 3) / 4);
  const bf16* Qo = static_cast<const bf16*>(q_obs);
  const bf16* K = static_cast<const bf16*>(k);
  float* stat_m = reinterpret_cast<float*>(ws + lay.stat_m);
  float* stat_l = reinterpret_cast<float*>(ws + lay.stat_l);
  float* row_m = reinterpret_cast<float*>(ws + lay.row_m);
  float* row_inv = reinterpret_cast<float*>(ws + lay.row_inv);
  float* mass = reinterpret_cast<float*>(ws + lay.mass);
  float* ent = reinterpret_cast<float*>(ws + lay.ent);
  if (sg != nullptr)
    obs_pass_kernel<D, RT, false, true><<<grid, 256, 0, st>>>(
        Qo, K, p.Hq, p.Hkv, p.r, p.L, p.Lk, p.W, lay.nch, sl2, stat_m, stat_l, row_m, row_inv,
        p.n_sink, kind, alpha, mass, ent, sg->cid, sg->bounds, sg->seg_base, sg->seg_v,
        sg->seg_m);
  else
    obs_pass_kernel<D, RT, false><<<grid, 256, 0, st>>>(Qo, K, p.Hq, p.Hkv, p.r, p.L, p.Lk, p.W,
                                                        lay.nch, sl2, stat_m, stat_l, row_m,
                                                        row_inv, p.n_sink, kind, alpha, mass, ent);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  obs_combine_kernel<<<p.B * p.Hq, 256, 0, st>>>(stat_m, stat_l, lay.nch, p.W, row_m, row_inv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  obs_pass_kernel<D, RT, true><<<grid, 256, 0, st>>>(Qo, K, p.Hq, p.Hkv, p.r, p.L, p.Lk, p.W,
                                                     lay.nch, sl2, stat_m, stat_l, row_m,
                                                     row_inv, p.n_sink, kind, alpha, mass, ent);
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
      raw_score_kernel<128><<<grid, 256, 0, st>>>(static_cast<const bf16*>(k), qsum, p.L, p.Lk, mu,
                                                  scores);
    else
      raw_score_kernel<64><<<grid, 256, 0, st>>>(static_cast<const bf16*>(k), qsum, p.L, p.Lk, mu,
                                                 scores);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (head_entropy != nullptr) {
      const int n = p.B * p.Hq;
      fill_zero_kernel<<<(n + 255) / 256, 256, 0, st>>>(head_entropy, n);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  float* mu = reinterpret_cast<float*>(ws + lay.mu);
  if (!raw) {
    const bool fuse = token_entropy != nullptr && prm.info_alpha < 1.0;
    float* tstats = reinterpret_cast<float*>(ws + lay.tstats);
    if (fuse) {
      token_softmax_stats_kernel<<<p.B, SEL_T, 0, st>>>(token_entropy, p.L, tstats);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    dim3 grid((p.L + 255) / 256, p.B * p.Hkv);
    retain_mu_kernel<<<grid, 256, 0, st>>>(
        reinterpret_cast<const float*>(ws + lay.mass),
        reinterpret_cast<const float*>(ws + lay.weight), fuse ? token_entropy : nullptr, tstats,
        (float)prm.info_alpha, p.Hq, p.Hkv, p.r, p.L, mu, scores);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = launch_retain_topk(p, lay, ws, mu, keep_idx, st)) != hipSuccess) return e;
  if (k_out != nullptr) {
    const long long units = (long long)p.B * p.Hkv * p.n_total * (p.D / 8);
    const unsigned blocks = (unsigned)((units + 255) / 256);
    if (p.D == 128)
      gather_kv_kernel<128><<<blocks, 256, 0, st>>>(
          static_cast<const bf16*>(k), static_cast<const bf16*>(v), keep_idx, p.L, p.Lk,
          p.n_total, units, static_cast<bf16*>(k_out), static_cast<bf16*>(v_out));
    else
      gather_kv_kernel<64><<<blocks, 256, 0, st>>>(
          static_cast<const bf16*>(k), static_cast<const bf16*>(v), keep_idx, p.L, p.Lk,
          p.n_total, units, static_cast<bf16*>(k_out), static_cast<bf16*>(v_out));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// K8: decode attention over the kept entries
// ---------------------------------------------------------------------------
// One workgroup per (split of spl kept entries, batch x KV group); the GQA
// group's query heads (one per wavefront, four at a time) share every 64-entry
// K / V stage, copied straight into LDS two stages deep.
//   QK: a lane owns one entry of the stage; the entry's K row is read as
//       swizzled 16-byte chunks and meets the head's bf16 query (one
//       broadcast LDS read per chunk) in v_dot2c_f32_bf16: exact products
//       of bf16 pairs, fp32 sums, no conversions.
//   softmax: online per head over the split (wave max / sum per stage).
//   PV: a lane owns one 16-byte chunk of the V rows for a quarter (d 128) or
//       an eighth (d 64) of the stage's entries (16-byte LDS reads); two keys
//       at a time, their probabilities as a bf16 pair (the row sums stay in
//       fp32) and each dimension's two V values as a pair go through
//       v_dot2c_f32_bf16; the lanes' partial outputs are summed once per
//       split.
// Each split leaves its unnormalised output, maximum and sum for the combine.
template <int D>
__global__ __launch_bounds__(256) void decode_attn_split_kernel(
    const bf16* __restrict__ Qn, const bf16* __restrict__ K, const bf16* __restrict__ V,
    int Hq, int Hkv, int r, int n, int ldk, int spl, int nsplit, float sl2,
    float* __restrict__ part) {
  constexpr int KCH = D / 8;           // 16-byte chunks per row
  constexpr int ST = 64;               // entries per stage
  constexpr int PIECES = ST * D * 2 / 1024;
  constexpr int PER_W = PIECES / 4;
  constexpr int KROWS = 1024 / (D * 2);
  static_assert(PIECES % 4 == 0, "stage copies must split over four waves");
  __shared__ __attribute__((aligned(1024))) bf16 Ks[2][ST * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[2][ST * D];
  __shared__ __attribute__((aligned(16))) bf16 qsb[4][D];
  __shared__ float psh[4][ST];
  const int sp = blockIdx.x, bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t_begin = sp * spl, t_end = min(n, t_begin + spl);
  const int nst = (t_end - t_begin + ST - 1) / ST;
  const bf16* Kg = K + (size_t)bg * ldk * D;
  const bf16* Vg = V + (size_t)bg * ldk * D;
  // K and V rows share one layout: swizzled 16-byte chunks
  auto copy_stage = [&](int st, int buf) {
    const int t0 = t_begin + st * ST;
#pragma unroll
    for (int ii = 0; ii < PER_W; ++ii) {
      const int pc = w * PER_W + ii;
      const int row = pc * KROWS + lane / KCH;
      const int c = (lane % KCH) ^ lds_swz<D * 2>(row);
      const int t = min(t0 + row, t_end - 1);   // past the split: a repeated row, masked
      const uint32_t off = (uint32_t)(((t - t0) * D + c * 8) * sizeof(bf16));
      copy16_to_lds(Kg + (size_t)t0 * D, off, Ks[buf] + pc * 512);
      copy16_to_lds(Vg + (size_t)t0 * D, off, Vs[buf] + pc * 512);
    }
  };
  for (int hl0 = 0; hl0 < r; hl0 += 4) {
    const int hl = hl0 + w;
    const bool hv = hl < r;
    const int h = g * r + (hv ? hl : 0);
    {
      const bf16* q = Qn + ((size_t)b * Hq + h) * D;
      for (int d = lane; d < D; d += 64) qsb[w][d] = hv ? q[d] : (bf16)0.f;
    }
    copy_stage(0, 0);
    // PV: lane = (key group kg, 16-byte chunk c of the V row): dims 8c .. 8c+7
    // over keys kg*KPG .. kg*KPG+KPG-1 of every stage (16-byte LDS reads); the
    // key groups are summed once after the last stage
    constexpr int KG = 64 / KCH, KPG = ST / KG;
    const int vc = lane % KCH, kg = lane / KCH;
    float m = kNegBig, l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int st = 0; st < nst; ++st) {
      wait_vmem();
      __syncthreads();   // stage st landed; every wave is done with stage st-1
      if (st + 1 < nst) copy_stage(st + 1, (st + 1) & 1);
      const bf16* ks = Ks[st & 1];
      const bf16* vs = Vs[st & 1];
      const int t = t_begin + st * ST + lane;
      // logit of this lane's entry (log2 units)
      // bf16 pairs straight into v_dot2c_f32_bf16 (exact products, fp32
      // sums); the query chunk is one broadcast LDS read
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const bf16x8 kv = load8(ks + lane * D + ((c ^ lds_swz<D * 2>(lane)) * 8));
        const bf16x8 qv = load8(&qsb[w][8 * c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 kp = {kv[2 * e], kv[2 * e + 1]};
          const bf16x2 qp = {qv[2 * e], qv[2 * e + 1]};
          z = __builtin_amdgcn_fdot2_f32_bf16(kp, qp, z, false);
        }
      }
      z *= sl2;
      if (t >= t_end) z = -INFINITY;
      const float mx = fmaxf(m, wave_max_v(z));
      const float pz = fast_exp2(z - mx);
      const float alpha = fast_exp2(m - mx);
      l = l * alpha + wave_sum_v(pz);
      m = mx;
      psh[w][lane] = pz;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
      // two keys at a time: their probabilities as a bf16 pair and, per
      // dimension, the two V values as a pair, into v_dot2c_f32_bf16
#pragma unroll
      for (int j = 0; j < KPG; j += 2) {
        const int k = kg * KPG + j;
        const bf16x2 pp = {(bf16)psh[w][k], (bf16)psh[w][k + 1]};
        const bf16x8 v0 = load8(vs + k * D + ((vc ^ lds_swz<D * 2>(k)) * 8));
        const bf16x8 v1 = load8(vs + (k + 1) * D + ((vc ^ lds_swz<D * 2>(k + 1)) * 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bf16x2 vp = {v0[e], v1[e]};
          o[e] = __builtin_amdgcn_fdot2_f32_bf16(vp, pp, o[e], false);
        }
      }
    }
    // sum the key groups (lanes vc, vc + KCH, ...)
    if constexpr (KCH < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], KCH);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = xhalf_sum(xrow_sum(o[e]));
    if (hv) {
      float* pp = part + (((size_t)b * Hq + h) * nsplit + sp) * (D + 2);
      if (kg == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pp[8 * vc + e] = o[e];
      }
      if (lane == 0) {
        pp[D] = m;
        pp[D + 1] = l;
      }
    }
    __syncthreads();   // the stage buffers are reused by the next head group
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_attn_combine_kernel(const float* __restrict__ part,
                                                                  int nsplit, bf16* __restrict__ out) {
  constexpr int DPL = D / 64;
  constexpr int NB = 8;   // splits per round, their loads issued together
  __shared__ float wm[4], wl[4], wo[4][D];
  const int bh = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* pp = part + (size_t)bh * nsplit * (D + 2);
  // wave w folds the splits of quarter w against that quarter's maximum
  const int qn = (nsplit + 3) / 4;
  const int s_lo = min(nsplit, w * qn), s_hi = min(nsplit, s_lo + qn);
  float M = kNegBig;
  for (int s0 = s_lo; s0 < s_hi; s0 += 64)
    M = fmaxf(M, wave_max(s0 + lane < s_hi ? pp[(size_t)(s0 + lane) * (D + 2) + D] : kNegBig));
  float Lr = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int s0 = s_lo; s0 < s_hi; s0 += NB) {
    float sm[NB], sl[NB], so[NB][DPL];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float* q = pp + (size_t)min(s0 + j, s_hi - 1) * (D + 2);   // clamped
      sm[j] = q[D];
      sl[j] = q[D + 1];
#pragma unroll
      for (int e = 0; e < DPL; ++e) so[j][e] = q[lane * DPL + e];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (s0 + j < s_hi) {
        const float f = fast_exp2(sm[j] - M);
        Lr += sl[j] * f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] += so[j][e] * f;
      }
  }
  if (lane == 0) {
    wm[w] = M;
    wl[w] = Lr;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) wo[w][lane * DPL + e] = o[e];
  __syncthreads();
  if (w == 0) {
    // the four quarters in order (an empty quarter holds kNegBig, 0)
    float Mt = wm[0];
#pragma unroll
    for (int v = 1; v < 4; ++v) Mt = fmaxf(Mt, wm[v]);
    float Lt = 0.f, ot[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) ot[e] = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float f = fast_exp2(wm[v] - Mt);
      Lt += wl[v] * f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) ot[e] += wo[v][lane * DPL + e] * f;
    }
    const float inv = 1.0f / Lt;
#pragma unroll
    for (int e = 0; e < DPL; ++e) out[(size_t)bh * D + lane * DPL + e] = f2bf(ot[e] * inv);
  }
}

// Split size: the largest multiple of 64 in [DA_SPL_MIN, DA_SPL_MAX] whose
// last round of workgroups still fills 90% of the 512 workgroup slots (256
// CUs x 2, LDS-bound); else the one that leaves the fewest slots idle.  Long
// caches take 1024 (fewer prologues and partials to combine); the 4,356 kept
// entries of a batch-8 step take 576 (8 splits x 64 rows: exactly one round,
// where 192-entry splits needed three).
static int decode_split(const DecodeDims& p, int n_total) {
  constexpr long kSlots = 512;
  const long rows = (long)p.B * p.Hkv;
  int best = DA_SPL_MAX;
  double best_eff = -1.0;
  for (int s = DA_SPL_MAX; s >= DA_SPL_MIN; s -= 64) {
    const long wg = rows * ((n_total + s - 1) / s);
    const long rounds = (wg + kSlots - 1) / kSlots;
    if (wg * 10 >= rounds * kSlots * 9) return s;
    const double eff = (double)wg / (double)(rounds * kSlots);
    if (eff > best_eff) {
      best_eff = eff;
      best = s;
    }
  }
  return best;
}

size_t decode_attn_workspace_bytes(const DecodeDims& p, int n_total) {
  const int spl = decode_split(p, n_total);
  const int nsplit = (n_total + spl - 1) / spl;
  return align_up((size_t)p.B * p.Hq * nsplit * (p.D + 2) * 4);
}

// The split count is not monotone in n (a shorter list can take a smaller
// split), so a buffer reused for every length up to `cap` is sized for the
// smallest split the launcher can choose: ceil(cap / DA_SPL_MIN) partials.
size_t decode_attn_workspace_bytes_upto(const DecodeDims& p, int cap) {
  const int nsplit = (cap + DA_SPL_MIN - 1) / DA_SPL_MIN;
  return align_up((size_t)p.B * p.Hq * nsplit * (p.D + 2) * 4);
}

hipError_t launch_decode_attn(const DecodeDims& p, const void* q_new, const void* k,
                              const void* v, int n_total, int ldk, void* out, void* ws,
                              hipStream_t st) {
  const int spl = decode_split(p, n_total);
  const int nsplit = (n_total + spl - 1) / spl;
  const float sl2 = p.sm_scale * kLog2e;
  float* part = static_cast<float*>(ws);
  dim3 grid(nsplit, p.B * p.Hkv);
  const bf16* Qn = static_cast<const bf16*>(q_new);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  if (p.D == 128)
    decode_attn_split_kernel<128><<<grid, 256, 0, st>>>(Qn, K, V, p.Hq, p.Hkv, p.r, n_total,
                                                        ldk, spl, nsplit, sl2, part);
  else
    decode_attn_split_kernel<64><<<grid, 256, 0, st>>>(Qn, K, V, p.Hq, p.Hkv, p.r, n_total,
                                                       ldk, spl, nsplit, sl2, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 128)
    decode_attn_combine_kernel<128><<<p.B * p.Hq, 256, 0, st>>>(part, nsplit,
                                                               static_cast<bf16*>(out));
  else
    decode_attn_combine_kernel<64><<<p.B * p.Hq, 256, 0, st>>>(part, nsplit,
                                                              static_cast<bf16*>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Chunk pruning (EntroPrefill Sec. 3.1-3.2, 4.1-4.2): the observer-pooled
// measure of one prompt (the retention passes with Renyi-2 head entropies,
// averaged over the KV groups), the mass every observer row puts on every
// candidate chunk, null-calibrated chunk priorities and the greedy feasible
// removal scan.
// ---------------------------------------------------------------------------
constexpr int PR_MAX_CHUNKS = 4096;
constexpr int PR_MAX_ROWS = 8192;

// The caller's chunk bounds (device memory) checked and copied: chunks must be
// ascending, disjoint, non-empty and end at or before limit = T - W.  The copy
// is clamped into that shape whatever the input, so every later index stays
// in range; ok[0] records whether the input already had it (the scan reports
// a failure through removed_tokens = -1 when it did not).  One thread: k is
// at most a few thousand.
__global__ __launch_bounds__(64) void chunk_bounds_kernel(const int32_t* __restrict__ in, int k,
                                                          int limit, int32_t* __restrict__ out,
                                                          int32_t* __restrict__ ok) {
  if (threadIdx.x != 0) return;
  int prev = 0, valid = 1;
  for (int i = 0; i < k; ++i) {
    const int b = in[2 * i], e = in[2 * i + 1];
    if (b < prev || e <= b || e > limit) valid = 0;
    const int bc = min(max(b, prev), limit);
    const int ec = min(max(e, bc), limit);
    out[2 * i] = bc;
    out[2 * i + 1] = ec;
    prev = ec;
  }
  ok[0] = valid;
}

// chunk id of every position (-1 outside the chunks); bounds [k][2] ascending
__global__ __launch_bounds__(256) void chunk_of_kernel(const int32_t* __restrict__ bounds, int k,
                                                       int T, int32_t* __restrict__ cid) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = k - 1, id = -1;
  while (lo <= hi) {   // the last chunk whose begin is <= t
    const int mid = (lo + hi) >> 1;
    if (bounds[2 * mid] <= t) {
      id = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  cid[t] = (id >= 0 && t < bounds[2 * id + 1]) ? id : -1;
}

// first segment of every chunk: seg_base[c] = sum over c' < c of the number of
// 2048-key spans chunk c' touches; seg_base[k] = the total.  One workgroup.
__global__ __launch_bounds__(SEL_T) void seg_base_kernel(const int32_t* __restrict__ bounds,
                                                         int k, int32_t* __restrict__ seg_base) {
  __shared__ int ired[SEL_T / 64];
  constexpr int PER = PR_MAX_CHUNKS / SEL_T;
  const int tid = threadIdx.x;
  int n[PER], own = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = tid * PER + j;
    n[j] = c < k ? (bounds[2 * c + 1] - 1) / RT_CK - bounds[2 * c] / RT_CK + 1 : 0;
    own += n[j];
  }
  int pos = block_excl_scan_1024(own, ired);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int c = tid * PER + j;
    if (c < k) seg_base[c] = pos;
    pos += n[j];
    if (c == k - 1) seg_base[k] = pos;
  }
}

// m[c][a] = sum over the segments of chunk c of seg_v exp2(seg_m - M_a) / L_a,
// with the row's final reference M_a and sum L_a (row_m, row_inv); workgroup
// per (chunk, 256 rows), thread per row a = h * W + u
__global__ __launch_bounds__(256) void chunk_norm_kernel(
    const int32_t* __restrict__ seg_base, const float* __restrict__ seg_v,
    const float* __restrict__ seg_m, const float* __restrict__ row_m,
    const float* __restrict__ row_inv, int R, float* __restrict__ m) {
  const int c = blockIdx.x;
  const int a = blockIdx.y * 256 + threadIdx.x;
  if (a >= R) return;
  const int s0 = seg_base[c], s1 = seg_base[c + 1];
  const float M = row_m[a], inv = row_inv[a];
  float acc = 0.f;
  for (int sg = s0; sg < s1; ++sg)
    acc += seg_v[(size_t)sg * R + a] * fast_exp2(seg_m[(size_t)sg * R + a] - M);
  m[(size_t)c * R + a] = acc * inv;
}

// pooled measure mu^l_t = (1/G) sum_g sum_{h in g} w_h a^h_t of one sequence
// (the group sums in head order, then the mean over groups); one thread per
// position, the head masses in rounds of eight loads issued together
__global__ __launch_bounds__(256) void pooled_mu_kernel(const float* __restrict__ mass,
                                                        const float* __restrict__ weight, int Hq,
                                                        int Hkv, int r, int L,
                                                        float* __restrict__ pooled) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= L) return;
  float tot = 0.f;
  for (int g = 0; g < Hkv; ++g) {
    float acc = 0.f;
    for (int h0 = 0; h0 < r; h0 += 8) {
      float mv[8], wh[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int h = g * r + min(h0 + j, r - 1);
        mv[j] = mass[(size_t)h * L + t];
        wh[j] = weight[h];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (h0 + j < r) acc += wh[j] * mv[j];
    }
    tot += acc;
  }
  pooled[t] = tot / (float)Hkv;
}

// per chunk: s[i] = (sum, sum of squares) of the pooled measure over the
// chunk; one workgroup per chunk, eight coalesced loads in flight per thread
__global__ __launch_bounds__(256) void chunk_stats_kernel(const float* __restrict__ pooled,
                                                          const int32_t* __restrict__ bounds,
                                                          float* __restrict__ stats) {
  __shared__ float red[2][4];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int b0 = bounds[2 * i], b1 = bounds[2 * i + 1];
  float s1 = 0.f, s2 = 0.f;
  for (int base = b0; base < b1; base += 8 * 256) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = pooled[min(base + j * 256 + tid, b1 - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (base + j * 256 + tid < b1) {
        s1 += v[j];
        s2 += v[j] * v[j];
      }
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = s1;
    red[1][tid >> 6] = s2;
  }
  __syncthreads();
  if (tid == 0) {
    stats[2 * i] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    stats[2 * i + 1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

// Block-wide AND of 32-bit masks (one bit per scan step).  Two LDS slots are
// used in turn, so one barrier per call suffices: a slot is written again only
// after every thread has passed the barrier of the call in between.
__device__ __forceinline__ uint32_t block_and_mask(uint32_t v, uint32_t (*red)[SEL_T / 64],
                                                   int& slot) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v &= (uint32_t)__shfl_xor((int)v, o);
  if ((threadIdx.x & 63) == 0) red[slot][threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = ~0u;
#pragma unroll
  for (int w = 0; w < SEL_T / 64; ++w) r &= red[slot][w];
  slot ^= 1;
  return r;
}

// priorities, their order and the greedy scan; one workgroup of 1024 threads,
// thread tid keeping the running sums of rows tid + j * 1024, j < RPT.
// Order: up to 512 chunks by rank (each thread counts the chunks that come
// before its own; the order (S, -n, index) is total), more by bitonic sort.
// Scan: the masses are >= 0, so the running sums only grow and a chunk that
// does not fit on its own never fits later.  The mass columns of PF sorted
// chunks are fetched at once; a round votes (1) which of them fit on their
// own and (2) which fit when every earlier one that fits on its own is also
// removed; the steps are then taken in order, and a round ends early only at
// a chunk that fits alone but not after the earlier ones (its rejection
// changes what the later ones see).  Two barriers per round instead of one per
// chunk.
template <int RPT>
__global__ __launch_bounds__(SEL_T) void prune_select_kernel(
    const float* __restrict__ stats, const int32_t* __restrict__ bounds, int k, int R,
    const float* __restrict__ m, float eps_s, float lam, float eps, int m0, int target,
    const int32_t* __restrict__ bounds_ok, float* __restrict__ prio,
    int8_t* __restrict__ removed, int32_t* __restrict__ removed_tokens) {
  if (bounds_ok[0] == 0) {   // the caller's chunks were not valid: nothing is removed
    for (int i = threadIdx.x; i < k; i += SEL_T) {
      removed[i] = 0;
      prio[i] = __builtin_nanf("");
    }
    if (threadIdx.x == 0) *removed_tokens = -1;
    return;
  }
  __shared__ float key_s[PR_MAX_CHUNKS];
  __shared__ int key_n[PR_MAX_CHUNKS];
  __shared__ int key_i[PR_MAX_CHUNKS];
  __shared__ int order[PR_MAX_CHUNKS];
  __shared__ float red[SEL_T / 64];
  __shared__ int ired[SEL_T / 64];
  __shared__ uint32_t vote[2][SEL_T / 64];
  const int tid = threadIdx.x;
  // totals: Z = sum of the chunks' pooled mass, N = candidate tokens
  float z = 0.f;
  int nn = 0;
  for (int i = tid; i < k; i += SEL_T) {
    z += stats[2 * i];
    nn += bounds[2 * i + 1] - bounds[2 * i];
  }
  z = wave_sum(z);
  if ((tid & 63) == 0) red[tid >> 6] = z;
  const int ntot = block_excl_scan_1024(nn, ired) + nn;   // the last thread holds the total
  __shared__ float shZ;
  __shared__ int shN;
  __syncthreads();
  if (tid == SEL_T - 1) {
    float a = 0.f;
    for (int j = 0; j < SEL_T / 64; ++j) a += red[j];
    shZ = a;
    shN = ntot;
  }
  __syncthreads();
  const float Z = shZ, N = (float)shN;
  const bool by_rank = k <= 512;
  int P = 1;
  while (P < k) P <<= 1;
  const int nkeys = by_rank ? k : P;
  for (int i = tid; i < nkeys; i += SEL_T) {
    if (i < k) {
      const int n = bounds[2 * i + 1] - bounds[2 * i];
      const float M = stats[2 * i] / Z, sq = stats[2 * i + 1] / (Z * Z);
      const float pi = (float)n / N;
      const float c = eps_s * pi / (float)n;
      const float den = M + eps_s * pi;
      const float ph2 = (sq + 2.f * c * M + (float)n * c * c) / (den * den);   // sum p_hat^2
      const float ell = den / ((1.f + eps_s) * pi);
      const float kap = n >= 2 ? logf(ph2) / logf((float)n) : 0.f;
      const float S = logf(ell) + lam * kap;
      prio[i] = S;
      // a NaN priority (all candidate mass underflowed) sorts last: the sort
      // keys must form a total order, or ranks would repeat
      key_s[i] = S == S ? S : INFINITY;
      key_n[i] = n;
      key_i[i] = i;
      removed[i] = 0;
    } else {
      key_s[i] = INFINITY;
      key_n[i] = 0;
      key_i[i] = 0x7fffffff;
    }
  }
  __syncthreads();
  // (S ascending, n descending, index ascending)
  auto before = [&](int a, int b) {
    if (key_s[a] != key_s[b]) return key_s[a] < key_s[b];
    if (key_n[a] != key_n[b]) return key_n[a] > key_n[b];
    return key_i[a] < key_i[b];
  };
  if (by_rank) {
    for (int i = tid; i < k; i += SEL_T) {
      const float si = key_s[i];
      const int ni = key_n[i];
      int rank = 0;
      for (int j = 0; j < k; ++j) {
        const float sj = key_s[j];
        const int nj = key_n[j];
        rank += (sj < si || (sj == si && (nj > ni || (nj == ni && j < i)))) ? 1 : 0;
      }
      order[rank] = i;
    }
  } else {
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int x = tid; x < P; x += SEL_T) {
          const int y = x ^ stride;
          if (y > x) {
            const bool up = (x & size) == 0;
            if (before(y, x) == up) {
              const float ts = key_s[x];
              key_s[x] = key_s[y];
              key_s[y] = ts;
              const int tn = key_n[x];
              key_n[x] = key_n[y];
              key_n[y] = tn;
              const int ti = key_i[x];
              key_i[x] = key_i[y];
              key_i[y] = ti;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int x = tid; x < k; x += SEL_T) order[x] = key_i[x];
  }
  __syncthreads();
  // key_n is indexed by chunk in the rank order and by position after the
  // bitonic sort
  auto n_of = [&](int o) { return by_rank ? key_n[order[o]] : key_n[o]; };

  float cur[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) cur[j] = 0.f;
  int tokens = 0, count = 0, slot = 0;
  bool done = false;
  constexpr int PF = 32 / RPT > 4 ? 32 / RPT : 4;
  for (int o0 = 0; o0 < k && !done; o0 += PF) {
    float mv[PF][RPT];
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const float* mi = m + (size_t)order[min(o0 + q, k - 1)] * R;
#pragma unroll
      for (int j = 0; j < RPT; ++j) mv[q][j] = mi[min(tid + j * SEL_T, R - 1)];
    }
    int q0 = 0;
    while (q0 < PF && !done) {
      // (1) fits on its own
      uint32_t alone = 0u;
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        bool ok = true;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
          ok = ok && (tid + j * SEL_T >= R || cur[j] + mv[q][j] <= eps);
        alone |= (ok ? 1u : 0u) << q;
      }
      alone = block_and_mask(alone, vote, slot);
      // (2) fits after every earlier chunk of the round that fits alone
      float acc[RPT];
#pragma unroll
      for (int j = 0; j < RPT; ++j) acc[j] = cur[j];
      uint32_t after = 0u;
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        if (q >= q0 && ((alone >> q) & 1u)) {
          bool ok = true;
#pragma unroll
          for (int j = 0; j < RPT; ++j) {
            acc[j] += mv[q][j];
            ok = ok && (tid + j * SEL_T >= R || acc[j] <= eps);
          }
          after |= (ok ? 1u : 0u) << q;
        }
      }
      after = block_and_mask(after, vote, slot);
      // take the steps in order
      int qn = PF;
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        if (q < q0 || qn < PF || done) continue;
        const int o = o0 + q;
        if (o >= k || tokens >= target || count + 1 > k - m0) {
          done = true;
          continue;
        }
        if (!((alone >> q) & 1u)) continue;   // never fits
        if ((after >> q) & 1u) {
#pragma unroll
          for (int j = 0; j < RPT; ++j) cur[j] += mv[q][j];
          tokens += n_of(o);
          count += 1;
          if (tid == 0) removed[order[o]] = 1;
        } else {
          qn = q + 1;   // rejected; the later ones need a new vote
        }
      }
      q0 = qn;
    }
  }
  if (tid == 0) *removed_tokens = tokens;
}

PruneLayout prune_layout(const DecodeDims& p, int k) {
  PruneLayout o;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  o.retain = take(retain_workspace_bytes(p));
  o.cid = take((size_t)p.L * sizeof(int32_t));
  o.bounds = take((size_t)2 * k * sizeof(int32_t));
  o.bounds_ok = take(sizeof(int32_t));
  o.segb = take((size_t)(k + 1) * sizeof(int32_t));
  o.stats = take((size_t)2 * k * sizeof(float));
  o.mtab = take((size_t)k * p.Hq * p.W * sizeof(float));
  // disjoint ascending chunks touch at most k + spans - 1 (span, chunk) pairs
  const size_t nseg = (size_t)k + (p.L + RT_CK - 1) / RT_CK;
  o.seg_v = take(nseg * p.Hq * p.W * sizeof(float));
  o.seg_m = take(nseg * p.Hq * p.W * sizeof(float));
  o.total = off;
  return o;
}

hipError_t launch_chunk_prune(const DecodeDims& p, const PruneArgs& a, const void* q_obs,
                              const void* k, const int32_t* bounds_in, int8_t* removed,
                              int32_t* removed_tokens, float* prio, float* row_mass, void* workspace,
                              hipStream_t st) {
  const PruneLayout ly = prune_layout(p, a.k);
  const RetainLayout lay = retain_layout(p);
  char* w = static_cast<char*>(workspace);
  char* rws = w + ly.retain;
  int32_t* bounds = reinterpret_cast<int32_t*>(w + ly.bounds);
  int32_t* cid = reinterpret_cast<int32_t*>(w + ly.cid);
  float* stats = reinterpret_cast<float*>(w + ly.stats);
  float* m = row_mass != nullptr ? row_mass : reinterpret_cast<float*>(w + ly.mtab);
  const int R = p.Hq * p.W;
  int32_t* bounds_ok = reinterpret_cast<int32_t*>(w + ly.bounds_ok);
  chunk_bounds_kernel<<<1, 64, 0, st>>>(bounds_in, a.k, p.L - p.W, bounds, bounds_ok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  chunk_of_kernel<<<(p.L + 255) / 256, 256, 0, st>>>(bounds, a.k, p.L, cid);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int32_t* segb = reinterpret_cast<int32_t*>(w + ly.segb);
  seg_base_kernel<<<1, SEL_T, 0, st>>>(bounds, a.k, segb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the retention passes with Renyi-2 head entropies; pass 1 also writes the
  // chunk segments of the row masses
  const SegArgs sg{cid, bounds, segb, reinterpret_cast<float*>(w + ly.seg_v),
                   reinterpret_cast<float*>(w + ly.seg_m)};
  const int RT = (p.W + 31) / 32;
#define EGS_RP(DD, RR) \
  e = retain_passes<DD, RR>(p, lay, rws, q_obs, k, EGS_RENYI, 2.0f, st, &sg)
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
  chunk_norm_kernel<<<dim3(a.k, (R + 255) / 256), 256, 0, st>>>(segb, sg.seg_v, sg.seg_m,
                                         reinterpret_cast<const float*>(rws + lay.row_m),
                                         reinterpret_cast<const float*>(rws + lay.row_inv), R, m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  head_weight_kernel<<<p.Hkv, 64, 0, st>>>(reinterpret_cast<const float*>(rws + lay.ent), p.Hq,
                                           p.Hkv, p.r, lay.nch, EGS_RENYI, 2.0f, a.zeta, a.tau,
                                           reinterpret_cast<float*>(rws + lay.weight), nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  float* pooled = reinterpret_cast<float*>(rws + lay.mu);
  pooled_mu_kernel<<<(p.L + 255) / 256, 256, 0, st>>>(
      reinterpret_cast<const float*>(rws + lay.mass),
      reinterpret_cast<const float*>(rws + lay.weight), p.Hq, p.Hkv, p.r, p.L, pooled);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  chunk_stats_kernel<<<a.k, 256, 0, st>>>(pooled, bounds, stats);
  if ((e = hipGetLastError()) != hipSuccess) return e;
#define EGS_PS(RPT)                                                                              \
  prune_select_kernel<RPT><<<1, SEL_T, 0, st>>>(stats, bounds, a.k, R, m, a.eps_s, a.lam, a.eps, \
                                                a.m0, a.target, bounds_ok, prio, removed,      \
                                                removed_tokens)
  if (R <= SEL_T) EGS_PS(1);
  else if (R <= 2 * SEL_T) EGS_PS(2);
  else if (R <= 4 * SEL_T) EGS_PS(4);
  else EGS_PS(8);
#undef EGS_PS
  return hipGetLastError();
}

// Optimality-gap certificate of a removal (EntroPrefill Sec. 4.2):
// U = eps sum_a y_a + t (k - m0) + sum_i [n_i - sum_a y_a m[i][a] - t]_+,
// in float64 over the float32 masses and prices.  Per chunk, one workgroup
// forms the priced mass and its hinge; one workgroup then adds the terms in
// index order (no atomics: the result does not depend on timing).
__device__ __forceinline__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();   // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double tot = 0.0;
  for (int j = 0; j < nw; ++j) tot += red[j];
  return tot;
}

__global__ __launch_bounds__(256) void cert_chunk_kernel(const int32_t* __restrict__ bounds,
                                                         const float* __restrict__ m,
                                                         const float* __restrict__ y, int R,
                                                         double t, double* __restrict__ hinge) {
  __shared__ double red[4];
  const int i = blockIdx.x;
  const float* mi = m + (size_t)i * R;
  double acc = 0.0;
  for (int a0 = 0; a0 < R; a0 += 4 * 256) {
    float mv[4], yv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int a = min(a0 + j * 256 + (int)threadIdx.x, R - 1);
      mv[j] = mi[a];
      yv[j] = y[a];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (a0 + j * 256 + (int)threadIdx.x < R) acc += (double)yv[j] * (double)mv[j];
  }
  const double priced = block_sum_d(acc, red);
  if (threadIdx.x == 0) {
    const double n = (double)(bounds[2 * i + 1] - bounds[2 * i]);
    hinge[i] = fmax(n - priced - t, 0.0);
  }
}

__global__ __launch_bounds__(SEL_T) void cert_total_kernel(const double* __restrict__ hinge,
                                                           int k, const float* __restrict__ y,
                                                           int R, double eps, int m0, double t,
                                                           double* __restrict__ out) {
  __shared__ double red[SEL_T / 64];
  double ys = 0.0, hs = 0.0;
  for (int a = threadIdx.x; a < R; a += SEL_T) ys += (double)y[a];
  for (int i = threadIdx.x; i < k; i += SEL_T) hs += hinge[i];
  ys = block_sum_d(ys, red);
  hs = block_sum_d(hs, red);
  if (threadIdx.x == 0) *out = eps * ys + t * (double)(k - m0) + hs;
}

size_t certificate_workspace_bytes(int k) {
  return align_up((size_t)k * sizeof(double));
}

hipError_t launch_prune_certificate(const int32_t* bounds, int k, int R, const float* m,
                                    const float* y, double eps, int m0, double t, double* out,
                                    void* workspace, hipStream_t st) {
  double* hinge = static_cast<double*>(workspace);
  cert_chunk_kernel<<<k, 256, 0, st>>>(bounds, m, y, R, t, hinge);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  cert_total_kernel<<<1, SEL_T, 0, st>>>(hinge, k, y, R, eps, m0, t, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Latent decoding (EntropyInfer Sec. 4.3, App. B): the cache grows by one
// entry per generated token and is compressed once n_delay tokens have been
// generated, then every `interval` tokens, with the latest queries (generated
// ones included) as the observation window.
// ---------------------------------------------------------------------------
// Append the new token: its query at the end of the window (rows move up by
// one, staged through LDS) and, from the first head of every group, its K / V
// row at position `pos` of the cache (rows ldk entries apart).  One workgroup
// per (batch, query head).
template <int D>
__global__ __launch_bounds__(256) void latent_append_kernel(
    const bf16* __restrict__ q_new, const bf16* __restrict__ k_new,
    const bf16* __restrict__ v_new, bf16* __restrict__ q_win, bf16* __restrict__ k_cache,
    bf16* __restrict__ v_cache, int Hq, int Hkv, int r, int W, int pos, int ldk) {
  __shared__ __attribute__((aligned(16))) bf16 win[128 * D];
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq, g = h / r;
  const int tid = threadIdx.x;
  bf16* wrow = q_win + (size_t)bh * W * D;
  // rows 1 .. W-1 move down one row, staged through LDS (the ranges
  // overlap), in 16-byte pieces (D is a multiple of 8)
  const int nv = (W - 1) * D / 8;
  for (int i = tid; i < nv; i += 256) store8(win + 8 * i, load8(wrow + D + 8 * i));
  __syncthreads();
  for (int i = tid; i < nv; i += 256) store8(wrow + 8 * i, load8(win + 8 * i));
  for (int d = tid; d < D; d += 256) wrow[(size_t)(W - 1) * D + d] = q_new[(size_t)bh * D + d];
  if (h % r == 0) {
    const size_t bg = (size_t)b * Hkv + g;
    for (int d = tid; d < D; d += 256) {
      k_cache[(bg * ldk + pos) * D + d] = k_new[bg * D + d];
      v_cache[(bg * ldk + pos) * D + d] = v_new[bg * D + d];
    }
  }
}

// kept rows (contiguous, n per (batch, KV group)) back into the cache rows
// 0 .. n-1 (rows ldk entries apart); one thread per 16 bytes
template <int D>
__global__ __launch_bounds__(256) void copy_rows_kernel(const bf16* __restrict__ sk,
                                                        const bf16* __restrict__ sv, int n,
                                                        int ldk, long long units,
                                                        bf16* __restrict__ dk,
                                                        bf16* __restrict__ dv) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= units) return;
  constexpr int CPR = D / 8;
  const long long row = i / CPR;
  const int c8 = (int)(i % CPR);
  const long long bg = row / n, t = row % n;
  const size_t src = (size_t)row * D + c8 * 8;
  const size_t dst = ((size_t)bg * ldk + t) * D + c8 * 8;
  *reinterpret_cast<u32x4*>(dk + dst) = *reinterpret_cast<const u32x4*>(sk + src);
  *reinterpret_cast<u32x4*>(dv + dst) = *reinterpret_cast<const u32x4*>(sv + src);
}

LatentLayout latent_layout(const DecodeDims& p) {
  // p.L is the cache capacity; every phase of a step fits the sizes for it
  LatentLayout o;
  const long long tot = (long long)p.n_sink + p.n_recent + p.n_keep;
  o.ntot_max = (int)std::min<long long>(p.L, tot);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  o.attn = take(decode_attn_workspace_bytes_upto(p, p.L));
  o.retain = take(retain_workspace_bytes(p));
  o.keep = take((size_t)p.B * p.Hkv * o.ntot_max * sizeof(int32_t));
  o.ks = take((size_t)p.B * p.Hkv * o.ntot_max * p.D * sizeof(bf16));
  o.vs = take((size_t)p.B * p.Hkv * o.ntot_max * p.D * sizeof(bf16));
  o.total = off;
  return o;
}

hipError_t launch_latent_append(const DecodeDims& p, const void* q_new, const void* k_new,
                                const void* v_new, void* q_win, void* k_cache, void* v_cache,
                                int pos, int ldk, hipStream_t st) {
  const bf16* qn = static_cast<const bf16*>(q_new);
  const bf16* kn = static_cast<const bf16*>(k_new);
  const bf16* vn = static_cast<const bf16*>(v_new);
  bf16* qw = static_cast<bf16*>(q_win);
  bf16* kc = static_cast<bf16*>(k_cache);
  bf16* vc = static_cast<bf16*>(v_cache);
  if (p.D == 128)
    latent_append_kernel<128><<<p.B * p.Hq, 256, 0, st>>>(qn, kn, vn, qw, kc, vc, p.Hq, p.Hkv,
                                                          p.r, p.W, pos, ldk);
  else
    latent_append_kernel<64><<<p.B * p.Hq, 256, 0, st>>>(qn, kn, vn, qw, kc, vc, p.Hq, p.Hkv,
                                                         p.r, p.W, pos, ldk);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const DecodeDims& p, const void* sk, const void* sv, int n, int ldk,
                            void* dk, void* dv, hipStream_t st) {
  const long long units = (long long)p.B * p.Hkv * n * (p.D / 8);
  if (units == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((units + 255) / 256);
  if (p.D == 128)
    copy_rows_kernel<128><<<blocks, 256, 0, st>>>(static_cast<const bf16*>(sk),
                                                  static_cast<const bf16*>(sv), n, ldk, units,
                                                  static_cast<bf16*>(dk), static_cast<bf16*>(dv));
  else
    copy_rows_kernel<64><<<blocks, 256, 0, st>>>(static_cast<const bf16*>(sk),
                                                 static_cast<const bf16*>(sv), n, ldk, units,
                                                 static_cast<bf16*>(dk), static_cast<bf16*>(dv));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Page-level retention (EntroPrefill Sec. 7): a page's importance is the
// largest token score it holds; every member (KV group or query head) keeps
// the pages that hold a sink or a recent position plus its n_keep best other
// pages; the head and layer modes take unions of the members' page sets.
// The forced pages are a prefix and a suffix of the page range, so the
// member selection is the token-level select run on the page scores.
// ---------------------------------------------------------------------------
constexpr int PG_MAX_WORDS = 8192;   // union bitmap: up to 262144 pages

PageDims page_dims(const DecodeDims& p, int S, int K, int mode) {
  PageDims q;
  q.S = S;
  q.K = K;
  q.mode = mode;
  q.NP = (p.L + S - 1) / S;
  q.X = mode == EGS_PAGE_HEAD_UNION ? p.Hq : p.Hkv;
  q.Y = mode == EGS_PAGE_LAYER_UNION ? 1 : p.Hkv;
  q.m = q.X / q.Y;
  q.ps = std::min(q.NP, (p.n_sink + S - 1) / S);                       // pages touching a sink
  q.pr = p.n_recent > 0 ? std::min(q.NP - 1, (p.L - p.n_recent) / S) : q.NP;   // first recent page
  const long long forced = (long long)q.ps + (q.NP - q.pr);
  q.ntl = (int)std::min<long long>(q.NP, forced + K);                 // pages per member
  q.cap = (int)std::min<long long>(q.NP, forced + (long long)q.m * K);  // pages per output set
  return q;
}

size_t page_retain_workspace_bytes(const DecodeDims& p, const PageDims& q) {
  const size_t a = ((size_t)p.B * q.X * q.NP * sizeof(float) + 255) / 256 * 256;
  return a + (size_t)p.B * q.X * std::max(q.ntl, 1) * sizeof(int32_t);
}

// I[row, i] = max of scores[row, i*S .. min(L, (i+1)*S) - 1]; one thread per page
__global__ __launch_bounds__(256) void page_max_kernel(const float* __restrict__ sc, int L, int S,
                                                       int NP, float* __restrict__ I) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int row = blockIdx.y;
  if (i >= NP) return;
  const float* src = sc + (size_t)row * L;
  const int lo = i * S, hi = min(L, lo + S);
  if ((S & 3) == 0 && (L & 3) == 0 && (reinterpret_cast<uintptr_t>(sc) & 15) == 0) {
    // 16-byte loads, eight in flight (the page and the row start 16-byte
    // aligned); clamped repeats do not change the maximum
    const floatx4* v4 = reinterpret_cast<const floatx4*>(src + lo);
    const int n4 = (hi - lo) / 4;
    float m = -INFINITY;
    for (int q0 = 0; q0 < n4; q0 += 8) {
      floatx4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v4[min(q0 + j, n4 - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        m = fmaxf(fmaxf(m, fmaxf(v[j][0], v[j][1])), fmaxf(v[j][2], v[j][3]));
    }
    I[(size_t)row * NP + i] = m;
    return;
  }
  // eight loads in flight; clamped repeats do not change the maximum
  float m = src[lo];
  for (int t0 = lo + 1; t0 < hi; t0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[min(t0 + j, hi - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, v[j]);
  }
  I[(size_t)row * NP + i] = m;
}

// union of the m member lists of output set (b, y) through an LDS bitmap,
// compacted in ascending order; -1 past the count
__global__ __launch_bounds__(SEL_T) void page_union_kernel(const int32_t* __restrict__ lists,
                                                           int ntl, int m, int X, int Y, int NP,
                                                           int cap, int32_t* __restrict__ page_idx,
                                                           int32_t* __restrict__ page_cnt) {
  __shared__ uint32_t bm[PG_MAX_WORDS];
  __shared__ int ired[SEL_T / 64];
  const int set = blockIdx.x, b = set / Y, y = set % Y;
  const int tid = threadIdx.x;
  const int nw = (NP + 31) / 32;
  for (int i = tid; i < nw; i += SEL_T) bm[i] = 0u;
  __syncthreads();
  for (int j = 0; j < m; ++j) {
    const int32_t* lst = lists + ((size_t)b * X + (size_t)y * m + j) * ntl;
    for (int e = tid; e < ntl; e += SEL_T) {
      const int pg = lst[e];
      atomicOr(&bm[pg >> 5], 1u << (pg & 31));
    }
  }
  __syncthreads();
  // thread tid owns words [tid * WPT, (tid + 1) * WPT)
  const int WPT = (nw + SEL_T - 1) / SEL_T;
  const int w0 = tid * WPT;
  int own = 0;
  for (int i = w0; i < min(nw, w0 + WPT); ++i) own += __popc(bm[i]);
  const int excl = block_excl_scan_1024(own, ired);
  int32_t* out = page_idx + (size_t)set * cap;
  int pos = excl;
  for (int i = w0; i < min(nw, w0 + WPT); ++i) {
    uint32_t bits = bm[i];
    while (bits) {
      const int t = __ffs(bits) - 1;
      bits &= bits - 1;
      if (pos < cap) out[pos] = i * 32 + t;
      ++pos;
    }
  }
  // the last thread ends at the total
  __shared__ int sh_total;
  if (tid == SEL_T - 1) {
    sh_total = min(pos, cap);
    page_cnt[set] = sh_total;
  }
  __syncthreads();
  for (int i = sh_total + tid; i < cap; i += SEL_T) out[i] = -1;
}

hipError_t launch_page_retain(const DecodeDims& p, const PageDims& q, const float* scores,
                              int32_t* page_idx, int32_t* page_cnt, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  float* I = reinterpret_cast<float*>(w);
  int32_t* lists = reinterpret_cast<int32_t*>(
      w + ((size_t)p.B * q.X * q.NP * sizeof(float) + 255) / 256 * 256);
  const int rows = p.B * q.X;
  page_max_kernel<<<dim3((q.NP + 255) / 256, rows), 256, 0, st>>>(scores, p.L, q.S, q.NP, I);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (q.ntl > 0) {
    retain_select_kernel<<<rows, SEL_T, 0, st>>>(I, q.NP, q.ps, q.NP - q.pr, q.K, q.ntl, lists);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  page_union_kernel<<<p.B * q.Y, SEL_T, 0, st>>>(lists, q.ntl, q.m, q.X, q.Y, q.NP, q.cap,
                                                 page_idx, page_cnt);
  return hipGetLastError();
}

}  // namespace egs
