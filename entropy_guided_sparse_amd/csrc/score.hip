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
// gfx950 design: four kernels, no logits stored.
//  * pool_keys streams K once from HBM: a workgroup of eight waves pools a
//    chunk of 8 key blocks (a wave takes one, 16-byte nontemporal loads
//    along d, 8 in flight per lane, fp32 sums reduced across the wave's row
//    phases) and writes the block means as a bf16 hi/lo pair (k_bar ~= hi +
//    lo to ~2^-17, so the logits run on bf16 MFMA with two products each).
//  * probe_stats and probe_mass take (piece, segment, KV group) work items,
//    only the pieces that hold causal blocks, 96-block pieces for the
//    statistics (three workgroups per CU: the 768 items of the 128k layer,
//    three per CU, run in one round) and 160-block pieces for the masses
//    (80 KB of LDS, two per CU: its 488 items, one round).  The piece's hi/lo block means are copied straight from
//    global memory into LDS (one round trip, shared by the r heads of the
//    group) while each wave loads the probe queries of its head into
//    registers; then v_mfma_f32_32x32x16_bf16 forms the piece's logits.
//      probe_stats  blocks as M (a lane owns a probe row): each row's maximum
//                   and sum of exponentials over the piece, one partial per
//                   (row, piece);
//      probe_mass   folds a row's partials (at most C_B / 96) into the row's
//                   log2 offset M + log2 L, recomputes the logits with the
//                   blocks as N (a lane owns a block, the probe mean is a
//                   register sum) and writes the piece's block scores and its
//                   entropy partial.
//    Items are numbered group-major and every XCD takes a contiguous range,
//    so a group's block means, probe queries and partials (~2 MB at 128k)
//    stay in one XCD's L2.
//  * probe_entropy adds the entropy partials of every (head, segment) in
//    piece order.
#include <algorithm>

#include "egs_device.h"
#include "egs_launch.h"

#include <mutex>

namespace egs {

constexpr int PS_NB = 8;      // key blocks per pool_keys workgroup
constexpr int PS_NW = 8;      // waves per pool_keys workgroup
constexpr int PS_U = 8;       // 16-byte key loads in flight per lane while pooling
constexpr int PC = 160;       // key blocks per probe_mass piece (and entropy partial)
constexpr int PC_S = 96;      // key blocks per probe_stats piece

struct ScoreLayout {
  size_t kb_hi, kb_lo, stat_m, stat_l, ent, total;
  int npool;    // pool_keys chunks per KV group
  int npc;      // probe_mass pieces per segment (at most)
  int npc_s;    // probe_stats pieces per segment (at most)
  int ipg;      // probe_mass pieces inside the causal ranges, per KV group
  int ipg_s;    // probe_stats pieces inside the causal ranges, per KV group
};

// Pieces of pc blocks that hold causal blocks, over the segments of one KV
// group: segment s sees blocks 0 .. (s + 1) bps - 1.
__host__ __device__ inline int causal_pieces(int CS, int bps, int pc) {
  int n = 0;
  for (int s = 0; s < CS; ++s) n += ((s + 1) * bps + pc - 1) / pc;
  return n;
}

static size_t sc_align(size_t x) {
  return (x + 255) / 256 * 256;
}

static ScoreLayout score_layout(const PrefillDims& p) {
  ScoreLayout o;
  o.npool = (p.CB + PS_NB - 1) / PS_NB;
  o.npc = (p.CB + PC - 1) / PC;
  o.npc_s = (p.CB + PC_S - 1) / PC_S;
  o.ipg = causal_pieces(p.CS, p.LS / p.LB, PC);
  o.ipg_s = causal_pieces(p.CS, p.LS / p.LB, PC_S);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += sc_align(bytes);
    return at;
  };
  o.kb_hi = take((size_t)p.Hkv * p.CB * p.D * sizeof(bf16));
  o.kb_lo = take((size_t)p.Hkv * p.CB * p.D * sizeof(bf16));
  const size_t rows = (size_t)p.Hq * p.CS * p.P;
  o.stat_m = take(rows * o.npc_s * sizeof(float));
  o.stat_l = take(rows * o.npc_s * sizeof(float));
  o.ent = take((size_t)p.Hq * p.CS * o.npc * sizeof(float));
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

// Add the elements of one 16-byte load (raw bits) to acc.
__device__ __forceinline__ void add16(const u32x4& v, float* acc, const bf16*) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += __uint_as_float(v[e] << 16);
    acc[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void add16(const u32x4& v, float* acc, const float*) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[e]);
}

// ---------------------------------------------------------------------------
// K1 pool_keys: one workgroup per (8-block chunk, KV group g);
//   kbar[g, j, :] = mean of keys j*LB .. (j+1)*LB-1, stored as bf16 hi + lo.
// Every chunk of one KV group runs on one XCD (workgroup id mod 8), in order.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW, 16 / NW) void pool_keys_kernel(
    const T* __restrict__ K, int N, int LB, int CB, int Hkv, int nch, bf16* __restrict__ kb_hi,
    bf16* __restrict__ kb_lo) {
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte load
  constexpr int CH = D / EPC;                // 16-byte chunks per key row
  constexpr int RPH = 64 / CH;               // key rows covered by one wave load
  static_assert(CH >= 1 && CH <= 64 && 64 % CH == 0, "row chunking");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int items = Hkv * nch, per_xcd = (items + 7) / 8;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= items) return;
  const int g = item / nch, c = item % nch;
  const int j0 = c * PS_NB, nb = min(PS_NB, CB - j0);
  // wave w takes blocks w, w + NW, ...; lane = (row phase, 16-byte chunk).
  // K is read once: nontemporal loads keep it from displacing reused data.
  const int cc = lane % CH, rp = lane / CH;
  const int nr = rp < LB ? (LB - rp + RPH - 1) / RPH : 0;
  const float inv_lb = 1.0f / (float)LB;
  for (int bi = w; bi < nb; bi += NW) {
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    const T* base = K + ((size_t)g * N + (size_t)(j0 + bi) * LB + rp) * D + cc * EPC;
    for (int i0 = 0; i0 < nr; i0 += PS_U) {
      u32x4 x[PS_U];
#pragma unroll
      for (int u = 0; u < PS_U; ++u) {
        const int i = min(i0 + u, nr - 1);   // clamped: every load stays in the block
        x[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(base + (size_t)i * RPH * D));
      }
#pragma unroll
      for (int u = 0; u < PS_U; ++u)
        if (i0 + u < nr) add16(x[u], acc, (const T*)nullptr);
    }
#pragma unroll
    for (int o = CH; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o);
    if (rp == 0) {
      const size_t go = ((size_t)g * CB + j0 + bi) * D + cc * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float mean = acc[e] * inv_lb;
        const bf16 hv = f2bf(mean);
        kb_hi[go + e] = hv;
        kb_lo[go + e] = f2bf(mean - bf2f(hv));
      }
    }
  }
}

// XOR swizzle of the 16-byte chunks of a D-wide bf16 row in LDS
template <int D>
__device__ __forceinline__ int kbar_swz(int row) {
  return lds_swz<D * 2>(row);
}

// 16 bf16 of pooled-key row `row`, d chunk (2c + hg), from the swizzled stage
template <int D>
__device__ __forceinline__ bf16x8 kbar_frag(const bf16* k, int row, int c, int hg) {
  return load8(k + row * D + (((2 * c + hg) ^ kbar_swz<D>(row)) * 8));
}

// Direct global -> LDS copies of the hi / lo block means of blocks
// c0 .. c0 + NB - 1 into the swizzled stage (4 waves).  Each copy lands at
// a fixed LDS slot; the lane fetches the global chunk that belongs there.
// Rows at or past nb repeat block c0 + nb - 1, whose logits every reader
// masks or discards.  Completion: wait_vmem() and a workgroup barrier.
template <int D, int NB>
__device__ __forceinline__ void stage_piece(bf16* kh, bf16* kl, const bf16* KH, const bf16* KL,
                                            int c0, int nb) {
  constexpr int KCH = D / 8;                    // 16-byte chunks per row
  constexpr int NI = (NB * KCH + 255) / 256;    // copies per lane per plane
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bf16* sh = uniform_ptr(KH + (size_t)c0 * D);
  const bf16* sl = uniform_ptr(KL + (size_t)c0 * D);
  const uint32_t dh = __builtin_amdgcn_readfirstlane(lds_u32(kh));
  const uint32_t dl = __builtin_amdgcn_readfirstlane(lds_u32(kl));
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int q = (w * NI + ii) * 64 + lane;    // destination chunk
    if (w * NI + ii >= NB * KCH / 64) break;      // (wave-uniform) past the stage
    const int row = q / KCH, slot = q % KCH;
    const int src = min(row, nb - 1);
    const uint32_t off = (uint32_t)((src * D + (slot ^ kbar_swz<D>(row)) * 8) * sizeof(bf16));
    const uint32_t at = (uint32_t)((w * NI + ii) * 1024);
    copy16_to_lds_at(sh, off, dh + at);
    copy16_to_lds_at(sl, off, dl + at);
  }
}

// 1-D grid -> (piece, segment, KV group) over the pieces that hold causal
// blocks only (ipg per group): the items are numbered group-major (group,
// segment, piece) and every XCD (workgroup id mod 8) takes one contiguous
// eighth of them, so a group's pooled keys, probe queries and partials are
// fetched into one L2 only.  No workgroups are launched for pieces past the
// causal ranges: the hardware hands a grid's workgroups to the CUs of an XCD
// in a fixed rotation, which with those pieces in the grid gave some CUs five
// causal items and others two (at 128k: 96 causal statistics items per XCD,
// now three per CU).  Returns false for padding ids.
__device__ __forceinline__ bool probe_item(int bid, int pc, int bps, int CS, int Hkv, int ipg,
                                           int& ch, int& s, int& g) {
  const int items = Hkv * ipg, per_xcd = (items + 7) / 8;
  const int item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= items) return false;
  g = item / ipg;
  int k = item % ipg;
  for (s = 0;; ++s) {
    const int n = ((s + 1) * bps + pc - 1) / pc;
    if (k < n) break;
    k -= n;
  }
  ch = k;
  return true;
}

// MFMA fragments of RTG 32-row probe tiles of head h, rows grp * 32 RTG ..:
// lane l holds row (l % 32) of each tile and d slots 16 c + 8 (l / 32) .. + 7
// (zero past the probe).
template <typename TQ, int D, int RTG>
__device__ __forceinline__ void load_probe(typename QFrag<TQ>::raw_t (&qr)[RTG][D / 16],
                                           const TQ* Q, int h, int N, size_t u_begin, int P,
                                           int grp) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hg = lane >> 5;
#pragma unroll
  for (int t = 0; t < RTG; ++t) {
    const int urow = grp * 32 * RTG + t * 32 + l32;
    const bool ok = urow < P;
    const TQ* qp = Q + ((size_t)h * N + u_begin + (ok ? urow : 0)) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qr[t][c] = QFrag<TQ>::load(qp + 16 * c + 8 * hg, ok);
  }
}

// ---------------------------------------------------------------------------
// K2a probe_stats: work item (piece of PC_S key blocks, segment s, KV group g).
// For each head of the group (one per wave at a time) and probe row u:
//   m = max_j z_uj, l = sum_j 2^(z_uj - m) over the piece's causal blocks
//   j < C_B(s) (z in log2 units), stored at stat[h, s, piece, u].
// Blocks are the MFMA M dimension: a lane owns a probe row, a register a block.
// ---------------------------------------------------------------------------
template <typename TQ, int D>
__global__ __launch_bounds__(256, 3) void probe_stats_kernel(
    const TQ* __restrict__ Q, const bf16* __restrict__ kb_hi, const bf16* __restrict__ kb_lo,
    int Hq, int r, int N, int LS, int LB, int P, int CS, int CB, int ipg, float scale_log2,
    float* __restrict__ stat_m, float* __restrict__ stat_l) {
  constexpr int NC = D / 16;
  constexpr int BT = PC_S / 32;
  constexpr int RTG = sizeof(TQ) == 2 ? 2 : 1;   // 32-row probe tiles per group
  typedef typename QFrag<TQ>::raw_t raw_t;
  __shared__ __attribute__((aligned(16))) bf16 kh[PC_S * D];
  __shared__ __attribute__((aligned(16))) bf16 kl[PC_S * D];
  int ch, s, g;
  if (!probe_item(blockIdx.x, PC_S, LS / LB, CS, Hq / r, ipg, ch, s, g)) return;
  const int cb = (s + 1) * (LS / LB);
  const int c0 = ch * PC_S;
  const int npc_s = (CB + PC_S - 1) / PC_S;   // partials per row (the stride)
  const int nb = min(PC_S, cb - c0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const size_t u_begin = (size_t)(s + 1) * LS - P;
  const int ngrp = (P + 32 * RTG - 1) / (32 * RTG);

  stage_piece<D, PC_S>(kh, kl, kb_hi + (size_t)g * CB * D, kb_lo + (size_t)g * CB * D, c0, nb);
  raw_t qr[RTG][NC];
  if (w < r) load_probe<TQ, D, RTG>(qr, Q, g * r + w, N, u_begin, P, 0);
  wait_vmem();
  __syncthreads();

  for (int hl = w; hl < r; hl += 4) {
    const int h = g * r + hl;
    for (int grp = 0; grp < ngrp; ++grp) {
      if (hl != w || grp != 0) load_probe<TQ, D, RTG>(qr, Q, h, N, u_begin, P, grp);
      bf16x8 qh[RTG][NC], ql[RTG][NC];
#pragma unroll
      for (int t = 0; t < RTG; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) QFrag<TQ>::split(qr[t][c], qh[t][c], ql[t][c]);
      float m[RTG], l[RTG];
#pragma unroll
      for (int t = 0; t < RTG; ++t) {
        m[t] = -INFINITY;
        l[t] = 0.f;
      }
      // block tiles outer, probe tiles inner: each LDS fragment is read once
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) {
        if (bt * 32 >= nb) break;
        floatx16 z[RTG];
#pragma unroll
        for (int t = 0; t < RTG; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) z[t][i] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 ah = kbar_frag<D>(kh, bt * 32 + l32, c, hg);
          const bf16x8 al = kbar_frag<D>(kl, bt * 32 + l32, c, hg);
#pragma unroll
          for (int t = 0; t < RTG; ++t) {
            z[t] = mfma32(ah, qh[t][c], z[t]);
            z[t] = mfma32(al, qh[t][c], z[t]);
            if (QFrag<TQ>::kSplit) z[t] = mfma32(ah, ql[t][c], z[t]);
          }
        }
        // z[t][i]: block c0 + bt*32 + acc_row(i, lane) against probe row l32 of
        // tile t.  Only the piece's last tile can hold blocks past it; the
        // maximum is taken on the raw logits and scaled once (scale_log2 > 0
        // and rounding keep the order), and each term is one FMA and one exp2.
        const bool ragged = bt * 32 + 32 > nb;
#pragma unroll
        for (int t = 0; t < RTG; ++t) {
          if (ragged) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (bt * 32 + acc_row(i, lane) >= nb) z[t][i] = -INFINITY;
          }
          float tmax = z[t][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, z[t][i]);
          tmax = xhalf_max(tmax) * scale_log2;   // finite: the tile's first block is causal
          const float mn = fmaxf(m[t], tmax);
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(z[t][i], scale_log2, -mn));
          l[t] = l[t] * fast_exp2(m[t] - mn) + xhalf_sum(sum);
          m[t] = mn;
        }
      }
#pragma unroll
      for (int t = 0; t < RTG; ++t) {
        const int urow = grp * 32 * RTG + t * 32 + l32;
        if (hg == 0 && urow < P) {
          const size_t o = (((size_t)h * CS + s) * npc_s + ch) * P + urow;
          stat_m[o] = m[t];
          stat_l[o] = l[t];
        }
      }
    }
  }
}

// Fold up to RP_B partials (m, l) of one probe row, starting at partial p0,
// into the running (M, L).  A row's partials lie P floats apart (lanes on
// consecutive rows read consecutive floats); indices past n are clamped to
// the last partial on load and ignored by the fold.
constexpr int RP_B = 8;
struct RowPartials {
  float m[RP_B], l[RP_B];
  __device__ void fetch(const float* sm, const float* sl, int p0, int n, int P) {
#pragma unroll
    for (int i = 0; i < RP_B; ++i) {
      const size_t at = (size_t)min(p0 + i, n - 1) * P;
      m[i] = sm[at];
      l[i] = sl[at];
    }
  }
  __device__ void fold(int p0, int n, float& M, float& L) const {
    float bm = M;
#pragma unroll
    for (int i = 0; i < RP_B; ++i)
      if (p0 + i < n) bm = fmaxf(bm, m[i]);
    float acc = L * fast_exp2(M - bm);
#pragma unroll
    for (int i = 0; i < RP_B; ++i)
      if (p0 + i < n) acc += l[i] * fast_exp2(m[i] - bm);
    M = bm;
    L = acc;
  }
};

// ---------------------------------------------------------------------------
// K2b probe_mass: work item (piece of PC key blocks, segment s, KV group g).
// For each head of the group (one per wave at a time) and each group of RTG
// 32-row probe tiles: the rows' partials are folded into the row's log2
// offset M + log2 L (a lane owns a row), the logits of the piece are
// recomputed with the blocks as the MFMA N dimension and the normalised
// probabilities are summed over the probe rows in registers.  Writes a_bar
// of the piece's causal blocks and the piece's entropy partial.
// ---------------------------------------------------------------------------
template <typename TQ, int D>
__global__ __launch_bounds__(256, 2) void probe_mass_kernel(
    const TQ* __restrict__ Q, const bf16* __restrict__ kb_hi, const bf16* __restrict__ kb_lo,
    int Hq, int r, int N, int LS, int LB, int P, int CS, int CB, int npc, int npc_s, int ipg,
    float scale_log2, int kind, float alpha, const float* __restrict__ stat_m,
    const float* __restrict__ stat_l,
    float* __restrict__ ent, float* __restrict__ scores) {
  constexpr int NC = D / 16;
  constexpr int BT = PC / 32;
  constexpr int RTG = sizeof(TQ) == 2 ? 2 : 1;   // 32-row probe tiles per group
  constexpr int RG = 32 * RTG;                   // probe rows per group
  typedef typename QFrag<TQ>::raw_t raw_t;
  __shared__ __attribute__((aligned(16))) bf16 kh[PC * D];
  __shared__ __attribute__((aligned(16))) bf16 kl[PC * D];
  int ch, s, g;
  if (!probe_item(blockIdx.x, PC, LS / LB, CS, Hq / r, ipg, ch, s, g)) return;
  const int cb = (s + 1) * (LS / LB);
  const int c0 = ch * PC;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hg = lane >> 5;
  const int nb = min(PC, cb - c0);
  const int nparts = (cb + PC_S - 1) / PC_S;   // probe_stats pieces of segment s
  const size_t u_begin = (size_t)(s + 1) * LS - P;
  const float invP = 1.0f / (float)P;
  const int ngrp = (P + RG - 1) / RG;
  auto part_ptrs = [&](int h, int grp, const float*& sm, const float*& sl) {
    const int urow = min(grp * RG + lane % RG, P - 1);
    const size_t o = ((size_t)h * CS + s) * npc_s * P + urow;
    sm = stat_m + o;
    sl = stat_l + o;
  };

  // one round trip: the piece's block means, the first head's queries and
  // its rows' first partials are all in flight together
  stage_piece<D, PC>(kh, kl, kb_hi + (size_t)g * CB * D, kb_lo + (size_t)g * CB * D, c0, nb);
  raw_t qr[RTG][NC];
  RowPartials rp;
  if (w < r) {
    const float *sm, *sl;
    load_probe<TQ, D, RTG>(qr, Q, g * r + w, N, u_begin, P, 0);
    part_ptrs(g * r + w, 0, sm, sl);
    rp.fetch(sm, sl, 0, nparts, P);
  }
  wait_vmem();
  __syncthreads();

  for (int hl = w; hl < r; hl += 4) {
    const int h = g * r + hl;
    float acc[BT];
#pragma unroll
    for (int bt = 0; bt < BT; ++bt) acc[bt] = 0.f;
    for (int grp = 0; grp < ngrp; ++grp) {
      const float *sm, *sl;
      part_ptrs(h, grp, sm, sl);
      if (hl != w || grp != 0) {
        load_probe<TQ, D, RTG>(qr, Q, h, N, u_begin, P, grp);
        rp.fetch(sm, sl, 0, nparts, P);
      }
      float M = kNegBig, L = 0.f;
      rp.fold(0, nparts, M, L);
      for (int p0 = RP_B; p0 < nparts; p0 += RP_B) {
        rp.fetch(sm, sl, p0, nparts, P);
        rp.fold(p0, nparts, M, L);
      }
      // a row's probabilities are 2^(z - off), off = M + log2 L; rows past
      // the probe take off = +inf, so they add nothing
      const bool own = grp * RG + (lane % RG) < P && L > 0.f;
      const float off = own ? M + __log2f(L) : INFINITY;
      // registers of the mass pass hold rows acc_row(i, lane): fetch their offsets
      float ro[RTG][16];
      bf16x8 qh[RTG][NC], ql[RTG][NC];
#pragma unroll
      for (int t = 0; t < RTG; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ro[t][i] = __shfl(off, t * 32 + acc_row(i, lane));
#pragma unroll
        for (int c = 0; c < NC; ++c) QFrag<TQ>::split(qr[t][c], qh[t][c], ql[t][c]);
      }
      // block tiles outer, probe tiles inner: each LDS fragment is read once
#pragma unroll
      for (int bt = 0; bt < BT; ++bt) {
        if (bt * 32 >= nb) break;
        floatx16 z[RTG];
#pragma unroll
        for (int t = 0; t < RTG; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) z[t][i] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 bh = kbar_frag<D>(kh, bt * 32 + l32, c, hg);
          const bf16x8 bl = kbar_frag<D>(kl, bt * 32 + l32, c, hg);
#pragma unroll
          for (int t = 0; t < RTG; ++t) {
            z[t] = mfma32(qh[t][c], bh, z[t]);
            z[t] = mfma32(qh[t][c], bl, z[t]);
            if (QFrag<TQ>::kSplit) z[t] = mfma32(ql[t][c], bh, z[t]);
          }
        }
        float colsum = 0.f;
#pragma unroll
        for (int t = 0; t < RTG; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            colsum += fast_exp2(__builtin_fmaf(z[t][i], scale_log2, -ro[t][i]));
        acc[bt] += xhalf_sum(colsum);
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
    // the segment's last causal piece also writes the sentinels of every
    // block past the causal range (no items are launched for those pieces)
    if (c0 + nb == cb)
      for (int j = cb + lane; j < CB; j += 64) out[j] = -1.0f;
    epart = wave_sum(epart);
    if (lane == 0) ent[((size_t)h * CS + s) * npc + ch] = epart;
  }
}

// one thread per (head, segment): E from the pieces' partial sums, in order
__global__ __launch_bounds__(256) void probe_entropy_kernel(const float* __restrict__ ent,
                                                            int Hq, int CS, int npc, int bps,
                                                            int kind, float alpha,
                                                            float* __restrict__ entropy) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= Hq * CS) return;
  const int s = i % CS;
  const int npieces = ((s + 1) * bps + PC - 1) / PC;
  const float* e = ent + (size_t)i * npc;
  float tot = 0.f;
  for (int c = 0; c < npieces; ++c) tot += e[c];
  entropy[i] = (kind == EGS_SHANNON) ? tot : logf(tot) / (1.0f - alpha);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
// entropy == nullptr: stop after the mass pass, leaving the per-piece entropy
// partials in the workspace for a later kernel to finish
template <typename T>
static hipError_t score_dispatch(const PrefillDims& p, const ScoreLayout& ly, const void* q,
                                 const void* k, char* ws, int kind, float alpha, float* scores,
                                 float* entropy, hipStream_t st) {
  const float sl2 = p.sm_scale * kLog2e;
  const T* Q = static_cast<const T*>(q);
  const T* K = static_cast<const T*>(k);
  bf16* H = reinterpret_cast<bf16*>(ws + ly.kb_hi);
  bf16* L = reinterpret_cast<bf16*>(ws + ly.kb_lo);
  float* sm = reinterpret_cast<float*>(ws + ly.stat_m);
  float* sl = reinterpret_cast<float*>(ws + ly.stat_l);
  float* en = reinterpret_cast<float*>(ws + ly.ent);
  const int g1 = (p.Hkv * ly.npool + 7) / 8 * 8;
  const int g2s = (p.Hkv * ly.ipg_s + 7) / 8 * 8;
  const int g2 = (p.Hkv * ly.ipg + 7) / 8 * 8;
  hipError_t e;
#define EGS_POOL(DD)                                                                         \
  pool_keys_kernel<T, DD, PS_NW><<<g1, 64 * PS_NW, 0, st>>>(K, p.N, p.LB, p.CB, p.Hkv,      \
                                                            ly.npool, H, L)
#define EGS_STATS(DD)                                                                        \
  probe_stats_kernel<T, DD><<<g2s, 256, 0, st>>>(Q, H, L, p.Hq, p.r, p.N, p.LS, p.LB, p.P,  \
                                                  p.CS, p.CB, ly.ipg_s, sl2, sm, sl)
#define EGS_MASS(DD)                                                                         \
  probe_mass_kernel<T, DD><<<g2, 256, 0, st>>>(Q, H, L, p.Hq, p.r, p.N, p.LS, p.LB, p.P,    \
                                                p.CS, p.CB, ly.npc, ly.npc_s, ly.ipg, sl2, \
                                                kind,                                      \
                                                alpha, sm, sl, en, scores)
#define EGS_D_SWITCH(M)              \
  switch (p.D) {                     \
    case 16: M(16); break;           \
    case 32: M(32); break;           \
    case 64: M(64); break;           \
    case 128: M(128); break;         \
    default: return hipErrorInvalidValue; \
  }                                  \
  if ((e = hipGetLastError()) != hipSuccess) return e;
  EGS_D_SWITCH(EGS_POOL)
  EGS_D_SWITCH(EGS_STATS)
  EGS_D_SWITCH(EGS_MASS)
#undef EGS_D_SWITCH
#undef EGS_POOL
#undef EGS_STATS
#undef EGS_MASS
  if (entropy == nullptr) return hipSuccess;
  probe_entropy_kernel<<<(p.Hq * p.CS + 255) / 256, 256, 0, st>>>(en, p.Hq, p.CS, ly.npc,
                                                                  p.LS / p.LB, kind, alpha,
                                                                  entropy);
  return hipGetLastError();
}

hipError_t launch_entropy_score(const PrefillDims& p, const void* q, const void* k, int kind,
                                float alpha, float* scores, float* entropy, void* ws,
                                hipStream_t st) {
  const ScoreLayout ly = score_layout(p);
  char* w = static_cast<char*>(ws);
  return p.dtype == EGS_F32
             ? score_dispatch<float>(p, ly, q, k, w, kind, alpha, scores, entropy, st)
             : score_dispatch<bf16>(p, ly, q, k, w, kind, alpha, scores, entropy, st);
}

EntropyParts entropy_parts(const PrefillDims& p, const void* ws) {
  const ScoreLayout ly = score_layout(p);
  EntropyParts e;
  e.part = reinterpret_cast<const float*>(static_cast<const char*>(ws) + ly.ent);
  e.npc = ly.npc;
  e.pc = PC;
  return e;
}

// ---------------------------------------------------------------------------
// Static scratch for egs_entropy_score_static: callers that cannot allocate
// get the workspace from this device array instead (each GPU holds its own
// copy from the code object's load until the process ends).  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address is taken once per device with hipGetSymbolAddress, with that device
// current, and only that address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[EGS_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_entropy_score_static(const PrefillDims& p, bool maxmin, const void* q,
                                       const void* k, int kind, float alpha, float* scores,
                                       float* entropy, hipStream_t st) {
  void* ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return e;
  return maxmin ? launch_entropy_score_maxmin(p, q, k, kind, alpha, scores, entropy, ws, st)
                : launch_entropy_score(p, q, k, kind, alpha, scores, entropy, ws, st);
}

}  // namespace egs
