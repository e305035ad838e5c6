// K5: block-sparse causal GQA attention over per-(head, segment) block lists.
//
// Method: EntropyInfer (arXiv 2606.09508) App. A eq. (3) computes attention of
// every segment only over its selected key blocks; the causal GQA softmax is
// the one of EntroPrefill Sec. 2.1 (query head h reads KV head g(h)).  Query
// block b of segment s attends { j in Sel(h, s) : j < b } plus its own block b
// under the causal mask, so a full budget reproduces dense causal attention.
//
// gfx950 design (bf16, head_dim 64/128, block 64/128):
//  * A pre-pass (vt_pack) rewrites V once per call into 64-key tiles stored
//    d-major ("V^T") with the keys of every 16-key group permuted into the
//    order in which the softmax probabilities leave the accumulator.  Every
//    MFMA operand of the main kernel is then one 16-byte LDS read, and no
//    transposition is repeated by the many query blocks that select a block.
//  * A work item is one (head, query block), run by a workgroup of L_B/32
//    wavefronts of 32 query rows.  The launch is a persistent grid that takes
//    items from work queues, one per (XCD, head of the group), each heaviest
//    (latest query block) first; a KV group's items stay on one XCD so its
//    shared K/V blocks meet in that XCD's L2 (details at the kernel).
//  * Transposed flash formulation, no cross-lane shuffles:
//        S^T = K Q^T     (A = K tile from LDS, B = Q^T held in registers)
//        P^T = exp2(S^T - m)   (a lane owns one query row)
//        O^T += V^T P^T  (A = V^T tile from LDS, B = P^T from the accumulator)
//    on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The running maximum
//    is only raised (and O rescaled) when some row's maximum grows by more
//    than 2^8 in probability; otherwise probabilities up to 2^8 accumulate
//    against the stale maximum, which fp32 and bf16 hold exactly enough.
//  * 64-key K and V^T stages are copied straight from global memory into LDS
//    (global_load_lds_dwordx4, no register staging) behind XOR-swizzled
//    16-byte chunks (conflict-free ds_read_b128), double-buffered: the copies
//    of stage n+1 are in flight while stage n is computed.  Two workgroups
//    share a CU, so one wavefront's softmax overlaps another's MFMAs.  (Also
//    holding S^T of the next stage in registers to overlap it within a
//    wavefront measured slower: the extra 32 registers cost LDS prefetch.)
//    The block list of the (head, segment) is staged in LDS once.
//
// Generic path: a VALU kernel (one thread per query row, fp32 math) serves
// fp32 inputs and shapes outside the MFMA kernel's range.
#include "egs_device.h"
#include "egs_launch.h"

namespace egs {

constexpr int AT_KT = 64;     // keys per LDS stage and per V^T tile
constexpr int AT_LCAP = 512;  // block-list entries staged in LDS at a time
constexpr int PV_AHEAD = 4;   // V^T fragments read ahead of their MFMA
constexpr int AT_NQUEUE = 8;  // XCDs, each with r work queues of the MFMA kernel
constexpr int AT_QSTRIDE = 16;   // ints between queue counters (one 64-byte line each)
constexpr int AT_QMAX = 128;     // queue counters zeroed by vt_pack (8 XCDs x r <= 16)

// The compiler schedules nothing across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Key order inside a 16-key group of a V^T tile: the k-slot order of the P^T
// operand as it leaves the S^T accumulator.  Keys 0-3 sit at positions 0-3,
// keys 8-11 at 4-7, keys 4-7 at 8-11 and keys 12-15 at 12-15 (bits 2 and 3
// swapped), so the map is its own inverse.
__device__ __forceinline__ int vt_swap23(int x16) {
  return (x16 & 3) | ((x16 & 4) << 1) | ((x16 & 8) >> 1);
}

// ---------------------------------------------------------------------------
// vt_pack: V [Hkv, N, D] -> Vt [Hkv, N/64, D, 64] with permuted keys.
// One workgroup per (64-key tile, KV head); coalesced 16-byte loads and stores.
// The first workgroup also zeroes the MFMA kernel's queue counters, which
// the launch that follows in stream order then finds at zero.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void vt_pack_kernel(const bf16* __restrict__ V, int N,
                                                      bf16* __restrict__ Vt,
                                                      int* __restrict__ queue) {
  constexpr int VP = D + 2;   // padded row (bf16) to spread the column reads
  __shared__ bf16 tile[AT_KT * VP];
  const int t = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  if (t == 0 && g == 0 && tid < AT_QMAX) queue[tid * AT_QSTRIDE] = 0;
  const bf16* src = V + ((size_t)g * N + (size_t)t * AT_KT) * D;
  constexpr int CH = AT_KT * D / 8;
  for (int q = tid; q < CH; q += 256) {
    const int row = q / (D / 8), c8 = q % (D / 8);
    const bf16x8 v = load8(src + (size_t)row * D + c8 * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row * VP + c8 * 8 + e] = v[e];
  }
  __syncthreads();
  bf16* dst = Vt + ((size_t)g * (N / AT_KT) + t) * (size_t)(D * AT_KT);
  for (int q = tid; q < CH; q += 256) {
    const int d = q / (AT_KT / 8), c8 = q % (AT_KT / 8);   // 8 positions per chunk
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = c8 * 8 + e;
      const int grp = pos >> 4;
      v[e] = tile[(grp * 16 + vt_swap23(pos & 15)) * VP + d];
    }
    store8(dst + (size_t)d * AT_KT + c8 * 8, v);
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
// Stage n of a workgroup is one 64-key piece of its key list: the selected
// blocks j < b in list order, then the own block b (each L_B / 64 stages).
// Iteration n issues the direct LDS copies of K(n+1) and V^T(n+1), computes
// S^T(n), its softmax and O^T += V^T(n) P^T(n), and ends with one barrier.
// K and V^T each live in two LDS buffers; the buffer a copy overwrites was
// last read before the previous barrier.
struct AtItem {
  int blk, sub;
  bool diag, valid;
};

//
// Work distribution.  The hardware hands a grid's workgroups to the CUs in a
// fixed rotation, whatever their length: with one workgroup per item, every
// CU of an XCD kept serving the same head, and the CUs of heads with short
// lists (rigid heads at a 5% budget against 30%) sat idle for a third of the
// launch while the others set its length.  The launch is therefore a
// persistent grid of as many workgroups as the CUs hold at once, and each
// workgroup takes items (KV group, query block, head) from counters in the
// workspace until they run out.  With xcd_remap there is one queue per
// (XCD x, head hl of the group): the items of head hl in KV groups x, x + 8,
// ..., latest (heaviest) query block first.  The workgroups of XCD x
// (workgroup id mod 8) form r sets (workgroup id / 8 mod r), and set hl
// drains queue (x, hl) first: a group's K / V blocks then meet in one XCD's
// L2, and the workgroups of one set run items of one head and one segment
// (the same block list, of near-equal lengths) side by side, so their tile
// reads stay close together in the list and hit in L2.  A set whose queue
// is empty takes items from the other heads' queues of its XCD; once those
// are empty too, wave 0 reads every counter (one lane each) and takes from
// the queue with the most items left, so the XCDs of heavy KV groups get
// help from all others at once.  The counters are zeroed by vt_pack before
// the launch and only ever incremented; a workgroup fails to take an item
// at most once per queue, so every workgroup leaves the loop.

template <int D, int LB>
__global__ __launch_bounds__(LB * 2) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_attn_mfma_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ Vt,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int k_max,
    bf16* __restrict__ O, float* __restrict__ lse, int Hkv, int r, int N, int LS, int CS,
    int CB, float scale_log2, int xcd_remap, int* __restrict__ queue) {
  constexpr int NW = LB / 32;
  constexpr int NT = NW * 64;
  constexpr int KT = AT_KT;
  constexpr int SUB = LB / KT;
  constexpr int NC = D / 16;            // 16-wide d chunks of Q / K
  constexpr int ND = D / 32;            // 32-row d tiles of O^T
  constexpr int KCH = D / 8;            // 16-byte chunks per K row
  constexpr int PIECES = KT * D * 2 / 1024;   // 1-KB wave copies per K (or V^T) stage
  constexpr int PER_W = PIECES / NW;
  static_assert(PIECES % NW == 0, "stage copies must split evenly over the waves");
  constexpr int KROWS = 1024 / (D * 2);       // K rows per 1-KB piece
  constexpr float kRescale = 8.0f;      // log2 of the largest unnormalised probability
  __shared__ __attribute__((aligned(1024))) bf16 Ks[2][KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[2][D * KT];
  __shared__ int lst[AT_LCAP];
  __shared__ int s_item;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hg = lane >> 5;
  // queue x * r + hl: XCD x, head hl; home: own XCD, set (workgroup id / 8) mod r
  const int nq = xcd_remap ? AT_NQUEUE * r : 1;
  const int per_q = Hkv * r * CB / nq;
  const int home = xcd_remap ? (int)((blockIdx.x & 7) * r + ((blockIdx.x >> 3) % r)) : 0;
  int tried = 0;   // wave 0: queues of the own XCD found empty (home first)

  for (;;) {
  // ---- next work item: pair grp = k * Hkv + g (heaviest first), head hl ----
  // (queue x * r + hl holds pairs grp = 8 k + x, k = 0, 1, ...)
  if (w == 0) {
    int item = -1;
    const int nown = xcd_remap ? r : 1;
    while (tried < nown) {
      const int qx = xcd_remap ? (home / r) * r + (home % r + tried) % r : 0;
      int slot = 0;
      if (lane == 0)
        slot = __hip_atomic_fetch_add(queue + qx * AT_QSTRIDE, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      slot = __shfl(slot, 0);
      if (slot < per_q) {
        item = qx * per_q + slot;
        break;
      }
      ++tried;
    }
    // the own XCD's queues are empty: the queue with the most items left
    // (ties: the first after home); a failed take means that queue emptied
    // meanwhile, and every retry sees one more empty queue
    while (item < 0 && tried >= nown) {
      int best = 0, bq = -1;
      for (int q0 = 0; q0 < nq; q0 += 64) {
        const int k = q0 + lane;
        const int qx = (home + k) % nq;
        int left = 0;
        if (k < nq)
          left = per_q - min(per_q, __hip_atomic_load(queue + qx * AT_QSTRIDE, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
        int key = left > 0 ? (min(left, (1 << 22) - 1) << 8) | (255 - k) : 0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o));
        if ((key >> 8) > best) {
          best = key >> 8;
          bq = (home + 255 - (key & 255)) % nq;
        }
      }
      if (best == 0) break;
      int slot = 0;
      if (lane == 0)
        slot = __hip_atomic_fetch_add(queue + bq * AT_QSTRIDE, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      slot = __shfl(slot, 0);
      if (slot < per_q) item = bq * per_q + slot;
    }
    if (lane == 0) s_item = item;
  }
  __syncthreads();
  const int item = __builtin_amdgcn_readfirstlane(s_item);
  if (item < 0) break;
  int grp, hl;
  if (xcd_remap) {
    const int qx = item / per_q, slot = item % per_q;
    grp = AT_NQUEUE * slot + qx / r;
    hl = qx % r;
  } else {
    grp = item / r;
    hl = item % r;
  }
  const int g = grp % Hkv;
  const int b = CB - 1 - grp / Hkv;
  const int h = g * r + hl;
  const int s = (b * LB) / LS;

  const size_t qrow0 = (size_t)b * LB + w * 32;
  const int row_local = w * 32 + l32;

  // block list of (h, s): staged in LDS, AT_LCAP entries at a time
  const int32_t* sel = idx + ((size_t)h * CS + s) * k_max;
  const int n = min(max(cnt[(size_t)h * CS + s], 0), k_max);
  int lbase = 0;
  for (int e = tid; e < min(n, AT_LCAP); e += NT) lst[e] = sel[e];

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
  float m_run = kNegBig, l_run = 0.f;   // m_run in raw (unscaled) logit units

  __syncthreads();   // lst ready
  int p = 0;
  auto next_sel = [&]() -> int {
    while (p < n) {
      if (p == lbase + AT_LCAP) {   // uniform: refill the staged list
        __syncthreads();
        lbase += AT_LCAP;
        for (int e = tid; e < AT_LCAP && lbase + e < n; e += NT) lst[e] = sel[lbase + e];
        __syncthreads();
      }
      const int j = lst[p - lbase];
      ++p;
      if (j >= 0 && j < b) return j;
    }
    return -1;
  };
  auto gen = [&](const AtItem& prev) -> AtItem {
    AtItem it{prev.blk, prev.sub + 1, prev.diag, prev.valid};
    if (!prev.valid || it.sub < SUB) return it;
    it.sub = 0;
    if (prev.diag) {
      it.valid = false;
      return it;
    }
    const int j = __builtin_amdgcn_readfirstlane(next_sel());
    it.diag = j < 0;
    it.blk = it.diag ? b : j;
    return it;
  };
  // a wave whose rows all precede the piece's first key has nothing to do
  auto active = [&](const AtItem& it) { return !(it.diag && it.sub * KT > w * 32 + 31); };

  const bf16* Kg = K + (size_t)g * N * D;
  const bf16* Vg = Vt + (size_t)g * N * D;

  // per-lane byte offsets of the 16-byte chunks this lane copies (the XOR
  // swizzle is a function of the row only, so they are the same every stage)
  uint32_t koff[PER_W], voff[PER_W];
#pragma unroll
  for (int ii = 0; ii < PER_W; ++ii) {
    const int pc = w * PER_W + ii;
    const int krow = pc * KROWS + lane / KCH;
    koff[ii] = (uint32_t)((krow * D + ((lane % KCH) ^ lds_swz<D * 2>(krow)) * 8) *
                          sizeof(bf16));
    const int vrow = pc * 8 + (lane >> 3);
    voff[ii] = (uint32_t)((vrow * KT + ((lane & 7) ^ lds_swz<KT * 2>(vrow)) * 8) * sizeof(bf16));
  }
  auto load_k = [&](const AtItem& it, bf16* kbuf) {
    const bf16* src = Kg + ((size_t)it.blk * LB + it.sub * KT) * D;
    const uint32_t dst = lds_u32(kbuf) + w * PER_W * 1024;
#pragma unroll
    for (int ii = 0; ii < PER_W; ++ii) copy16_to_lds_at(src, koff[ii], dst + ii * 1024);
  };
  auto load_v = [&](const AtItem& it, bf16* vbuf) {
    // V^T tile of the piece: D rows of 64 keys, contiguous
    const bf16* src = Vg + ((size_t)it.blk * LB + it.sub * KT) * D;
    const uint32_t dst = lds_u32(vbuf) + w * PER_W * 1024;
#pragma unroll
    for (int ii = 0; ii < PER_W; ++ii) copy16_to_lds_at(src, voff[ii], dst + ii * 1024);
  };
  // LDS operand reads run ahead of their use: K fragments two d chunks
  // ahead (three register slots), V^T fragments PV_AHEAD MFMAs ahead.  The
  // loops unroll fully, so every slot index is a compile-time constant, and a
  // scheduling fence after each read group keeps the compiler from sinking
  // the reads back next to their use (it does so to save registers, and
  // every MFMA then waits out a full LDS latency).
  auto kfrag = [&](const bf16* ks, int c, bf16x8 (&f)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int row = kt * 32 + l32;
      f[kt] = load8(ks + row * D + (((2 * c + hg) ^ lds_swz<D * 2>(row)) * 8));
    }
  };
  auto mma_s = [&](const bf16* ks, floatx16 (&st)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
    bf16x8 fa[3][2];
    kfrag(ks, 0, fa[0]);
    if (NC > 1) kfrag(ks, 1, fa[1]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 2 < NC) kfrag(ks, c + 2, fa[(c + 2) % 3]);
      sched_fence();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[kt] = mfma32(fa[c % 3][kt], qf[c], st[kt]);
      sched_fence();
    }
  };
  // V^T fragment f in PV order: 16-key group q = f / ND, d tile f % ND
  auto vfrag = [&](const bf16* vs, int f) -> bf16x8 {
    const int row = (f % ND) * 32 + l32, ch = f / ND;
    return load8(vs + row * KT + (((2 * ch + hg) ^ lds_swz<KT * 2>(row)) * 8));
  };
  // probabilities of 16-key group q = exp2(S^T - m) (accumulator tile q / 2,
  // slots 8 (q % 2) .. 8 (q % 2) + 7)
  auto group_exp = [&](const floatx16 (&st)[2], int q, float moff, float (&pv)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pv[e] = fast_exp2(__builtin_fmaf(st[q >> 1][8 * (q & 1) + e], scale_log2, -moff));
  };
  // their bf16 B operand; their row sum joins l_run
  auto group_operand = [&](const float (&pv)[8]) -> bf16x8 {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = f2bf(pv[e]);
    l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    return r;
  };
  auto softmax_exp = [&](const floatx16 (&st)[2], int q, float moff) -> bf16x8 {
    float pv[8];
    group_exp(st, q, moff, pv);
    return group_operand(pv);
  };
  // Causal mask of the own block, row maximum and (rarely) a raised maximum.
  // Beside the maximum's serial chain the VALU forms group 0's probabilities
  // against the current maximum (formed again in the rare stage that raises
  // it); returns them as the first P^T operand.
  auto softmax_max = [&](floatx16 (&st)[2], const AtItem& it) -> bf16x8 {
    if (it.diag && (it.sub * KT + KT - 1 > w * 32)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (it.sub * KT + kt * 32 + acc_row(i, lane) > row_local) st[kt][i] = -INFINITY;
    }
    float pv0[8];
    group_exp(st, 0, m_run * scale_log2, pv0);
    float mx = st[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kt][i]);
    mx = xhalf_max(mx);
    // raise the running maximum only when a row grew by more than 2^kRescale
    if (__any((mx - m_run) * scale_log2 > kRescale)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2((m_run - m_new) * scale_log2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      group_exp(st, 0, m_run * scale_log2, pv0);
    }
    return group_operand(pv0);
  };
  // O^T += V^T P^T, 16-key group outer: the ND MFMAs of group q run while the
  // VALU forms the probabilities of group q + 1.  fv[0 .. PV_AHEAD-1] hold
  // the first V^T fragments and pcur group 0's P^T on entry.
  auto mma_pv = [&](const floatx16 (&st)[2], const bf16* vs, bf16x8 (&fv)[PV_AHEAD + 1],
                    bf16x8 pcur) {
    constexpr int NF = ND * 4;
    const float moff = m_run * scale_log2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sched_fence();
      bf16x8 pnx;
      if (q < 3) pnx = softmax_exp(st, q + 1, moff);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int f = q * ND + dt;
        if (f + PV_AHEAD < NF) fv[(f + PV_AHEAD) % (PV_AHEAD + 1)] = vfrag(vs, f + PV_AHEAD);
        o[dt] = mfma32(fv[f % (PV_AHEAD + 1)], pcur, o[dt]);
      }
      pcur = pnx;
    }
    sched_fence();
  };

  // ---- prologue: K(0), V^T(0) ----
  AtItem it0;
  {
    const int j = __builtin_amdgcn_readfirstlane(next_sel());
    it0.diag = j < 0;
    it0.blk = it0.diag ? b : j;
    it0.sub = 0;
    it0.valid = true;
  }
  AtItem it1 = gen(it0);
  load_k(it0, Ks[0]);
  load_v(it0, Vs[0]);
  wait_vmem();
  __syncthreads();

  // one pipeline step over buffers fixed at compile time (even / odd stage):
  // the copies of stage n+1 fly while stage n is computed; returns false
  // after the last piece
  auto step = [&](bf16* k_cur, bf16* k_nxt, bf16* v_cur, bf16* v_nxt) -> bool {
    if (it1.valid) {
      load_k(it1, k_nxt);
      load_v(it1, v_nxt);
    }
    if (active(it0)) {
      floatx16 st[2];
      bf16x8 fv[PV_AHEAD + 1];
      mma_s(k_cur, st);
#pragma unroll
      for (int f = 0; f < PV_AHEAD; ++f) fv[f] = vfrag(v_cur, f);   // in flight during the max
      sched_fence();
      const bf16x8 p0 = softmax_max(st, it0);
      mma_pv(st, v_cur, fv, p0);
    }
    if (!it1.valid) return false;
    wait_vmem();
    __syncthreads();
    it0 = it1;
    it1 = gen(it1);
    return true;
  };
  while (step(Ks[0], Ks[1], Vs[0], Vs[1]) && step(Ks[1], Ks[0], Vs[1], Vs[0])) {
  }

  const float lt = xhalf_sum(l_run);
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
  if (lse != nullptr && hg == 0)
    lse[(size_t)h * N + qrow0 + l32] = (m_run * scale_log2 + log2f(lt)) * kLn2;
  }
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
        const float alpha = fast_exp2(m - mx);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
        m = mx;
        for (int kk = 0; kk < KT; ++kk) {
          const float pv = fast_exp2(sc[kk] - mx);
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

static bool mfma_path(const PrefillDims& p) {
  return p.dtype == EGS_BF16 && (p.D == 64 || p.D == 128) && (p.LB == 64 || p.LB == 128);
}

// V^T tiles, then the work-queue counters
static size_t vt_bytes(const PrefillDims& p) { return (size_t)p.Hkv * p.N * p.D * sizeof(bf16); }
constexpr size_t kQueueBytes = AT_QMAX * AT_QSTRIDE * sizeof(int);
static_assert(AT_QMAX <= 256, "vt_pack zeroes the counters with its 256 threads");

size_t sparse_attn_workspace_bytes(const PrefillDims& p) {
  // V^T tiles and the queue counters for the MFMA path; nothing otherwise
  return mfma_path(p) ? vt_bytes(p) + kQueueBytes : 0;
}

// Workgroups of the MFMA kernel that the device holds at once.
template <typename Kern>
static int resident_workgroups(Kern kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

hipError_t launch_sparse_attn(const PrefillDims& p, const void* q, const void* k,
                              const void* v, const int32_t* idx, const int32_t* cnt,
                              int k_max, void* out, float* lse, void* ws, hipStream_t st) {
  if (p.dtype == EGS_F32) return generic_dispatch<float>(p, q, k, v, idx, cnt, k_max, out, lse, st);
  if (!mfma_path(p)) return generic_dispatch<bf16>(p, q, k, v, idx, cnt, k_max, out, lse, st);
  const bf16* Q = static_cast<const bf16*>(q);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  bf16* Vt = static_cast<bf16*>(ws);
  int* queue = reinterpret_cast<int*>(static_cast<char*>(ws) + vt_bytes(p));
  bf16* O = static_cast<bf16*>(out);
  const dim3 pgrid(p.N / AT_KT, p.Hkv);
  if (p.D == 128) vt_pack_kernel<128><<<pgrid, 256, 0, st>>>(V, p.N, Vt, queue);
  else vt_pack_kernel<64><<<pgrid, 256, 0, st>>>(V, p.N, Vt, queue);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items = p.Hq * p.CB;
  const int remap = ((p.Hkv * p.CB) % AT_NQUEUE == 0 && AT_NQUEUE * p.r <= AT_QMAX) ? 1 : 0;
  const float sl2 = p.sm_scale * kLog2e;
#define EGS_MF(DD, BB)                                                                    \
  {                                                                                       \
    const int slots = resident_workgroups(sparse_attn_mfma_kernel<DD, BB>, BB * 2);       \
    if (slots <= 0) return hipErrorInvalidDeviceFunction;                                 \
    sparse_attn_mfma_kernel<DD, BB><<<std::min(items, slots), BB * 2, 0, st>>>(           \
        Q, K, Vt, idx, cnt, k_max, O, lse, p.Hkv, p.r, p.N, p.LS, p.CS, p.CB, sl2, remap, \
        queue);                                                                           \
  }
  if (p.D == 128 && p.LB == 128) EGS_MF(128, 128)
  else if (p.D == 128 && p.LB == 64) EGS_MF(128, 64)
  else if (p.D == 64 && p.LB == 128) EGS_MF(64, 128)
  else EGS_MF(64, 64)
#undef EGS_MF
  return hipGetLastError();
}

}  // namespace egs
