// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, conversions and wavefront reductions.  CDNA4 only (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace egs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Operand layout (both A and B): lane l holds row/column (l % 32) and the
// 8 consecutive k-slots of group (l / 32).  Accumulator: lane l holds column
// (l % 32), register i holds row 8*(i/4) + 4*(l/32) + (i%4).
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l holds row (A) / column (B) l % 16 and 8 k-slots of group l / 16 (the
// same slots in both operands, so any fixed assignment of k to slots gives the
// same product).  Accumulator: lane l holds column l % 16, register i holds
// row 4 * (l / 16) + i.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 2^x with one v_exp_f32.  Results below 2^-126 may flush to zero: every
// caller exponentiates a logit minus a running maximum, where such terms are
// far below the fp32 resolution of the sum they join.  exp2f() would add a
// denormal-preserving range reduction (five more VALU operations).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }   // RNE

__device__ __forceinline__ bf16x8 load8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void store8(bf16* p, bf16x8 v) {
  *reinterpret_cast<bf16x8*>(p) = v;
}

// Load 8 consecutive elements as floats from bf16 or float storage.
__device__ __forceinline__ void load8f(const bf16* p, float* out) {
  bf16x8 v = load8(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
__device__ __forceinline__ void load8f(const float* p, float* out) {
  floatx4 a = *reinterpret_cast<const floatx4*>(p);
  floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[e + 4] = b[e]; }
}

// Split 8 floats into bf16 hi + lo parts (x ~= hi + lo to ~2^-17 relative).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 h = (bf16)x[e];
    hi[e] = h;
    lo[e] = (bf16)(x[e] - (float)h);
  }
}

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap: the two
// halves of the wave trade places without going through LDS).
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's bytes land at lds_base + 16 * i, lds_base being wave-uniform (M0).
// Issued through inline assembly so that the compiler does not track the copy
// as an LDS write: it would otherwise wait for every copy in flight before any
// later LDS read, including reads of other buffers.  Callers order reads of
// the destination with wait_vmem() and a workgroup barrier.
typedef __attribute__((address_space(3))) void lds_void_t;
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}
// lds_addr must be wave-uniform (it goes to M0 through an SGPR).
__device__ __forceinline__ void copy16_to_lds_at(const void* sbase, uint32_t voff,
                                                 uint32_t lds_addr) {
  // sbase: wave-uniform global base; voff: this lane's byte offset from it
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory", "m0");
}
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, void* lds_base) {
  copy16_to_lds_at(sbase, voff, __builtin_amdgcn_readfirstlane(lds_u32(lds_base)));
}
// A pointer the compiler cannot prove wave-uniform, moved into SGPRs (the
// value of lane 0; callers pass a pointer that is the same on every lane).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// Wait until at most N of this wave's vector-memory operations are in flight.
// Loads retire in issue order, so with only direct LDS copies outstanding this
// waits for every copy except the N issued last.  The wait goes through the
// s_waitcnt builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their maxima) rather than inline assembly, so the compiler's
// own wait tracking sees it: loads it issued earlier (e.g. register operands
// fetched before a pipelined loop) are then known to be complete, and it does
// not wait for them again inside the loop, where such a wait would also stall
// on the copies in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait for all of this wave's outstanding vector-memory loads (direct LDS
// copies included).
__device__ __forceinline__ void wait_vmem() { wait_vmem_upto<0>(); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// XOR swizzle of the 16-byte chunks of LDS rows of ROW_BYTES bytes.  The LDS
// serves 256 bytes (16 chunks) per cycle, i.e. the 16 lanes of a quarter
// wave per ds_read_b128; operand reads have those lanes on 16 consecutive
// rows at one logical chunk.  Rows sharing a 256-byte window are told apart
// by their offset in it, rows in different windows by the XOR, so the 16
// reads land in 16 distinct chunk slots.
template <int ROW_BYTES>
__device__ __forceinline__ int lds_swz(int row) {
  constexpr int CPR = ROW_BYTES / 16;               // chunks per row
  constexpr int RPW = CPR >= 16 ? 1 : 16 / CPR;     // rows per 256-byte window
  constexpr int MASK = (CPR >= 16 ? 16 : CPR) - 1;
  return (row / RPW) & MASK;
}

// Order-preserving map of float bits onto unsigned integers.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace egs
