// mifa_common.h -- device helpers shared by the libmifa kernels (gfx950): vector types, LDS
// operand reads with explicit waits, the 16-byte chunk swizzles of K/V-style tiles, and small
// VALU reductions across the two 32-lane halves of a wave.
#ifndef MIFA_COMMON_H
#define MIFA_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <utility>

namespace mifa_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

template <int V>
using IC = std::integral_constant<int, V>;

constexpr int kXcds = 8;

// 16-byte chunk swizzles.  K rows are read 16 rows at a time at one logical chunk; V rows are
// read 4 rows at a time in 32-byte (2-chunk) pieces by the transpose read, so V only XORs with
// even values to keep chunk pairs adjacent.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt at their maxima (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- LDS operand reads ------------------------------------------------------------------------
// Issued as inline asm so that the compiler does not treat them as reads of the LDS buffer the
// next DMA is filling (which would make it drain that DMA first).  Every consumer waits through
// lgkm_wait, which ties the registers that must have landed to the s_waitcnt; LDS reads complete
// in issue order, so "at most N outstanding" means everything but the N most recent is done.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read_b128(unsigned addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ i16x4 lds_read_tr(unsigned addr) {
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N, typename R>
__device__ __forceinline__ void lgkm_wait(R& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
template <int N, typename R>
__device__ __forceinline__ void lgkm_wait(R& a, R& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// ---- small VALU helpers ------------------------------------------------------------------------
// Maximum without the NaN-quieting canonicalisation that fmaxf needs (scores are never NaN);
// three-operand forms map onto v_maximum3_f32.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmax2(fmax2(a, b), c); }

// v_permlane32_swap exchanges the two 32-lane halves of a wave.  Every lane then holds its own
// value and the value of the lane 32 away.  (The pair is read back through a 64-bit bit cast:
// subscripting the returned vector loses its second element with this compiler.)
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  const uint64_t both = __builtin_bit_cast(uint64_t, r);
  a = __builtin_bit_cast(float, (unsigned)both);
  b = __builtin_bit_cast(float, (unsigned)(both >> 32));
}
__device__ __forceinline__ float half_max(float x) {
  float a, b;
  swap_halves(x, a, b);
  return fmax2(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a, b;
  swap_halves(x, a, b);
  return a + b;
}

// ---- host: the dynamic-LDS limit of a kernel ----------------------------------------------------
// Kernels that use more than the default dynamic LDS need the limit raised once on every device
// they run on; `done` (one per kernel) records the devices already set.  Thread-safe: two
// threads may both set it, which is harmless.
inline hipError_t raise_lds_limit(const void* fn, int bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace mifa_detail

#endif  // MIFA_COMMON_H
