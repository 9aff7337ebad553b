// mifa_softmax.hip -- stand-alone row softmax with the online normaliser, for MI355X (gfx950).
//
// What is computed: for every row r of X [rows, cols] (bf16 or fp32) and a scale c,
//   y_rj = exp(c x_rj - m_r) / l_r,  m_r = max_j c x_rj,  l_r = sum_j exp(c x_rj - m_r),
//   lse_r = m_r + ln l_r,
// i.e. the softmax over a row that the online-softmax trick of the interview "Tri Dao:
// prediction" (transcript) computes with one pass for the maximum and the sum: a running max
// and a running sum that is rescaled by exp(m_old - m_new) whenever the max grows.  Partial
// (max, sum) pairs of disjoint parts of a row merge with the same rule, which is how the
// threads of a row combine their parts.
//
// Design (the operation moves bytes and does little arithmetic, so HBM bandwidth bounds it):
//  * Rows of up to 32,768 elements stay in registers between the reduction and the output:
//    every input byte is read from HBM once and every output byte written once.  Each thread
//    loads 16-byte vectors (8 bf16 or 4 fp32) at a stride that keeps a wave's loads contiguous.
//    Rows of up to 4,096 elements get one wave each (four rows per 256-thread workgroup, no
//    LDS); longer rows get the whole workgroup, which combines its four waves through LDS.
//  * Longer rows stream: pass 1 reads the row once and keeps a per-thread running (max, sum)
//    with the online rescale; the pairs are merged across the workgroup; pass 2 reads the row
//    again and writes the output (two reads, one write, against three reads for a separate
//    max pass, sum pass and normalising pass).
//  * Arithmetic is fp32 in the log2 domain (exp2 on v_exp_f32 with c*log2(e) folded into one
//    FMA); bf16 outputs are rounded to nearest even.  Rows or bases that are not 16-byte
//    aligned fall back to element loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mifa.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// c * x in log2 units, with an input of -inf taking no weight for every scale (0 * -inf and a
// negative scale would otherwise turn a masked entry into NaN or +inf).
__device__ __forceinline__ float scaled(float xv, float c) { return xv == -__builtin_inff() ? xv : xv * c; }

// ---- element access ------------------------------------------------------------------------
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  static constexpr int kVec = 8;  // elements per 16-byte vector
  __device__ static float load(const __bf16* p) { return (float)*p; }
  __device__ static void store(__bf16* p, float v) { *p = (__bf16)v; }
  __device__ static void load_vec(const __bf16* p, float* v) {
    const u32x4 raw = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
      v[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xffff0000u);
    }
  }
  __device__ static void store_vec(__bf16* p, const float* v) {
    u32x4 raw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 lo = (__bf16)v[2 * i], hi = (__bf16)v[2 * i + 1];
      raw[i] = (unsigned)__builtin_bit_cast(unsigned short, lo) | ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
    }
    *(u32x4*)p = raw;
  }
};
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
  __device__ static void load_vec(const float* p, float* v) {
    const f32x4 r = *(const f32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r[i];
  }
  __device__ static void store_vec(float* p, const float* v) { *(f32x4*)p = (f32x4){v[0], v[1], v[2], v[3]}; }
};

// ---- merging (max, sum) pairs: the online rule -----------------------------------------------
// (m1, l1) + (m2, l2) -> (m, l1 2^(m1-m) + l2 2^(m2-m)), m = max(m1, m2); a pair with m = -inf is
// empty (l = 0) and must not produce -inf - (-inf).
__device__ __forceinline__ void merge(float& m, float& l, float m2, float l2) {
  const float mn = fmax2(m, m2);
  if (mn == -__builtin_inff()) return;
  l = l * __builtin_amdgcn_exp2f(m - mn) + l2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void wave_merge(float& m, float& l) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64);
    merge(m, l, m2, l2);
  }
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmax2(m, __shfl_xor(m, off, 64));
  return m;
}
__device__ __forceinline__ float wave_sum(float s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}

// ---- register-resident rows ----------------------------------------------------------------
// WPR waves per row (1 or 4), EPT elements per thread.  Thread t of a row group of G = 64 WPR
// threads holds vector k (k = 0 .. EPT/V - 1) at element offset (k G + t) V.
// bf16 rows of 64 or more elements per thread keep the raw bf16 pairs in registers (EPT/2
// per thread instead of EPT floats) and widen them again in each pass; the passes then
// recompute exp2(c x - m) where the float version kept it.  The arithmetic is the same
// sequence of float operations, so the results are identical, and twice as many waves fit
// on a SIMD to overlap one row's loads with another's stores (measured on MI355X: 32,768-element
// rows 18% faster; at 32 elements per thread occupancy was already high and the recomputed
// exponentials made 2,048-element rows 9% slower).
template <typename T, int EPT>
constexpr bool kPackedRow = sizeof(T) == 2 && EPT >= 64;

// NT threads per workgroup (NT/64 waves), WPR waves per row, EPT elements per thread.
template <typename T, int WPR, int EPT, int NT>
// y may be x (in place): every store of a row follows the reduction over all of its loaded values.
__global__ __launch_bounds__(NT) void softmax_resident(const T* x, T* y,
                                                       float* __restrict__ lse, int64_t rows, int cols, float c,
                                                       int vec_ok) {
  using E = Elem<T>;
  constexpr int V = E::kVec, G = 64 * WPR, NV = EPT / V, NW = NT / 64;
  constexpr bool kPacked = kPackedRow<T, EPT>;
  static_assert(EPT % V == 0, "whole vectors per thread");
  static_assert(NW % WPR == 0, "whole rows per workgroup");
  __shared__ float red[2][NW];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int w0 = wave - wave % WPR;  // first wave of this row
  const int t = tid & (G - 1);
  const int64_t row = (int64_t)blockIdx.x * (NW / WPR) + wave / WPR;
  const bool live = row < rows;
  const T* xr = x + (live ? row : 0) * (int64_t)cols;
  T* yr = y + (live ? row : 0) * (int64_t)cols;

  // Element (k, i) of this thread: (k G + t) V + i with 16-byte vectors, or (k V + i) G + t with
  // element loads (consecutive lanes then read consecutive elements).  It is v[k V + i], or
  // the low (i even) / high half of raw[(k V + i) / 2] when packed.
  float v[kPacked ? 1 : EPT];
  unsigned raw[kPacked ? EPT / 2 : 1];
  constexpr unsigned kNegInfBits = 0xff80u;  // bf16 -inf
  // The compiler would otherwise keep the widened values of one pass for the next (they are
  // the same expressions), undoing the packing: each pass starts from registers it cannot see
  // through.
  auto opaque = [&]() {
    if constexpr (kPacked) {
#pragma unroll
      for (int j = 0; j < EPT / 2; ++j) asm volatile("" : "+v"(raw[j]));
    }
  };
  auto elem = [&](int idx) -> float {
    if constexpr (kPacked) {
      const unsigned w = raw[idx >> 1];
      return __builtin_bit_cast(float, (idx & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return v[idx];
    }
  };
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (vec_ok) {
      const int e0 = (k * G + t) * V;
      if (live && e0 + V <= cols) {
        if constexpr (kPacked) {
          const u32x4 r = *(const u32x4*)(xr + e0);
#pragma unroll
          for (int j = 0; j < 4; ++j) raw[k * 4 + j] = r[j];
        } else {
          E::load_vec(xr + e0, v + k * V);
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const bool in = live && e0 + i < cols;
          if constexpr (kPacked) {
            const unsigned b = in ? (unsigned)__builtin_bit_cast(unsigned short, xr[e0 + i]) : kNegInfBits;
            if (i & 1) raw[(k * V + i) >> 1] |= b << 16;
            else raw[(k * V + i) >> 1] = b;
          } else {
            v[k * V + i] = in ? E::load(xr + e0 + i) : -__builtin_inff();
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = (k * V + i) * G + t;
        const bool in = live && e < cols;
        if constexpr (kPacked) {
          const unsigned b = in ? (unsigned)__builtin_bit_cast(unsigned short, xr[e]) : kNegInfBits;
          if (i & 1) raw[(k * V + i) >> 1] |= b << 16;
          else raw[(k * V + i) >> 1] = b;
        } else {
          v[k * V + i] = in ? E::load(xr + e) : -__builtin_inff();
        }
      }
    }
  }
  // row max (log2 units: s = c x; the max of s is c max x for c > 0 and c min x for c < 0,
  // so take the max of the scaled values)
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const float sv = scaled(elem(i), c);
    if constexpr (!kPacked) v[i] = sv;
    m = fmax2(m, sv);
  }
  m = wave_max(m);
  if constexpr (WPR > 1) {
    if ((tid & 63) == 0) red[0][wave] = m;
    __syncthreads();
    m = red[0][w0];
#pragma unroll
    for (int w = 1; w < WPR; ++w) m = fmax2(m, red[0][w0 + w]);
  }
  float l = 0.f;
  opaque();
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if constexpr (kPacked) {
      l += __builtin_amdgcn_exp2f(scaled(elem(i), c) - m);
    } else {
      v[i] = __builtin_amdgcn_exp2f(v[i] - m);
      l += v[i];
    }
  }
  l = wave_sum(l);
  if constexpr (WPR > 1) {
    if ((tid & 63) == 0) red[1][wave] = l;
    __syncthreads();
    if constexpr (WPR == 4) {
      l = (red[1][w0] + red[1][w0 + 1]) + (red[1][w0 + 2] + red[1][w0 + 3]);
    } else {
      l = red[1][w0];
#pragma unroll
      for (int w = 1; w < WPR; ++w) l += red[1][w0 + w];
    }
  }
  if (!live) return;
  const float inv = 1.f / l;
  opaque();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    float o[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if constexpr (kPacked) o[i] = __builtin_amdgcn_exp2f(scaled(elem(k * V + i), c) - m) * inv;
      else o[i] = v[k * V + i] * inv;
    }
    if (vec_ok) {
      const int e0 = (k * G + t) * V;
      if (e0 + V <= cols) {
        E::store_vec(yr + e0, o);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (e0 + i < cols) E::store(yr + e0 + i, o[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = (k * V + i) * G + t;
        if (e < cols) E::store(yr + e, o[i]);
      }
    }
  }
  if (lse && t == 0) lse[row] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
}

// ---- 256-thread row pieces: part u of step `base` -------------------------------------------
// With 16-byte vectors thread tid holds elements base + (u 256 + tid) V + i; with element loads
// it holds base + (u V + i) 256 + tid.  Elements past the row read as -inf and are not stored.
template <typename T>
__device__ __forceinline__ int part_elem(int base, int u, int i, int tid, int vec_ok) {
  constexpr int V = Elem<T>::kVec;
  return vec_ok ? base + (u * kThreads + tid) * V + i : base + (u * V + i) * kThreads + tid;
}
template <typename T>
__device__ __forceinline__ void load_part(const T* xr, int cols, int base, int u, int tid, int vec_ok, float* v) {
  using E = Elem<T>;
  constexpr int V = E::kVec;
  const int e0 = part_elem<T>(base, u, 0, tid, vec_ok);
  if (vec_ok && e0 + V <= cols) {
    E::load_vec(xr + e0, v);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = part_elem<T>(base, u, i, tid, vec_ok);
      v[i] = e < cols ? E::load(xr + e) : -__builtin_inff();
    }
  }
}
template <typename T>
__device__ __forceinline__ void store_part(T* yr, int cols, int base, int u, int tid, int vec_ok, const float* v) {
  using E = Elem<T>;
  constexpr int V = E::kVec;
  const int e0 = part_elem<T>(base, u, 0, tid, vec_ok);
  if (vec_ok && e0 + V <= cols) {
    E::store_vec(yr + e0, v);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = part_elem<T>(base, u, i, tid, vec_ok);
      if (e < cols) E::store(yr + e, v[i]);
    }
  }
}

// ---- streaming rows (longer than a workgroup's registers hold) ------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_stream(const T* x, T* y,
                                                            float* __restrict__ lse, int cols, float c, int vec_ok) {
  using E = Elem<T>;
  constexpr int V = E::kVec, U = 4;  // U vectors in flight per thread per step
  constexpr int kStep = kThreads * V * U;
  __shared__ float red[2][4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const T* xr = x + row * (int64_t)cols;
  T* yr = y + row * (int64_t)cols;

  // pass 1: running (max, sum) per thread, rescaled when the max grows
  float m = -__builtin_inff(), l = 0.f;
  for (int base = 0; base < cols; base += kStep) {
    float v[U * V];
#pragma unroll
    for (int u = 0; u < U; ++u) load_part<T>(xr, cols, base, u, tid, vec_ok, v + u * V);
    float bm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < U * V; ++i) {
      v[i] = scaled(v[i], c);
      bm = fmax2(bm, v[i]);
    }
    if (bm == -__builtin_inff()) continue;
    const float mn = fmax2(m, bm);
    float bl = 0.f;
#pragma unroll
    for (int i = 0; i < U * V; ++i) bl += __builtin_amdgcn_exp2f(v[i] - mn);
    l = l * __builtin_amdgcn_exp2f(m - mn) + bl;
    m = mn;
  }
  wave_merge(m, l);
  if ((tid & 63) == 0) {
    red[0][wave] = m;
    red[1][wave] = l;
  }
  __syncthreads();
  m = red[0][0];
  l = red[1][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) merge(m, l, red[0][w], red[1][w]);
  const float inv = 1.f / l;

  // pass 2: normalise.  y may be x (in place): every element is read and written by the same
  // thread, and a step's U loads are all issued before its stores, so no store overtakes a load.
  for (int base = 0; base < cols; base += kStep) {
    float v[U * V];
#pragma unroll
    for (int u = 0; u < U; ++u) load_part<T>(xr, cols, base, u, tid, vec_ok, v + u * V);
#pragma unroll
    for (int i = 0; i < U * V; ++i) v[i] = __builtin_amdgcn_exp2f(scaled(v[i], c) - m) * inv;
#pragma unroll
    for (int u = 0; u < U; ++u) store_part<T>(yr, cols, base, u, tid, vec_ok, v + u * V);
  }
  if (lse && tid == 0) lse[row] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
}

template <typename T, int WPR, int EPT, int NT = kThreads>
hipError_t launch_resident(const void* x, void* y, float* lse, int64_t rows, int cols, float c, int vec_ok,
                           hipStream_t s) {
  constexpr int rpb = NT / 64 / WPR;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  hipLaunchKernelGGL((softmax_resident<T, WPR, EPT, NT>), dim3((unsigned)blocks), dim3(NT), 0, s, (const T*)x, (T*)y,
                     lse, rows, cols, c, vec_ok);
  return hipGetLastError();
}

// Launch choice by row length: one wave per row up to 64*64 elements, one 256-thread workgroup
// with the row in registers up to 256*128, one 1024-thread workgroup with the row in registers
// up to 1024*128 (bf16) or 1024*64 (float), streaming (two reads) beyond.  Measured on MI355X:
// keeping 32,768-element rows in registers runs 1.2-1.5x faster than staging them in LDS or
// streaming them.  EPT is the smallest whole number of vectors that covers the row.
template <typename T>
hipError_t dispatch_softmax(const void* x, void* y, float* lse, int64_t rows, int cols, float c, int vec_ok,
                            hipStream_t s) {
  constexpr int V = Elem<T>::kVec;
  if (cols <= 64 * 64) {
    if (cols <= 64 * V) return launch_resident<T, 1, V>(x, y, lse, rows, cols, c, vec_ok, s);
    if (cols <= 64 * 2 * V) return launch_resident<T, 1, 2 * V>(x, y, lse, rows, cols, c, vec_ok, s);
    if (cols <= 64 * 4 * V) return launch_resident<T, 1, 4 * V>(x, y, lse, rows, cols, c, vec_ok, s);
    if (cols <= 64 * 8 * V) return launch_resident<T, 1, 8 * V>(x, y, lse, rows, cols, c, vec_ok, s);
    return launch_resident<T, 1, 64>(x, y, lse, rows, cols, c, vec_ok, s);
  }
  if (cols <= 256 * 16) return launch_resident<T, 4, 16>(x, y, lse, rows, cols, c, vec_ok, s);
  if (cols <= 256 * 32) return launch_resident<T, 4, 32>(x, y, lse, rows, cols, c, vec_ok, s);
  if (cols <= 256 * 64) return launch_resident<T, 4, 64>(x, y, lse, rows, cols, c, vec_ok, s);
  if (cols <= 256 * 128) return launch_resident<T, 4, 128>(x, y, lse, rows, cols, c, vec_ok, s);
  // Up to 131,072 bf16 (65,536 float) elements: one 1024-thread workgroup per row, the row still
  // in registers (bf16 packed two per register), so it is read once instead of twice.
  if constexpr (sizeof(T) == 2) {
    if (cols <= 1024 * 128) return launch_resident<T, 16, 128, 1024>(x, y, lse, rows, cols, c, vec_ok, s);
  } else {
    if (cols <= 1024 * 64) return launch_resident<T, 16, 64, 1024>(x, y, lse, rows, cols, c, vec_ok, s);
  }
  hipLaunchKernelGGL(softmax_stream<T>, dim3((unsigned)rows), dim3(kThreads), 0, s, (const T*)x, (T*)y, lse, cols, c,
                     vec_ok);
  return hipGetLastError();
}

}  // namespace

// Records a HIP error code for mifa_last_hip_error (defined beside it).
extern "C" __attribute__((visibility("hidden"))) void mifa_record_hip_error(int e);

extern "C" int mifa_softmax_rows(const void* x, void* y, float* lse, int64_t rows, int64_t cols, int dtype,
                                 float scale, void* stream) {
  if (!x || !y) return MIFA_ERR_NULL_POINTER;
  if (rows < 1 || cols < 1) return MIFA_ERR_BAD_SHAPE;
  if (dtype != MIFA_DTYPE_BF16 && dtype != MIFA_DTYPE_F32) return MIFA_ERR_BAD_DTYPE;
  const uintptr_t esize = dtype == MIFA_DTYPE_BF16 ? 2 : 4;
  if ((((uintptr_t)x | (uintptr_t)y) & (esize - 1)) != 0 || ((uintptr_t)lse & 3u) != 0) return MIFA_ERR_MISALIGNED;
  if (!__builtin_isfinite(scale)) return MIFA_ERR_BAD_SCALE;
  if (rows >= ((int64_t)1 << 31) || cols >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  const int vec_ok = ((((uintptr_t)x | (uintptr_t)y) & 15u) == 0 && ((uint64_t)cols * esize) % 16 == 0) ? 1 : 0;
  const float c = (float)((double)scale * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = dtype == MIFA_DTYPE_BF16 ? dispatch_softmax<__bf16>(x, y, lse, rows, (int)cols, c, vec_ok, s)
                                                : dispatch_softmax<float>(x, y, lse, rows, (int)cols, c, vec_ok, s);
  if (e != hipSuccess) {
    mifa_record_hip_error((int)e);
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}
