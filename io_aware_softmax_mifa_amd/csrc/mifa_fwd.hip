// mifa_fwd.hip -- exact FlashAttention forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// What is computed: O = softmax(scale * Q K^T [+ causal mask]) V and the per-row log-sum-exp,
// for bf16 Q, K, V in [B, H, N, d] (d = 64 or 128) with fp32 O and LSE.  The method is the one
// the interview "Tri Dao: prediction" (transcript) describes: kernel fusion (every step below
// runs inside one kernel, so the scores and probabilities never go to HBM), tiling into fast
// on-chip memory, and the online-softmax trick, which splits each row's softmax into key blocks
// whose partial sums and outputs are rescaled when the running maximum grows and still give
// the exact result.  The causal variant is the softmax of the lower-triangular score matrix
// (FlashAttention-2 remark in the Hacker News FlashAttention-3 thread); blocks wholly above
// the diagonal are never loaded.
//
// Design on gfx950 (one workgroup = 4 waves = 128 query rows of one (b, h)):
//  * Each wave owns 32 query rows.  Its Q rows stay in VGPRs for the whole kernel, already in
//    the B-operand layout of v_mfma_f32_32x32x16_bf16.
//  * K and V blocks of BC keys are streamed from HBM/L2 into double-buffered LDS with the
//    16-byte global->LDS DMA (global_load_lds_dwordx4), so loads of block j+1 overlap the math
//    of block j without passing through VGPRs.  A wait on the vector-memory counter plus a
//    workgroup barrier guards each buffer before use: the threads fill the tile cooperatively,
//    so nobody may read it before everyone's part has landed (the point made about shared
//    SRAM in "Show HN: Flash Attention in ~100 lines of CUDA").
//  * Scores are computed transposed, S^T = K Q^T, on MFMA.  In the 32x32 accumulator layout a
//    lane then holds 16 scores of ONE query (its lane % 32), so the row max and row sum are
//    in-lane reductions plus a single exchange with lane ^ 32.
//  * Softmax runs in the log2 domain (exp2 on v_exp_f32, with scale * log2(e) folded into one
//    FMA per score).  The running max used for exponentiation is only raised when a block's
//    max exceeds it by more than kRescaleSlack (2^8): the output and row sum are then
//    rescaled once; otherwise the stale max is kept and the weights are at most 2^8.  The
//    final division by the row sum taken with the same max makes this exact, and it removes
//    almost every per-block O rescale.
//  * O^T = V^T P^T on MFMA: the probabilities (rounded to bf16) feed the B operand straight from
//    the score accumulators (the key order inside one MFMA is a free permutation of the
//    contraction index), and V^T comes from LDS with ds_read_b64_tr_b16, which transposes a
//    4 x 16 block of bf16 across each 16-lane group.  Each lane accumulates O for its own
//    query, so the per-row rescale and the final 1/l are in-lane multiplies.
//  * LDS tiles are XOR-swizzled in 16-byte chunks to spread the K reads and the V transpose
//    reads over the banks.
//  * Grid: one workgroup per (b, h, q-tile), heaviest causal tiles first, and when the tile
//    count allows it, all tiles of one head are placed on the same XCD (workgroups are handed
//    to the 8 XCDs round-robin) so K/V re-reads hit that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mifa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleSlack = 8.0f;       // log2 units: weights stay <= 2^8 between rescales
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
  return D == 128 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1);
}

__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt with expcnt and lgkmcnt at their maxima: only the vector-memory count is waited on.
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14].
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

template <int D, int BC, bool CAUSAL>
struct Tile {
  static constexpr int kChunksPerRow = D / 8;             // 16-byte chunks per K/V row
  static constexpr int kRowsPerInst = 64 / kChunksPerRow; // rows one wave-wide DMA covers
  static constexpr int kInstPerTensor = BC / kRowsPerInst;
  static constexpr int kInstPerWave = kInstPerTensor / kWaves;
  static constexpr int kLoadsPerBlock = 2 * kInstPerWave; // K and V DMA ops per thread per block
  static constexpr int kTensorBytes = BC * D * 2;
  static constexpr int kBufBytes = 2 * kTensorBytes;      // K then V
  static constexpr int kLdsBytes = 2 * kBufBytes;         // double buffered
  static_assert(kInstPerTensor % kWaves == 0, "block must split evenly over the waves");
  static_assert(BC % 32 == 0, "key block must be a multiple of the 32-key MFMA tile");
};

// Issue the DMA of key block `blk` (rows blk*BC ..) of K and V into LDS buffer `buf`.
// Rows past N are clamped to N-1: they are masked out of the softmax, and clamping keeps every
// global address inside the tensors.
template <int D, int BC, bool CAUSAL>
__device__ __forceinline__ void issue_kv(const __bf16* __restrict__ kbase, const __bf16* __restrict__ vbase,
                                        char* smem_buf, int blk, int N, int wave, int lane) {
  using T = Tile<D, BC, CAUSAL>;
#pragma unroll
  for (int t = 0; t < T::kInstPerWave; ++t) {
    const int inst = wave * T::kInstPerWave + t;
    const int r = inst * T::kRowsPerInst + lane / T::kChunksPerRow;
    const int pc = lane % T::kChunksPerRow;
    int grow = blk * BC + r;
    grow = grow < N ? grow : N - 1;
    const __bf16* ks = kbase + (int64_t)grow * D + ((pc ^ swz_k<D>(r)) * 8);
    const __bf16* vs = vbase + (int64_t)grow * D + ((pc ^ swz_v<D>(r)) * 8);
    __builtin_amdgcn_global_load_lds((global_cvoid*)ks, (lds_void*)(smem_buf + inst * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_cvoid*)vs,
                                     (lds_void*)(smem_buf + T::kTensorBytes + inst * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

template <int D, int BC, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void mifa_fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
                     int N, int BH, int n_qtiles, float c_log2, int negate_q, int xcd_group) {
  using T = Tile<D, BC, CAUSAL>;
  constexpr int kDS = D / 16;  // 16-wide d slices of the S^T MFMA
  constexpr int kDT = D / 32;  // 32-row dv tiles of O^T
  constexpr int kKT = BC / 32; // 32-key tiles per block
  constexpr int kKS = BC / 16; // 16-key slices per block (PV k-steps)

  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;

  // ---- which (b*H + h, q-tile) this workgroup owns ----
  int bh, qt;
  {
    const int w = blockIdx.x;
    if (xcd_group) {
      // Workgroup w runs on XCD w % 8; give XCD x the heads bh = x, x + 8, ... and walk them
      // heaviest tile first.
      const int x = w % kXcds, kk = w / kXcds;
      const int heads_per_xcd = BH / kXcds;
      const int rank = kk / heads_per_xcd;
      bh = (kk % heads_per_xcd) * kXcds + x;
      qt = CAUSAL ? n_qtiles - 1 - rank : rank;
    } else {
      const int rank = w / BH;
      bh = w % BH;
      qt = CAUSAL ? n_qtiles - 1 - rank : rank;
    }
  }
  const int64_t head_off = (int64_t)bh * N * D;
  const __bf16* __restrict__ qh = q + head_off;
  const __bf16* __restrict__ kh = k + head_off;
  const __bf16* __restrict__ vh = v + head_off;

  const int row0 = qt * kBR + wave * kRowsPerWave;  // first query row of this wave
  const int my_row = row0 + ln;

  // ---- Q rows into VGPRs (B operand of S^T = K Q^T: lane holds q[row][16s + 8hf .. +7]) ----
  bf16x8 qf[kDS];
  {
    const int r = my_row < N ? my_row : N - 1;
    const __bf16* src = qh + (int64_t)r * D + 8 * hf;
#pragma unroll
    for (int s = 0; s < kDS; ++s) {
      u32x4 raw = *(const u32x4*)(src + 16 * s);
      if (negate_q) raw ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  const int n_kblocks = (N + BC - 1) / BC;
  int nblk = n_kblocks;
  if (CAUSAL) {
    const int last_row = min(N - 1, qt * kBR + kBR - 1);
    nblk = last_row / BC + 1;
  }

  f32x16 oacc[kDT];
#pragma unroll
  for (int t = 0; t < kDT; ++t) oacc[t] = (f32x16){};
  float m_run = -__builtin_inff();  // running max in log2 units (stale by at most kRescaleSlack)
  float l_run = 0.f;                // this lane's half of the row sum

  issue_kv<D, BC, CAUSAL>(kh, vh, smem, 0, N, wave, lane);

  for (int j = 0; j < nblk; ++j) {
    char* buf = smem + (j & 1) * T::kBufBytes;
    if (j + 1 < nblk) {
      issue_kv<D, BC, CAUSAL>(kh, vh, smem + ((j + 1) & 1) * T::kBufBytes, j + 1, N, wave, lane);
      wait_vmcnt(T::kLoadsPerBlock);
    } else {
      wait_vmcnt(0);
    }
    __builtin_amdgcn_s_barrier();

    const int key0 = j * BC;
    // Wave-uniform facts about this block.
    const bool wave_dead = CAUSAL && key0 > row0 + kRowsPerWave - 1;  // all keys above the diagonal
    const bool need_mask = (CAUSAL && key0 + BC - 1 > row0) || (key0 + BC > N);

    if (!wave_dead) {
      const char* sk = buf;
      const char* sv = buf + T::kTensorBytes;

      // ---- S^T = K_j Q^T on MFMA ----
      f32x16 sacc[kKT];
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        sacc[kt] = (f32x16){};
        const bool tile_live = !CAUSAL || key0 + 32 * kt <= row0 + kRowsPerWave - 1;
        if (tile_live) {
          const int r = 32 * kt + ln;
#pragma unroll
          for (int s = 0; s < kDS; ++s) {
            const int c = 2 * s + hf;
            const bf16x8 a = *(const bf16x8*)(sk + r * (D * 2) + ((c ^ swz_k<D>(r)) * 16));
            sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
          }
        }
      }

      // ---- mask, block row max ----
      // Lane holds S^T[key][my_row] for key = key0 + 32kt + 8(i/4) + 4hf + (i%4).
      float mx = -__builtin_inff();
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * hf + (i & 3);
            const bool vis = key < N && (!CAUSAL || key <= my_row);
            sacc[kt][i] = vis ? sacc[kt][i] : -__builtin_inff();
          }
      }
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[kt][i], sacc[kt][i + 1]));
      mx = fmaxf(mx, xor32(mx));
      // Block max in log2 units; c_log2 >= 0, and an all-masked row stays at -inf.
      const float bm = mx == -__builtin_inff() ? mx : mx * c_log2;

      // ---- lazy rescale: only when the block max outgrows the running max by the slack ----
      const bool grow = bm > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? bm : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < kDT; ++t) oacc[t] *= alpha;
        m_run = m_new;
      }

      // ---- P = exp2(S * c - m), row sum, bf16 pack (B operand of O^T += V^T P^T) ----
      bf16x8 pb[kKS];
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][i], c_log2, -m_run));
          if (need_mask) p = sacc[kt][i] == -__builtin_inff() ? 0.f : p;
          lsum += p;
          pb[2 * kt + (i >> 3)][i & 7] = (__bf16)p;
        }
      l_run += lsum;

      // ---- O^T += V_j^T P^T on MFMA; V^T operand via the LDS transpose read ----
      // Lane (dv row 32t + ln, half hf) needs V[key][dv] for keys 16ks + 4hf + 0..3 and
      // 16ks + 8 + 4hf + 0..3.  Within a 16-lane group, lane p addresses key row (p / 4) of the
      // 4-row slab and dv column 4 * (p % 4) of the group's 16 columns; the transpose read then
      // hands lane i the group's column i of those 4 rows.
      const int g = lane >> 4, p = lane & 15;
      const int dvh = g & 1;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bool slice_live = !CAUSAL || key0 + 16 * ks <= row0 + kRowsPerWave - 1;
        if (!slice_live) continue;
#pragma unroll
        for (int t = 0; t < kDT; ++t) {
          const int c = 4 * t + 2 * dvh + ((p & 3) >> 1);
          const int sub = (p & 1) * 8;
          const int r0 = 16 * ks + 4 * hf + (p >> 2);
          const int r1 = r0 + 8;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(lds_void*)(sv + r0 * (D * 2) + ((c ^ swz_v<D>(r0)) * 16) + sub));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(lds_void*)(sv + r1 * (D * 2) + ((c ^ swz_v<D>(r1)) * 16) + sub));
          const i16x8 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16), pb[ks], oacc[t], 0, 0, 0);
        }
      }
    }
    // Everyone is done with this buffer before the next iteration's DMA overwrites it.
    __builtin_amdgcn_s_barrier();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ----
  const float l_tot = l_run + xor32(l_run);
  if (my_row < N) {
    const float inv = 1.f / l_tot;
    float* orow = o + head_off + (int64_t)my_row * D;
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 val = {oacc[t][4 * g4] * inv, oacc[t][4 * g4 + 1] * inv, oacc[t][4 * g4 + 2] * inv,
                     oacc[t][4 * g4 + 3] * inv};
        *(f32x4*)(orow + 32 * t + 8 * g4 + 4 * hf) = val;
      }
    if (hf == 0) lse[(int64_t)bh * N + my_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int BC, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, float* o, float* lse, int N, int BH,
                  float scale, hipStream_t stream) {
  using T = Tile<D, BC, CAUSAL>;
  const int n_qtiles = (N + kBR - 1) / kBR;
  const int64_t tiles = (int64_t)BH * n_qtiles;
  const int xcd_group = (BH % kXcds == 0) ? 1 : 0;
  const int negate_q = scale < 0.f ? 1 : 0;
  const float c_log2 = (float)((double)(negate_q ? -scale : scale) * 1.4426950408889634);
  auto kern = mifa_fwd_kernel<D, BC, CAUSAL>;
  static bool configured = false;  // per-instantiation attribute, idempotent
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, T::kLdsBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kThreads), T::kLdsBytes, stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, o, lse, N, BH, n_qtiles, c_log2,
                     negate_q, xcd_group);
  return hipGetLastError();
}

thread_local int g_last_hip_error = 0;

}  // namespace

extern "C" {

int mifa_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int64_t B, int64_t H,
             int64_t N, int64_t d, int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return MIFA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || N < 1) return MIFA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return MIFA_ERR_UNSUPPORTED_D;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return MIFA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3u) return MIFA_ERR_MISALIGNED;
  if (!__builtin_isfinite(scale)) return MIFA_ERR_BAD_SCALE;
  // Per-head offsets inside the kernel are 32-bit (N*d), the grid is 1-D (B*H*tiles).
  if (N * d >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  if (B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  const int64_t BH = B * H;
  const int64_t tiles = BH * ((N + kBR - 1) / kBR);
  if (BH >= ((int64_t)1 << 31) || tiles >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;

  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d == 128)
    e = causal ? launch<128, 64, true>(q, k, v, o, lse, (int)N, (int)BH, scale, s)
               : launch<128, 64, false>(q, k, v, o, lse, (int)N, (int)BH, scale, s);
  else
    e = causal ? launch<64, 64, true>(q, k, v, o, lse, (int)N, (int)BH, scale, s)
               : launch<64, 64, false>(q, k, v, o, lse, (int)N, (int)BH, scale, s);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}

const char* mifa_status_string(int status) {
  switch (status) {
    case MIFA_OK: return "ok";
    case MIFA_ERR_NULL_POINTER: return "null pointer argument";
    case MIFA_ERR_BAD_SHAPE: return "B, H and N must be >= 1";
    case MIFA_ERR_UNSUPPORTED_D: return "head dimension d must be 64 or 128";
    case MIFA_ERR_MISALIGNED: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case MIFA_ERR_BAD_SCALE: return "scale must be finite";
    case MIFA_ERR_TOO_LARGE: return "problem too large (N*d or the tile count reaches 2^31)";
    case MIFA_ERR_HIP: return "HIP runtime error (see mifa_last_hip_error)";
    default: return "unknown status";
  }
}

const char* mifa_version(void) { return "mifa 0.1.0 gfx950"; }

int mifa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
