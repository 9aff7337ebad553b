// mifa_bwd.hip -- gradients of exact attention for MI355X (gfx950).
//
// What is computed: for the forward O = P V, P = softmax(S) row by row, S = c Q K^T (the causal
// variant masks key j for query i iff j > i + Nk - Nq) and an upstream gradient dO,
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_t dO_it O_it,   dS = P * (dP - D),
//     dQ = c dS K,   dK = c dS^T Q.
// The pages stop at the forward pass ("Show HN: Flash Attention in ~100 lines of CUDA" leaves
// the matrix derivatives out); this is the next step, built the same way as the forward: fused
// and tiled, with P recomputed block by block from the forward's saved LSE
// (P_ij = exp(c s_ij - LSE_i)) instead of being stored, so no N x N matrix reaches HBM.
//
// Three kernels, no atomics (results are bitwise reproducible):
//  * row_dot: D_i = dO_i . O_i per query row (one pass over O and dO).
//  * dq: one workgroup per (b*h, 128-query tile), like the forward: each wave keeps 32 query
//    rows of Q and dO in registers, streams K and V blocks of 64 keys through LDS, computes
//    S^T = K Q^T and dP^T = V dO^T on MFMA, then dS^T, and accumulates dQ^T += K^T dS^T (K^T
//    read from the K tile with the transposing LDS read).
//  * dkdv: one workgroup per (b*h, 128-key tile), the roles swapped: each wave keeps 32 keys
//    of K and V in registers, streams Q and dO blocks of 64 queries (with their LSE and D,
//    three buffers), computes S = Q K^T and dP = dO V^T, then P and dS, and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS.  Software-pipelined: the score arithmetic of one
//    32-query tile runs beside the S and dP products of the next and the dV/dK products of
//    the previous one.  With the causal mask, dkdv_split instead: 8 waves, the two waves of a
//    SIMD sharing 32 keys in two roles (one computes S, P and dV, the other dP, dS and dK,
//    with P passed through LDS), so two waves per SIMD overlap each other's arithmetic.
// In both, the probabilities / dS feed the second product straight from the accumulator
// layout (the contraction index inside one MFMA is a free permutation), as in the forward.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "mifa.h"
#include "mifa_common.h"

namespace {

using namespace mifa_detail;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // rows (queries or keys) a workgroup owns
constexpr int kBlk = 64;            // rows of a streamed block (keys or queries)

template <int D, int W = kWaves>
struct Geo {
  static constexpr int kDS = D / 16;                // 16-wide d slices
  static constexpr int kDT = D / 32;                // 32-row d tiles of a transposed product
  static constexpr int kTile = kBlk * D * 2;        // bytes of one bf16 block
  static constexpr int kChunksPerRow = D / 8;       // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunksPerRow;
  static constexpr int kInstPerTile = kBlk / kRowsPerInst;
  static constexpr int kInstPerWave = kInstPerTile / W;
  static constexpr int kLds = 2 * 2 * kTile;        // dq: two tensors (K, V), double buffered
  static_assert(kInstPerWave * W == kInstPerTile, "tile splits evenly over the waves");
};

// ---- tiles in LDS --------------------------------------------------------------------------
// Every tile here is read both row-major (16 bytes of one row per lane: 16 lanes, 16 rows, per
// LDS cycle) and transposed (8 bytes per lane: 32 lanes, 4 rows x 4 chunks, per cycle).  The XOR
// swizzle of the 16-byte chunk index puts each cycle's accesses in distinct bank groups for both
// patterns (64 banks of 4 bytes; measured on MI355X with SQ_LDS_BANK_CONFLICT: zero conflict
// cycles for both).  d = 128 (256-byte rows): ((r & 3) << 2) | ((r >> 2) & 3).  d = 64 (two rows
// per bank row): (((r >> 1) & 1) << 2) | ((r >> 2) & 3).  Both depend on r mod 16 only and stay
// inside the row.
template <int D>
__device__ __forceinline__ int swz_b(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// A block of kBlk rows x D bf16, rows of D*2 bytes, 16-byte chunk c of row r at c ^ swz_b<D>(r).
// DMA instruction t of this wave covers rows (wave*kInstPerWave + t)*kRowsPerInst ...; rows past
// row_limit are clamped to it (the last, partial block).  Source rows are rsb bytes apart; the
// workgroup's W waves share the tile.
template <int D, int W = kWaves>
__device__ __forceinline__ void dma_tile(const __bf16* src, char* dst, int wave, int lane, int row_limit,
                                         unsigned rsb) {
  using G = Geo<D, W>;
  const char* s = (const char*)src;
#pragma unroll
  for (int t = 0; t < G::kInstPerWave; ++t) {
    const int inst = wave * G::kInstPerWave + t;
    const int r = inst * G::kRowsPerInst + lane / G::kChunksPerRow;
    const int pc = lane % G::kChunksPerRow;
    const int rr = r < row_limit ? r : row_limit;
    const unsigned off = (unsigned)rr * rsb + (unsigned)((pc ^ swz_b<D>(r)) * 16);
    __builtin_amdgcn_global_load_lds((global_cvoid*)(s + off), (lds_void*)(dst + inst * 1024), 16, 0, 0);
  }
}
template <int D>
constexpr int dma_ops() {
  return Geo<D>::kInstPerWave;
}

// Row-major operand read (A operand of X Y^T, X the tile): lane l reads row l%32 (+32*rt) of
// the tile at logical chunk 2s + l/32.  base = this lane's row address in tile 0, chunk part
// applied here.
template <int D>
__device__ __forceinline__ unsigned row_addr(unsigned tile, int row, int s, int hf) {
  return tile + row * (D * 2) + ((((2 * s + hf) ^ swz_b<D>(row))) * 16);
}

// Transposing operand read (A operand of X^T Y): lane (g = lane/16, p = lane%16) reads, for
// column tile t, the 4 rows r = 4 hf + p/4 (+8 for the high half, +16 ks) at column chunk
// 4t + 2(g%2) + (p%4)/2, byte (p%2)*8.  Each 16-lane group then holds one column of 4 rows.
template <int D>
__device__ __forceinline__ unsigned tr_addr(unsigned tile, int lane, int t, int hi) {
  const int g = lane >> 4, p = lane & 15, hf = lane >> 5;
  const int r = 4 * hf + (p >> 2) + 8 * hi;
  const int cl = 2 * (g & 1) + ((p & 3) >> 1);
  return tile + r * (D * 2) + (p & 1) * 8 + (((4 * t + cl) ^ swz_b<D>(r)) * 16);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Load 32 rows x D of a bf16 tensor (rows rs elements apart) into the B-operand layout of a
// 32x32x16 MFMA: lane l holds row l%32, elements 16s + 8(l/32) .. +7 of slice s.  Rows at or
// past `rows` are clamped; flip = 1 negates (sign bit) every element.
template <int D>
__device__ __forceinline__ void load_rows(const __bf16* base, int64_t rs, int row, int rows, int hf, int flip,
                                          bf16x8 (&f)[D / 16]) {
  const int r = row < rows ? row : rows - 1;
  const __bf16* src = base + r * rs + 8 * hf;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 raw = *(const u32x4*)(src + 16 * s);
    if (flip) raw ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    f[s] = __builtin_bit_cast(bf16x8, raw);
  }
}

// Pack a 32x32 accumulator pair (two 32-row tiles along the contraction) into the B operand of
// the following product: slice ks (16 contraction rows) takes elements 8(ks%2) .. +7 of tile
// ks/2, converted to bf16.
__device__ __forceinline__ void pack(const f32x16 (&x)[2], bf16x8 (&pb)[4]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) pb[2 * tt + (i >> 3)][i & 7] = (__bf16)x[tt][i];
}

// Store a transposed accumulator (lane = output row, 16 values of a 32-column tile t) scaled by
// `mul` to the row at element offset `off` of a float32 (or, with as_bf16, bf16) tensor.
template <int D>
__device__ __forceinline__ void store_row(void* base, int64_t off, int hf, const f32x16 (&acc)[D / 32], float mul,
                                          int as_bf16) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 v = {acc[t][4 * g4] * mul, acc[t][4 * g4 + 1] * mul, acc[t][4 * g4 + 2] * mul,
                       acc[t][4 * g4 + 3] * mul};
      const int64_t e = off + 32 * t + 8 * g4 + 4 * hf;
      if (as_bf16) {
        const __bf16 r[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *(uint64_t*)((__bf16*)base + e) = __builtin_bit_cast(uint64_t, r);
      } else {
        *(f32x4*)((float*)base + e) = v;
      }
    }
}

// Row-major A-operand products of the two 32-row tiles of a block with the wave's registers:
// acc[tt] = sum_s tile[rows 32 tt + l%32][slice s] (x) f[s].  All reads of a tile are issued
// first; each MFMA waits only for its own operand (LDS reads complete in order).
template <int D, int S>
__device__ __forceinline__ void rm_step(bf16x8 (&a)[D / 16], const bf16x8 (&f)[D / 16], f32x16& acc, IC<S>) {
  lgkm_wait<D / 16 - 1 - S>(a[S]);
  acc = mfma(a[S], f[S], S == 0 ? (f32x16){} : acc);
}
template <int D>
__device__ __forceinline__ void rowmajor_tile(unsigned tile, int row, int hf, const bf16x8 (&f)[D / 16], f32x16& acc) {
  bf16x8 a[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) a[s] = lds_read_b128<0>(row_addr<D>(tile, row, s, hf));
  [&]<int... S>(std::integer_sequence<int, S...>) { (rm_step<D>(a, f, acc, IC<S>{}), ...); }(
      std::make_integer_sequence<int, D / 16>{});
}
template <int D>
__device__ __forceinline__ void rowmajor_products(unsigned tile, int ln, int hf, const bf16x8 (&f)[D / 16],
                                                  f32x16 (&acc)[2]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) rowmajor_tile<D>(tile, 32 * tt + ln, hf, f, acc[tt]);
}

// Transposed A-operand products: acc[t] += tile^T[cols 32 t ..][rows 16 ks ..] (x) pb[ks], the
// 16 contraction rows of slice ks in the order the accumulator layout hands them over.
template <int D, int KS, int NP>
__device__ __forceinline__ void tp_step(const unsigned (&tra)[D / 32][2], const bf16x8 (&pb)[NP],
                                        f32x16 (&acc)[D / 32], int pidx, IC<KS>) {
  constexpr int kDT = D / 32, off = KS * 16 * D * 2;
  i16x4 lo[kDT], hi[kDT];
#pragma unroll
  for (int t = 0; t < kDT; ++t) {
    lo[t] = lds_read_tr<off>(tra[t][0]);
    hi[t] = lds_read_tr<off>(tra[t][1]);
  }
  [&]<int... T>(std::integer_sequence<int, T...>) {
    ((lgkm_wait<2 * (kDT - 1 - T)>(lo[T], hi[T]),
      acc[T] = mfma(__builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[T], hi[T], 0, 1, 2, 3, 4, 5, 6, 7)),
                    pb[pidx], acc[T])),
     ...);
  }(std::make_integer_sequence<int, kDT>{});
}
template <int D>
__device__ __forceinline__ void transposed_products(const unsigned (&tra)[D / 32][2], const bf16x8 (&pb)[4],
                                                    f32x16 (&acc)[D / 32]) {
  [&]<int... KS>(std::integer_sequence<int, KS...>) { (tp_step<D>(tra, pb, acc, KS, IC<KS>{}), ...); }(
      std::make_integer_sequence<int, 4>{});
}

template <int D>
__device__ __forceinline__ void tr_addrs(unsigned tile, int lane, unsigned (&tra)[D / 32][2]) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    tra[t][0] = tr_addr<D>(tile, lane, t, 0);
    tra[t][1] = tr_addr<D>(tile, lane, t, 1);
  }
}

// ---- launch parameters ------------------------------------------------------------------------
// Element (b, h, i, t) of q sits at b q[0] + h q[1] + i q[2] + t (strides in elements); likewise
// the other tensors.  LSE and D are [B*H, Nq], contiguous.
struct Strides {
  int64_t b, h, n;
};
struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dO;
  const float* lse2;  // forward LSE times log2(e), [BH, Nq] (written by row_dot)
  const float* dd;    // D = rowsum(dO * O), [BH, Nq]
  void* dq;
  void* dk;
  void* dv;
  Strides sq, sk, sv, sdo, sdq, sdk, sdv;
  int H, g_bf16;      // g_bf16: dq, dk, dv in bf16 (else float32)
  int Nq, Nk, BH;
  float c_log2;       // |scale| * log2(e)
  float scale;        // signed, for dQ and dK
  int negate;         // scale < 0: the sign is moved onto Q (dq kernel) or K (dkdv kernel)
};

// ---- D = rowsum(dO * O) --------------------------------------------------------------------
// O is float32, or bf16 when o_bf16 is set; row r of D is (b*H + h)*Nq + i.  Also writes the
// forward's LSE in log2 units, the form in which the gradient kernels use it.
template <int D>
__global__ __launch_bounds__(64) void row_dot_kernel(const __bf16* __restrict__ dO, Strides sdo,
                                                     const void* __restrict__ o, Strides so, int o_bf16,
                                                     const float* __restrict__ lse, float* __restrict__ dd,
                                                     float* __restrict__ lse2, int H, int Nq, int64_t rows) {
  constexpr int TPR = D / 4, RPB = 64 / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  float s = 0.f;
  if (row < rows) {
    const int64_t bh = row / Nq, i = row - bh * Nq, b = bh / H, h = bh - b * H;
    const int64_t oe = b * so.b + h * so.h + i * so.n + 4 * t;
    f32x4 ov;
    if (o_bf16) {
      const uint64_t raw = *(const uint64_t*)((const __bf16*)o + oe);
#pragma unroll
      for (int j = 0; j < 4; ++j) ov[j] = __builtin_bit_cast(float, (unsigned)((raw >> (16 * j)) & 0xffffu) << 16);
    } else {
      ov = *(const f32x4*)((const float*)o + oe);
    }
    const uint64_t raw = *(const uint64_t*)(dO + b * sdo.b + h * sdo.h + i * sdo.n + 4 * t);
#pragma unroll
    for (int j = 0; j < 4; ++j) s += __builtin_bit_cast(float, (unsigned)((raw >> (16 * j)) & 0xffffu) << 16) * ov[j];
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, TPR);
  if (row < rows && t == 0) {
    dd[row] = s;
    lse2[row] = lse[row] * 1.4426950408889634f;  // log2 units, once per row instead of per score
  }
}

// ---- dQ ------------------------------------------------------------------------------------
// W waves of 32 query rows each: 4 (two workgroups per CU) or, for long sequences, 8 (one
// per CU; every K/V block in LDS then serves 256 queries).
template <int D, bool CAUSAL, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(2, 2)))
void dq_kernel(BwdParams p) {
  using G = Geo<D, W>;
  constexpr int kQRows = 32 * W;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int BH = p.BH, Nq = p.Nq, Nk = p.Nk, kshift = Nk - Nq;
  // Workgroup w runs on XCD w % 8, so with BH a multiple of 8 all tiles of a head share one
  // XCD's L2.  Causal tiles go heaviest first: tiles that start together have about the same
  // length and stream the same K/V blocks in step, which keeps those blocks in L2.
  const int n_qt = (Nq + kQRows - 1) / kQRows;
  const int bh = blockIdx.x % BH, rank = blockIdx.x / BH;
  const int qt = CAUSAL ? n_qt - 1 - rank : rank;
  const int my_row = qt * kQRows + wave * 32 + ln;

  const int b = bh / p.H, h = bh - b * p.H;
  bf16x8 qf[G::kDS], dof[G::kDS];
  load_rows<D>(p.q + b * p.sq.b + h * p.sq.h, p.sq.n, my_row, Nq, hf, p.negate, qf);
  load_rows<D>(p.dO + b * p.sdo.b + h * p.sdo.h, p.sdo.n, my_row, Nq, hf, 0, dof);
  const int rc = my_row < Nq ? my_row : Nq - 1;
  const float lse2 = p.lse2[(int64_t)bh * Nq + rc];
  const float drow = p.dd[(int64_t)bh * Nq + rc];
  f32x16 acc[G::kDT];
#pragma unroll
  for (int t = 0; t < G::kDT; ++t) acc[t] = (f32x16){};

  const int n_kb = (Nk + kBlk - 1) / kBlk;
  int nblk = n_kb, j_mask = Nk / kBlk;
  if (CAUSAL) {
    const int last_row = min(Nq - 1, qt * kQRows + kQRows - 1);
    nblk = min(n_kb, (last_row + kshift) / kBlk + 1);
    j_mask = min(j_mask, (qt * kQRows + kshift) / kBlk);
  }
  const __bf16* kh = p.k + b * p.sk.b + h * p.sk.h;
  const __bf16* vh = p.v + b * p.sv.b + h * p.sv.h;
  const unsigned ksb = (unsigned)(p.sk.n * 2), vsb = (unsigned)(p.sv.n * 2);
  const unsigned base = (unsigned)(uintptr_t)(lds_void*)smem;
  const int my_pos = my_row + kshift;

  // Buffer bf holds K at smem + 2 bf kTile and V at smem + (2 bf + 1) kTile.
  dma_tile<D, W>(kh, smem, wave, lane, Nk - 1, ksb);
  dma_tile<D, W>(vh, smem + G::kTile, wave, lane, Nk - 1, vsb);
  for (int j = 0; j < nblk; ++j) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // block j has landed for every wave; block j-1 is done
    const int bf = j & 1;
    if (j + 1 < nblk) {
      const int nb = (j + 1) & 1;
      const int limit = Nk - 1 - (j + 1) * kBlk;
      dma_tile<D, W>(kh + (int64_t)(j + 1) * kBlk * p.sk.n, smem + 2 * nb * G::kTile, wave, lane, limit, ksb);
      dma_tile<D, W>(vh + (int64_t)(j + 1) * kBlk * p.sv.n, smem + (2 * nb + 1) * G::kTile, wave, lane, limit, vsb);
    }
    const unsigned kt_base = base + 2 * bf * G::kTile, vt_base = kt_base + G::kTile;
    f32x16 s[2], dp[2];
    rowmajor_products<D>(kt_base, ln, hf, qf, s);
    rowmajor_products<D>(vt_base, ln, hf, dof, dp);
    const int key0 = j * kBlk;
    if (j >= j_mask) {
      int lim = Nk - 1 - key0 - 4 * hf;
      if (CAUSAL) lim = min(lim, my_pos - key0 - 4 * hf);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kt + 8 * (i >> 2) + (i & 3) > lim) s[kt][i] = -__builtin_inff();
    }
    f32x16 ds[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], p.c_log2, -lse2));
        ds[kt][i] = pr * (dp[kt][i] - drow);
      }
    bf16x8 dsb[4];
    pack(ds, dsb);
    unsigned tra[G::kDT][2];
    tr_addrs<D>(kt_base, lane, tra);
    transposed_products<D>(tra, dsb, acc);
  }
  wait_vmcnt<0>();
  if (my_row < Nq)
    store_row<D>(p.dq, b * p.sdq.b + h * p.sdq.h + my_row * p.sdq.n, hf, acc, p.scale, p.g_bf16);
}

// ---- dK, dV -------------------------------------------------------------------------------
// At one wave per SIMD nothing else hides an LDS round trip, so every LDS read is issued ahead
// of the MFMA that consumes it (see the pipelined step below).  Waits count the reads issued
// after the one needed (LDS reads complete in order); counts above the 4-bit field are clamped,
// which only waits longer.
template <int N>
constexpr int kClampLgkm = N < 15 ? N : 15;

// The lane-dependent part of every LDS address of the dV/dK kernel, computed once: the
// row-major reads of row l%32 (one register per d slice) and the transposed reads (one per d
// tile and half), both for tile 0.  Each block moves them to its buffer with one add per
// register; the Q/dO tile, the 32-row tile and the contraction slice go into the instructions'
// immediate offsets (the swizzles depend on the row mod 16 only, so those displacements are
// plain byte offsets, and within one buffer they fit the 16-bit field).
template <int D>
struct LaneAddrs {
  unsigned row[D / 16];
  unsigned tr[D / 32][2];
  __device__ __forceinline__ void init(unsigned base, int lane) {
    const int ln = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) row[s] = row_addr<D>(base, ln, s, hf);
    tr_addrs<D>(base, lane, tr);
  }
  __device__ __forceinline__ void shift(const LaneAddrs& a, unsigned by) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) row[s] = a.row[s] + by;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) tr[t][0] = a.tr[t][0] + by, tr[t][1] = a.tr[t][1] + by;
  }
};
template <int D, int OFF>
__device__ __forceinline__ void issue_rows(const unsigned (&ra)[D / 16], bf16x8 (&a)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) a[s] = lds_read_b128<OFF>(ra[s]);
}
// acc = sum_s a[s] (x) f[s]; AFTER reads were issued after a[] (their order is a, then those).
template <int D, int AFTER, int S>
__device__ __forceinline__ void rows_mfma(bf16x8 (&a)[D / 16], const bf16x8 (&f)[D / 16], f32x16& acc, IC<S>) {
  lgkm_wait<kClampLgkm<AFTER + D / 16 - 1 - S>>(a[S]);
  acc = mfma(a[S], f[S], S == 0 ? (f32x16){} : acc);
}
template <int D, int AFTER>
__device__ __forceinline__ void rows_product(bf16x8 (&a)[D / 16], const bf16x8 (&f)[D / 16], f32x16& acc) {
  [&]<int... S>(std::integer_sequence<int, S...>) { (rows_mfma<D, AFTER>(a, f, acc, IC<S>{}), ...); }(
      std::make_integer_sequence<int, D / 16>{});
}

// Transposed operand reads of contraction slice KS for every d tile (2 per tile).
template <int D, int KS>
struct TrReads {
  i16x4 lo[D / 32], hi[D / 32];
  template <int BOFF>
  __device__ __forceinline__ void issue(const unsigned (&tra)[D / 32][2]) {
    constexpr int off = BOFF + KS * 16 * D * 2;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      lo[t] = lds_read_tr<off>(tra[t][0]);
      hi[t] = lds_read_tr<off>(tra[t][1]);
    }
  }
};

template <int OFF>
__device__ __forceinline__ f32x4 lds_read_f32x4(unsigned addr) {
  f32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// dV/dK products of one 32-query tile are deferred into the next step, where they run during
// that step's softmax arithmetic (one wave per SIMD: no other wave overlaps them).  Only the
// tile's P and dS (bf16) cross steps in registers; the transposed dO and Q operands are read
// again from LDS in the next step, which is why the query blocks are triple-buffered: the
// buffer of block j is refilled only after block j+1's first step has read it.
struct Pending {
  bf16x8 pb[2], dsb[2];
};

// The dV/dK products of tile TT of a block, all at once (the last tile's, after the loop):
// dO^T and Q^T sit at byte offsets DO_OFF / Q_OFF from the addresses tra_do / tra_q;
// dV^T += dO^T P, dK^T += Q^T dS.  All transposed reads go out first; MFMA m of the 4 kDT waits
// for its own pair.
template <int D, int TT>
struct DeferredReads {
  static constexpr int kDT = D / 32, kReads = 8 * kDT;
  TrReads<D, 2 * TT> do0, q0;
  TrReads<D, 2 * TT + 1> do1, q1;
  template <int DO_OFF, int Q_OFF>
  __device__ __forceinline__ void issue(const unsigned (&tra_do)[kDT][2], const unsigned (&tra_q)[kDT][2]) {
    do0.template issue<DO_OFF>(tra_do);
    do1.template issue<DO_OFF>(tra_do);
    q0.template issue<Q_OFF>(tra_q);
    q1.template issue<Q_OFF>(tra_q);
  }
  template <int M>
  __device__ __forceinline__ void mfma_m(const Pending& pd, f32x16 (&dv)[kDT], f32x16 (&dk)[kDT]) {
    constexpr int t = M % kDT, part = M / kDT;
    // reads issued after this MFMA's pair: the rest of its group and the later groups
    constexpr int after = kReads - (part * 2 * kDT + 2 * t + 2);
    auto op = [](const i16x4& lo, const i16x4& hi) {
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    if constexpr (part == 0) {
      lgkm_wait<kClampLgkm<after>>(do0.lo[t], do0.hi[t]);
      dv[t] = mfma(op(do0.lo[t], do0.hi[t]), pd.pb[0], dv[t]);
    } else if constexpr (part == 1) {
      lgkm_wait<kClampLgkm<after>>(do1.lo[t], do1.hi[t]);
      dv[t] = mfma(op(do1.lo[t], do1.hi[t]), pd.pb[1], dv[t]);
    } else if constexpr (part == 2) {
      lgkm_wait<kClampLgkm<after>>(q0.lo[t], q0.hi[t]);
      dk[t] = mfma(op(q0.lo[t], q0.hi[t]), pd.dsb[0], dk[t]);
    } else {
      lgkm_wait<kClampLgkm<after>>(q1.lo[t], q1.hi[t]);
      dk[t] = mfma(op(q1.lo[t], q1.hi[t]), pd.dsb[1], dk[t]);
    }
  }
};

// P and dS of score i of this lane (query row 32 TT + 8 (i/4) + 4 hf + i%4 of the block).
template <int I>
__device__ __forceinline__ void score(const f32x16& s, const f32x16& dp, const f32x4 (&lv)[4], const f32x4 (&dvv)[4],
                                      float c_log2, Pending& cur) {
  const float sv = s[I];
  const float l2 = lv[I >> 2][I & 3];
  const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c_log2, -l2));
  cur.pb[I >> 3][I & 7] = (__bf16)pr;
  cur.dsb[I >> 3][I & 7] = (__bf16)(pr * (dp[I] - dvv[I >> 2][I & 3]));
}

// Scores I0 .. I0 + N - 1.
template <int I0, int N>
__device__ __forceinline__ void scores(const f32x16& s, const f32x16& dp, const f32x4 (&lv)[4], const f32x4 (&dvv)[4],
                                       float c_log2, Pending& cur) {
  if constexpr (N > 0) {
    score<I0>(s, dp, lv, dvv, c_log2, cur);
    scores<I0 + 1, N - 1>(s, dp, lv, dvv, c_log2, cur);
  }
}

// ---- the software-pipelined step ----------------------------------------------------------
// Step g (query tile g, 32 rows) runs three things at once: the softmax arithmetic of tile g (its
// S and dP were computed in step g - 1), the S = Q K^T and dP = dO V^T chains of tile g + 1, and
// the dV/dK products of tile g - 1.  Both product sets go to the MFMA pipe between the scores,
// so the pipe has independent work while the VALU turns S and dP into P and dS.  With D/8 chain
// MFMAs and D/8 deferred MFMAs per step, step g pairs chain MFMA i with deferred MFMA i; the
// operands of pair i are one row-major read and two transposed reads, issued kLookahead pairs
// ahead of their use.
constexpr int kLookahead = 4;

struct PairOps {
  bf16x8 c;
  i16x4 lo, hi;
};
// Operands of pair I: chain MFMA I reads slice I of the next tile's Q rows (I < D/16), then of
// its dO rows; deferred MFMA I (d tile t = I mod D/32, part I / (D/32)) reads dO^T (parts 0, 1)
// or Q^T (parts 2, 3) of the previous tile, contraction slice 2 TTP + part mod 2.
template <int D, int TTN, int TTP, int I>
__device__ __forceinline__ void issue_pair(const LaneAddrs<D>& nat, const LaneAddrs<D>& pat, PairOps& o) {
  constexpr int kDS = D / 16, kDT = D / 32, kTile = Geo<D>::kTile, kRowOff = 32 * TTN * D * 2;
  if constexpr (I < kDS)
    o.c = lds_read_b128<kRowOff>(nat.row[I]);
  else
    o.c = lds_read_b128<kTile + kRowOff>(nat.row[I - kDS]);
  constexpr int t = I % kDT, part = I / kDT;
  constexpr int off = (part < 2 ? kTile : 0) + (2 * TTP + (part & 1)) * 16 * D * 2;
  o.lo = lds_read_tr<off>(pat.tr[t][0]);
  o.hi = lds_read_tr<off>(pat.tr[t][1]);
}

// Step TT (0 or 1) of a query block: scores of this block's tile TT from s_in / dp_in (P and dS
// into cur; rows' LSE and D at rvr); chains of the next tile (its Q rows at nat, dO one tile up)
// into s_out / dp_out; dV/dK products of the previous tile (P and dS in prev, Q^T at pat, dO^T
// one tile up).  The next and the previous tile both sit at position 1 - TT of their blocks.
template <int D, bool CAUSAL, int TT>
__device__ __forceinline__ void step(bool masked, const LaneAddrs<D>& nat, const LaneAddrs<D>& pat, unsigned rvr,
                                     int hf, const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16], int q0, int Nq,
                                     int my_key, int kshift, float c_log2, const Pending& prev, Pending& cur,
                                     const f32x16& s_in, const f32x16& dp_in, f32x16& s_out, f32x16& dp_out,
                                     f32x16 (&dv)[D / 32], f32x16 (&dk)[D / 32]) {
  constexpr int kDS = D / 16, kDT = D / 32, kNP = D / 8, kSPP = 16 / kNP;
  constexpr int kTTN = 1 - TT, kTTP = 1 - TT;
  f32x4 lv[4], dvv[4];
  [&]<int... G>(std::integer_sequence<int, G...>) {
    ((lv[G] = lds_read_f32x4<(32 * TT + 8 * G) * 4>(rvr), dvv[G] = lds_read_f32x4<256 + (32 * TT + 8 * G) * 4>(rvr)),
     ...);
  }(std::make_integer_sequence<int, 4>{});
  PairOps ops[kNP];
  [&]<int... P>(std::integer_sequence<int, P...>) {
    (issue_pair<D, kTTN, kTTP, P>(nat, pat, ops[P]), ...);
  }(std::make_integer_sequence<int, (kLookahead < kNP ? kLookahead : kNP)>{});
  // Blocks on the causal diagonal or past the last query: hidden scores get -inf (P = 0).
  f32x16 s = s_in;
  if (masked) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qg = q0 + 32 * TT + 8 * (i >> 2) + 4 * hf + (i & 3);
      const bool vis = qg < Nq && (!CAUSAL || my_key <= qg + kshift);
      s[i] = vis ? s[i] : -__builtin_inff();
    }
  }
  auto op = [](const i16x4& lo, const i16x4& hi) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (([&] {
       if constexpr (I + kLookahead < kNP) issue_pair<D, kTTN, kTTP, I + kLookahead>(nat, pat, ops[I + kLookahead]);
       // LDS reads complete in order: count the reads issued after the one needed
       constexpr int issued = I + kLookahead + 1 < kNP ? I + kLookahead + 1 : kNP;
       lgkm_wait<kClampLgkm<3 * (issued - I - 1) + 2>>(ops[I].c);
       if constexpr (I == 0) {
         // the row values went out before every pair: they have landed
#pragma unroll
         for (int g = 0; g < 4; ++g) asm volatile("" : "+v"(lv[g]), "+v"(dvv[g]));
       }
       if constexpr (I < kDS)
         s_out = mfma(ops[I].c, kf[I], I == 0 ? (f32x16){} : s_out);
       else
         dp_out = mfma(ops[I].c, vf[I - kDS], I == kDS ? (f32x16){} : dp_out);
       scores<I * kSPP, kSPP>(s, dp_in, lv, dvv, c_log2, cur);
       // Keep the scores in this pair: their only users are the next step's MFMAs, and without
       // the tie they would sink past the barrier that follows the step.
       if constexpr (((I + 1) * kSPP) % 2 == 0) {
         constexpr int v = ((I + 1) * kSPP - 1) >> 3;
         asm volatile("" : "+v"(cur.pb[v]), "+v"(cur.dsb[v]));
       }
       lgkm_wait<kClampLgkm<3 * (issued - I - 1)>>(ops[I].lo, ops[I].hi);
       constexpr int t = I % kDT, part = I / kDT;
       if constexpr (part == 0)
         dv[t] = mfma(op(ops[I].lo, ops[I].hi), prev.pb[0], dv[t]);
       else if constexpr (part == 1)
         dv[t] = mfma(op(ops[I].lo, ops[I].hi), prev.pb[1], dv[t]);
       else if constexpr (part == 2)
         dk[t] = mfma(op(ops[I].lo, ops[I].hi), prev.dsb[0], dk[t]);
       else
         dk[t] = mfma(op(ops[I].lo, ops[I].hi), prev.dsb[1], dk[t]);
     }()),
     ...);
  }(std::make_integer_sequence<int, kNP>{});
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(BwdParams p) {
  using G = Geo<D>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int BH = p.BH, Nq = p.Nq, Nk = p.Nk, kshift = Nk - Nq;
  // Key tile kb sees the query blocks from about kb on (causal), so ascending kb is already
  // heaviest first; see dq_kernel for the XCD placement.
  const int bh = blockIdx.x % BH, kb = blockIdx.x / BH;
  const int tile_key0 = kb * kRows;
  const int my_key = tile_key0 + wave * 32 + ln;

  const int b = bh / p.H, h = bh - b * p.H;
  bf16x8 kf[G::kDS], vf[G::kDS];
  load_rows<D>(p.k + b * p.sk.b + h * p.sk.h, p.sk.n, my_key, Nk, hf, p.negate, kf);
  load_rows<D>(p.v + b * p.sv.b + h * p.sv.h, p.sv.n, my_key, Nk, hf, 0, vf);
  f32x16 dv[G::kDT], dk[G::kDT];
#pragma unroll
  for (int t = 0; t < G::kDT; ++t) dv[t] = dk[t] = (f32x16){};

  // Query blocks [jb, n_qb): with the causal mask a query sees this tile's keys only from
  // position tile_key0 on.  Blocks whose first query sits before the tile's last key, and the
  // last partial block, take the masked path.
  const int n_qb = (Nq + kBlk - 1) / kBlk;
  int jb = 0;
  if (CAUSAL) jb = max(0, tile_key0 - kshift) / kBlk;
  const __bf16* qh = p.q + b * p.sq.b + h * p.sq.h;
  const __bf16* doh = p.dO + b * p.sdo.b + h * p.sdo.h;
  const unsigned qsb = (unsigned)(p.sq.n * 2), dosb = (unsigned)(p.sdo.n * 2);
  const float* lh = p.lse2 + (int64_t)bh * Nq;
  const float* dh = p.dd + (int64_t)bh * Nq;
  const unsigned base = (unsigned)(uintptr_t)(lds_void*)smem;
  // LDS: buffer u (0..2) holds Q at smem + 2u kTile, dO at smem + (2u + 1) kTile; the rows'
  // LSE and D follow the six tiles (64 floats each, 512 bytes per buffer).
  char* rowvals = smem + 6 * G::kTile;
  auto load_block = [&](int jq, int buf) {
    const int limit = Nq - 1 - jq * kBlk;
    dma_tile<D>(qh + (int64_t)jq * kBlk * p.sq.n, smem + 2 * buf * G::kTile, wave, lane, limit, qsb);
    dma_tile<D>(doh + (int64_t)jq * kBlk * p.sdo.n, smem + (2 * buf + 1) * G::kTile, wave, lane, limit, dosb);
    // The rows' LSE (wave 1) and D (wave 2): a load instruction costs the issuing wave tens of
    // cycles, and every wave waits for the slowest at the next barrier.
    if (wave == 1 || wave == 2) {
      const int r = lane < limit ? lane : limit;
      const float* src = (wave == 1 ? lh : dh) + (int64_t)jq * kBlk + r;
      __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)(rowvals + buf * 512 + (wave - 1) * 256), 4, 0,
                                       0);
    }
  };
  // The first step's deferred products read buffer 2 with P = dS = 0; zero it so that those
  // products add exactly nothing (uninitialised LDS could hold NaN patterns).
  {
    u32x4* z = (u32x4*)(smem + 4 * G::kTile);
#pragma unroll
    for (int i = 0; i < 2 * G::kTile / 16 / kThreads; ++i) z[tid + i * kThreads] = (u32x4){};
  }
  Pending pend0, pend1;  // tile 0 / tile 1 of the latest block
#pragma unroll
  for (int i = 0; i < 2; ++i) pend1.pb[i] = pend1.dsb[i] = (bf16x8){};
  LaneAddrs<D> lo;
  lo.init(base, lane);
  const unsigned rv0 = base + 6 * G::kTile + 16 * hf;
  const float c = p.c_log2;
  // S and dP of the tile whose scores the next step computes: [0] for a block's first tile,
  // [1] for its second.
  f32x16 sa[2], dpa[2];
  if (jb < n_qb) {
    load_block(jb, 0);
    if (jb + 1 < n_qb) load_block(jb + 1, 1);
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // blocks jb, jb + 1 and the zeroed buffer 2 are in place
    bf16x8 qa[G::kDS], oa[G::kDS];
    issue_rows<D, 0>(lo.row, qa);
    issue_rows<D, G::kTile>(lo.row, oa);
    rows_product<D, G::kDS>(qa, kf, sa[0]);
    rows_product<D, 0>(oa, vf, dpa[0]);
  }
  // Block jb + i sits in buffer i mod 3.  Step 0 of block jq reads its own buffer and the
  // previous block's; step 1 reads its own and the next block's.  Between the two steps every
  // wave has finished with the previous block, which is refilled with block jq + 2.
  int pbuf = 2;  // buffer of the tile pending after the loop (the zeroed one if there was no block)
  for (int jq = jb; jq < n_qb; ++jq) {
    const int u = (jq - jb) % 3, un = u == 2 ? 0 : u + 1, up = u == 0 ? 2 : u - 1;
    LaneAddrs<D> at, pat;
    at.shift(lo, (unsigned)(2 * u * G::kTile));
    pat.shift(lo, (unsigned)(2 * up * G::kTile));
    const unsigned rvr = rv0 + u * 512;
    const int q0 = jq * kBlk;
    const bool masked = (CAUSAL && q0 + kshift < tile_key0 + kRows - 1) || q0 + kBlk > Nq;
    step<D, CAUSAL, 0>(masked, at, pat, rvr, hf, kf, vf, q0, Nq, my_key, kshift, c, pend1, pend0, sa[0], dpa[0], sa[1],
                       dpa[1], dv, dk);
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // block jq + 1 has landed; block jq - 1's buffer is free
    if (jq + 2 < n_qb) load_block(jq + 2, up);
    // After the last block the chains read a stale buffer; their S and dP are never used.
    LaneAddrs<D> nat;
    nat.shift(lo, (unsigned)(2 * un * G::kTile));
    step<D, CAUSAL, 1>(masked, nat, at, rvr, hf, kf, vf, q0, Nq, my_key, kshift, c, pend0, pend1, sa[1], dpa[1], sa[0],
                       dpa[0], dv, dk);
    pbuf = u;
  }
  // the last tile's dV/dK products
  {
    LaneAddrs<D> pat;
    pat.shift(lo, (unsigned)(2 * pbuf * G::kTile));
    DeferredReads<D, 1> pr;
    pr.template issue<G::kTile, 0>(pat.tr, pat.tr);
    [&]<int... M>(std::integer_sequence<int, M...>) { (pr.template mfma_m<M>(pend1, dv, dk), ...); }(
        std::make_integer_sequence<int, 4 * G::kDT>{});
  }
  wait_vmcnt<0>();
  if (my_key < Nk) {
    store_row<D>(p.dv, b * p.sdv.b + h * p.sdv.h + my_key * p.sdv.n, hf, dv, 1.f, p.g_bf16);
    store_row<D>(p.dk, b * p.sdk.b + h * p.sdk.h + my_key * p.sdk.n, hf, dk, p.scale, p.g_bf16);
  }
}

constexpr int kRowValsBytes = 3 * 512;
// dkdv: three Q/dO buffer pairs and their row values
template <int D>
constexpr int kDkdvLds = 6 * Geo<D>::kTile + kRowValsBytes;

// ---- dK/dV with the two waves of each SIMD in two roles -------------------------------------
// 8 waves, 128 keys per workgroup (256 registers per wave, two waves per SIMD).  Waves g and
// g + 4 share a SIMD and the 32 keys 32 g .. 32 g + 31:
//  * wave g keeps K: S = Q K^T, P = exp2(c S - LSE2) (masked scores give 0), P to LDS as bf16
//    for its partner, dV^T += dO^T P;
//  * wave g + 4 keeps V: dP = dO V^T; one block later, with the partner's P of that block,
//    dS = P (dP - D) and dK^T += Q^T dS.
// Each wave runs two of the four products per 64-query block, and while one wave of a SIMD
// turns scores into P or dS the other keeps the matrix unit busy.  One barrier per block: it
// publishes the block's P and releases the buffers of the block before, which is refilled with
// the block two ahead (three Q/dO buffers, since Q of a block is read again one block later).
// P reaches dS rounded to bf16 (the form it takes in the dV product as well).
// Causal problems take the role-split kernel (same-box A/B, medians, against dkdv_kernel: B=1
// H=32 N=16384 -2.8% per backward call, B=2 H=16 N=4096 -5.7%, B=8 H=16 N=2048 -5.2%).  Without
// the mask the compiler keeps more lane addresses live across its loop and spills at d = 128,
// so non-causal problems keep dkdv_kernel.
template <bool CAUSAL>
constexpr bool kDkdvRoleSplit = CAUSAL;
constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kPexBytes = 2 * 4 * 4096;  // 2 blocks x 4 key groups x (4 x 64 lanes x 16 bytes)
template <int D>
constexpr int kDkdvSplitLds = 6 * Geo<D>::kTile + kRowValsBytes + kPexBytes;

// Query row (within a 64-query block) of accumulator element i of 32-query tile tt, for the lane
// half hf: the row order of a 32x32 accumulator.
__device__ __forceinline__ int query_of(int tt, int i, int hf) {
  return 32 * tt + 8 * (i >> 2) + 4 * hf + (i & 3);
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kSplitThreads, kSplitThreads), amdgpu_waves_per_eu(2, 2)))
void dkdv_split_kernel(BwdParams p) {
  using G = Geo<D, kSplitWaves>;
  constexpr int kDT = D / 32;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const int kg = wave & 3, role = wave >> 2;  // role 0 keeps K (P, dV), role 1 keeps V (dS, dK)
  const int BH = p.BH, Nq = p.Nq, Nk = p.Nk, kshift = Nk - Nq;
  // ascending kb is heaviest first (causal), as in dkdv_kernel
  const int bh = blockIdx.x % BH, kb = blockIdx.x / BH;
  const int tile_key0 = kb * kRows;
  const int my_key = tile_key0 + kg * 32 + ln;
  const int b = bh / p.H, h = bh - b * p.H;

  bf16x8 kvf[D / 16];
  if (role == 0)
    load_rows<D>(p.k + b * p.sk.b + h * p.sk.h, p.sk.n, my_key, Nk, hf, p.negate, kvf);
  else
    load_rows<D>(p.v + b * p.sv.b + h * p.sv.h, p.sv.n, my_key, Nk, hf, 0, kvf);
  f32x16 acc[kDT];  // dV^T (role 0) or dK^T (role 1) of this lane's key
#pragma unroll
  for (int t = 0; t < kDT; ++t) acc[t] = (f32x16){};

  const int n_qb = (Nq + kBlk - 1) / kBlk;
  int jb = 0;
  if (CAUSAL) jb = max(0, tile_key0 - kshift) / kBlk;
  const __bf16* qh = p.q + b * p.sq.b + h * p.sq.h;
  const __bf16* doh = p.dO + b * p.sdo.b + h * p.sdo.h;
  const unsigned qsb = (unsigned)(p.sq.n * 2), dosb = (unsigned)(p.sdo.n * 2);
  const float* lh = p.lse2 + (int64_t)bh * Nq;
  const float* dh = p.dd + (int64_t)bh * Nq;
  const unsigned base = (unsigned)(uintptr_t)(lds_void*)smem;
  // LDS: buffer u (0..2) holds Q at 2u kTile and dO at (2u + 1) kTile; then the rows' LSE2 and D
  // (512 bytes per buffer); then P of two blocks, per key group 4 slices x 64 lanes x 16 bytes.
  char* rowvals = smem + 6 * G::kTile;
  char* pex = rowvals + kRowValsBytes;
  auto load_block = [&](int jq, int buf) {
    const int limit = Nq - 1 - jq * kBlk;
    dma_tile<D, kSplitWaves>(qh + (int64_t)jq * kBlk * p.sq.n, smem + 2 * buf * G::kTile, wave, lane, limit, qsb);
    dma_tile<D, kSplitWaves>(doh + (int64_t)jq * kBlk * p.sdo.n, smem + (2 * buf + 1) * G::kTile, wave, lane, limit,
                             dosb);
    // the rows' LSE2 (wave 5) and D (wave 6): role-1 waves, which have less arithmetic
    if (wave == 5 || wave == 6) {
      const int r = lane < limit ? lane : limit;
      const float* src = (wave == 5 ? lh : dh) + (int64_t)jq * kBlk + r;
      __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)(rowvals + buf * 512 + (wave - 5) * 256), 4, 0,
                                       0);
    }
  };
  if (jb < n_qb) {
    load_block(jb, 0);
    if (jb + 1 < n_qb) load_block(jb + 1, 1);
    wait_vmcnt<0>();
    __syncthreads();
  }
  const float c = p.c_log2;
  f32x16 dpp[2];  // role 1: dP of the block before
  // role 1, for the block in buffer ub whose P sits in exchange slot par: dS and dK^T += Q^T dS
  // role 1, for the block in buffer ub whose P sits in exchange slot par: dS = P (dP - D) and
  // dK^T += Q^T dS, tile by tile; with `next` >= 0 the dP chain of the following block (dO in
  // buffer next) goes out after each tile's dK slices, into that tile's dP registers.
  // LDS operand addresses: this lane's part for buffer 0, computed once; a buffer's are these
  // plus its offset (one add per register), the 32-row tile an immediate offset.
  LaneAddrs<D> la;
  la.init(base, lane);
  auto ds_dk = [&](int ub, int par, int next) {
    const bf16x8* pr = (const bf16x8*)(pex + (par * 4 + kg) * 4096);
    const float* dvals = (const float*)(rowvals + ub * 512 + 256);
    LaneAddrs<D> aq, ado;
    aq.shift(la, (unsigned)(2 * ub * G::kTile));
    if (next >= 0) ado.shift(la, (unsigned)((2 * next + 1) * G::kTile));
    bf16x8 dsb[4];
    auto tile_ds = [&]<int TT>(IC<TT>) {
      const bf16x8 p0 = pr[(2 * TT) * 64 + lane], p1 = pr[(2 * TT + 1) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = (float)(i < 8 ? p0[i & 7] : p1[i & 7]);
        dsb[2 * TT + (i >> 3)][i & 7] = (__bf16)(pv * (dpp[TT][i] - dvals[query_of(TT, i, hf)]));
      }
      tp_step<D>(aq.tr, dsb, acc, 2 * TT, IC<2 * TT>{});  // dK^T += Q^T dS
      tp_step<D>(aq.tr, dsb, acc, 2 * TT + 1, IC<2 * TT + 1>{});
      if (next >= 0) {  // dP = dO V^T of the next block, tile TT
        bf16x8 a[D / 16];
        issue_rows<D, 32 * TT * D * 2>(ado.row, a);
        rows_product<D, 0>(a, kvf, dpp[TT]);
      }
    };
    tile_ds(IC<0>{});
    tile_ds(IC<1>{});
  };
  // The role is fixed per wave, so each role runs its own copy of the block loop (same barriers):
  // values one role carries across blocks then take no registers in the other's code.
  if (role == 0) {
    for (int jq = jb; jq < n_qb; ++jq) {
      const int u = (jq - jb) % 3, up = u == 0 ? 2 : u - 1;
      const int par = (jq - jb) & 1;
      const int q0 = jq * kBlk;
      const bool masked = (CAUSAL && q0 + kshift < tile_key0 + kRows - 1) || q0 + kBlk > Nq;
      // S of both 32-query tiles first (independent chains), then per tile: P, its half of the
      // exchange, and its two dV^T slices, so that tile 1's exponentials run beside tile 0's MFMAs.
      LaneAddrs<D> aq, ado;
      aq.shift(la, (unsigned)(2 * u * G::kTile));
      ado.shift(la, (unsigned)((2 * u + 1) * G::kTile));
      f32x16 sc[2];
      {
        bf16x8 a[D / 16];  // S = Q K^T, tile 0 then tile 1
        issue_rows<D, 0>(aq.row, a);
        rows_product<D, 0>(a, kvf, sc[0]);
        issue_rows<D, 32 * D * 2>(aq.row, a);
        rows_product<D, 0>(a, kvf, sc[1]);
      }
      const float* lv = (const float*)(rowvals + u * 512);
      bf16x8* pw = (bf16x8*)(pex + (par * 4 + kg) * 4096);
      bf16x8 pb[4];
      auto tile_p = [&]<int TT>(IC<TT>) {
        if (masked) {  // hidden scores get -inf (P = 0)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qg = q0 + query_of(TT, i, hf);
            const bool vis = qg < Nq && (!CAUSAL || my_key <= qg + kshift);
            sc[TT][i] = vis ? sc[TT][i] : -__builtin_inff();
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pb[2 * TT + (i >> 3)][i & 7] =
              (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[TT][i], c, -lv[query_of(TT, i, hf)]));
        pw[(2 * TT) * 64 + lane] = pb[2 * TT];
        pw[(2 * TT + 1) * 64 + lane] = pb[2 * TT + 1];
        tp_step<D>(ado.tr, pb, acc, 2 * TT, IC<2 * TT>{});  // dV^T += dO^T P
        tp_step<D>(ado.tr, pb, acc, 2 * TT + 1, IC<2 * TT + 1>{});
      };
      tile_p(IC<0>{});
      tile_p(IC<1>{});
      wait_vmcnt<0>();
      __syncthreads();  // P of block jq is in LDS; block jq + 1 has landed; block jq - 1 is done with
      if (jq + 2 < n_qb) load_block(jq + 2, up);
    }
  } else {
    for (int jq = jb; jq < n_qb; ++jq) {
      const int u = (jq - jb) % 3, up = u == 0 ? 2 : u - 1;
      const int par = (jq - jb) & 1;
      if (jq > jb) {
        ds_dk(up, par ^ 1, u);  // block jq - 1, then dP = dO V^T of block jq
      } else {
        LaneAddrs<D> ado;
        ado.shift(la, (unsigned)((2 * u + 1) * G::kTile));
        bf16x8 a[D / 16];
        issue_rows<D, 0>(ado.row, a);
        rows_product<D, 0>(a, kvf, dpp[0]);
        issue_rows<D, 32 * D * 2>(ado.row, a);
        rows_product<D, 0>(a, kvf, dpp[1]);
      }
      wait_vmcnt<0>();
      __syncthreads();  // (the partner's side of the same barrier)
      if (jq + 2 < n_qb) load_block(jq + 2, up);
    }
    if (jb < n_qb) ds_dk((n_qb - 1 - jb) % 3, (n_qb - 1 - jb) & 1, -1);
  }
  wait_vmcnt<0>();
  if (my_key < Nk) {
    if (role == 0)
      store_row<D>(p.dv, b * p.sdv.b + h * p.sdv.h + my_key * p.sdv.n, hf, acc, 1.f, p.g_bf16);
    else
      store_row<D>(p.dk, b * p.sdk.b + h * p.sdk.h + my_key * p.sdk.n, hf, acc, p.scale, p.g_bf16);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const BwdParams& p, const void* o, Strides so, int o_bf16, const float* lse, float* dd,
                      float* lse2, hipStream_t s) {
  using G = Geo<D>;
  hipError_t e;
  // dynamic-LDS limits first, so that a failure leaves nothing half launched
  static std::atomic<unsigned long long> done_dq4{0}, done_dq8{0}, done_dkdv{0};
  if ((e = raise_lds_limit((const void*)dq_kernel<D, CAUSAL, 4>, G::kLds, done_dq4)) != hipSuccess) return e;
  if ((e = raise_lds_limit((const void*)dq_kernel<D, CAUSAL, 8>, G::kLds, done_dq8)) != hipSuccess) return e;
  if constexpr (kDkdvRoleSplit<CAUSAL>) {
    if ((e = raise_lds_limit((const void*)dkdv_split_kernel<D, CAUSAL>, kDkdvSplitLds<D>, done_dkdv)) != hipSuccess)
      return e;
  } else {
    if ((e = raise_lds_limit((const void*)dkdv_kernel<D, CAUSAL>, kDkdvLds<D>, done_dkdv)) != hipSuccess) return e;
  }
  const int64_t rows = (int64_t)p.BH * p.Nq;
  constexpr int rpb = 64 / (D / 4);
  hipLaunchKernelGGL(row_dot_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(64), 0, s, p.dO, p.sdo, o, so,
                     o_bf16, lse, dd, lse2, p.H, p.Nq, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 8-wave dq workgroups for long sequences with more than one such workgroup per CU (causal:
  // with exactly one per CU, nothing evens out the unequal causal tiles, and 4-wave workgroups,
  // two per CU, are faster: B=1 H=8 N=8192 and B=1 H=4 N=16384 -10% per backward call in a
  // same-box A/B); without the mask one per CU suffices.
  const int64_t big_q = (int64_t)p.BH * ((p.Nq + 255) / 256);
  const bool dq8 = CAUSAL ? (p.Nq > 4096 && big_q > 256) : (p.Nq >= 4096 && big_q >= 256);
  const unsigned gq = (unsigned)(dq8 ? big_q : (int64_t)p.BH * ((p.Nq + kRows - 1) / kRows));
  const unsigned gk = (unsigned)((int64_t)p.BH * ((p.Nk + kRows - 1) / kRows));
  if (dq8)
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL, 8>), dim3(gq), dim3(512), G::kLds, s, p);
  else
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL, 4>), dim3(gq), dim3(kThreads), G::kLds, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (kDkdvRoleSplit<CAUSAL>)
    hipLaunchKernelGGL((dkdv_split_kernel<D, CAUSAL>), dim3(gk), dim3(kSplitThreads), kDkdvSplitLds<D>, s, p);
  else
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(gk), dim3(kThreads), kDkdvLds<D>, s, p);
  return hipGetLastError();
}

}  // namespace

extern "C" __attribute__((visibility("hidden"))) void mifa_record_hip_error(int e);

extern "C" int64_t mifa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq) {
  if (B < 1 || H < 1 || Nq < 1 || B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31)) return 0;
  return B * H * Nq * 8;  // D, then LSE in log2 units
}

namespace {

// Argument checks and launch shared by both entry points.  st: (batch, head, row) strides in
// elements of q, k, v, o, dO, dq, dk, dv.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
            void* dk, void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, const int64_t* st,
            int o_bf16, int g_bf16, int causal, float scale, void* workspace, int64_t workspace_bytes,
            void* stream) {
  const int64_t BH = B * H;
  if (!workspace || ((uintptr_t)workspace & 15u) || workspace_bytes < BH * Nq * 8) return MIFA_ERR_WORKSPACE;
  BwdParams p;
  p.q = (const __bf16*)q;
  p.k = (const __bf16*)k;
  p.v = (const __bf16*)v;
  p.dO = (const __bf16*)dO;
  float* dd = (float*)workspace;
  float* lse2 = dd + BH * Nq;
  p.lse2 = lse2;
  p.dd = dd;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.sq = Strides{st[0], st[1], st[2]};
  p.sk = Strides{st[3], st[4], st[5]};
  p.sv = Strides{st[6], st[7], st[8]};
  const Strides so{st[9], st[10], st[11]};
  p.sdo = Strides{st[12], st[13], st[14]};
  p.sdq = Strides{st[15], st[16], st[17]};
  p.sdk = Strides{st[18], st[19], st[20]};
  p.sdv = Strides{st[21], st[22], st[23]};
  p.H = (int)H;
  p.g_bf16 = g_bf16;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.BH = (int)BH;
  p.negate = scale < 0.f ? 1 : 0;
  double c_exact = (double)(p.negate ? -scale : scale) * 1.4426950408889634;
  if (c_exact < 1e-30) c_exact = 1e-30;
  p.c_log2 = (float)c_exact;
  p.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d == 128)
    e = causal ? launch_bwd<128, true>(p, o, so, o_bf16, lse, dd, lse2, s)
               : launch_bwd<128, false>(p, o, so, o_bf16, lse, dd, lse2, s);
  else
    e = causal ? launch_bwd<64, true>(p, o, so, o_bf16, lse, dd, lse2, s)
               : launch_bwd<64, false>(p, o, so, o_bf16, lse, dd, lse2, s);
  if (e != hipSuccess) {
    mifa_record_hip_error((int)e);
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}

// The checks of mifa_bwd, in its documented order, up to (not including) the workspace.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
              const void* dq, const void* dk, const void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
              int causal, float scale) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return MIFA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (causal && Nq > Nk)) return MIFA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return MIFA_ERR_UNSUPPORTED_D;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dO | (uintptr_t)dq | (uintptr_t)dk |
       (uintptr_t)dv) & 15u)
    return MIFA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3u) return MIFA_ERR_MISALIGNED;
  if (!__builtin_isfinite(scale)) return MIFA_ERR_BAD_SCALE;
  if (Nq * d >= ((int64_t)1 << 31) || Nk * d >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  if (B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  const int64_t BH = B * H;
  if (BH >= ((int64_t)1 << 31) || BH * ((Nq + 127) / 128) >= ((int64_t)1 << 31) ||
      BH * ((Nk + 127) / 128) >= ((int64_t)1 << 31))
    return MIFA_ERR_TOO_LARGE;
  return MIFA_OK;
}

// The stride rules of the strided entry points, for n (batch, head, row) triples.
int check_bwd_strides(const int64_t* st, int n) {
  for (int i = 0; i < 3 * n; ++i)
    if (st[i] < 0) return MIFA_ERR_BAD_STRIDE;
  for (int i = 0; i < 3 * n; ++i)
    if (st[i] % 8) return MIFA_ERR_MISALIGNED;
  for (int i = 0; i < n; ++i)
    if (st[3 * i + 2] >= ((int64_t)1 << 24)) return MIFA_ERR_TOO_LARGE;
  return MIFA_OK;
}

}  // namespace

extern "C" int mifa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dO,
                        float* dq, float* dk, float* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                        int causal, float scale, void* workspace, int64_t workspace_bytes, void* stream) {
  const int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, causal, scale);
  if (st != MIFA_OK) return st;
  const int64_t sq[3] = {H * Nq * d, Nq * d, d}, sk[3] = {H * Nk * d, Nk * d, d};
  int64_t strides[24];
  // q, k, v, o, dO, dq, dk, dv
  const int64_t* per[8] = {sq, sk, sk, sq, sq, sq, sk, sk};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i) strides[3 * t + i] = per[t][i];
  return run_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, strides, 0, 0, causal, scale, workspace,
                 workspace_bytes, stream);
}

extern "C" int mifa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq,
                                int64_t Nk, int64_t d, const int64_t* strides, int o_dtype, int grad_dtype,
                                int causal, float scale, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!strides) return MIFA_ERR_NULL_POINTER;
  int st = check_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, causal, scale);
  if (st != MIFA_OK) return st;
  if ((o_dtype != MIFA_DTYPE_BF16 && o_dtype != MIFA_DTYPE_F32) ||
      (grad_dtype != MIFA_DTYPE_BF16 && grad_dtype != MIFA_DTYPE_F32))
    return MIFA_ERR_BAD_DTYPE;
  st = check_bwd_strides(strides, 8);
  if (st != MIFA_OK) return st;
  return run_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Nq, Nk, d, strides, o_dtype == MIFA_DTYPE_BF16 ? 1 : 0,
                 grad_dtype == MIFA_DTYPE_BF16 ? 1 : 0, causal, scale, workspace, workspace_bytes, stream);
}
