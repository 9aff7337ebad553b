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
// Design on gfx950 (one workgroup = 4 or 8 waves = 128 or 256 query rows of one (b, h)):
//  * Each wave owns 32 query rows.  Its Q rows stay in VGPRs for the whole kernel, already in
//    the B-operand layout of v_mfma_f32_32x32x16_bf16.
//  * K and V blocks of BC keys are streamed from HBM/L2 into 2 or 4 LDS buffers each with the
//    16-byte global->LDS DMA (global_load_lds_dwordx4), without passing through VGPRs.  The
//    threads fill a tile cooperatively, so nobody may read it before everyone's part has
//    landed (the point made about shared SRAM in "Show HN: Flash Attention in ~100 lines of
//    CUDA"): a wait on the vector-memory counter and a workgroup barrier come before the
//    blocks that use a tile, and the DMA into a buffer is issued only after a barrier that
//    every wave passes once it is done with that buffer.  With 4 buffers the waves meet once
//    every two blocks and each DMA has two block-times to land.
//  * Long sequences use 8-wave workgroups (one per CU, 128 KB of LDS): every K/V block brought
//    into LDS then serves 256 query rows, which halves the L2->LDS stream; shorter ones use
//    4-wave workgroups (two per CU, three at d = 64), whose tiles are shorter and which fill the
//    256 CUs more evenly.
//  * Scores are computed transposed, S^T = K Q^T, on MFMA.  In the 32x32 accumulator layout a
//    lane then holds 16 scores of ONE query (its lane % 32), so the row max and row sum are
//    in-lane reductions plus one v_permlane32_swap with the other half of the wave.
//  * Each wave is software-pipelined over key blocks: while its VALU runs the softmax of block
//    j, its MFMAs compute the scores of block j+1 (K runs one block ahead of V in LDS), and
//    then the PV product of block j follows, one chunk of 16-key slices at a time as soon as
//    that chunk's weights exist, beside the exponentials of the next chunk.  K and V^T operands
//    are read from LDS through small register rings with explicit waits, so the MFMA chains
//    never stall on a read that could have been issued earlier.
//  * Softmax runs in the log2 domain (exp2 on v_exp_f32, with scale * log2(e) folded into one
//    FMA per score).  The running max used for exponentiation is only raised when a block's
//    max exceeds it by more than kRescaleSlack (2^16): the output and row sum are then
//    rescaled once; otherwise the stale max is kept and the weights are at most 2^16.  The
//    final division by the row sum taken with the same max makes this exact, and it removes
//    almost every per-block O rescale (with logits of std 4, as in B=8 H=16 N=2048 with large
//    logits, a slack of 2^16 instead of 2^8 is 2-4% faster; with std-1 logits no rescale
//    happens after the first block either way).
//  * O^T = V^T P^T on MFMA: the probabilities (rounded to bf16) feed the B operand straight from
//    the score accumulators (the key order inside one MFMA is a free permutation of the
//    contraction index), and V^T comes from LDS with ds_read_b64_tr_b16, which transposes a
//    4 x 16 block of bf16 across each 16-lane group.  Each lane accumulates O for its own
//    query, so the per-row rescale and the final 1/l are in-lane multiplies.
//  * Only the blocks that straddle the causal diagonal or the end of the sequence run the
//    masking code; all other blocks take a mask-free path.  A wave stops computing after the
//    last block any of its rows can see (it keeps joining the workgroup's barriers).
//  * LDS tiles are XOR-swizzled in 16-byte chunks to spread the K reads and the V transpose
//    reads over the banks.  The main loop is unrolled over the buffer ring, so every LDS read
//    address is a per-lane register plus an immediate offset.
//  * The first half of the waves run at a raised issue priority, so the two waves sharing a
//    SIMD drift out of step and their MFMA-only and VALU-heavy stretches overlap.
//  * Grid: one workgroup per (b, h, q-tile) -- with the causal mask and 256-row tiles one per
//    pair of tiles (n-1-r, r) of a head, run one after the other, so that all workgroups carry
//    the same number of key blocks --, heaviest causal tiles first, and when the tile
//    count allows it, all tiles of one head are placed on the same XCD (workgroups are handed
//    to the 8 XCDs round-robin) so K/V re-reads hit that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "mifa.h"
#include "mifa_common.h"

namespace {

using namespace mifa_detail;

constexpr int kRowsPerWave = 32;
constexpr float kRescaleSlack = 16.0f;      // log2 units: weights stay <= 2^16 between rescales

// ---- tile geometry -----------------------------------------------------------------------------
// GROUPS_ = 2: the waves form two groups that share the rows and split the key blocks (even
// blocks to group 0, odd ones to group 1); their partial results merge at the end.
template <int D_, int BC_, int WAVES_, int NBUF_, int GROUPS_ = 1>
struct Cfg {
  static constexpr int D = D_, BC = BC_, WAVES = WAVES_, NBUF = NBUF_, kGroups = GROUPS_;
  static constexpr int kWavesPerGroup = WAVES / kGroups;
  static constexpr int kBR = kWavesPerGroup * kRowsPerWave;  // query rows per workgroup
  static constexpr int kThreads = WAVES * 64;
  static constexpr int kChunksPerRow = D / 8;              // 16-byte chunks per K/V row
  static constexpr int kRowsPerInst = 64 / kChunksPerRow;  // rows one wave-wide DMA covers
  static constexpr int kInstPerTensor = BC / kRowsPerInst;
  static constexpr int kInstPerWave = kInstPerTensor / WAVES;
  static constexpr int kTensorBytes = BC * D * 2;
  // LDS: NBUF K buffers, then NBUF V buffers.
  static constexpr int kVBase = NBUF * kTensorBytes;
  static constexpr int kLdsBytes = 2 * NBUF * kTensorBytes;
  static constexpr int kDS = D / 16;  // 16-wide d slices of the S^T MFMA
  static constexpr int kDT = D / 32;  // 32-row dv tiles of O^T
  static constexpr int kKT = BC / 32; // 32-key tiles per block
  static constexpr int kKS = BC / 16; // 16-key slices per block (PV k-steps)
  static constexpr int kSSteps = kKT * kDS;  // MFMAs per S^T block
  static constexpr int kPVSteps = kKS * kDT; // MFMAs per PV block
  static_assert(kInstPerTensor % WAVES == 0 && kInstPerWave >= 1, "block must split evenly over the waves");
  static_assert(BC % 32 == 0, "key block must be a multiple of the 32-key MFMA tile");
  static_assert(NBUF == 2 || NBUF == 4, "two or four K/V buffers");
  static_assert(kGroups == 1 || (kGroups == 2 && NBUF == 4 && WAVES == 8), "key-split groups: 8 waves, 4 buffers");
  static constexpr int kUnroll = NBUF % 2 == 0 ? NBUF : 2 * NBUF;  // blocks per loop trip
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one workgroup");
  static_assert((NBUF - 1) * kTensorBytes + (kKT - 1) * 32 * D * 2 <= 65535, "K read immediates fit in 16 bits");
  static_assert((NBUF - 1) * kTensorBytes + (kKS - 1) * 16 * D * 2 + 8 * D * 2 <= 65535,
                "V read immediates fit in 16 bits");
};

// ---- per-lane addressing, fixed for the whole kernel -----------------------------------------
template <typename C>
struct Lane {
  unsigned k;                   // K operand of slice 0, tile 0, K buffer 0; slice s XORs 32*s
  unsigned ka[C::kDS];          // k ^ 32*s: slice s (buffer and key tile go in the immediate)
  unsigned v[C::kDT];           // V^T operand of dv tile t, key slice 0, V buffer 0
  unsigned dk[C::kInstPerWave]; // DMA source byte offsets within a key block (K)
  unsigned dv[C::kInstPerWave]; // (V)
  unsigned pdk[C::kInstPerWave], pdv[C::kInstPerWave];  // the same for wave + WAVES/2
  unsigned ksb, vsb;            // K and V row strides in bytes (wave-uniform)
};

// DMA: instruction t of this wave covers rows inst*kRowsPerInst .. of the block; lane ->
// (row, physical chunk); the source is the logical chunk that the swizzle places there.  Rows
// past `row_limit` are clamped to it (only the last, partial block needs that).
template <typename C>
__device__ __forceinline__ void dma_offsets(unsigned* dk, unsigned* dv, int wave, int lane, int row_limit, unsigned ksb,
                                            unsigned vsb) {
  constexpr int D = C::D;
#pragma unroll
  for (int t = 0; t < C::kInstPerWave; ++t) {
    const int inst = wave * C::kInstPerWave + t;
    const int r = inst * C::kRowsPerInst + lane / C::kChunksPerRow;
    const int pc = lane % C::kChunksPerRow;
    const int rr = r < row_limit ? r : row_limit;
    dk[t] = (unsigned)rr * ksb + (unsigned)((pc ^ swz_k<D>(r)) * 16);
    dv[t] = (unsigned)rr * vsb + (unsigned)((pc ^ swz_v<D>(r)) * 16);
  }
}

template <typename C>
__device__ __forceinline__ Lane<C> lane_setup(unsigned smem_base, int wave, int lane, unsigned ksb, unsigned vsb) {
  constexpr int D = C::D;
  Lane<C> a;
  const int ln = lane & 31, hf = lane >> 5;
  a.k = smem_base + ln * (D * 2) + ((hf ^ swz_k<D>(ln)) * 16);
#pragma unroll
  for (int s = 0; s < C::kDS; ++s) a.ka[s] = a.k ^ (32u * s);
  const int g = lane >> 4, p = lane & 15;
  const int dvh = g & 1;
  const int r = 4 * hf + (p >> 2);          // row within a 16-key slice, half e = 0
  const int cl = 2 * dvh + ((p & 3) >> 1);  // chunk within a 32-wide dv tile
  const unsigned base = smem_base + C::kVBase + r * (D * 2) + (p & 1) * 8;
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) a.v[t] = base + (((4 * t + cl) ^ swz_v<D>(r)) * 16);
  a.ksb = ksb;
  a.vsb = vsb;
  dma_offsets<C>(a.dk, a.dv, wave, lane, C::BC, ksb, vsb);
  dma_offsets<C>(a.pdk, a.pdv, wave + C::WAVES / 2, lane, C::BC, ksb, vsb);
  return a;
}

// Wave `wave`'s share of the DMA of key block blk of K (IS_V false) or V into that tensor's
// LDS buffer buf; od: that share's per-lane source offsets within a full block.  Block bases are
// wave-uniform, the per-lane parts 32-bit byte offsets.  In the last, partial block, rows past
// the end of the sequence are clamped to the last row: they are masked out of the softmax, and
// clamping keeps every global address inside the tensors.
template <typename C, bool IS_V>
__device__ __forceinline__ void issue_one(const __bf16* __restrict__ base, char* smem, int blk, int buf, int N,
                                          int wave, int lane, const Lane<C>& la,
                                          const unsigned (&od)[C::kInstPerWave]) {
  constexpr int BC = C::BC;
  const char* src = (const char*)base + (int64_t)blk * BC * (IS_V ? la.vsb : la.ksb);
  unsigned o[C::kInstPerWave];
#pragma unroll
  for (int t = 0; t < C::kInstPerWave; ++t) o[t] = od[t];
  if (blk * BC + BC > N) {
    unsigned ok[C::kInstPerWave], ov[C::kInstPerWave];
    dma_offsets<C>(ok, ov, wave, lane, N - 1 - blk * BC, la.ksb, la.vsb);
#pragma unroll
    for (int t = 0; t < C::kInstPerWave; ++t) o[t] = IS_V ? ov[t] : ok[t];
  }
  char* dst = smem + (IS_V ? C::kVBase : 0) + buf * C::kTensorBytes;
#pragma unroll
  for (int t = 0; t < C::kInstPerWave; ++t) {
    const int inst = wave * C::kInstPerWave + t;
    __builtin_amdgcn_global_load_lds((global_cvoid*)(src + o[t]), (lds_void*)(dst + inst * 1024), 16, 0, 0);
  }
}

// ---- the per-wave pipeline stages -------------------------------------------------------------
template <typename C, bool CAUSAL>
struct Wave {
  static constexpr int D = C::D, BC = C::BC;
  // Operand ring depths.  K operand reads run kKR-1 MFMAs ahead, V^T reads kVLook PV steps.  At
  // d = 64 the shallower rings keep a wave within 168 registers, so that three waves fit on a
  // SIMD (the 4-wave launch then holds three workgroups per CU): same results, 1-2% faster on
  // B=4 H=8 N=1024 and 11% on B=16 H=16 N=512 causal (1,024 four-wave workgroups), same-box A/B.
  static constexpr int kKR = D == 64 ? 4 : 6;
  static constexpr int kVLook = D == 64 ? 3 : 8;
  static constexpr int kVR = 2 * (kVLook + 1);

  bf16x8 qf[C::kDS];
  f32x16 oacc[C::kDT];
  float m_run;  // running max in log2 units (stale by at most kRescaleSlack)
  float l_run;  // this lane's half of the row sum
  float c;      // |scale| * log2(e), >= 1e-30
  int N;       // keys from this workgroup's first key block to the end of the sequence
  int row0, my_row, hf;
  int my_pos;  // causal: this row's last visible key, counted from the first key block
  Lane<C> la;

  // ---- S^T = K Q^T for one block: step i is d slice i / kKT of key tile i % kKT ----
  // kaddr is this lane's K address in the block's K buffer.
  template <int KB, int I>
  __device__ __forceinline__ void issue_k(bf16x8 (&kr)[kKR], IC<I>) {
    constexpr int s = I / C::kKT, kt = I % C::kKT;
    kr[I % kKR] = lds_read_b128<KB * C::kTensorBytes + kt * 32 * D * 2>(la.ka[s]);
  }
  template <int KB>
  __device__ __forceinline__ void s_start(bf16x8 (&kr)[kKR]) {
    [&]<int... I>(std::integer_sequence<int, I...>) { (issue_k<KB>(kr, IC<I>{}), ...); }(
        std::make_integer_sequence<int, kKR>{});
  }
  template <int KB, int I>
  __device__ __forceinline__ void s_step(f32x16 (&sacc)[C::kKT], bf16x8 (&kr)[kKR], IC<I>) {
    constexpr int n = C::kSSteps;
    constexpr int after = (I + kKR < n ? I + kKR : n) - I - 1;  // K reads issued after read I
    lgkm_wait<after>(kr[I % kKR]);
    const bf16x8 a = kr[I % kKR];
    if constexpr (I + kKR < n) issue_k<KB>(kr, IC<I + kKR>{});
    constexpr int s = I / C::kKT, kt = I % C::kKT;
    if constexpr (s == 0)
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], (f32x16){}, 0, 0, 0);
    else
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
  }
  template <int KB, int LO, int HI>
  __device__ __forceinline__ void s_steps(f32x16 (&sacc)[C::kKT], bf16x8 (&kr)[kKR]) {
    [&]<int... I>(std::integer_sequence<int, I...>) { (s_step<KB>(sacc, kr, IC<LO + I>{}), ...); }(
        std::make_integer_sequence<int, HI - LO>{});
  }

  // ---- softmax, part 1: mask (diagonal / tail blocks), block row max, rescale decision ----
  __device__ __forceinline__ void apply_mask(f32x16 (&sacc)[C::kKT], int key0) {
    // Key offset 32kt + 8(i/4) + (i%4) within the block is visible iff it is <= lim.
    int lim = N - 1 - key0 - 4 * hf;
    if (CAUSAL) lim = min(lim, my_pos - key0 - 4 * hf);
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 32 * kt + 8 * (i >> 2) + (i & 3);
        sacc[kt][i] = off <= lim ? sacc[kt][i] : -__builtin_inff();
      }
  }
  __device__ __forceinline__ bool softmax_max(const f32x16 (&sacc)[C::kKT], float& bm) {
    float mx4[2 * C::kKT];
#pragma unroll
    for (int kt = 0; kt < C::kKT; ++kt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 8 * h;
        float m = fmax3(sacc[kt][i], sacc[kt][i + 1], sacc[kt][i + 2]);
        m = fmax3(m, sacc[kt][i + 3], sacc[kt][i + 4]);
        m = fmax3(m, sacc[kt][i + 5], sacc[kt][i + 6]);
        mx4[2 * kt + h] = fmax2(m, sacc[kt][i + 7]);
      }
    static_assert(C::kKT == 2, "row max written for two 32-key tiles");
    const float mx = half_max(fmax2(fmax3(mx4[0], mx4[1], mx4[2]), mx4[3]));
    bm = mx * c;  // block max in log2 units; c > 0 keeps an all-masked row at -inf
    return bm > m_run + kRescaleSlack;
  }

  __device__ __forceinline__ void rescale(bool grow, float bm) {
    const float m_new = grow ? bm : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < C::kDT; ++t) oacc[t] *= alpha;
    m_run = m_new;
  }

  // ---- softmax, part 2: P = exp2(S * c - m) packed to bf16, and the row sum ----
  // A masked score is -inf and c > 0, so its weight is exp2(-inf) = 0.  The weights are produced
  // one 16-key slice at a time (slice ks -> pb[ks]), so that the PV steps of a slice can start
  // while later slices are still being exponentiated.  ls4 collects the row sum in the same
  // order whatever the chunking.
  // A row that has seen no visible key yet (m = -inf; possible when the workgroup covers a key
  // range that starts after the row's last key) must get weight exp2(-inf) = 0, not
  // exp2(-inf + inf): neg_m is then 0.
  __device__ __forceinline__ float neg_max() const { return m_run == -__builtin_inff() ? 0.f : -m_run; }
  template <int KS>
  __device__ __forceinline__ void softmax_exp_slice(const f32x16 (&sacc)[C::kKT], bf16x8 (&pb)[C::kKS], float neg_m,
                                                    float (&ls4)[4]) {
    constexpr int kt = KS / 2, i0 = 8 * (KS % 2);
#pragma unroll
    for (int i = i0; i < i0 + 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][i], c, neg_m));
      if (KS == 0 && i < 4)
        ls4[i] = p;
      else
        ls4[i & 3] += p;
      pb[KS][i & 7] = (__bf16)p;
    }
  }
  template <int K0, int K1>
  __device__ __forceinline__ void softmax_exp_slices(const f32x16 (&sacc)[C::kKT], bf16x8 (&pb)[C::kKS], float neg_m,
                                                     float (&ls4)[4]) {
    [&]<int... K>(std::integer_sequence<int, K...>) { (softmax_exp_slice<K0 + K>(sacc, pb, neg_m, ls4), ...); }(
        std::make_integer_sequence<int, K1 - K0>{});
  }

  // ---- O^T += V^T P^T for one block ----
  // Step st multiplies key slice st / kDT into dv tile st % kDT.  Lane (dv row 32t + ln, half hf)
  // needs V[key][dv] for keys 16ks + 4hf + 0..3 (read "lo") and 16ks + 8 + 4hf + 0..3 (read
  // "hi"); the transpose read hands each lane of a 16-lane group its dv column of a 4-key slab.
  // vbuf is the byte offset of the block's V buffer.
  template <int VB, int ST>
  __device__ __forceinline__ void issue_v(i16x4 (&vr)[kVR], IC<ST>) {
    constexpr int ks = ST / C::kDT, t = ST % C::kDT;
    constexpr int slot = ST % (kVLook + 1);
    constexpr int off = VB * C::kTensorBytes + ks * 16 * D * 2;
    vr[2 * slot] = lds_read_tr<off>(la.v[t]);
    vr[2 * slot + 1] = lds_read_tr<off + 8 * D * 2>(la.v[t]);
  }
  template <int VB>
  __device__ __forceinline__ void pv_start(i16x4 (&vr)[kVR]) {
    [&]<int... I>(std::integer_sequence<int, I...>) { (issue_v<VB>(vr, IC<I>{}), ...); }(
        std::make_integer_sequence<int, kVLook>{});
  }
  template <int VB, int ST>
  __device__ __forceinline__ void pv_step(const bf16x8 (&pb)[C::kKS], i16x4 (&vr)[kVR], IC<ST>) {
    constexpr int n = C::kPVSteps;
    constexpr int ks = ST / C::kDT, t = ST % C::kDT;
    constexpr int slot = ST % (kVLook + 1);
    constexpr int ahead = (ST + kVLook < n ? ST + kVLook : n) - ST - 1;  // steps issued after this one
    lgkm_wait<2 * ahead>(vr[2 * slot], vr[2 * slot + 1]);
    const i16x8 a16 = __builtin_shufflevector(vr[2 * slot], vr[2 * slot + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    if constexpr (ST + kVLook < n) issue_v<VB>(vr, IC<ST + kVLook>{});
    // (On the causal diagonal, slices above this wave's rows have all-zero weights; they are
    // multiplied anyway, which keeps this path free of branches.)
    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16), pb[ks], oacc[t], 0, 0, 0);
  }
  // PV steps of key slices K0 .. K1-1.
  template <int VB, int K0, int K1>
  __device__ __forceinline__ void pv_slices(const bf16x8 (&pb)[C::kKS], i16x4 (&vr)[kVR]) {
    [&]<int... St>(std::integer_sequence<int, St...>) { (pv_step<VB>(pb, vr, IC<K0 * C::kDT + St>{}), ...); }(
        std::make_integer_sequence<int, (K1 - K0) * C::kDT>{});
  }

  // ---- one key block j, with the scores of block j+1 computed alongside ----
  // `cur` holds S^T(j) on entry and `nxt` holds S^T(j+1) on exit.  kbuf / vbuf are the byte
  // offsets of the buffers holding K(j+1) and V(j).  The first half of the S^T(j+1) MFMAs sits
  // with the row max, the second half with the first chunk of exponentials; the PV steps of each
  // chunk of key slices then run beside the exponentials of the next chunk, so that no long
  // stretch of the wave is all VALU or all MFMA.  Chunks of one slice suit the 8-wave kernel
  // (one workgroup per CU), chunks of two the 4-wave kernel (two per CU), by measurement.
  // On the last block the K buffer holds no new block and the scores computed from it are
  // unused.
  static constexpr int kExpChunk = C::WAVES == 8 ? 1 : 2;  // key slices per chunk
  static_assert(C::kKS % kExpChunk == 0, "chunks tile the key slices");
  template <int VB, int G>
  __device__ __forceinline__ void pv_chunk(const f32x16 (&cur)[C::kKT], bf16x8 (&pb)[C::kKS], i16x4 (&vr)[kVR],
                                           float neg_m, float (&ls4)[4]) {
    constexpr int k0 = G * kExpChunk, k1 = k0 + kExpChunk;
    pv_slices<VB, k0, k1>(pb, vr);
    if constexpr (k1 < C::kKS) softmax_exp_slices<k1, k1 + kExpChunk>(cur, pb, neg_m, ls4);
  }
  template <int KB, int VB>
  __device__ __forceinline__ void block(f32x16 (&cur)[C::kKT], f32x16 (&nxt)[C::kKT], int key0, bool masked) {
    bf16x8 kr[kKR];
    constexpr int half = C::kSSteps / 2;
    if (masked) apply_mask(cur, key0);
    s_start<KB>(kr);
    s_steps<KB, 0, half>(nxt, kr);
    float bm;
    const bool grow = softmax_max(cur, bm);
    if (__builtin_amdgcn_ballot_w64(grow)) rescale(grow, bm);
    bf16x8 pb[C::kKS];
    s_steps<KB, half, C::kSSteps>(nxt, kr);
    const float neg_m = neg_max();
    float ls4[4];
    softmax_exp_slices<0, kExpChunk>(cur, pb, neg_m, ls4);
    i16x4 vr[kVR];
    pv_start<VB>(vr);
    [&]<int... G>(std::integer_sequence<int, G...>) { (pv_chunk<VB, G>(cur, pb, vr, neg_m, ls4), ...); }(
        std::make_integer_sequence<int, C::kKS / kExpChunk>{});
    l_run += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
  }

  // Scores of the first block (no softmax to overlap with); K(0) is in K buffer 0.
  __device__ __forceinline__ void first_scores(f32x16 (&s)[C::kKT]) {
    bf16x8 kr[kKR];
    s_start<0>(kr);
    s_steps<0, 0, C::kSSteps>(s, kr);
  }
};

// Four consecutive O elements at element offset off: float32, or bf16 (round to nearest even).
__device__ __forceinline__ void store_o4(void* o, int64_t off, f32x4 v, int as_bf16) {
  if (as_bf16) {
    const __bf16 r[4] = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *(uint64_t*)((__bf16*)o + off) = __builtin_bit_cast(uint64_t, r);
  } else {
    *(f32x4*)((float*)o + off) = v;
  }
}

// Launch parameters.  Nq query rows and Nk keys per head; query i sits at position
// i + Nk - Nq (so with Nq < Nk the queries are the newest positions, and the causal mask keeps
// key j iff j <= i + Nk - Nq).  With n_splits > 1 the keys are cut into ranges of split_blocks
// key blocks and split s writes the attention over its range alone (O normalised over that
// range, LSE of that range; O = 0 and LSE = -inf where the range holds no visible key) to
// o + s o_split and lse + s lse_split.  Element (b, h, i, t) of q sits at
// b q_sb + h q_sh + i q_sn + t (strides in elements; likewise k, v, o); LSE is [B*H, Nq].
// O is float32, or bf16 when o_bf16 is set.
struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn, o_sb, o_sh, o_sn;
  int H, o_bf16;
  int Nq, Nk, BH, n_qtiles;
  float c_log2;
  int negate_q, xcd_group;
  int n_splits, split_blocks;
  int64_t o_split, lse_split;
};

// One query tile (qt) of head bh, key range `split`: the whole pipeline from the Q load to the
// O and LSE stores.
template <typename C, bool CAUSAL>
__device__ __forceinline__ void fwd_tile(const FwdParams& p, int bh, int qt, int split) {
  constexpr int BC = C::BC, NBUF = C::NBUF, kBR = C::kBR;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk, kshift = Nk - Nq;

  // Blocks [jb0, jb1) of the head's keys are visited: the tile's visible blocks, cut to this
  // workgroup's key range.  Blocks from j_mask on straddle the diagonal or the end of the
  // sequence and take the masked path.
  const int n_kblocks = (Nk + BC - 1) / BC;
  int nblk_all = n_kblocks;
  int j_mask_all = Nk / BC;
  if (CAUSAL) {
    const int last_row = min(Nq - 1, qt * kBR + kBR - 1);
    nblk_all = min(n_kblocks, (last_row + kshift) / BC + 1);
    j_mask_all = min(j_mask_all, (qt * kBR + kshift) / BC);
  }
  const int jb0 = split * p.split_blocks;
  const int jb1 = min(nblk_all, jb0 + p.split_blocks);
  const int nblk = jb1 - jb0;
  const int j_mask = j_mask_all - jb0;
  const int key_base = jb0 * BC;

  const int b = bh / p.H, h = bh - b * p.H;
  const __bf16* __restrict__ qh = p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* __restrict__ kh = p.k + b * p.k_sb + h * p.k_sh + key_base * p.k_sn;
  const __bf16* __restrict__ vh = p.v + b * p.v_sb + h * p.v_sh + key_base * p.v_sn;
  const int64_t o_off = split * p.o_split + b * p.o_sb + h * p.o_sh;
  float* __restrict__ lse_out = p.lse + split * p.lse_split + (int64_t)bh * Nq;

  Wave<C, CAUSAL> W;
  const int N = Nk - key_base;
  W.N = N;
  const int grp = wave / C::kWavesPerGroup;  // key-split group (0 unless kGroups == 2)
  W.row0 = qt * kBR + (wave - grp * C::kWavesPerGroup) * kRowsPerWave;
  W.my_row = W.row0 + ln;
  W.my_pos = W.my_row + kshift - key_base;
  // Key blocks this wave needs: with the causal mask, up to the last visible key of its last
  // row (the blocks after that are fully masked for all its rows and would add exp2(-inf) = 0
  // weights); none when all its rows lie past the end.  The wave still takes part in every
  // barrier and DMA of the workgroup's longer loop.
  int nblk_w = nblk;
  if (CAUSAL) {
    const int wave_last = min(Nq - 1, W.row0 + kRowsPerWave - 1);
    nblk_w = min(nblk, min(n_kblocks, (wave_last + kshift) / BC + 1) - jb0);
  }
  if (W.row0 >= Nq) nblk_w = 0;
  nblk_w = __builtin_amdgcn_readfirstlane(nblk_w);
  W.hf = hf;
  W.c = p.c_log2;
  W.m_run = -__builtin_inff();
  W.l_run = 0.f;
#pragma unroll
  for (int t = 0; t < C::kDT; ++t) W.oacc[t] = (f32x16){};

  // ---- Q rows into VGPRs (B operand of S^T = K Q^T: lane holds q[row][16s + 8hf .. +7]) ----
  {
    const int r = W.my_row < Nq ? W.my_row : Nq - 1;
    const __bf16* src = qh + r * p.q_sn + 8 * hf;
#pragma unroll
    for (int s = 0; s < C::kDS; ++s) {
      u32x4 raw = *(const u32x4*)(src + 16 * s);
      if (p.negate_q) raw ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      W.qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // A key range that holds no block of this tile (a split past the causal diagonal) still
  // writes its part: no weight (O = 0, LSE = -inf).  The test is uniform over the workgroup.
  if (nblk <= 0) {
    if (W.my_row < Nq) {
      const int64_t orow = o_off + W.my_row * p.o_sn;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) store_o4(p.o, orow + 32 * t + 8 * g4 + 4 * hf, (f32x4){}, p.o_bf16);
      if (hf == 0) lse_out[W.my_row] = -__builtin_inff();
    }
    return;
  }

  const unsigned smem_base = (unsigned)(uintptr_t)(lds_void*)smem;
  W.la = lane_setup<C>(smem_base, wave, lane, (unsigned)(p.k_sn * 2), (unsigned)(p.v_sn * 2));
  // The two waves that share a SIMD run the same blocks between the same barriers.  A static
  // priority for the first half of the waves lets one of them run ahead, so that its MFMA-only
  // stretches (PV) line up with the other's VALU-heavy ones (softmax).
  if (wave < C::WAVES / 2) __builtin_amdgcn_s_setprio(1);

  f32x16 sA[C::kKT], sB[C::kKT];
  const int last = nblk - 1;
  if constexpr (C::kGroups == 2) {
    // ---- two groups of four waves over the same 128 rows, one barrier per two blocks ----
    // Group g runs the blocks j = g, g+2, g+4, ...; between two barriers group 0 runs block j and
    // group 1 block j+1 (j even), side by side, so each wave walks half of the key blocks.  K(i)
    // lives in K buffer i % 4 and V(i) in V buffer i % 4.  The period from the barrier before
    // block j reads K(j+2), K(j+3) (the next scores of the two groups) and V(j), V(j+1); right
    // after that barrier the waves of group 0 issue K(j+4), K(j+5), V(j+2), V(j+3), their share
    // and that of the group-1 wave on their SIMD, into the buffers the previous period read.
    auto ld = [&](int blk, int w, const unsigned (&odk)[C::kInstPerWave], const unsigned (&odv)[C::kInstPerWave],
                  bool is_v) {
      if (blk > last) return;
      if (is_v)
        issue_one<C, true>(vh, smem, blk, blk % NBUF, N, w, lane, W.la, odv);
      else
        issue_one<C, false>(kh, smem, blk, blk % NBUF, N, w, lane, W.la, odk);
    };
    auto both = [&](int blk, bool is_v) {
      ld(blk, wave, W.la.dk, W.la.dv, is_v);
      ld(blk, wave + C::WAVES / 2, W.la.pdk, W.la.pdv, is_v);
    };
    // Prologue, every wave its own share: K(0) .. K(3), V(0), V(1).
    for (int b = 0; b < 4; ++b) ld(b, wave, W.la.dk, W.la.dv, false);
    ld(0, wave, W.la.dk, W.la.dv, true);
    ld(1, wave, W.la.dk, W.la.dv, true);
    // Group 0 always reads an even buffer and group 1 the next one, so group 1's LDS read
    // addresses start one buffer further and both groups run the same code.
    if (grp == 1) {
      W.la.k += C::kTensorBytes;
#pragma unroll
      for (int s = 0; s < C::kDS; ++s) W.la.ka[s] += C::kTensorBytes;
#pragma unroll
      for (int t = 0; t < C::kDT; ++t) W.la.v[t] += C::kTensorBytes;
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    W.first_scores(sA);
    // Period U2 of a trip of two periods (four blocks): group g runs block j0 + 2 U2 + g, whose
    // scores were computed into cur and whose next scores (block + 2) go to nxt.
    auto period = [&]<int U2>(int j, f32x16(&cur)[C::kKT], f32x16(&nxt)[C::kKT], IC<U2>) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (grp == 0) {
        both(j + 4, false);
        both(j + 2, true);
        both(j + 5, false);
        both(j + 3, true);
      }
      const int jb = j + grp;
      if (jb < nblk_w) W.template block<(2 * U2 + 2) % NBUF, (2 * U2) % NBUF>(cur, nxt, jb * BC, jb >= j_mask);
    };
    for (int j0 = 0; j0 < nblk; j0 += 4) {
      period(j0, sA, sB, IC<0>{});
      if (j0 + 2 < nblk) period(j0 + 2, sB, sA, IC<1>{});
    }
  } else if constexpr (NBUF == 4) {
    // ---- DMA schedule: one barrier per two blocks ----
    // K(i) lives in K buffer i % 4 and V(i) in V buffer i % 4.  Before every even block j all
    // waves meet at a barrier, and right after it the DMA of K(j+3), K(j+4), V(j+2), V(j+3)
    // goes out: the buffers blocks j-2 and j-1 have released.  Blocks j and j+1 read K(j+1),
    // K(j+2), V(j), V(j+1), all issued at the previous even barrier and waited for (vmcnt 0)
    // before this one.  Loads past the last block are skipped.  Between barriers the waves drift
    // up to a block apart.
    //   A load instruction holds up its wave for tens of cycles.  Inside the loop only the
    // high-priority waves issue, each its own share and that of the wave it shares a SIMD with:
    // they run ahead and would wait at the next barrier anyway, and while they issue, the other
    // wave of the SIMD keeps the matrix unit busy.
    auto ld = [&](int blk, int w, const unsigned (&odk)[C::kInstPerWave], const unsigned (&odv)[C::kInstPerWave],
                  bool is_v) {
      if (blk > last) return;
      if (is_v)
        issue_one<C, true>(vh, smem, blk, blk % NBUF, N, w, lane, W.la, odv);
      else
        issue_one<C, false>(kh, smem, blk, blk % NBUF, N, w, lane, W.la, odk);
    };
    auto both = [&](int blk, bool is_v) {
      ld(blk, wave, W.la.dk, W.la.dv, is_v);
      ld(blk, wave + C::WAVES / 2, W.la.pdk, W.la.pdv, is_v);
    };
    // Prologue, every wave its own share: K(0), V(0), K(1), V(1), K(2).
    ld(0, wave, W.la.dk, W.la.dv, false);
    ld(0, wave, W.la.dk, W.la.dv, true);
    ld(1, wave, W.la.dk, W.la.dv, false);
    ld(1, wave, W.la.dk, W.la.dv, true);
    ld(2, wave, W.la.dk, W.la.dv, false);
    if (last >= 2)  // K(0) has landed (the loads issued after it may still be in flight)
      wait_vmcnt<4 * C::kInstPerWave>();
    else if (last == 1)
      wait_vmcnt<3 * C::kInstPerWave>();
    else
      wait_vmcnt<C::kInstPerWave>();
    __builtin_amdgcn_s_barrier();
    W.first_scores(sA);
    auto step = [&]<int U>(int j, f32x16(&cur)[C::kKT], f32x16(&nxt)[C::kKT], IC<U>) {
      if constexpr (U % 2 == 0) {
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (wave < C::WAVES / 2) {
          both(j + 3, false);
          both(j + 2, true);
          both(j + 4, false);
          both(j + 3, true);
        }
      }
      if (j < nblk_w) W.template block<(U + 1) % NBUF, U % NBUF>(cur, nxt, j * BC, j >= j_mask);
    };
    for (int j0 = 0; j0 < nblk; j0 += C::kUnroll) {
      [&]<int... U>(std::integer_sequence<int, U...>) {
        (void)((j0 + U < nblk ? (U % 2 == 0 ? step(j0 + U, sA, sB, IC<U>{}) : step(j0 + U, sB, sA, IC<U>{})), true : false) && ...);
      }(std::make_integer_sequence<int, C::kUnroll>{});
    }
  } else {
  // ---- DMA schedule (two buffers) ----
  // K(i) lives in K buffer i % 2 and V(i) in V buffer i % 2.  Right after the barrier before block
  // j, K(j+2) and V(j+1) go out into the buffers block j-1 has just released; block j reads K(j+1)
  // and V(j), issued at the previous barrier and waited for (vmcnt 0) before this one.  Loads past
  // the last block are skipped.
  static_assert(NBUF == 2, "the short-sequence schedule has two buffers");
  auto ld = [&](int blk, bool is_v) {
    if (blk > last) return;
    if (is_v)
      issue_one<C, true>(vh, smem, blk, blk % 2, N, wave, lane, W.la, W.la.dv);
    else
      issue_one<C, false>(kh, smem, blk, blk % 2, N, wave, lane, W.la, W.la.dk);
  };
  auto group = [&](int g) {
    ld(g + 2, false);
    ld(g + 1, true);
  };
  // Prologue: K(0), then V(0) and K(1); K(0) must land before the scores of block 0.
  ld(0, false);
  ld(0, true);
  ld(1, false);
  if (last >= 1)
    wait_vmcnt<2 * C::kInstPerWave>();
  else
    wait_vmcnt<C::kInstPerWave>();
  __builtin_amdgcn_s_barrier();

  W.first_scores(sA);

  // ---- main loop, unrolled so that buffer indices and score-register roles are static ----
  // (trip of kUnroll blocks: a multiple of NBUF and of 2)
  auto step = [&]<int U>(int j, f32x16(&cur)[C::kKT], f32x16(&nxt)[C::kKT], IC<U>) {
    wait_vmcnt<0>();               // K(j+1) and V(j) have landed
    __builtin_amdgcn_s_barrier();  // ... for every wave; block j-1 is done
    group(j);
    if (j < nblk_w) W.template block<(U + 1) % NBUF, U % NBUF>(cur, nxt, j * BC, j >= j_mask);
  };
  for (int j0 = 0; j0 < nblk; j0 += C::kUnroll) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (void)((j0 + U < nblk ? (U % 2 == 0 ? step(j0 + U, sA, sB, IC<U>{}) : step(j0 + U, sB, sA, IC<U>{})), true : false) && ...);
    }(std::make_integer_sequence<int, C::kUnroll>{});
  }
  }
  // No load is left in flight when the workgroup's LDS is handed to another workgroup.
  wait_vmcnt<0>();

  float l_tot = half_sum(W.l_run);
  if constexpr (C::kGroups == 2) {
    // ---- merge of the two groups' partial results (same rows, disjoint key blocks) ----
    // Each holds O, the row sum l and the max m it was taken against; with m = max(m0, m1) the
    // rows combine as O = 2^(m0-m) O0 + 2^(m1-m) O1 and l likewise (a partial with no visible
    // key has m = -inf and weight 0).  Group 1 passes its values through LDS (the K/V buffers,
    // free once every wave is past its last block); both waves of a pair hold the same rows
    // in the same lane layout, so the exchange is element by element.
    constexpr int kVals = C::kDT * 16 + 2;
    static_assert(C::kWavesPerGroup * kVals * 64 * 4 <= C::kLdsBytes, "merge buffer fits the K/V buffers");
    float* xch = (float*)smem + (wave - grp * C::kWavesPerGroup) * kVals * 64 + lane;
    __syncthreads();  // every wave is done reading K and V
    if (grp == 1) {
#pragma unroll
      for (int t = 0; t < C::kDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(16 * t + i) * 64] = W.oacc[t][i];
      xch[(kVals - 2) * 64] = W.m_run;
      xch[(kVals - 1) * 64] = l_tot;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xch[(kVals - 2) * 64], l1 = xch[(kVals - 1) * 64];
    const float m = fmax2(W.m_run, m1);
    const float a0 = W.m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(W.m_run - m);
    const float a1 = m1 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int t = 0; t < C::kDT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) W.oacc[t][i] = a0 * W.oacc[t][i] + a1 * xch[(16 * t + i) * 64];
    l_tot = a0 * l_tot + a1 * l1;
    W.m_run = m;
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ----
  // (A row with no visible key in this workgroup's key range has l = 0: O = 0, LSE = -inf.)
  if (W.my_row < Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t orow = o_off + W.my_row * p.o_sn;
#pragma unroll
    for (int t = 0; t < C::kDT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 val = {W.oacc[t][4 * g4] * inv, W.oacc[t][4 * g4 + 1] * inv, W.oacc[t][4 * g4 + 2] * inv,
                     W.oacc[t][4 * g4 + 3] * inv};
        store_o4(p.o, orow + 32 * t + 8 * g4 + 4 * hf, val, p.o_bf16);
      }
    if (hf == 0) lse_out[W.my_row] = (W.m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f;
  }
}

// Register budget: two waves per SIMD (256 registers each), three at d = 64 (168 each).
template <typename C>
constexpr int kWavesPerSimd = C::D == 64 ? 3 : 2;

template <typename C, bool CAUSAL, bool PAIR>
__global__ __attribute__((amdgpu_flat_work_group_size(C::kThreads, C::kThreads),
                          amdgpu_waves_per_eu(kWavesPerSimd<C>, kWavesPerSimd<C>)))
void mifa_fwd_kernel(FwdParams p) {
  const int BH = p.BH, n_qtiles = p.n_qtiles;
  // ---- which (key range, b*H + h, q-tile) this workgroup owns ----
  // PAIR (causal only): a workgroup owns the tile pair (n-1-r, r) of one head, the heavy tile
  // first, then the light one, so that every workgroup has the same number of key blocks.
  const int slots = BH * (PAIR ? (n_qtiles + 1) / 2 : n_qtiles);
  const int split = blockIdx.x / slots;
  int bh, rank;
  {
    const int w = blockIdx.x - split * slots;
    if (p.xcd_group) {
      // Workgroup w runs on XCD w % 8; give XCD x the heads bh = x, x + 8, ...  Single tiles are
      // walked heaviest first across those heads; tile pairs (all equally heavy) head by head,
      // so that the pairs running side by side on an XCD read the same head's K and V through
      // its L2 (B=8 H=16 N=2048 causal: -4.6% against the order of single tiles, same-box A/B).
      const int x = w % kXcds, kk = w / kXcds;
      const int heads_per_xcd = BH / kXcds;
      if constexpr (PAIR) {
        const int npairs = (n_qtiles + 1) / 2;
        rank = kk % npairs;
        bh = (kk / npairs) * kXcds + x;
      } else {
        rank = kk / heads_per_xcd;
        bh = (kk % heads_per_xcd) * kXcds + x;
      }
    } else {
      rank = w / BH;
      bh = w % BH;
    }
  }
  fwd_tile<C, CAUSAL>(p, bh, CAUSAL ? n_qtiles - 1 - rank : rank, split);
  if (PAIR && n_qtiles - 1 - rank > rank) {
    __syncthreads();  // every wave is done with the first tile's LDS buffers
    fwd_tile<C, CAUSAL>(p, bh, rank, split);
  }
}

// Shape of one launch on the host side.
struct Problem {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int Nq, Nk, BH;
  float scale;
  int n_splits, split_blocks;
  int64_t o_split, lse_split;
  int H, o_bf16;
  int64_t st[12];  // q, k, v, o: (batch, head, row) strides in elements
};

template <typename C, bool CAUSAL>
hipError_t launch(const Problem& pr, hipStream_t stream, bool pair_tiles = true) {
  FwdParams p;
  p.q = (const __bf16*)pr.q;
  p.k = (const __bf16*)pr.k;
  p.v = (const __bf16*)pr.v;
  p.o = pr.o;
  p.lse = pr.lse;
  p.q_sb = pr.st[0], p.q_sh = pr.st[1], p.q_sn = pr.st[2];
  p.k_sb = pr.st[3], p.k_sh = pr.st[4], p.k_sn = pr.st[5];
  p.v_sb = pr.st[6], p.v_sh = pr.st[7], p.v_sn = pr.st[8];
  p.o_sb = pr.st[9], p.o_sh = pr.st[10], p.o_sn = pr.st[11];
  p.H = pr.H;
  p.o_bf16 = pr.o_bf16;
  p.Nq = pr.Nq;
  p.Nk = pr.Nk;
  p.BH = pr.BH;
  p.n_qtiles = (pr.Nq + C::kBR - 1) / C::kBR;
  p.xcd_group = (pr.BH % kXcds == 0) ? 1 : 0;
  p.negate_q = pr.scale < 0.f ? 1 : 0;
  // The exponent factor c = |scale| * log2(e) is kept >= 1e-30 so that a masked score (-inf)
  // always maps to exp2(-inf) = 0.  For |scale| below that every logit is under 1e-29 in
  // magnitude and exp2 of it rounds to exactly 1 in fp32, the same as with scale = 0.
  double c_exact = (double)(p.negate_q ? -pr.scale : pr.scale) * 1.4426950408889634;
  if (c_exact < 1e-30) c_exact = 1e-30;
  p.c_log2 = (float)c_exact;
  p.n_splits = pr.n_splits;
  p.split_blocks = pr.split_blocks;
  p.o_split = pr.o_split;
  p.lse_split = pr.lse_split;
  // Causal 8-wave launches over the whole key range pair their tiles (n-1-r with r): every
  // workgroup then has n+1 key blocks, and half as many workgroups are dispatched.  Measured
  // on MI355X (same-box A/B, medians, identical output): B=2 H=16 N=4096 -4.8%, B=8 H=16 N=2048
  // -0.9%, B=1 H=32 N=16384 -0.6%.  The key-split launch pairs only when asked (`pair_tiles`).
  constexpr bool kCanPair = CAUSAL && C::WAVES == 8;
  const bool pair = kCanPair && pair_tiles && pr.n_splits == 1 && p.n_qtiles > 1;
  const int64_t grid = (int64_t)pr.BH * (pair ? (p.n_qtiles + 1) / 2 : p.n_qtiles) * pr.n_splits;
  auto kern = mifa_fwd_kernel<C, CAUSAL, false>;
  if constexpr (kCanPair) {
    if (pair) kern = mifa_fwd_kernel<C, CAUSAL, true>;
  }
  // Raise the dynamic-LDS limit once per instantiation and device.
  static std::atomic<unsigned long long> done[2] = {0, 0};  // per kernel: single tiles, tile pairs
  const hipError_t attr = raise_lds_limit((const void*)kern, C::kLdsBytes, done[pair ? 1 : 0]);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, stream, p);
  return hipGetLastError();
}

// Launch-shape choice: 8-wave workgroups (256 rows, one per CU) for sequences longer than 1024
// with more of them than CUs; 8-wave workgroups with two key-split groups (128 rows) for few
// tiles; otherwise 4-wave workgroups (128 rows, two per CU; three at d = 64).  Measured on
// MI355X (same-box A/B): with 8 waves B=1 H=32 N=16384 causal runs ~8 % faster, B=2 H=16
// N=4096 causal ~7 % and B=8 H=16 N=2048 causal ~3 %; with exactly one 256-row tile per CU
// (B=1 H=4 N=16384, B=1 H=8 N=8192) 4 waves are 1-2.5 % faster, since two workgroups per CU
// even out the causal triangle a little.  Key-range splits always use 4-wave workgroups.
constexpr int kCUs = 256;
constexpr int kLongN = 1024;
template <int D, bool CAUSAL>
hipError_t dispatch(const Problem& pr, hipStream_t stream) {
  const int64_t big_tiles = (int64_t)pr.BH * ((pr.Nq + 255) / 256);
  const int64_t tiles = (int64_t)pr.BH * ((pr.Nq + 127) / 128);
  if (pr.n_splits == 1 && pr.Nq > kLongN && big_tiles > kCUs) return launch<Cfg<D, 64, 8, 4>, CAUSAL>(pr, stream);
  // Without the mask every tile is equally heavy, so exactly one 256-row tile per CU already
  // fills the GPU evenly: 8 waves there too (same-box A/B, medians, against 4-wave workgroups:
  // B=1 H=8 N=8192 d=128 -8%, B=1 H=4 N=16384 -8%, B=1 H=16 N=4096 d=64 -11%, B=4 H=16 N=1024
  // d=128 -6%).
  if (!CAUSAL && pr.n_splits == 1 && pr.Nq >= kLongN && big_tiles >= kCUs)
    return launch<Cfg<D, 64, 8, 4>, CAUSAL>(pr, stream);
  // Few 128-row tiles (at most one per CU) over at least 512 keys: two groups of four waves per
  // tile split the key blocks, so twice as many waves share the work of a tile.  Measured on
  // MI355X (same-box A/B, medians): B=4 H=8 N=1024 d=64 -8% causal and non-causal against one
  // 4-wave workgroup per tile; N=128 (one tile, two key blocks) +15%, and with 512 tiles, where
  // 4-wave workgroups fit twice per CU, +13%, so those keep the 4-wave launch.
  if (pr.n_splits == 1 && tiles <= kCUs && pr.Nk >= 512) return launch<Cfg<D, 64, 8, 4, 2>, CAUSAL>(pr, stream, false);
  // Causal, longer than 1024, between one and two 128-row tiles per CU: the key-split launch over
  // tile pairs (n-1-r, r) gives every CU one workgroup with the same n+1 key blocks, where
  // 128-row tiles two per CU leave the causal triangle unbalanced.  Measured on MI355X
  // (same-box A/B, medians, against 4-wave workgroups): B=1 H=4 N=16384 d=128 -28.5%,
  // B=1 H=8 N=8192 -26% (d=64 -29%), B=1 H=16 N=4096 -23%; at N=1024 (B=4 H=16) +13%, so
  // shorter sequences keep the 4-wave launch.
  if (CAUSAL && pr.n_splits == 1 && pr.Nq > kLongN && tiles > kCUs && tiles <= 2 * kCUs)
    return launch<Cfg<D, 64, 8, 4, 2>, CAUSAL>(pr, stream, true);
  return launch<Cfg<D, 64, 4, 2>, CAUSAL>(pr, stream);
}

hipError_t dispatch_d(const Problem& pr, int d, bool causal, hipStream_t s) {
  if (d == 128) return causal ? dispatch<128, true>(pr, s) : dispatch<128, false>(pr, s);
  return causal ? dispatch<64, true>(pr, s) : dispatch<64, false>(pr, s);
}

// ---- merge of key-range partials: the associative rule on (O_s, LSE_s) ----------------------
// O = sum_s w_s O_s / sum_s w_s and LSE = m + ln sum_s w_s, with w_s = exp(LSE_s - m) and
// m = max_s LSE_s.  One row per D/4 threads (four O elements each), 64-thread workgroups so that
// even a few hundred rows spread over the CUs; the loops over ranges are unrolled so their loads
// are in flight together.
constexpr int kMergeThreads = 64;
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_splits(const float* __restrict__ o_part,
                                                              const float* __restrict__ lse_part, float* __restrict__ o,
                                                              float* __restrict__ lse, int64_t rows, int n_splits,
                                                              int64_t o_split, int64_t lse_split) {
  constexpr int TPR = D / 4, RPB = kMergeThreads / TPR;
  const int t = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  float m = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < n_splits; ++s) m = __builtin_elementwise_maximum(m, lse_part[s * lse_split + row]);
  f32x4 acc = {};
  float wsum = 0.f;
#pragma unroll 8
  for (int s = 0; s < n_splits; ++s) {
    const float ls = lse_part[s * lse_split + row];
    const float w = ls == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((ls - m) * 1.4426950408889634f);
    wsum += w;
    acc += w * *(const f32x4*)(o_part + s * o_split + row * D + 4 * t);
  }
  *(f32x4*)(o + row * D + 4 * t) = acc * (1.f / wsum);
  if (t == 0) lse[row] = m + __builtin_amdgcn_logf(wsum) * 0.69314718055994531f;
}

// Key-range split for the split-KV entry point: enough workgroups to fill the machine twice
// over (two 4-wave workgroups per CU), each range at least four key blocks long.
struct Split {
  int n_splits, split_blocks;
};
Split choose_split(int64_t BH, int64_t Nq, int64_t Nk) {
  const int64_t tiles = BH * ((Nq + 127) / 128);
  const int64_t kblocks = (Nk + 63) / 64;
  int64_t want = (4 * kCUs + tiles - 1) / tiles;
  want = want < 1 ? 1 : want;
  int64_t most = (kblocks + 3) / 4;
  most = most < 1 ? 1 : most;
  const int64_t n = want < most ? want : most;
  const int64_t per = (kblocks + n - 1) / n;
  return Split{(int)((kblocks + per - 1) / per), (int)per};
}

int64_t workspace_bytes(int64_t BH, int64_t Nq, int64_t d, int n_splits) {
  return (int64_t)n_splits * BH * Nq * (d + 1) * 4;
}

// Argument checks shared by the attention entry points, in the documented order.
int check_attention(const void* q, const void* k, const void* v, const float* o, const float* lse, int64_t B,
                    int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return MIFA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (causal && Nq > Nk)) return MIFA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return MIFA_ERR_UNSUPPORTED_D;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return MIFA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3u) return MIFA_ERR_MISALIGNED;
  if (!__builtin_isfinite(scale)) return MIFA_ERR_BAD_SCALE;
  // Per-head offsets inside the kernel are 32-bit (N*d), the grid is 1-D (B*H*tiles*splits).
  if (Nq * d >= ((int64_t)1 << 31) || Nk * d >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  if (B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  const int64_t BH = B * H;
  const int64_t tiles = BH * ((Nq + 127) / 128);
  if (BH >= ((int64_t)1 << 31) || tiles >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  return MIFA_OK;
}

// Strides of dense [B, H, N, d] tensors: q and o with Nq rows, k and v with Nk rows.
void dense_strides(int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t* st) {
  const int64_t sq[3] = {H * Nq * d, Nq * d, d}, sk[3] = {H * Nk * d, Nk * d, d};
  for (int i = 0; i < 3; ++i) {
    st[i] = sq[i];
    st[3 + i] = sk[i];
    st[6 + i] = sk[i];
    st[9 + i] = sq[i];
  }
}

// Stride checks for n (batch, head, row) triples, in elements: none negative, every one a
// multiple of 8 elements (16-byte rows for bf16, the unit of the kernels' vector loads), and
// row strides below 2^24 elements (per-lane offsets inside a 64-row block are 32-bit).
int check_strides(const int64_t* st, int n) {
  for (int i = 0; i < 3 * n; ++i)
    if (st[i] < 0) return MIFA_ERR_BAD_STRIDE;
  for (int i = 0; i < 3 * n; ++i)
    if (st[i] % 8) return MIFA_ERR_MISALIGNED;
  for (int i = 0; i < n; ++i)
    if (st[3 * i + 2] >= ((int64_t)1 << 24)) return MIFA_ERR_TOO_LARGE;
  return MIFA_OK;
}

thread_local int g_last_hip_error = 0;

// The split-KV launches after validation: the split kernel writes each key range's partial O and
// LSE to `workspace` (unused when one range suffices), then merge_splits combines them.
int splitkv_run(const void* q, const void* k, const void* v, float* o, float* lse, int64_t H, int64_t BH, int64_t Nq,
                int64_t Nk, int64_t d, int causal, float scale, const Split& sp, void* workspace, hipStream_t s) {
  hipError_t e;
  if (sp.n_splits == 1) {
    Problem pr{q, k, v, o, lse, (int)Nq, (int)Nk, (int)BH, scale, 1, sp.split_blocks, 0, 0, (int)H, 0, {}};
    dense_strides(H, Nq, Nk, d, pr.st);
    e = dispatch_d(pr, (int)d, causal != 0, s);
  } else {
    float* o_part = (float*)workspace;
    float* lse_part = o_part + (int64_t)sp.n_splits * BH * Nq * d;
    Problem pr{q,          k,  v,  o_part, lse_part, (int)Nq, (int)Nk, (int)BH, scale, sp.n_splits, sp.split_blocks,
               BH * Nq * d, BH * Nq, (int)H, 0, {}};
    dense_strides(H, Nq, Nk, d, pr.st);
    e = dispatch_d(pr, (int)d, causal != 0, s);
    if (e == hipSuccess) {
      const int64_t rows = BH * Nq;
      const int rpb = kMergeThreads / ((int)d / 4);
      const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
      if (d == 128)
        hipLaunchKernelGGL(merge_splits<128>, dim3(blocks), dim3(kMergeThreads), 0, s, o_part, lse_part, o, lse, rows,
                           sp.n_splits, BH * Nq * d, BH * Nq);
      else
        hipLaunchKernelGGL(merge_splits<64>, dim3(blocks), dim3(kMergeThreads), 0, s, o_part, lse_part, o, lse, rows,
                           sp.n_splits, BH * Nq * d, BH * Nq);
      e = hipGetLastError();
    }
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}

// ---- allocation-free split-KV: the partials live in a static device array ----------------------
// For callers that cannot allocate device memory (code under HIP graph capture, serving loops that
// forbid hipMalloc).  Each device the library runs on holds its own copy of `scratch` until the
// process ends.  In host code the array's name is only a stand-in for the symbol, not a device
// address: the address is resolved with hipGetSymbolAddress once per device (with that device
// current) and kept here; kernels receive that address.  Calls on one device share the array,
// so calls that may overlap on one device must be ordered on a stream.  The split kernel writes
// every row of every range before the merge reads it, so nothing needs clearing between calls.
constexpr int64_t kScratchBytes = (int64_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(p, std::memory_order_release);  // two threads may both resolve it: same value
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int mifa_attention(const void* q, const void* k, const void* v, float* o, float* lse, int64_t B, int64_t H,
                   int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, void* stream) {
  const int st = check_attention(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale);
  if (st != MIFA_OK) return st;
  Problem pr{q, k, v, o, lse, (int)Nq, (int)Nk, (int)(B * H), scale, 1, 1 << 30, 0, 0, (int)H, 0, {}};
  dense_strides(H, Nq, Nk, d, pr.st);
  const hipError_t e = dispatch_d(pr, (int)d, causal != 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}

int mifa_attention_strided(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                           int64_t Nq, int64_t Nk, int64_t d, const int64_t* strides, int o_dtype, int causal,
                           float scale, void* stream) {
  if (!strides) return MIFA_ERR_NULL_POINTER;
  int st = check_attention(q, k, v, (const float*)o, lse, B, H, Nq, Nk, d, causal, scale);
  if (st != MIFA_OK) return st;
  if (o_dtype != MIFA_DTYPE_BF16 && o_dtype != MIFA_DTYPE_F32) return MIFA_ERR_BAD_DTYPE;
  st = check_strides(strides, 4);
  if (st != MIFA_OK) return st;
  Problem pr{q, k, v, o, lse, (int)Nq, (int)Nk, (int)(B * H), scale, 1, 1 << 30, 0, 0, (int)H,
             o_dtype == MIFA_DTYPE_BF16 ? 1 : 0, {}};
  for (int i = 0; i < 12; ++i) pr.st[i] = strides[i];
  const hipError_t e = dispatch_d(pr, (int)d, causal != 0, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}

int mifa_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int64_t B, int64_t H,
             int64_t N, int64_t d, int causal, float scale, void* stream) {
  return mifa_attention(q, k, v, o, lse, B, H, N, N, d, causal, scale, stream);
}

int64_t mifa_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
  if (B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31) || Nq >= ((int64_t)1 << 31) || Nk >= ((int64_t)1 << 31)) return 0;
  const Split sp = choose_split(B * H, Nq, Nk);
  return workspace_bytes(B * H, Nq, d, sp.n_splits);
}

int mifa_attention_splitkv(const void* q, const void* k, const void* v, float* o, float* lse, int64_t B, int64_t H,
                           int64_t Nq, int64_t Nk, int64_t d, int causal, float scale, void* workspace,
                           int64_t workspace_bytes_given, void* stream) {
  const int st = check_attention(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale);
  if (st != MIFA_OK) return st;
  const int64_t BH = B * H;
  const Split sp = choose_split(BH, Nq, Nk);
  if (!workspace || ((uintptr_t)workspace & 15u) || workspace_bytes_given < workspace_bytes(BH, Nq, d, sp.n_splits))
    return MIFA_ERR_WORKSPACE;
  if (BH * ((Nq + 127) / 128) * sp.n_splits >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  return splitkv_run(q, k, v, o, lse, H, BH, Nq, Nk, d, causal, scale, sp, workspace, (hipStream_t)stream);
}

int mifa_attention_splitkv_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int64_t B,
                                   int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                                   void* stream) {
  const int st = check_attention(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale);
  if (st != MIFA_OK) return st;
  const int64_t BH = B * H;
  const Split sp = choose_split(BH, Nq, Nk);
  if (sp.n_splits > 1 && workspace_bytes(BH, Nq, d, sp.n_splits) > kScratchBytes) return MIFA_ERR_SCRATCH;
  if (BH * ((Nq + 127) / 128) * sp.n_splits >= ((int64_t)1 << 31)) return MIFA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (sp.n_splits > 1) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return MIFA_ERR_HIP;
    }
  }
  return splitkv_run(q, k, v, o, lse, H, BH, Nq, Nk, d, causal, scale, sp, ws, (hipStream_t)stream);
}

const char* mifa_status_string(int status) {
  switch (status) {
    case MIFA_OK: return "ok";
    case MIFA_ERR_NULL_POINTER: return "null pointer argument";
    case MIFA_ERR_BAD_SHAPE: return "B, H, N (Nq, Nk) must be >= 1, and causal needs Nq <= Nk";
    case MIFA_ERR_UNSUPPORTED_D: return "head dimension d must be 64 or 128";
    case MIFA_ERR_MISALIGNED: return "tensors must be 16-byte aligned (lse 4-byte) and strides multiples of 8 elements";
    case MIFA_ERR_BAD_SCALE: return "scale must be finite";
    case MIFA_ERR_TOO_LARGE: return "problem too large (N*d or the tile count reaches 2^31)";
    case MIFA_ERR_HIP: return "HIP runtime error (see mifa_last_hip_error)";
    case MIFA_ERR_BAD_DTYPE: return "dtype must be MIFA_DTYPE_BF16 or MIFA_DTYPE_F32";
    case MIFA_ERR_WORKSPACE: return "workspace NULL, not 16-byte aligned, or smaller than the entry point's *_workspace_bytes";
    case MIFA_ERR_BAD_STRIDE: return "a stride is negative";
    case MIFA_ERR_SCRATCH:
      return "the key-range partials need more than the 32 MiB static scratch array of the allocation-free entry point";
    default: return "unknown status";
  }
}

const char* mifa_version(void) { return "mifa 0.1.0 gfx950"; }

int mifa_last_hip_error(void) { return g_last_hip_error; }

__attribute__((visibility("hidden"))) void mifa_record_hip_error(int e) { g_last_hip_error = e; }

}  // extern "C"
