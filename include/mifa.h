/*
 * mifa.h -- C ABI of libmifa, an exact FlashAttention forward pass for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation.  For every batch b and head h,
 *
 *     O[b,h]   = softmax(scale * Q[b,h] K[b,h]^T  [+ causal mask]) V[b,h]
 *     LSE[b,h,i] = ln sum_j exp(scale * q_i . k_j)      (over the visible keys j)
 *
 * computed in one fused, tiled kernel with the online-softmax trick: the row softmax is
 * split into key blocks whose partial results are rescaled as the running row maximum
 * grows, so the N x N score matrix never leaves the chip and the result is still the exact
 * one (the combination of kernel fusion, tiling into fast on-chip memory and the online
 * softmax described in the interview "Tri Dao: prediction", transcript).  The causal
 * variant is the softmax over the lower-triangular score matrix mentioned in the Hacker
 * News FlashAttention-3 thread: query i sees key j iff j <= i.  LSE is not on the pages;
 * it is the per-row log partition sum, natural log, of the scaled logits, which lets
 * partial results over disjoint key sets be merged.
 *
 * Conventions for every entry point:
 *   - Pointers named q, k, v, o, lse, x, y are DEVICE pointers (hipMalloc'd or equivalent) on
 *     the current HIP device.  The caller allocates and owns them; the library calls no
 *     allocator and keeps no caller pointer after returning.  Its state across calls is the
 *     per-thread code read by mifa_last_hip_error; per kernel, an atomic record of the devices
 *     on which that kernel's dynamic-LDS limit has already been raised (set on its first
 *     launch there); and, for mifa_attention_splitkv_noalloc only, a 32 MiB device array held
 *     by each GPU the library runs on, with its device address cached per device on first
 *     use.  Calls are thread-safe and re-entrant (the one exception, overlapping calls of
 *     mifa_attention_splitkv_noalloc on one GPU, is stated at that entry point).
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.  Work is
 *     enqueued asynchronously on it and the library never synchronises.  The caller must
 *     keep every buffer alive and unmodified until the stream has passed the kernel.
 *   - Return value: MIFA_OK (0) or one of the mifa_status codes below.  Every argument
 *     check runs before any HIP call, so a rejected call has no side effect on the device.
 */
#ifndef MIFA_H
#define MIFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mifa_status {
  MIFA_OK = 0,
  MIFA_ERR_NULL_POINTER = 1,   /* q, k, v, o or lse is NULL */
  MIFA_ERR_BAD_SHAPE = 2,      /* B, H or N (Nq, Nk) < 1, or causal with Nq > Nk */
  MIFA_ERR_UNSUPPORTED_D = 3,  /* head dimension d is not 64 or 128 */
  MIFA_ERR_MISALIGNED = 4,     /* a tensor not 16-byte aligned (lse: 4-byte), or a stride not a
                                  multiple of 8 elements */
  MIFA_ERR_BAD_SCALE = 5,      /* scale is NaN or infinite */
  MIFA_ERR_TOO_LARGE = 6,      /* N*d >= 2^31, or B*H*ceil(N/128) >= 2^31 work tiles */
  MIFA_ERR_HIP = 7,            /* the HIP runtime rejected the launch; see mifa_last_hip_error */
  MIFA_ERR_BAD_DTYPE = 8,      /* dtype is not one of mifa_dtype (mifa_softmax_rows) */
  MIFA_ERR_WORKSPACE = 9,      /* workspace NULL, misaligned or too small (mifa_attention_splitkv,
                                  mifa_bwd) */
  MIFA_ERR_BAD_STRIDE = 10,    /* a stride is negative (the *_strided entry points) */
  MIFA_ERR_SCRATCH = 11        /* mifa_attention_splitkv_noalloc: partials exceed its 32 MiB array */
} mifa_status;

/* Element types of mifa_softmax_rows. */
typedef enum mifa_dtype {
  MIFA_DTYPE_BF16 = 0,         /* bfloat16 bit patterns, 2 bytes */
  MIFA_DTYPE_F32 = 1           /* IEEE float32, 4 bytes */
} mifa_dtype;

/*
 * mifa_fwd -- exact attention forward, FlashAttention style.
 *
 *   q, k, v  bf16 (bfloat16 bit patterns), shape [B, H, N, d], contiguous, d fastest:
 *            element (b,h,i,t) lives at ((b*H + h)*N + i)*d + t.  Read only.
 *   o        float32, shape [B, H, N, d], same layout.  Fully overwritten.
 *   lse      float32, shape [B, H, N]: lse[(b*H + h)*N + i].  Fully overwritten.
 *   B, H, N  batch, heads, sequence length (queries = keys = N); each >= 1.  Any N is
 *            supported; it need not be a multiple of the tile sizes.
 *   d        head dimension of q, k and v; 64 or 128.
 *   causal   0: every query sees all N keys.  Non-zero: query i sees keys j <= i.
 *   scale    softmax scale applied to q . k (usually 1/sqrt(d)); any finite value,
 *            including 0 and negative values.
 *   stream   hipStream_t (as void*) to enqueue on; NULL for the null stream.
 *
 * o and lse must not overlap q, k, v or each other (not checked).  Inputs must be finite
 * (not checked; non-finite inputs give unspecified outputs).
 * Accuracy: products are exact, accumulation is float32, and the softmax weights are
 * rounded to bf16 before they multiply V.
 */
int mifa_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
             void* stream);

/*
 * mifa_attention -- the same operation with Nq queries and Nk keys per head (Nq != Nk allowed).
 *
 *   q        bf16 [B, H, Nq, d]; k, v bf16 [B, H, Nk, d]; o float32 [B, H, Nq, d];
 *            lse float32 [B, H, Nq].  Layout, alignment and ownership as for mifa_fwd.
 *   causal   Non-zero: the queries are the last Nq positions of the Nk-long sequence, so query
 *            i sees keys j <= i + (Nk - Nq) -- the lower-triangular mask of the square case
 *            (the causal remark in the Hacker News FlashAttention-3 thread) restricted to
 *            those rows.  Requires Nq <= Nk (MIFA_ERR_BAD_SHAPE otherwise).
 * mifa_fwd(..., N, ...) is mifa_attention(..., N, N, ...).  Errors as for mifa_fwd.
 */
int mifa_attention(const void* q, const void* k, const void* v, float* o, float* lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                   void* stream);

/*
 * mifa_attention_strided -- mifa_attention on tensors of any (batch, head, row) strides, with O
 * in float32 or bf16: the layouts of the scaled-dot-product-attention call the Hacker News
 * FlashAttention-3 thread names as the user-facing entry ([B, H, N, d], or [B, N, H, d] views
 * of one projection output) are read in place, without copies.
 *
 *   strides  host array of 12 int64: the (batch, head, row) strides, in elements, of q, k, v
 *            and o in that order.  Element (b,h,i,t) of q lives at
 *            q[b*strides[0] + h*strides[1] + i*strides[2] + t]; d is contiguous.  Strides must
 *            be >= 0 (MIFA_ERR_BAD_STRIDE) and multiples of 8 (MIFA_ERR_MISALIGNED); row
 *            strides below 2^24 (MIFA_ERR_TOO_LARGE).  A zero stride on q, k or v broadcasts
 *            it; o must not overlap itself or the inputs (not checked).
 *   o_dtype  MIFA_DTYPE_F32 or MIFA_DTYPE_BF16 (rounded to nearest even); MIFA_ERR_BAD_DTYPE
 *            otherwise.
 *   lse      float32 [B, H, Nq], contiguous, as for mifa_attention.
 * Other arguments as for mifa_attention.  Errors in the order NULL (strides too), shape, d,
 * alignment of the pointers, scale, size, then o_dtype, then the strides.
 */
int mifa_attention_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                           const int64_t* strides, int o_dtype, int causal, float scale,
                           void* stream);

/*
 * mifa_attention_splitkv -- mifa_attention with the keys of each head cut into ranges that
 * separate workgroups process in parallel, for few queries against many keys (decoding with a
 * key/value cache).  Each range produces the attention over its keys alone, a partial O and
 * its LSE; a second kernel merges the ranges with the associative rule
 *     LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s
 * (the partial softmax states combine as aggregates, as the Hacker News FlashAttention-3 thread
 * puts it; the same rescaling as the online softmax).  The result equals mifa_attention's up
 * to fp32 rounding order.
 *
 *   workspace        device memory the caller owns, 16-byte aligned, at least
 *                    mifa_splitkv_workspace_bytes(B, H, Nq, Nk, d) bytes; overwritten (it holds
 *                    the partial O and LSE); the caller must not touch it until the stream has
 *                    passed the call.  Calls that share a workspace must be ordered on a stream.
 *   workspace_bytes  its size in bytes.
 * Other arguments and errors as for mifa_attention, plus MIFA_ERR_WORKSPACE (checked after the
 * other arguments).  When one range suffices the workspace is not used.
 */
int mifa_attention_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes mifa_attention_splitkv needs for this shape (0 for an invalid shape). */
int64_t mifa_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d);

/*
 * mifa_attention_splitkv_noalloc -- mifa_attention_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses that forbid hipMalloc):
 * the key-range partials live in a static 32 MiB device array of the library instead of a
 * caller workspace.  Same arguments (no workspace), same kernels and the same result, bit for bit.
 *   - The call itself calls no hipMalloc, hipFree or other allocating routine.  Each device holds
 *     its own copy of the array from the library's loading until the process ends; its address is
 *     resolved on the first call on that device.
 *   - The array is shared by every call on one device and keeps the last call's contents; calls
 *     that may overlap on one device race and must be ordered on one stream.  Nothing in it needs
 *     clearing: every call writes all the partials it reads.
 *   - MIFA_ERR_SCRATCH, checked after the other arguments and before any HIP call, when the
 *     partials (mifa_splitkv_workspace_bytes of the shape) exceed 32 MiB.  Errors otherwise as for
 *     mifa_attention_splitkv without MIFA_ERR_WORKSPACE.
 */
int mifa_attention_splitkv_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                                   float scale, void* stream);

/*
 * mifa_bwd -- gradients of mifa_attention with respect to q, k and v.
 *
 * The pages give the forward only (the ~100-line kernel of "Show HN: Flash Attention in ~100
 * lines of CUDA" leaves the matrix derivatives out); this is its backward by the chain rule,
 * with P = softmax(c q k^T [+ causal mask]) recomputed from the saved lse:
 *     dv = P^T dO,  dP = dO v^T,  D_i = sum_t dO_it o_it,  dS = P * (dP - D),
 *     dq = c dS k,  dk = c dS^T q.
 *
 *   q, k, v, causal, scale, B, H, Nq, Nk, d   exactly as passed to mifa_attention.
 *   o, lse   float32 [B, H, Nq, d] and [B, H, Nq]: that call's outputs.  Read only.
 *   dO       bf16 [B, H, Nq, d]: gradient of the loss with respect to o.  Read only.
 *   dq       float32 [B, H, Nq, d]; dk, dv float32 [B, H, Nk, d].  Fully overwritten.
 *   workspace  device memory of at least mifa_bwd_workspace_bytes(B, H, Nq) bytes, 16-byte
 *            aligned; overwritten (it holds D and the LSE in log2 units).  Not to be touched until the stream has passed
 *            the call; calls that share a workspace must be ordered on a stream.
 *   workspace_bytes  its size in bytes.
 *   stream   hipStream_t (as void*); NULL for the null stream.
 * Layouts as for mifa_fwd (d fastest).  q, k, v, o, dO, dq, dk, dv 16-byte aligned; lse 4-byte.
 * Outputs must not overlap the inputs or each other (not checked).  Rows of a causal problem
 * that see no key do not occur (Nq <= Nk is required).  The result does not depend on the
 * launch: no atomics are used, and repeated calls give identical bits.
 * Errors: as for mifa_attention (NULL_POINTER also for o, dO, dq, dk, dv; MISALIGNED also for
 * o, dO, dq, dk, dv), plus MIFA_ERR_WORKSPACE, checked last.
 * Accuracy: products are exact, accumulation is float32, and P and dS are rounded to bf16 before
 * they multiply dO, q and k.
 */
int mifa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dO, float* dq, float* dk, float* dv, int64_t B, int64_t H, int64_t Nq,
             int64_t Nk, int64_t d, int causal, float scale, void* workspace,
             int64_t workspace_bytes, void* stream);

/*
 * mifa_bwd_strided -- mifa_bwd on tensors of any (batch, head, row) strides, with O read as
 * float32 or bf16 and the gradients written as float32 or bf16 (what an autograd function over
 * mifa_attention_strided needs: gradients in the inputs' layout and type, without copies).
 *
 *   strides     host array of 24 int64: the (batch, head, row) strides, in elements, of q, k,
 *               v, o, dO, dq, dk, dv in that order; d is contiguous.  Rules as for
 *               mifa_attention_strided (>= 0, multiples of 8, row strides below 2^24).
 *   o_dtype     type of o: MIFA_DTYPE_F32 or MIFA_DTYPE_BF16.
 *   grad_dtype  type of dq, dk, dv: MIFA_DTYPE_F32 or MIFA_DTYPE_BF16 (rounded to nearest even).
 * Other arguments as for mifa_bwd.  Errors in the order NULL (strides too), shape, d, pointer
 * alignment, scale, size, then the dtypes, then the strides, then the workspace.
 */
int mifa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                     int64_t Nq, int64_t Nk, int64_t d, const int64_t* strides, int o_dtype,
                     int grad_dtype, int causal, float scale, void* workspace,
                     int64_t workspace_bytes, void* stream);

/* Workspace bytes mifa_bwd needs for this shape (0 for an invalid shape). */
int64_t mifa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq);

/*
 * mifa_softmax_rows -- the row softmax on its own, with the online normaliser.
 *
 * For every row r of X and s_rj = scale * x_rj:
 *
 *     y_rj  = exp(s_rj - m_r) / l_r,   m_r = max_j s_rj,   l_r = sum_j exp(s_rj - m_r)
 *     lse_r = m_r + ln l_r
 *
 * This is the online-softmax trick of the interview "Tri Dao: prediction" (transcript) taken
 * by itself: the maximum and the sum come from one pass over the row, the sum being rescaled
 * whenever the running maximum grows, and a second pass normalises.  Rows of up to 32,768
 * elements are read from memory once (they stay on chip between the passes).
 *
 *   x      device pointer, `rows` rows of `cols` elements of type `dtype`, contiguous, the
 *          column index fastest: element (r, j) at r*cols + j.  Read only.  An entry equal to
 *          -inf takes no weight (for every scale); each row needs at least one finite entry
 *          (a row of -inf only gives unspecified values).  Other entries must be finite.
 *   y      device pointer, same shape and type, fully overwritten.  y may equal x (in place);
 *          any other overlap is undefined.  bf16 outputs are rounded to nearest even.
 *   lse    device pointer to `rows` float32 values, fully overwritten; or NULL to skip it.
 *   rows, cols  each >= 1 and < 2^31.
 *   dtype  MIFA_DTYPE_BF16 or MIFA_DTYPE_F32 (for both x and y).
 *   scale  multiplies x before the softmax; any finite value, including 0 and negatives.
 *   stream hipStream_t (as void*); NULL for the null stream.
 *
 * Alignment: x and y aligned to the element size, lse to 4 bytes (MIFA_ERR_MISALIGNED
 * otherwise).  16-byte aligned bases with rows a multiple of 16 bytes take vector loads.
 * Errors, in order: MIFA_ERR_NULL_POINTER (x or y NULL), MIFA_ERR_BAD_SHAPE,
 * MIFA_ERR_BAD_DTYPE, MIFA_ERR_MISALIGNED, MIFA_ERR_BAD_SCALE, MIFA_ERR_TOO_LARGE,
 * MIFA_ERR_HIP.  Ownership, streams and threading as for every entry point (see the top of
 * this file).
 * Accuracy: fp32 arithmetic (exp2 with scale*log2(e) folded in); about 1e-6 relative for
 * fp32 outputs, one bf16 rounding for bf16 outputs.
 */
int mifa_softmax_rows(const void* x, void* y, float* lse, int64_t rows, int64_t cols, int dtype,
                      float scale, void* stream);

/*
 * mifa_clock_probe -- measures the engine clock the GPU sustains while other work runs
 * (a measurement aid, not part of the attention path).  Roofline fractions of the
 * compute-bound kernels are quoted against the bf16 MFMA peak at the nominal 2.4 GHz clock;
 * the fraction of the peak at the clock actually sustained separates the kernel's share of
 * the gap from the clock's.
 *
 * Launches 8 single-wave workgroups on `stream`.  Each reads the shader-clock counter
 * (s_memtime, one count per engine-clock cycle) and the fixed-rate real-time counter
 * (s_memrealtime) at its start, sleeps for span_us microseconds of real time, and reads both
 * again.  Launch it on a second stream while the work to be measured keeps the GPU busy on
 * another, with a short span (tens of microseconds) repeated as often as needed: a probe wave
 * holds a slot on its CU for the whole span, and a kernel that fills every CU's register file
 * cannot place a workgroup beside it.  The mean engine clock of probe w in MHz is
 *     (out[4w+2] - out[4w+0]) / (out[4w+3] - out[4w+1]) * realtime_khz / 1000.
 *   out          device pointer to 32 int64 values (8-byte aligned), overwritten when the
 *                kernel has run: {memtime start, realtime start, memtime end, realtime end}
 *                for each of the 8 probes.
 *   span_us      1 .. 2,000,000.  Each probe also stops after a bounded number of sleeps,
 *                so it ends even if the real-time counter were to stall.
 *   realtime_khz host pointer; receives the real-time counter's rate (kHz) before the launch.
 *   stream       hipStream_t (as void*); NULL for the null stream.
 * Errors: MIFA_ERR_NULL_POINTER (out or realtime_khz NULL), MIFA_ERR_BAD_SHAPE (span_us out
 * of range), MIFA_ERR_MISALIGNED, MIFA_ERR_HIP.
 */
int mifa_clock_probe(long long* out, int64_t span_us, int* realtime_khz, void* stream);

/* Human-readable name of a status code; never NULL (unknown codes give "unknown status"). */
const char* mifa_status_string(int status);

/* Library version string, e.g. "mifa 0.1.0 gfx950". */
const char* mifa_version(void);

/* The hipError_t of the last MIFA_ERR_HIP returned on the calling thread (0 if none). */
int mifa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MIFA_H */
