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
 *   - Pointers named q, k, v, o, lse are DEVICE pointers (hipMalloc'd or equivalent) on
 *     the current HIP device.  The caller allocates and owns them; the library allocates
 *     nothing, keeps no pointer after returning and has no mutable global state, so calls
 *     are thread-safe and re-entrant.
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
  MIFA_ERR_BAD_SHAPE = 2,      /* B, H or N < 1 */
  MIFA_ERR_UNSUPPORTED_D = 3,  /* head dimension d is not 64 or 128 */
  MIFA_ERR_MISALIGNED = 4,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  MIFA_ERR_BAD_SCALE = 5,      /* scale is NaN or infinite */
  MIFA_ERR_TOO_LARGE = 6,      /* N*d >= 2^31, or B*H*ceil(N/128) >= 2^31 work tiles */
  MIFA_ERR_HIP = 7             /* the HIP runtime rejected the launch; see mifa_last_hip_error */
} mifa_status;

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
