/*
 * fa.h -- C ABI of the MI355X (gfx950) attention forward library, libfa.so.
 *
 * One operation: O = softmax(scale * Q K^T [+ causal mask]) V and the per-row log-sum-exp, computed
 * tile by tile with a running row maximum m and running exponential sum l, so that the N x N score
 * matrix never reaches device memory.
 *   - The formula and its three steps: page "FlashAttention：让长文本推理不再"卡显存"" (ai6s.net,
 *     6a0d42d8...), section "Attention 的显存黑洞".
 *   - Tiling and the (m, l) online-softmax update: same page, sections "1. 分块计算（Tiling）" and
 *     "2. 在线归一化（Online Softmax）".
 *   - The per-row log-sum-exp output, shape [B, H, rows]: page ai6s.net/6a140d07..., section
 *     "第二层：数值稳定性增强".
 *   - A causal flag instead of a mask tensor, key j visible to query i iff j <= i: page
 *     ai6s.net/6a0d3bfb..., the causal-mask section (mask = triu(ones, diagonal=1) marks hidden
 *     entries); diagonal tile skipping: page hwcomputing.csdn.net/6a0d4681..., section
 *     "Causal Mask的实现差异", mode 2.
 *   - Layouts [batch, seq, heads, dim] and [batch, heads, seq, dim]: page hwcomputing.csdn.net/
 *     6a0d4444... (the BSND smoke test and the model hook that transposes [b, h, s, d] to BSND) and
 *     page hwcomputing.csdn.net/6a0d4681..., section "数据布局：这步做错后面全白搭".
 *   - Errors are reported as status codes, never as a crash (the deployment page's error table lists
 *     a segfault for host tensors, a wrong-layout error and a head-count mismatch).
 *
 * Everything here is plain C: pointers, 64-bit sizes, ints and a float.  No framework types.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor layouts.  Both are packed and contiguous, with the head dimension D innermost.
 * FA_LAYOUT_BHSD: [B][H][N][D]  element (b,h,i,d) at ((b*H + h)*N + i)*D + d
 * FA_LAYOUT_BSND: [B][N][H][D]  element (b,h,i,d) at ((b*N + i)*H + h)*D + d
 * (N is the sequence length here; the pages' "BSND" names heads "N" and sequence "S".) */
#define FA_LAYOUT_BHSD 0
#define FA_LAYOUT_BSND 1

/* Element types of q, k, v and o. */
#define FA_DTYPE_FP32 0 /* IEEE binary32; computed in fp32 end to end */
#define FA_DTYPE_FP16 1 /* IEEE binary16; fp16 MFMA products, fp32 accumulation and softmax */
#define FA_DTYPE_BF16 2 /* bfloat16;      bf16 MFMA products, fp32 accumulation and softmax */

/* Status codes. */
#define FA_OK 0
#define FA_ERR_NULL 1              /* a required pointer is NULL */
#define FA_ERR_BAD_DIM 2           /* B, H, N or D < 1 */
#define FA_ERR_BAD_LAYOUT 3        /* layout is not FA_LAYOUT_* */
#define FA_ERR_BAD_DTYPE 4         /* dtype is not FA_DTYPE_* */
#define FA_ERR_UNSUPPORTED 5       /* D not in {64, 128}, or sizes beyond the limits below */
#define FA_ERR_BAD_SCALE 6         /* scale is NaN or infinite, or |scale|*log2(e) overflows fp32 */
#define FA_ERR_MISALIGNED 7        /* a base pointer is not 16-byte aligned */
#define FA_ERR_ALIAS 8             /* o or lse overlaps an input, or o overlaps lse */
#define FA_ERR_NOT_DEVICE_MEMORY 9 /* a pointer is not device memory of the current device */
#define FA_ERR_HIP 10              /* the HIP runtime reported an error; see fa_last_error() */

/* Limits: 1 <= N <= 2^30, B*H <= 2^31 - 1, every tensor's byte size must fit in int64, and one head's
 * span -- (N - 1) * (bytes between consecutive positions) + D * element size -- must be below 2^31
 * (BHSD bf16 D=128: N up to 8M; BSND: N * H * D * element size below 2 GiB). */

/*
 * fa_fwd -- enqueue the attention forward on `stream` and return.
 *
 * q, k, v  : device pointers to B*H*N*D elements of `dtype`, in `layout`.  Read only.
 * o        : device pointer, same shape, layout and dtype as q.  Fully overwritten with
 *            O[b,h,i,:] = sum_j softmax_j(scale * q_i . k_j) v_j over the visible keys j,
 *            rounded to nearest-even into `dtype`.
 * lse      : device pointer to B*H*N fp32 values in [B][H][N] order whatever the layout.  Fully
 *            overwritten with lse[b,h,i] = ln sum_j exp(scale * q_i . k_j) over the visible keys.
 * B, H, N, D : batch, heads, sequence length (queries = keys = N), head dimension (64 or 128).
 * layout   : FA_LAYOUT_BHSD or FA_LAYOUT_BSND.
 * causal   : 0 = every key visible; 1 = key j visible to query i iff j <= i.
 * scale    : logit multiplier, used as given (0 gives the plain mean of the visible V rows; any
 *            finite value, negative included, is accepted).  Callers wanting 1/sqrt(D) pass it.
 * dtype    : FA_DTYPE_*.
 * stream   : a hipStream_t (NULL = the default stream).
 *
 * Ownership: the caller owns all five buffers.  The library allocates no device memory, keeps no
 * state between calls, never synchronises and never frees.  Results are valid once the stream has
 * reached this point.  Thread-safe and reentrant.
 *
 * Errors: arguments are checked before any HIP call, in the order NULL, layout, dtype, dims, D and
 * limits, scale, alignment, aliasing; then device residency.  On any error nothing is launched and
 * o, lse are untouched.  NaN or infinite input elements are not checked; they propagate.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
           int64_t N, int64_t D, int layout, int causal, float scale, int dtype, void* stream);

/* Static description of a status code ("ok", "null pointer", ...).  Never NULL. */
const char* fa_status_str(int status);

/* The calling thread's message for its most recent FA_ERR_HIP (empty string if none). */
const char* fa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
