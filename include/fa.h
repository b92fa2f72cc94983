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
#define FA_ERR_BAD_RANGE 11        /* fa_fwd_ex / fa_bwd_ex: key chunk outside [0, Nk], a window without
                                      causal, or |q_offset| > 2^30; fa_fwd_varlen: max_seqlen_q > total_q;
                                      fa_bwd_varlen: max_seqlen_q > total_q or max_seqlen_k > total_k */
#define FA_ERR_SCRATCH_LIMIT 12    /* fa_bwd_noalloc: B*H*N exceeds FA_NOALLOC_MAX_ROWS */

/* Rows (B*H*N) fa_bwd_noalloc accepts: the size of its per-GPU scratch array of floats (16 MiB). */
#define FA_NOALLOC_MAX_ROWS 4194304

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

/*
 * fa_fwd_ex -- the same forward over a chunk of keys, for queries placed anywhere in the sequence, with an
 * optional sliding window.  fa_fwd(...) is fa_fwd_ex(..., Nq = Nk = N, window = -1, q_offset = 0,
 * kv_start = 0, kv_len = N, ...).
 *
 * Processing one long key sequence in chunks and combining the partial results through their lse is the
 * single-GPU building block of ring and block-wise attention (page ai6s.net/6a0d3bfb..., section
 * "ops-transformer仓库里还有什么？"; a 64K sequence split into 8K pieces: page ai6s.net/6a140d07...,
 * section "多卡并行"); fa_merge below does the combination.  Sliding-window attention is one of the
 * variants the same page compares in section "与其他优化方法对比".
 *
 * q, o     : B*H*Nq*D elements of `dtype` in `layout` ([B][H][Nq][D] or [B][Nq][H][D]).
 * k, v     : B*H*Nk*D elements, same dtype and layout ([B][H][Nk][D] or [B][Nk][H][D]).
 * lse      : B*H*Nq fp32 values, [B][H][Nq].
 * Positions: query row i is at sequence position q_offset + i; key row j at position j.  Only the keys
 *            j in [kv_start, kv_start + kv_len) take part (the chunk; kv_len may be 0).  Key j is visible
 *            to query i iff it is in the chunk, j <= q_offset + i when causal, and
 *            j >= q_offset + i - window when window >= 0 (window >= 0 requires causal; window < 0: none).
 *            Queries that are the last Nq positions of an Nk-long sequence (prefill with a key cache) use
 *            q_offset = Nk - Nq.
 * Rows with no visible key get O = 0 and lse = -inf (the identity of the lse combination).
 * Limits: Nq, Nk <= 2^30, |q_offset| <= 2^30, and the other limits of fa_fwd with Nk for the key span.
 * Ownership, errors and check order as fa_fwd; FA_ERR_BAD_RANGE comes after the size limits.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
              int64_t Nq, int64_t Nk, int64_t D, int layout, int causal, int64_t window, int64_t q_offset,
              int64_t kv_start, int64_t kv_len, float scale, int dtype, void* stream);

/*
 * fa_merge -- combine n_parts partial results over disjoint key sets into the result over their union:
 * with M = max_s lse_s,  lse = M + ln sum_s exp(lse_s - M)  and  O = sum_s exp(lse_s - lse) O_s
 * (the max-shifted log-sum-exp combination of page ai6s.net/6a140d07..., section
 * "第二层：数值稳定性增强", for any number of parts).  Parts with lse = -inf contribute nothing; a row
 * where every part has lse = -inf gets O = 0 and lse = -inf.  Computed in fp32, rounded to `dtype`.
 *
 * o_parts  : n_parts consecutive tensors of B*H*N*D elements of `dtype` in `layout` (part s starts at
 *            element s*B*H*N*D).  Read only.
 * lse_parts: n_parts consecutive [B][H][N] fp32 arrays.  Read only.
 * o, lse   : the combined result, same shapes as one part.  Must not overlap the parts or each other.
 * Ownership and error conventions as fa_fwd (FA_ERR_BAD_DIM for n_parts < 1).
 */
int fa_merge(const void* o_parts, const float* lse_parts, int64_t n_parts, void* o, float* lse, int64_t B,
             int64_t H, int64_t N, int64_t D, int layout, int dtype, void* stream);

/*
 * fa_fwd_varlen -- the forward over a packed batch of sequences of different lengths, without padding
 * (the padding to a multiple of 128 that page hwcomputing.csdn.net/6a0d4444... needs, in its section on
 * sequence-length alignment, is not needed here).  Sequence b owns the query rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1]-1 of q and o and the key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v, and
 * attends only to its own keys.  With causal the two ends are aligned: query i of a sequence with Nq
 * queries and Nk keys sees its keys 0 .. Nk - Nq + i (a query that sees none gets O = 0, lse = -inf);
 * with Nq = Nk that is the ordinary causal mask.
 *
 * q, o       : [total_q][H][D] of `dtype` (each sequence is a [len][H][D] block, the BSND layout without
 *              the batch dimension).  k, v: [total_k][H][D].  q, k, v read only; o fully overwritten.
 * lse        : [H][total_q] fp32, fully overwritten.
 * cu_seqlens_q, cu_seqlens_k: device int32 arrays of B + 1 offsets; non-decreasing, starting at 0 and
 *              ending at total_q / total_k.  Read only.  The library cannot check their contents without
 *              synchronising; a sequence whose offsets fall outside [0, total] or decrease is skipped (its
 *              rows are left unwritten), so no offset array can cause an access outside the tensors.
 * max_seqlen_q: at least the longest query count (it sizes the launch grid); query rows of a sequence
 *              beyond it are left unwritten.  1 <= max_seqlen_q <= total_q.
 * dtype      : FA_DTYPE_FP16 or FA_DTYPE_BF16 (FA_DTYPE_FP32 returns FA_ERR_UNSUPPORTED).  D in {64, 128}.
 * total_q, total_k >= 1.  No window.  Ownership, stream semantics and error conventions as fa_fwd
 * (FA_ERR_BAD_RANGE for max_seqlen_q > total_q; cu arrays must be 4-byte aligned).
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int64_t B, int64_t H, int64_t total_q, int64_t total_k,
                  int64_t max_seqlen_q, int64_t D, int causal, float scale, int dtype, void* stream);

/*
 * fa_bwd -- gradients of the attention forward: for O = softmax(scale * Q K^T [+ causal]) V (the call
 * fa_fwd(q, k, v, o, lse, B, H, N, D, layout, causal, scale, dtype, ...) made) and the upstream gradient
 * dout = dL/dO, writes dq = dL/dQ, dk = dL/dK, dv = dL/dV.  The N x N probabilities are recomputed from
 * lse instead of being stored (page ai6s.net/6a0d3bfb..., section "FlashAttention在昇腾NPU上怎么跑？",
 * item 3).  No atomics: the result is the same bit for bit on every run, i.e. the deterministic mode of
 * page hwcomputing.csdn.net/6a0d4681..., section "反向传播的特殊处理" (fa_bwd_atomic is the other mode).
 *
 * q, k, v, o, dout: same shape, layout and dtype as in fa_fwd; o is the forward's output.  Read only.
 * lse   : the forward's [B][H][N] fp32 log-sum-exp (natural log).  Read only.
 * dq, dk, dv: outputs, shaped like q, in `dtype`; fully overwritten.
 * delta : caller-owned fp32 workspace of B*H*N floats; on return it holds D_i = sum_d dout_id o_id.
 * Outputs and workspace must not overlap each other or any input.
 * dtype : FA_DTYPE_FP32, FA_DTYPE_FP16 or FA_DTYPE_BF16 (fp32: fp32 MFMA end to end).  D in {64, 128}.
 * The call enqueues two kernels on `stream`; results are valid after the stream synchronises.  The
 * library allocates nothing.  Check order and error codes as fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t N, int64_t D, int layout,
           int causal, float scale, int dtype, void* stream);

/*
 * fa_bwd_atomic -- fa_bwd's gradients in the mode that accumulates with atomics (page
 * hwcomputing.csdn.net/6a0d4681..., section "反向传播的特殊处理": a deterministic mode next to a faster
 * one built on atomic adds).  One kernel per 128-key tile forms dK, dV and that tile's part of dQ from a
 * single pass over the queries; the dQ parts of all key tiles are summed into `dq_accum` with fp32
 * atomic adds, whose order varies from run to run, so dq can differ between runs in its last bits (dk,
 * dv and delta do not).  dq is then written from dq_accum, scaled and rounded to `dtype`.
 *
 * Arguments, layouts and ownership as fa_bwd, plus
 * dq_accum : caller-owned fp32 workspace shaped like q (B*H*N*D floats, same layout); overwritten (the
 *            call clears it first).  Must not overlap any input, output or delta.
 * dtype    : FA_DTYPE_FP16 or FA_DTYPE_BF16 (FA_DTYPE_FP32 returns FA_ERR_UNSUPPORTED).  D in {64, 128}.
 * The call enqueues three kernels on `stream`; results are valid after the stream synchronises.  The
 * library allocates nothing.  Errors as fa_bwd (FA_ERR_NULL for a null delta or dq_accum).
 */
int fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, float* dq_accum, int64_t B, int64_t H, int64_t N,
                  int64_t D, int layout, int causal, float scale, int dtype, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments without `delta`.  The D
 * workspace is a static device array of the library, FA_NOALLOC_MAX_ROWS floats per GPU, held until the
 * process ends; B*H*N beyond it returns FA_ERR_SCRATCH_LIMIT (checked with the other sizes, before any
 * HIP call).  The call allocates nothing.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be serialised by the caller.  Results
 * equal fa_bwd's bit for bit.  Other checks and errors as fa_bwd.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t D, int layout, int causal,
                   float scale, int dtype, void* stream);

/*
 * fa_bwd_ex -- the backward of fa_fwd_ex's rule: query row i at position q_offset + i, key row j at j,
 * causal hides keys after the query, a window (causal only) keys more than `window` before it.  P and
 * D are those of the softmax over every visible key of [0, Nk): pass the lse and O of the forward over
 * all of them (for a forward computed in key chunks, the merged lse and O).  The key chunk
 * [kv_start, kv_start + kv_len) restricts the work: dq (all Nq rows, overwritten) receives the chunk's
 * part of dQ, sum_{j in chunk} dS_ij k_j * scale, so the dq of disjoint chunks covering all keys add up
 * to dQ; dk and dv receive the chunk's rows and are left untouched elsewhere, so successive chunks can
 * fill one dk/dv.  This is the backward of attention computed in key chunks (page ai6s.net/6a0d3bfb...,
 * section "ops-transformer仓库里还有什么？", ring / block-wise attention).  fa_bwd(...) is
 * fa_bwd_ex(..., Nq = Nk = N, window = -1, q_offset = 0, kv_start = 0, kv_len = N, ...).
 *
 * q, o, dout, dq: [B][H][Nq][D] or [B][Nq][H][D]; k, v, dk, dv: [B][H][Nk][D] or [B][Nk][H][D]; lse and
 * delta: [B][H][Nq] fp32.  Checks, ownership and errors as fa_bwd, plus FA_ERR_BAD_RANGE as fa_fwd_ex.
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
              int layout, int causal, int64_t window, int64_t q_offset, int64_t kv_start, int64_t kv_len,
              float scale, int dtype, void* stream);

/*
 * fa_bwd_varlen -- the backward of fa_fwd_varlen: dQ, dK, dV of B packed sequences of different lengths
 * (page ai6s.net/6a0d3bfb..., section "FlashAttention在昇腾NPU上怎么跑？", item 3 for the recomputing
 * backward; the packed layout and the per-sequence rule are fa_fwd_varlen's).
 *
 * q, o, dout, dq: [total_q][H][D]; k, v, dk, dv: [total_k][H][D]; lse (the forward's) and delta (the
 * caller's fp32 workspace, written with D_i = sum_d dout_id o_id): [H][total_q].  cu_seqlens_q,
 * cu_seqlens_k: int32 device arrays of B+1 offsets as in fa_fwd_varlen; under causal each sequence's
 * query and key ends are aligned.  max_seqlen_q and max_seqlen_k bound the sequences' query and key
 * counts (the launch grid).  A sequence whose offsets fall outside [0, total] or decrease is skipped:
 * its rows of dq, dk, dv and delta are left untouched.  Rows of a sequence without queries get dK = dV
 * = 0, rows without keys dQ = 0.
 * dtype: FA_DTYPE_FP16 or FA_DTYPE_BF16 (FA_DTYPE_FP32 returns FA_ERR_UNSUPPORTED).  D in {64, 128}.
 * Errors as fa_fwd_varlen, plus the aliasing rules of fa_bwd; FA_ERR_BAD_RANGE when max_seqlen_q >
 * total_q or max_seqlen_k > total_k.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int64_t B, int64_t H, int64_t total_q, int64_t total_k,
                  int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, int causal, float scale, int dtype,
                  void* stream);

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
