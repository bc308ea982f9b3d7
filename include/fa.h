/*
 * fa.h — C ABI of the exact softmax attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact softmax attention
 *
 *     O = softmax(scale * Q K^T) V
 *
 * (the materialised attention of the "standard attention" code block in
 * "FlashAttention V2深度解析：反向传播显存优化让大模型训练不再OOM", section
 * "Attention反向传播的「内存泄漏」难题"), without ever storing the N x N score
 * matrix: the forward pass tiles Q and K/V and keeps a running row maximum and
 * exponential sum (the online / incremental softmax of "【词汇专栏】FlashAttention",
 * section 2.2 在线Softmax, and of "FlashAttention 在昇腾NPU上到底快在哪",
 * section 三、增量 Softmax), and saves one log-sum-exp per query row.  The
 * backward pass recomputes the probabilities from Q, K and that log-sum-exp
 * instead of reading a stored attention matrix (the recomputation principle of
 * "FlashAttention V2深度解析", section 改进1：IO感知的算子调度), so its extra memory
 * is O(N).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (memory of the current HIP device),
 *    16-byte aligned, densely packed, row-major:
 *        q, o, dO, dq : [B, H,   N, d]
 *        k, v, dk, dv : [B, Hkv, N, d]
 *        lse          : [B, H,   N]      float32
 *    Element type of q, k, v, o, dO, dq, dk, dv is given by `dtype`.
 *  - GQA / MQA: query head h reads KV head h / (H / Hkv) (contiguous groups);
 *    H must be a multiple of Hkv.  Hkv == H is ordinary multi-head attention.
 *  - `causal` != 0 applies the square causal mask: key j is visible to query i
 *    iff j <= i.
 *  - d must be 64 or 128.  N may be any value >= 1 (ragged tails are masked);
 *    one head's N x d slab must stay below 2 GiB.
 *  - `scale` multiplies Q K^T (typically 1/sqrt(d)); it must be finite and > 0.
 *  - lse[b,h,i] is the natural-log log-sum-exp of the scaled, masked scores of
 *    query row i.
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    backward workspace.  The library never allocates device memory, keeps no
 *    state across calls, and is safe to call from several threads.  Outputs must
 *    not alias inputs.
 *  - All work is enqueued on `stream` (0 = the default stream) and is
 *    asynchronous: a call returns once its kernels are launched.  Faults inside
 *    kernels surface at the caller's next synchronisation.
 *  - Errors: arguments are validated before anything is launched; an invalid
 *    call returns a non-zero status and enqueues nothing.  Nothing is printed,
 *    thrown or aborted across this boundary.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_BF16 = 0, /* bfloat16 storage, float32 accumulation and statistics */
  FA_F32 = 1   /* float32 storage and arithmetic throughout             */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad sizes, H % Hkv != 0, scale not finite and > 0 */
  FA_ERR_UNSUPPORTED = 2, /* d not in {64, 128}, unknown dtype                                   */
  FA_ERR_WORKSPACE = 3,   /* workspace null, misaligned or smaller than fa_bwd_workspace_size    */
  FA_ERR_HIP = 4,         /* a kernel launch failed                                              */
  FA_ERR_TOO_LARGE = 5    /* fa_bwd_noalloc: the sizes need more than its fixed scratch holds    */
} fa_status_t;

/*
 * Forward pass.  Writes o = softmax(scale * q k^T) v and lse.
 * Inputs q, k, v; outputs o and lse (see layouts above).
 *
 * Input domain of FA_BF16: the P V product runs on the fp16 matrix cores
 * (the pages' forward runs in fp16: "FlashAttention V2深度解析", section
 * 性能调优技巧, 混合精度训练), with V converted from bf16 to fp16.  That
 * conversion is exact for 2^-14 <= |v| <= 65280, the largest bfloat16 below
 * fp16's overflow threshold; smaller magnitudes keep an absolute error below
 * 2^-25.  Every element of v must satisfy |v| <= 65280: a larger one becomes
 * inf and makes o inf or NaN while the call still returns FA_OK (values are
 * not inspected).  FA_F32 has no such limit.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v,
                   void* o, float* lse,
                   int B, int H, int Hkv, int N, int d,
                   float scale, int causal, fa_dtype_t dtype, hipStream_t stream);

/*
 * Forward pass on 8-bit float inputs.  q, k, v hold OCP e4m3 codes (one byte
 * per element: sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 * finite 448) in the layouts above; the value of an element is its code
 * times the tensor's scale (q_scale, k_scale, v_scale: finite, > 0).  Writes
 * o in bf16 and lse as fa_fwd does, for o = softmax(scale * Q K^T) V of those
 * values.  Both products run on the 8-bit matrix cores with float32
 * accumulation; the probabilities are rounded to e4m3 for the P V product
 * (relative error at most 2^-4 each), while the row sums and lse use them
 * unrounded.  The fp8 variant of the pages' kernel family ("【词汇专栏】
 * FlashAttention", section 3.3, FA3) fixes no scaling recipe; this is
 * per-tensor scaling.  d must be 128 (FA_ERR_UNSUPPORTED otherwise).
 */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* v,
                       void* o, float* lse,
                       int B, int H, int Hkv, int N, int d,
                       float scale, float q_scale, float k_scale, float v_scale,
                       int causal, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: two float32 per
 * query row (-D_i = -sum_c dO_ic * O_ic and lse_i * log2 e) and, only for GQA
 * shapes whose query heads are spread over several workgroups of the dK/dV
 * kernel, float32 partial sums of dK and dV (at most 8 * B * H * N * d
 * bytes).  Linear in the sequence length N.  Valid for both values of
 * `causal`.  Returns 0 when the sizes are invalid.
 */
size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d, fa_dtype_t dtype);

/*
 * Backward pass of L = sum(dO * O) for the forward above (the FlashAttention-2
 * backward of "FlashAttention V2深度解析：反向传播显存优化让大模型训练不再OOM",
 * section 改进1：IO感知的算子调度: P is recomputed from q, k and lse, never
 * read from memory).  Inputs q, k, v, the forward's o and lse, and dO; outputs
 * dq, dk, dv (same dtype and layout as q, k, v).  dk and dv sum over the query
 * heads of each GQA group.  `workspace` is device memory of at least
 * fa_bwd_workspace_size(...) bytes, 256-byte aligned, owned by the caller and
 * not touched by anything else until the enqueued work has finished; its
 * contents on entry do not matter.  Results are deterministic (no atomics).
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v,
                   const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv,
                   int B, int H, int Hkv, int N, int d,
                   float scale, int causal, fa_dtype_t dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (minus the workspace), layouts, results
 * and errors as fa_bwd; the workspace is a fixed 32 MiB device array inside
 * the library, one per GPU it runs on, held until the process ends (its
 * device address is looked up on the first call on each device; nothing is
 * allocated or freed by any call).  Sizes whose workspace
 * (fa_bwd_workspace_size) exceeds 32 MiB return FA_ERR_TOO_LARGE and enqueue
 * nothing.  Every call on one GPU shares that array and leaves its last
 * contents there (nothing in it needs to start at zero): calls whose work
 * overlaps on one GPU (other streams, other host threads without ordering)
 * race on it and must be serialised by the caller.
 */
fa_status_t fa_bwd_noalloc(const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           void* dq, void* dk, void* dv,
                           int B, int H, int Hkv, int N, int d,
                           float scale, int causal, fa_dtype_t dtype, hipStream_t stream);

/*
 * The phases of fa_bwd, callable one by one (same arguments, layouts,
 * workspace and error rules as fa_bwd).  fa_bwd is fa_bwd_dq followed by
 * fa_bwd_dkdv on its stream; these exist so that callers and benchmarks can
 * time or schedule the phases separately.
 *
 * fa_bwd_preprocess: -D_i = -sum_c dO_ic * O_ic and lse_i * log2 e into the
 *   workspace.  Reads o, dO and lse.
 * fa_bwd_dq: recomputes P = exp(scale q k^T - lse) and dS = P * (dO v^T - D)
 *   and writes dq = scale dS k.  It forms D and lse * log2 e itself (reading
 *   o, dO and lse) and writes them to the workspace too, with the same bits
 *   as fa_bwd_preprocess.
 * fa_bwd_dkdv: recomputes P and dS the same way and writes dv = P^T dO and
 *   dk = scale dS^T q.  Reads D and lse * log2 e from the workspace: enqueue
 *   fa_bwd_dq or fa_bwd_preprocess (same sizes, same workspace) before it.
 * Any such order gives exactly fa_bwd's results.
 */
fa_status_t fa_bwd_preprocess(const void* o, const void* dO, const float* lse,
                              int B, int H, int Hkv, int N, int d, fa_dtype_t dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

fa_status_t fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                        void* dk, void* dv,
                        int B, int H, int Hkv, int N, int d,
                        float scale, int causal, fa_dtype_t dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v,
                      const void* o, const void* dO, const float* lse,
                      void* dq,
                      int B, int H, int Hkv, int N, int d,
                      float scale, int causal, fa_dtype_t dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Attention with dropout on the probabilities, fused into the forward and
 * backward passes ("FlashAttention 在昇腾NPU上到底快在哪", section 二, names
 * dropout fused into the attention operator together with the softmax; the
 * rate argument is that of PyTorch's fused attention in "【词汇专栏】FlashAttention",
 * section 5.1).  The pages give neither the generator nor the keep rule; this
 * library defines them:
 *
 *     P = softmax(scale * Q K^T) (masks as in fa_fwd),  O = (P * M / keep) V
 *     lse: as in fa_fwd (the mask M does not enter it)
 *
 * M[b,h,i,j] is 1 when the byte of element (i, j) is >= t, t = round(256 * p_drop),
 * keep = (256 - t) / 256.  The bytes come from Philox4x32-10 (Salmon et al.,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011): one call per 4 x 4
 * block of query rows 4a..4a+3 and keys 4c..4c+3, with counter
 * (c, a, b*H + h, offset) and key (seed & 0xffffffff, seed >> 32); word r of
 * the result belongs to query 4a + r, its byte e (little-endian) to key 4c + e.
 * The mask depends on (seed, offset, b, h, i, j) only, so fa_bwd_dropout with
 * the same seed and offset regenerates it instead of reading it, and a caller
 * that varies `offset` per call (or per layer) gets fresh masks.
 *
 * p_drop: finite, 0 <= p_drop with round(256 * p_drop) <= 255 (the rate is
 * quantised to t/256); t == 0 runs fa_fwd / fa_bwd.  Otherwise the same
 * arguments, layouts, workspace, ownership and errors as fa_fwd and fa_bwd.
 * fa_bwd_dropout takes the O written by fa_fwd_dropout and returns the
 * gradients of sum(O * dO) for that same mask.  fa_fwd_dropout has fa_fwd's
 * input domain: for FA_BF16 every |v| <= 65280.
 */
fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int N, int d,
                           float scale, int causal, float p_drop,
                           unsigned long long seed, unsigned int offset,
                           fa_dtype_t dtype, hipStream_t stream);

fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           void* dq, void* dk, void* dv,
                           int B, int H, int Hkv, int N, int d,
                           float scale, int causal, float p_drop,
                           unsigned long long seed, unsigned int offset,
                           fa_dtype_t dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Attention over a key/value cache: Nq query rows against Nk keys.
 *
 *   q, o : [B, H, Nq, d]    k, v : [B, Hkv, Nk, d]    lse : [B, H, Nq] float32
 *
 * Same conventions as fa_fwd (device pointers, GQA mapping, d, dtype, scale,
 * lse, ownership, errors), except for the mask: `causal` != 0 aligns it at the
 * bottom right, key j is visible to query i iff j <= i + (Nk - Nq), so the
 * last query row sees the whole cache (decoding Nq new tokens against Nk
 * cached ones, of which they are the last; Nq == Nk is fa_fwd's square mask).
 * Causal calls need Nq <= Nk.  Nq = 1 is decoding one token.
 *
 * The keys are split into `nsplit` ranges of equal length (a multiple of 64;
 * 0 lets the library choose from the sizes, at least 256 keys per range and
 * enough workgroups to fill the GPU), each processed by its own workgroups,
 * which write float32 partial results (O over the range, normalised over the
 * range, and the range's log-sum-exp) into `workspace`; fa_merge then
 * combines them into o and lse on the same stream.  When the sizes give a
 * single range, its workgroups write o and lse directly (the values the
 * merge would produce) and no merge runs.  The partials are the
 * per-block results of the incremental softmax of "FlashAttention 在昇腾NPU上到底
 * 快在哪", section 三、增量 Softmax, the merge its correction step, here across
 * workgroups: short query blocks (the cache reuse of section 七 of the same
 * page) get their parallelism from the keys.
 *
 * Input domain: as fa_fwd, for FA_BF16 every |v| <= 65280 (the kernel for
 * more than 32 query rows per KV head runs P V in fp16; the one for at most
 * 32 rows in bf16, which has no such limit, but callers cannot rely on which
 * one runs).
 *
 * `workspace`: device memory of at least fa_fwd_splitkv_workspace_size(...)
 * bytes for the same sizes and nsplit, 256-byte aligned, owned by the caller;
 * contents on entry do not matter.  Returns FA_ERR_WORKSPACE when it is
 * missing, misaligned or too small, FA_ERR_INVALID_ARG for causal calls with
 * Nq > Nk, nsplit < 0 or sizes out of range.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, fa_dtype_t dtype, int nsplit);

fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           int B, int H, int Hkv, int Nq, int Nk, int d,
                           float scale, int causal, fa_dtype_t dtype, int nsplit,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Merge of attention results computed over disjoint key ranges (on this
 * device by fa_fwd_splitkv, or elsewhere, e.g. one range per device of a
 * sequence-sharded cache):
 *
 *   o_parts   : [nsplit, rows, d] float32, each range's output normalised over the range
 *   lse_parts : [nsplit, rows]    float32, each range's log-sum-exp (-inf: the range
 *                                  holds no key visible to the row; its o_parts row is ignored)
 *   o         : [rows, d]  dtype          lse : [rows] float32
 *
 * lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s, i.e. the
 * attention over the union of the ranges.  A row with lse_s = -inf in every
 * range gets o = 0, lse = -inf.  All pointers are 16-byte aligned device
 * pointers; nsplit >= 1, rows >= 1, d in {64, 128}.
 */
fa_status_t fa_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                     int nsplit, long rows, int d, fa_dtype_t dtype, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(fa_status_t s);

/*
 * Identifies the sources this library was built from: 16 hex digits of a
 * SHA-256 over its source files, this header and the compile flags (a static
 * string, never NULL).  A binding compares it with the hash of the sources it
 * ships with and refuses a stale binary.
 */
const char* fa_build_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
