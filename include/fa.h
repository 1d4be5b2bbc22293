/*
 * fa.h - C ABI of the MI355X (gfx950) O(N)-memory fused attention library.
 *
 * The library computes scaled-dot-product attention for training without ever
 * materialising an (N, N) score or mask matrix.  The forward saves only the
 * output O and the per-row log-sum-exp; the backward recomputes the softmax
 * tile by tile from Q, K and that log-sum-exp (mlx-train-perf 0.5.1 README,
 * section "Flash-attention training path": O(N) saved state, tiles recomputed).
 * Masking is causal, optionally block-diagonal by a per-token segment id, so a
 * token attends another only when both belong to the same packed sequence
 * (same README, section "Sequence packing"; mlx-train-perf changelog, section
 * "Added": PACKED variants of the forward, dQ and dK/dV kernels driven by an
 * O(N) per-token segment id, never a materialised mask).
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous, row-major (B, H, N, D) device buffers of
 *     the element type `dtype` (bf16 or fp32), D in {64, 96, 128}, as in the
 *     README's "If you maintain a trainer" section ((B, H, N, D) with head_dim
 *     in {64, 96, 128}).
 *   - Grouped-query heads (same section: grouped query heads mapped
 *     contiguously): k, v, dk and dv have Hkv heads, H a multiple of Hkv, and
 *     query head h reads key/value head h / (H / Hkv).  Hkv = H is plain
 *     multi-head attention.  dk and dv of a key/value head are the sums over
 *     its H / Hkv query heads, formed inside one workgroup (no atomics).
 *   - `lse` is a (B, H, N) fp32 device buffer holding the natural-log
 *     log-sum-exp of scale * q_i . k_j over the keys row i may see.
 *   - `seg` is NULL (no packing) or a (B, N) int32 device buffer of segment ids
 *     that must be non-decreasing along each row (contiguous segments).  Query
 *     i sees key j iff (causal == 0 or j <= i) and (seg == NULL or
 *     seg[b][i] == seg[b][j]).  A row whose ids decrease gives unspecified
 *     values but every access stays in bounds; fa_check_seg validates a host
 *     copy, and the int32 at workspace offset 0 is set non-zero by the device
 *     when a decrease is seen.
 *   - Tensor pointers must be 16-byte aligned, lse and seg 4-byte aligned, the
 *     workspace 256-byte aligned.
 *   - The caller owns every buffer, including the workspace (size from
 *     fa_workspace_bytes).  The library never allocates device memory and keeps
 *     no state between calls beyond a per-device record of the architecture
 *     check and the compute-unit count (which sets the launch order of small
 *     causal grids, never a result).
 *   - Calls are asynchronous on `stream` (a hipStream_t of the current device;
 *     NULL means the default stream).  Outputs are overwritten, never
 *     accumulated; inputs are only read.  Two calls that share a workspace
 *     must be ordered on one stream.
 *   - Errors: arguments are validated on the host before any HIP call; a
 *     refused call returns a non-zero fa_status and launches nothing
 *     ("typed refusals, never silent fallbacks": README, "If you maintain a
 *     trainer").  FA_ERR_HIP reports a failed launch.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,       /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,      /* B, H, Hkv or N < 1, H not a multiple of Hkv, or sizes
                              beyond the supported range */
    FA_ERR_HEAD_DIM = 3,   /* D not in {64, 96, 128} */
    FA_ERR_DTYPE = 4,      /* dtype is neither FA_BF16 nor FA_FP32 (fp16 is refused) */
    FA_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than fa_workspace_bytes() */
    FA_ERR_ALIGN = 6,      /* a pointer violates the alignment rules above */
    FA_ERR_SCALE = 7,      /* scale is not a finite positive number */
    FA_ERR_SEG = 8,        /* fa_check_seg: ids decrease somewhere along a row */
    FA_ERR_HIP = 9,        /* a HIP call or kernel launch failed */
    FA_ERR_DEVICE = 10,    /* the current device is not a gfx950 GPU (or none) */
    FA_ERR_SCRATCH = 11    /* fa_bwd_noalloc: the shape needs more workspace than
                              FA_NOALLOC_MAX_BYTES */
} fa_status;

typedef enum fa_dtype {
    FA_BF16 = 0,
    FA_FP32 = 1
} fa_dtype;

/* Largest supported sequence length (rows per head).  In addition one head's
 * (N, D) matrix must stay below 2^31 bytes (N * D * element size), else
 * FA_ERR_SHAPE. */
#define FA_MAX_N (1 << 22)

/*
 * Bytes of workspace fa_fwd (for_bwd = 0) or fa_bwd (for_bwd = 1) needs for
 * this shape.  The method keeps O(N) state per head (mlx-train-perf 0.5.1
 * README, "Flash-attention training path": the forward saves only the
 * output and the log-sum-exp, and the backward recomputes tiles from them),
 * so the workspace is O(B*H*N): 256 bytes of flags, plus
 * for the backward two fp32 (B, H, N) arrays (the row sums
 * D_i = dO_i . O_i and LSE / scale, both stored negated, written by the dQ
 * kernel for dK/dV), plus with has_seg two per-tile range tables of
 * B * ceil(N/32) int32 pairs and two longest-first work lists of
 * B * ceil(N/32) int32 quadruples (the packed schedule: changelog, "Added",
 * cross-segment block skipping).  Never the (N, N) scores or mask.
 * Returns 0 for shapes fa_fwd / fa_bwd would refuse.  Makes no HIP call.
 */
size_t fa_workspace_bytes(int B, int H, int N, int D, int has_seg, int for_bwd);

/*
 * Forward pass.  Writes o = softmax(scale * q k^T, masked) v and lse.
 *   q       : (B, H, N, D) `dtype`, read only.
 *   k, v    : (B, Hkv, N, D) `dtype`, read only.
 *   seg     : (B, N) int32 or NULL.
 *   scale   : softmax scale (typically 1/sqrt(D)), finite and > 0.
 *   causal  : non-zero for causal masking.
 *   o       : (B, H, N, D) `dtype`, written.
 *   lse     : (B, H, N) fp32, written.
 *   ws      : workspace of at least fa_workspace_bytes(B,H,N,D,seg!=NULL,0)
 *             bytes (may be NULL when that is 0).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, const int32_t* seg,
                 float scale, int causal, void* o, float* lse,
                 int B, int H, int Hkv, int N, int D, fa_dtype dtype,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Backward pass from the output gradient dO (no gradient flows into lse).
 * Recomputes P = exp(scale q k^T - lse) tile by tile and writes
 *   dq = scale * dS k,  dk = scale * dS^T q,  dv = P^T dO,
 * with dS = P * (dO v^T - D_i) and D_i = dO_i . O_i taken from the stored o.
 *   q, o, dO       : (B, H, N, D) `dtype`, read only; o and lse come from
 *                    fa_fwd with the same q, k, v, seg, scale and causal.
 *   k, v           : (B, Hkv, N, D) `dtype`, read only.
 *   lse            : (B, H, N) fp32 from fa_fwd.
 *   seg, scale, causal : must equal the forward's.
 *   dq             : (B, H, N, D) `dtype`, written.
 *   dk, dv         : (B, Hkv, N, D) `dtype`, written (summed over each
 *                    key/value head's query heads).
 *   ws             : workspace of at least fa_workspace_bytes(..., 1) bytes.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dO, const float* lse, const int32_t* seg,
                 float scale, int causal, void* dq, void* dk, void* dv,
                 int B, int H, int Hkv, int N, int D, fa_dtype dtype,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * fa_bwd with per-stage HIP events, for profiling callers that need the time
 * of each backward kernel on its own stream.  `events` is NULL (then this is
 * fa_bwd) or points to 3 hipEvent_t handles, each may be NULL, created by the
 * caller on the current device.  They are recorded on `stream`: events[0]
 * before the dQ kernel (which also computes D_i), events[1] after it, before
 * the dK/dV kernel, events[2] after that.  Any segment schedule kernels run
 * before events[0].  Same arguments and errors as fa_bwd, plus FA_ERR_HIP if
 * recording an event fails.
 */
fa_status fa_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                       const void* dO, const float* lse, const int32_t* seg,
                       float scale, int causal, void* dq, void* dk, void* dv,
                       int B, int H, int Hkv, int N, int D, fa_dtype dtype,
                       void* ws, size_t ws_bytes, void* stream, void* const* events);

/*
 * fa_bwd without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * training loops, harnesses that forbid hipMalloc.  The workspace is a
 * static device array of FA_NOALLOC_MAX_BYTES inside the library, one per GPU,
 * held from the first call on that GPU until the process ends; the call makes
 * no hipMalloc, hipFree or other allocating call.  Arguments, outputs and
 * results are those of fa_bwd (the same kernels run), plus FA_ERR_SCRATCH,
 * returned before any HIP call, when fa_workspace_bytes(B, H, N, D,
 * seg != NULL, 1) exceeds FA_NOALLOC_MAX_BYTES (for example B * H * N above
 * about 4 million rows without seg).  Nothing in the array needs to start at
 * zero: every call writes each word it later reads.  All calls on one GPU
 * share its array, which keeps the last call's contents: calls that overlap
 * on one GPU (two streams, or two threads) race and must be ordered by the
 * caller.  FA_ERR_HIP if the array's device address cannot be obtained.
 */
#define FA_NOALLOC_MAX_BYTES ((size_t)32 << 20)
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, const int32_t* seg,
                         float scale, int causal, void* dq, void* dk, void* dv,
                         int B, int H, int Hkv, int N, int D, fa_dtype dtype,
                         void* stream);

/*
 * Host-side precondition check of a HOST copy of seg (B, N int32, row-major):
 * FA_OK when every row is non-decreasing, i.e. every segment is one
 * contiguous run of tokens, the form sequence packing produces (README,
 * "Sequence packing": short sequences concatenated into fixed-length rows,
 * a token attending only inside its own sequence) and the one the kernels'
 * tile ranges assume; FA_ERR_SEG otherwise, FA_ERR_NULL / FA_ERR_SHAPE for bad
 * arguments.  A refusal "naming the reason" rather than a silent wrong
 * answer (README, "If you maintain a trainer").  Reads B * N ints, makes no
 * HIP call; the caller keeps ownership of host_seg.
 */
fa_status fa_check_seg(const int32_t* host_seg, int B, int N);

/* Static, human-readable name of a status code. */
const char* fa_status_string(fa_status status);

/*
 * Fused linear cross-entropy: the loss layer of a language model without the
 * (N, V) logits tensor (mlx-train-perf README, section "The fused
 * cross-entropy loss": the forward regenerates the logits tile by tile and
 * returns the per-token NLL, log-sum-exp and target logit; the backward
 * recomputes the tiles it needs).  Logits are Z = h w^T, accumulated in fp32.
 *   h       : (N, D) bf16 hidden states; w : (V, D) bf16 dense output head.
 *   targets : (N,) int32, each in [0, V) (an id outside gives unspecified
 *             values for that token; every access stays in bounds).
 * bf16 only (FA_ERR_DTYPE otherwise); D a multiple of 256, and V * D, N * D
 * and N * FA_LCE_VOCAB_CHUNK elements below 2^30 (FA_ERR_SHAPE otherwise).
 * The backward walks the vocabulary in chunks of FA_LCE_VOCAB_CHUNK rows.
 * Same alignment, ownership, stream and refusal rules as the attention calls
 * (4-byte alignment for targets and the fp32 arrays).
 */
#define FA_LCE_VOCAB_CHUNK 8192

/* Workspace bytes of fa_lce_fwd (for_bwd = 0) or fa_lce_bwd (for_bwd = 1):
 * forward ceil(V/256) * N float pairs (per-tile partial maxima and sums);
 * backward an (N, FA_LCE_VOCAB_CHUNK) bf16 dZ chunk plus, when V spans more
 * than one chunk, an (N, D) fp32 dh accumulator.  0 for refused shapes. */
size_t fa_lce_workspace_bytes(int N, int V, int D, int for_bwd);

/* Forward: nll[i] = lse[i] - tlogit[i], lse[i] = ln sum_v exp(Z[i][v]),
 * tlogit[i] = Z[i][targets[i]]; all (N,) fp32, written.  Targets are not
 * validated on the host (they live on the device): a target outside [0, V)
 * gives NaN tlogit and nll for that token, and in fa_lce_bwd a gradient row
 * without the one-hot term.  No access goes out of bounds either way. */
fa_status fa_lce_fwd(const void* h, const void* w, const int32_t* targets,
                     float* nll, float* lse, float* tlogit,
                     int N, int V, int D, fa_dtype dtype,
                     void* ws, size_t ws_bytes, void* stream);

/* Backward from dnll (N,) fp32, the gradient of the loss with respect to
 * each token's NLL (1/N for a mean): with dZ = dnll[i] (softmax(Z[i]) -
 * onehot(targets[i])), writes dh = dZ w (N, D) bf16 and, when dw is not NULL,
 * dw = dZ^T h (V, D) bf16.  lse is the forward's. */
fa_status fa_lce_bwd(const void* h, const void* w, const int32_t* targets,
                     const float* lse, const float* dnll, void* dh, void* dw,
                     int N, int V, int D, fa_dtype dtype,
                     void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
