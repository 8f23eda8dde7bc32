/*
 * fa2.h -- C ABI of libfa2: exact attention forward and backward passes for AMD gfx950.
 *
 * The operation (all four pages agree on it):
 *
 *   O[b,h,i,:] = sum_j P[i,j] * V[b,h,j,:],
 *   P[i,j]     = exp(S[i,j] - L[b,h,i]),   S[i,j] = scale * <Q[b,h,i,:], K[b,h,j,:]>,
 *   L[b,h,i]   = log sum_{j visible} exp(S[i,j])  (natural log of the scaled scores)
 *
 * i.e. O = softmax(scale * Q K^T) V, optionally causal, plus the per-row
 * logsumexp L = m + log(l) of the online softmax.  Sources:
 *  - "From FlashAttention to FlashAttention 2", section "Background:
 *    FlashAttention 1" (the definition of standard attention) and section
 *    "Backward Pass: Recomputation" (L = m + log(l) is stored per row);
 *  - "FlashAttention-2 from PyTorch to Triton", opening description of the
 *    forward pass and of the second output L;
 *  - "Writing FlashAttention 2 in Triton", Step 1 (grid over Q tiles and
 *    batch*head), Step 4 (causal visibility: key <= query) and Step 6 (the
 *    wrapper's [B,H,N,D] tensors and fp32 L of shape [B,H,N_Q]);
 *  - "From FlashAttention to FlashAttention 2", section "Layer 2: C++ Entry
 *    Point" (dispatch on dtype, head dimension and causal onto a stream).
 * The M x N score matrix is never materialised: the kernels stream K/V tiles
 * and keep the running max m, sum l and unnormalised O in registers.
 */
#ifndef FA2_H_
#define FA2_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  lse is always float32. */
typedef enum {
    FA2_DTYPE_F32 = 0,  /* IEEE binary32 */
    FA2_DTYPE_BF16 = 1, /* bfloat16 (1-8-7); o is rounded to nearest-even */
    FA2_DTYPE_F16 = 2   /* IEEE binary16 (1-5-10); o is rounded to nearest-even */
} fa2_dtype;

typedef enum {
    FA2_OK = 0,
    FA2_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, bad scale */
    FA2_ERR_UNSUPPORTED = 2,      /* valid request this build does not implement (e.g. D) */
    FA2_ERR_LAUNCH = 3,           /* the HIP runtime refused the launch */
    FA2_ERR_NO_DEVICE = 4,        /* the runtime has no device, or none this build's gfx950
                                     code runs on, for the launch */
    FA2_ERR_SCRATCH = 5           /* fa2_fwd_ex_noalloc: the split partials would not fit
                                     the static scratch array */
} fa2_status;

/*
 * fa2_fwd -- attention forward pass on one HIP stream.
 *
 * Layout: every tensor is a contiguous row-major device array.
 *   q   [B, H, M, D]   element type `dtype`
 *   k   [B, H, N, D]   element type `dtype`
 *   v   [B, H, N, D]   element type `dtype`
 *   o   [B, H, M, D]   element type `dtype` (output)
 *   lse [B, H, M]      float32 (output): natural-log logsumexp of the scaled
 *                      scores of each query row over its visible keys
 * Q and K/V lengths may differ (cross-attention), as the pages' wrappers
 * allow ("Writing FlashAttention 2 in Triton", bug catalogue on separate
 * Q and KV strides).
 *
 * Arguments:
 *   B, H   batch and heads, >= 0 (the kernels see only the product B*H)
 *   M      query rows per head, >= 0
 *   N      key/value rows per head, >= 1
 *   D      head dimension; this build supports D = 64 and D = 128
 *   scale  multiplier of Q K^T, finite and > 0 (callers pass 1/sqrt(D) for
 *          standard attention)
 *   causal 0: every key is visible; 1: key j is visible to query i iff
 *          j <= i (top-left aligned, also when M != N)
 *   dtype  a fa2_dtype value
 *   stream a hipStream_t, or NULL for the null stream of the current device
 *
 * Ownership: all buffers are allocated and owned by the caller on the
 * current HIP device; the library allocates nothing and keeps no state, so
 * concurrent calls on different streams are safe (fa2_fwd_ex_noalloc, which
 * shares one static array per device, is the exception).  o must not overlap q, k or
 * v, and lse must not overlap any other buffer.  Every entry point of this
 * header only enqueues kernels on `stream` (no allocation, no memset, no
 * synchronisation), so a call may be captured into a HIP graph and replayed;
 * the replay reads whatever the captured buffers hold at that time.
 *
 * Runtime: libfa2 needs libamdhip64.so.7.  In a process that already uses a
 * HIP runtime (for instance the copy bundled with PyTorch), load that runtime
 * before libfa2 so both share one runtime: pointers and streams from one HIP
 * runtime are meaningless to another.
 *
 * Alignment: q, k, v, o must be 16-byte aligned, lse 4-byte aligned.  A
 * pointer may be NULL only when its buffer holds no element (q, o, lse when
 * B*H*M == 0; k, v when B == 0).
 *
 * Sizes: one head's q (o) and one head's k (v) must each stay under 2^31
 * bytes (the kernels address a head through 32-bit byte offsets), i.e.
 * M * D * elt < 2^31 and N * D * elt < 2^31 with elt = 4 for F32 and 2 for
 * BF16 / F16; B * H and the grid must stay under 2^31 as well.  Larger
 * problems are FA2_ERR_UNSUPPORTED, found before any launch.
 *
 * Errors: all argument checks run before any HIP call; on failure nothing is
 * launched and the outputs are untouched.  M == 0 or B*H == 0 returns FA2_OK
 * without a launch.  On success one kernel is enqueued on `stream` and the
 * call returns without synchronising; faults inside the kernel surface at
 * the caller's next synchronisation.  When the runtime rejects the launch
 * the call returns FA2_ERR_NO_DEVICE if it found no device, or no code object
 * for the current one (the library holds gfx950 code only), and
 * FA2_ERR_LAUNCH for any other refusal.
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
            float scale, int causal, int dtype, void* stream);

/* Upper bound of the n_splits argument of fa2_fwd_ex. */
#define FA2_MAX_SPLITS 128

/*
 * fa2_fwd_ex -- fa2_fwd with the other options of the pages' C++ entry point
 * ("From FlashAttention to FlashAttention 2", section "Layer 2": dispatch on
 * dtype, head dimension, causal and the number of K/V splits; section
 * "Layer 8": grouped-query attention).
 *
 * Differences from fa2_fwd:
 *   Hk        key/value heads, 1 <= Hk <= H with H % Hk == 0 (any Hk >= 1 when
 *             H == 0).  k and v are [B, Hk, N, D]; query head h reads K/V head
 *             h / (H / Hk).  Hk == H is multi-head attention (fa2_fwd),
 *             Hk == 1 multi-query attention.  Without a causal mask the
 *             H / Hk query heads of a group are processed as one sequence of
 *             (H / Hk) * M rows (they are consecutive in q, o and lse), so
 *             each K/V tile is read once per group.
 *   n_splits  0: the library chooses (fa2_fwd_num_splits); 1: one kernel over
 *             the whole key range, no workspace; 2..FA2_MAX_SPLITS: the key
 *             range [0, N) is cut into n_splits ranges of whole K/V tiles,
 *             each processed by its own workgroups, which write a partial O
 *             (fp32, normalised within the range) and the range's logsumexp;
 *             a second kernel combines them, O = sum_s exp(L_s - L) O_s with
 *             L = log sum_s exp(L_s).  Ranges past a causal row's diagonal
 *             are empty and contribute nothing.  The result matches the
 *             unsplit one to rounding (not bitwise); it is deterministic.
 *   workspace, workspace_size
 *             device memory the caller owns for the partial results when the
 *             effective split count is > 1: at least
 *             fa2_fwd_workspace_bytes(B, H, M, D, splits) bytes, 16-byte
 *             aligned, overlapping no other buffer; its contents on entry do
 *             not matter and on return are unspecified.  Ignored (may be NULL)
 *             when the effective split count is 1.
 * Both kernels are enqueued on `stream`; with splits the call returns after
 * enqueueing the second.  Errors as for fa2_fwd; a missing or short
 * workspace, or n_splits outside [0, FA2_MAX_SPLITS], is
 * FA2_ERR_INVALID_ARGUMENT.
 */
int fa2_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
               int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
               float scale, int causal, int dtype, int n_splits,
               void* workspace, int64_t workspace_size, void* stream);

/* Bytes of the static device scratch array behind fa2_fwd_ex_noalloc. */
#define FA2_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * fa2_fwd_ex_noalloc -- fa2_fwd_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the split-K/V partials go to a static device array of
 * FA2_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends, instead of a caller workspace.
 *
 * Arguments, layout, results and errors as for fa2_fwd_ex without the
 * workspace arguments; the output is bitwise the same as fa2_fwd_ex's with
 * the same effective split count.  A problem whose partials need more than
 * the array holds (fa2_fwd_workspace_bytes(B, H, M, D, splits) >
 * FA2_NOALLOC_SCRATCH_BYTES) returns FA2_ERR_SCRATCH before any HIP call;
 * pass a smaller n_splits (1 needs no scratch) or use fa2_fwd_ex.
 *
 * The call allocates nothing: it enqueues the same kernels as fa2_fwd_ex.
 * On its first call on a device (with that device current) it looks up the
 * array's device address with hipGetSymbolAddress and keeps it.  Nothing in
 * the array needs to start at zero (every partial a launch reads was written
 * by the same launch), but all calls on one device share the one array:
 * calls whose kernels overlap in time on one device (concurrent streams, or
 * host threads) race on it and give undefined results.  Serialise them, or
 * use fa2_fwd_ex with a workspace per stream.
 */
int fa2_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                       float scale, int causal, int dtype, int n_splits, void* stream);

/*
 * fa2_fwd_workspace_bytes -- workspace fa2_fwd_ex needs for n_splits splits
 * (0 when n_splits == 1); -1 for invalid arguments (negative sizes, D <= 0,
 * n_splits outside [1, FA2_MAX_SPLITS]).  Pure host computation.
 */
int64_t fa2_fwd_workspace_bytes(int64_t B, int64_t H, int64_t M, int64_t D, int n_splits);

/*
 * fa2_fwd_num_splits -- the split count fa2_fwd_ex uses for n_splits == 0:
 * 1 when the workgroups of the unsplit grid already fill about three
 * quarters of the GPU's workgroup slots (256 CUs), else enough splits to fill
 * them, keeping at least two K/V tiles per split.  (Without a causal mask the
 * query heads of one K/V group share their workgroups, see fa2_fwd_ex.)
 * Returns 1 for arguments fa2_fwd_ex would reject.  Pure host computation.
 */
int fa2_fwd_num_splits(int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D, int causal,
                       int dtype);

/*
 * fa2_fwd_local -- fa2_fwd_ex (unsplit) with a sliding-window mask, the
 * window_size = (left, right) option of the pages' Python entry point ("From
 * FlashAttention to FlashAttention 2", section "Layer 1"; "Writing
 * FlashAttention 2 in Triton", its list of next steps: a sliding-window
 * variant of the causal mask formula).
 *
 * Query row i sees key j iff
 *   (window_left  == -1 or j >= i - window_left) and
 *   (window_right == -1 or j <= i + window_right) and
 *   (!causal or j <= i),
 * measured from the top-left diagonal j = i like the causal mask (causal is
 * window_right = 0).  window_left, window_right >= -1; -1 leaves that side
 * unbounded, so (-1, -1) is plain fa2_fwd_ex attention.  A row that sees no
 * key (possible once a window is set, e.g. M > N with a finite left side)
 * gets o = 0 and lse = -inf.
 *
 * Layout, other arguments, ownership and errors as for fa2_fwd_ex with
 * n_splits = 1 (k, v are [B, Hk, N, D]); dtype F32, BF16 or F16; D = 64 or
 * 128.  One kernel is enqueued on `stream`.
 */
int fa2_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                  float scale, int causal, int64_t window_left, int64_t window_right,
                  int dtype, void* stream);

/*
 * fa2_fwd_varlen -- the forward pass over a batch of sequences of different
 * lengths packed without padding, the cu_seqlens interface of the pages'
 * variable-length entry point ("From FlashAttention to FlashAttention 2",
 * section "Layer 1": cu_seqlens_q / cu_seqlens_k for packed batching).
 *
 * Layout (head-major packing; each head's rows of all sequences are
 * contiguous, sequence after sequence):
 *   q, o   [H,  total_q, D]   element type `dtype`
 *   k, v   [Hk, total_k, D]   element type `dtype`
 *   lse    [H,  total_q]      float32
 *   cu_seqlens_q, cu_seqlens_k  int32 device arrays of B + 1 offsets:
 *          sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *          and keys cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of every head;
 *          offsets start at 0, never decrease and end at total_q (total_k).
 * Each sequence attends only to its own keys, with the causal / window
 * rules of fa2_fwd_local applied to its own row and key indices (query head
 * h reads K/V head h / (H / Hk)).  A sequence without keys gets o = 0 and
 * lse = -inf.
 *
 * max_seqlen_q: an upper bound of every sequence's query count (it sizes the
 * grid; rows of a longer sequence past it are not computed); 0 <=
 * max_seqlen_q <= total_q.
 *
 * The offsets live in device memory and are not read by the host: offsets
 * outside [0, total] or decreasing are clamped by the kernel (a sequence
 * then covers fewer rows or none), so they cannot make it address memory
 * outside q, k, v, o or lse, but the result for such a batch is
 * unspecified.  Other checks and errors as for fa2_fwd_local; B == 0, H ==
 * 0 or max_seqlen_q == 0 launches nothing.  One kernel on `stream`.
 */
int fa2_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   int64_t B, int64_t H, int64_t Hk, int64_t total_q, int64_t total_k,
                   int64_t max_seqlen_q, int64_t D, float scale, int causal,
                   int64_t window_left, int64_t window_right, int dtype, void* stream);

/*
 * fa2_bwd -- gradients of the attention forward pass on one HIP stream.
 *
 * For the forward O = softmax(S) V with S = scale * Q K^T (optionally causal,
 * grouped K/V heads as in fa2_fwd_ex) and an upstream gradient dO, it
 * computes
 *   P     = exp(S - L)                     recomputed from the stored lse
 *   delta = rowsum(dO o O)                 per query row, fp32
 *   dV    = P^T dO,   dP = dO V^T,   dS = P o (dP - delta)
 *   dQ    = scale * dS K,   dK = scale * dS^T Q
 * where dK, dV of a K/V head sum over the H / Hk query heads that read it.
 * Sources: "From FlashAttention to FlashAttention 2", section "Layer 7: The
 * Backward Kernel" (recompute P from L; dP, the rowsum(dO o O) correction,
 * dS and the products for dV, dK, dQ) and section "Backward Pass:
 * Recomputation"; "FlashAttention-2 from PyTorch to Triton", opening section
 * (L kept from the forward for the backward).
 *
 * Layout: contiguous row-major device arrays.
 *   q, o, dout, dq  [B, H, M, D]    element type `dtype`
 *   k, v, dk, dv    [B, Hk, N, D]   element type `dtype`
 *   lse             [B, H, M]       float32, the forward's logsumexp output
 *   delta           [B, H, M]       float32 (output): rowsum(dout o o)
 * o and lse must be the forward's outputs for the same q, k, v, scale and
 * causal flag.  16-bit dq, dk, dv are rounded to nearest even.
 *
 * Arguments as for fa2_fwd_ex (B, H, Hk, M, N >= 1, D, scale, causal, dtype,
 * stream).  This build supports dtype F32, BF16 and F16 with D = 64 or 128
 * (F32: fp32 products throughout, P and dS included).  Size limits as for
 * fa2_fwd (per head of q, dout: M * D * elt < 2^31 bytes, taken over the
 * H / Hk query heads of a K/V head together when there is no mask; per head
 * of k, v: N * D * elt < 2^31).
 *
 * Ownership: every buffer is caller-allocated device memory; the library
 * allocates nothing.  The outputs dq, dk, dv and delta must not overlap each
 * other or any input; q, k, v, o, dout, dq, dk, dv 16-byte aligned, lse and
 * delta 4-byte aligned.  A pointer may be NULL only when its buffer holds no
 * element (q, o, lse, dout, dq, delta when B*H*M == 0; k, v, dk, dv when
 * B == 0).
 *
 * Execution: on `stream`, for bf16 / fp16 two kernels (dQ, which also
 * computes delta; then dK and dV), for fp32 three (delta; dK and dV; dQ); no
 * synchronisation; every output element is written exactly once, by one
 * workgroup, so results are identical run to run.  M == 0 writes dk = dv = 0;
 * B * Hk == 0 launches nothing.  Errors as for fa2_fwd: every argument check
 * runs before any HIP call, and on failure nothing is launched.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* delta,
            int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
            float scale, int causal, int dtype, void* stream);

/*
 * fa2_bwd_local -- fa2_bwd for the sliding-window forward (fa2_fwd_local):
 * the same window_left / window_right rule decides which (query, key) pairs
 * carry a gradient.  o and lse must come from fa2_fwd_local with the same
 * window.  A row that saw no key (lse = -inf) gets dq = 0 and adds nothing
 * to dk, dv.  Arguments, layout and errors as for fa2_bwd; window sides >= -1.
 */
int fa2_bwd_local(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* delta,
                  int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                  float scale, int causal, int64_t window_left, int64_t window_right,
                  int dtype, void* stream);

/*
 * fa2_bwd_varlen -- fa2_bwd for packed variable-length sequences
 * (fa2_fwd_varlen): q, o, dout, dq [H, total_q, D]; k, v, dk, dv
 * [Hk, total_k, D]; lse, delta [H, total_q]; cu_seqlens_q / cu_seqlens_k
 * int32 device offsets [B + 1] as for fa2_fwd_varlen.  max_seqlen_q and
 * max_seqlen_k bound every sequence's query and key counts (they size the
 * grids: rows or keys of a longer sequence past them are not computed);
 * 0 <= max_seqlen_q <= total_q, 0 <= max_seqlen_k <= total_k.  Every key of
 * a sequence gets dk, dv written (zero for keys no query sees).  Offsets are
 * clamped on the device as in fa2_fwd_varlen.  Other arguments and errors as
 * for fa2_bwd_local.
 */
int fa2_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* delta,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   int64_t B, int64_t H, int64_t Hk, int64_t total_q, int64_t total_k,
                   int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, float scale, int causal,
                   int64_t window_left, int64_t window_right, int dtype, void* stream);

/* Static, NUL-terminated description of a fa2_status value. */
const char* fa2_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H_ */
