/*
 * fa.h -- C ABI of libfa: exact tiled scaled-dot-product attention on MI355X (gfx950).
 *
 * The operation is Attention(Q,K,V) = softmax(scale * Q K^T) V, the equation of
 * "FlashAttention Explained: How AI Models Process Attention Faster and Use Less
 * Memory", section "Understanding Attention in Transformer Models" (there
 * scale = 1/sqrt(d_k)).  It is computed in Q/K/V tiles with a running row
 * maximum, a running denominator and a rescaled partial output (same page, "How
 * FlashAttention Works", parts 1 and 3; "Flash Attention Explained: Same Maths,
 * Far Less Memory", section "The idea: never materialise the matrix"), so the
 * N_q x N_kv score matrix is never written to device memory and is not an output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout     Contiguous row-major [B, H, N, d] with d innermost, for q, k, v and o.
 *             lse is float32 [B, H, N_q]: the natural-log log-sum-exp of each row,
 *             ln sum_{allowed j} exp(scale * q_i . k_j), scale included.
 *  Pointers   Device pointers (or any pointer the device can read/write), q/k/v/o
 *             and workspaces 16-byte aligned, lse 4-byte aligned.  Outputs must
 *             not overlap inputs.  lse may be NULL (then it is not written).
 *  Mask       causal != 0 allows key j for query i iff j <= i + (N_kv - N_q)
 *             (bottom-right alignment; equal to the lower triangle when N_q == N_kv).
 *             It requires N_q <= N_kv so that every row has at least one key.
 *  Domain     d in {64, 128}; B, H, N_q, N_kv >= 1; scale finite (0 and negative
 *             allowed); B*H*N*d*elem_size and the launch grid must fit the device
 *             limits.  Anything else is an error code -- never a silent slower path.
 *  Ownership  The caller owns every buffer, including workspaces.  The library
 *             never allocates, frees or synchronises, and never changes the current
 *             device.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *             stream of the current device) and the call returns; outputs are valid
 *             once the caller has synchronised that stream.  Inputs are read-only.
 *  Errors     Every argument is validated on the host before anything is launched:
 *             on FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_WORKSPACE nothing
 *             was enqueued and the outputs are untouched.  FA_ERR_DEVICE means the
 *             HIP runtime refused a launch; an entry point that enqueues two kernels
 *             (fa_decode, fa_fwd_split, fa_decode_gqa, fa_decode_paged, fa_bwd) may
 *             then have enqueued the first, so its outputs are undefined.  An error
 *             already pending on the calling thread from earlier work (the HIP
 *             runtime's last-error state) is reported as FA_ERR_DEVICE before any
 *             launch instead of being cleared.  fa_last_error() gives a thread-local
 *             description of the last non-OK status.  No exception or abort crosses
 *             this boundary.
 *  Threads    Re-entrant; the global state is the thread-local error text and a
 *             per-device cache of the compute-unit count, read once on first use
 *             (launch heuristics such as causal tile pairing, wave counts and the
 *             automatic split counts are sized by it).
 *  Results    Bitwise deterministic run to run for the same arguments.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* NULL/misaligned/overlapping pointer, size < 1, causal with N_q > N_kv, ... */
  FA_ERR_UNSUPPORTED = 2, /* valid request outside the built domain (head size, dtype) */
  FA_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than fa_decode_workspace_bytes() */
  FA_ERR_DEVICE = 4       /* the HIP runtime refused a launch, or an error from earlier work was pending */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_F32 = 1 } fa_dtype;

/*
 * fa_fwd -- attention forward for N_q queries against N_kv keys per (batch, head).
 *
 * q [B,H,N_q,d], k [B,H,N_kv,d], v [B,H,N_kv,d] in `dtype`; writes o [B,H,N_q,d] in
 * `dtype` and, if lse != NULL, lse [B,H,N_q] float32.
 * bf16: scores and value sums accumulate in fp32 on the matrix cores, the
 * softmax runs in fp32, the probabilities enter the value product as bf16 and
 * o is rounded to bf16 to nearest-even.  f32: fp32 throughout.
 * bf16 additionally needs N_kv * d * 2 <= 2^31 - 1 (one head's K or V within a
 * 32-bit byte range); larger heads return FA_ERR_UNSUPPORTED.
 * Passage: the attention equation and "How FlashAttention Works" of the page
 * named at the top; prefill is "Where you actually feel it" of "Flash Attention
 * Explained: Same Maths, Far Less Memory".
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                 int N_kv, int d, float scale, int causal, void* stream, fa_dtype dtype);

/* fa_fwd with the element type fixed (bf16 / f32); arguments as for fa_fwd. */
fa_status fa_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                      int N_kv, int d, float scale, int causal, void* stream);
fa_status fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                     int N_kv, int d, float scale, int causal, void* stream);

/*
 * Split-KV decode: one query per sequence against its cached keys and values,
 * no mask ("Flash Attention Explained: Same Maths, Far Less Memory", section
 * "Where you actually feel it": during decode the score matrix is a single row).
 *
 * The N_kv keys are cut into S contiguous ranges; split s covers keys
 * [s*c, min((s+1)*c, N_kv)) with c = ceil(N_kv / S) (a range may be empty).  The
 * split kernel writes, per (b, h, s), the normalised partial output O_s and its
 * log-sum-exp lse_s (lse_s = -inf and O_s = 0 for an empty range) into the
 * workspace; the combine kernel merges them:
 *   M = max_s lse_s,  w_s = exp(lse_s - M),  o = sum_s w_s O_s / sum_s w_s,
 *   lse = M + ln sum_s w_s.
 *
 * Workspace layout (caller-owned, 16-byte aligned, fa_decode_workspace_bytes()):
 *   float O_s  [B, H, S, d]      at byte offset 0
 *   float lse_s[B, H, S]         at byte offset B*H*S*d*4
 */

/* The split count fa_decode uses for num_splits == 0 (auto): enough (b, h, split)
 * work-groups for eight per compute unit of the current device, no split shorter than
 * 256 keys; >= 1.  Returns 0 on invalid sizes. */
int fa_decode_num_splits(int B, int H, int N_kv, int d, int num_splits);

/* Workspace bytes fa_decode needs for these sizes (num_splits 0 = auto). Returns 0 on invalid sizes. */
size_t fa_decode_workspace_bytes(int B, int H, int N_kv, int d, int num_splits);

/*
 * fa_decode -- q [B,H,d], k [B,H,N_kv,d], v [B,H,N_kv,d] (bf16); writes o [B,H,d] (bf16,
 * rounded to nearest-even) and, if lse != NULL, lse [B,H] float32.
 * num_splits in [0, N_kv] (0 = auto).  The workspace holds the partials afterwards.
 * dtype must be FA_DTYPE_BF16 (FA_DTYPE_F32 returns FA_ERR_UNSUPPORTED).
 */
fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_kv,
                    int d, float scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream,
                    fa_dtype dtype);

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * split partials go to a scratch array built into the library (FA_NOALLOC_SCRATCH_BYTES
 * of device memory per GPU, held from the first call on that GPU until the process ends)
 * instead of a caller workspace; the caller passes only inputs and outputs.  Arguments,
 * layouts, split count and results are those of fa_decode (same kernels: bit-identical
 * o and lse for the same num_splits).
 *   - Calls no hipMalloc/hipFree.  The first call on a device looks up that device's
 *     copy of the array (hipGetSymbolAddress) and keeps its address.
 *   - FA_ERR_WORKSPACE when the partials, fa_decode_workspace_bytes(B, H, N_kv, d,
 *     num_splits), exceed FA_NOALLOC_SCRATCH_BYTES (e.g. B*H*S*(d+1)*4 > 32 MiB); use
 *     fa_decode with a workspace then.  Nothing is launched on any error.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     partials: calls that overlap in time on one GPU (different streams or threads)
 *     race and may return wrong results; issue them in one stream order.  Nothing in
 *     the array needs to start at zero: the split kernel writes every partial (empty
 *     key ranges included) before the combine reads it.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                            int N_kv, int d, float scale, int num_splits, void* stream, fa_dtype dtype);

/*
 * The two halves of fa_decode, for callers that time or reuse them separately.
 * fa_decode_split writes only the workspace partials; fa_decode_combine reads
 * partials laid out as above (S = num_splits, which must be >= 1 here) and writes
 * o (bf16) and lse.  The combine is also the merge a caller needs when the key
 * ranges of one row were processed elsewhere.
 */
fa_status fa_decode_split(const void* q, const void* k, const void* v, int B, int H, int N_kv, int d, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream, fa_dtype dtype);
fa_status fa_decode_combine(const void* workspace, size_t workspace_bytes, void* o, float* lse, int B, int H,
                            int d, int num_splits, void* stream, fa_dtype dtype);

/*
 * fa_fwd_split -- fa_fwd with the keys of every query tile cut into num_splits
 * contiguous ranges of 64-key tiles, processed by separate work-groups, and the
 * per-range partials merged by their log-sum-exp (the combine of fa_decode).
 * Same result as fa_fwd within rounding; use it when B*H*ceil(N_q/128) is too
 * small to fill the GPU (a short chunk of queries against a long cache).
 * Arguments as fa_fwd (bf16 only; FA_DTYPE_F32 returns FA_ERR_UNSUPPORTED),
 * plus num_splits in [1, N_kv] and a caller-owned workspace of at least
 * fa_fwd_split_workspace_bytes(B, H, N_q, d, num_splits) bytes, 16-byte aligned:
 *   float O_s[B*H*N_q][S][d] at byte offset 0, float lse_s[B*H*N_q][S] after it.
 * Passage: as fa_fwd; the merge is the decode combine of "Where you actually feel
 * it" ("Flash Attention Explained: Same Maths, Far Less Memory").
 */
size_t fa_fwd_split_workspace_bytes(int B, int H, int N_q, int d, int num_splits);
/* A split count for fa_fwd_split: enough work-groups for two per compute unit of the
 * current device (B*H*ceil(N_q/128)*S ~ 2 * CUs), no split shorter than 512 keys, at
 * least 1.  0 for sizes fa_fwd_split rejects (B, H, N_q, N_kv < 1; d not 64 or 128).
 * Host-only apart from the one-time CU-count query. */
int fa_fwd_split_num_splits(int B, int H, int N_q, int N_kv, int d);
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N_q,
                       int N_kv, int d, float scale, int causal, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream, fa_dtype dtype);

/*
 * fa_decode_gqa -- decode with grouped key/value heads: q [B,H,d] against
 * k, v [B,H_kv,N_kv,d] where query head h uses key/value head h / (H / H_kv)
 * (H a multiple of H_kv; H_kv == 1 is multi-query attention).  Writes o [B,H,d]
 * bf16 and, if lse != NULL, lse [B,H] float32; no mask.  Each key/value head is
 * read once for all H / H_kv query heads that share it, which is what makes the
 * KV cache cheaper ("Flash Attention Explained: Same Maths, Far Less Memory",
 * "Where you actually feel it": the KV cache dominates decode).
 * num_splits in [0, N_kv] (0 = auto over B*H_kv sequences); the workspace needs
 * fa_decode_gqa_workspace_bytes(B, H, H_kv, N_kv, d, num_splits) bytes (the
 * layout of fa_fwd_split with N_q = H / H_kv).  bf16 only.
 */
int fa_decode_gqa_num_splits(int B, int H, int H_kv, int N_kv, int d, int num_splits);
size_t fa_decode_gqa_workspace_bytes(int B, int H, int H_kv, int N_kv, int d, int num_splits);
fa_status fa_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                        int N_kv, int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                        void* stream, fa_dtype dtype);

/*
 * fa_decode_paged -- decode against a paged KV cache (the paging scheme of the
 * post "Paged Attention: Fixing the KV Cache Memory Problem", listed among the
 * related posts of "Flash Attention Explained: Speed From Memory Movement": the
 * cache is cut into fixed-size pages so that no sequence reserves memory for its
 * maximum length, and a table maps each sequence's logical blocks to pages).
 *
 *   q            [B, H, d] bf16, one query per sequence and head.
 *   k_pages,
 *   v_pages      [num_pages, H_kv, page_size, d] bf16: the shared page pool.
 *   block_table  [B, max_blocks] int32 (device): token t of sequence b is row
 *                t % page_size of page block_table[b][t / page_size].  An entry
 *                outside [0, num_pages) marks its tokens absent: they are not
 *                read and take no part in the softmax (use -1 for padding).
 *   seq_lens     [B] int32 (device): tokens of sequence b, used as
 *                min(max(seq_lens[b], 0), max_blocks * page_size).
 *   o            [B, H, d] bf16; lse [B, H] float32 or NULL.  A sequence with no
 *                present token gets o = 0 and lse = -inf.
 *
 * Query head h reads key/value head h / (H / H_kv), H a multiple of H_kv.  With
 * H / H_kv >= 2 and page_size >= 8 the group's query heads are the query rows of a
 * matrix-core split forward over the pages (any group size); otherwise a vector
 * kernel serves the group, which must then be 1, 2, 4 or 8 heads (else
 * FA_ERR_UNSUPPORTED).  page_size is a power of two in [1, 2^20] and
 * max_blocks * page_size <= 2^30.  No mask (every present token is seen).
 * Lengths and the table are read on the device, so the host needs only the bound
 * max_seq_len = max_blocks * page_size to size the work: num_splits in
 * [0, max_blocks * page_size] (0 = auto, as fa_decode_num_splits for B*H_kv
 * sequences of that length); each sequence's own length is cut into that many
 * ranges.  workspace: >= fa_decode_paged_workspace_bytes(B, H, H_kv,
 * max_blocks * page_size, d, num_splits) bytes, 16-byte aligned, overlapping no
 * other argument.  Table entries and lengths are trusted only as far as the
 * clamping above: any int32 value is memory-safe.  bf16 only.
 */
int fa_decode_paged_num_splits(int B, int H_kv, int max_seq_len, int d, int num_splits);
size_t fa_decode_paged_workspace_bytes(int B, int H, int H_kv, int max_seq_len, int d, int num_splits);
fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                          const int* seq_lens, void* o, float* lse, int B, int H, int H_kv, int num_pages,
                          int page_size, int max_blocks, int d, float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream, fa_dtype dtype);

/*
 * fa_bwd -- gradients of fa_fwd: given the forward's inputs, its output o and
 * log-sum-exp lse, and the upstream gradient dout = dL/dO, writes
 * dq = dL/dQ, dk = dL/dK, dv = dL/dV.
 *
 * q, o, dout, dq [B,H,N_q,d]; k, v, dk, dv [B,H,N_kv,d]; all bf16, row-major,
 * 16-byte aligned; lse [B,H,N_q] float32 exactly as fa_fwd wrote it (natural
 * log, scale included).  scale and causal must be the forward's.
 * The probabilities are recomputed from q, k and lse rather than stored
 * (passage: the training section, "More Efficient Backpropagation", of
 * "FlashAttention Explained: How AI Models Process Attention Faster and Use
 * Less Memory"; "Recompute probabilities for training" in the contents of "How
 * FlashAttention Speeds Up LLM Attention").  With P = softmax(scale q k^T):
 *   dv = P^T dout,  dP = dout v^T,  dS = P * (dP - rowsum(dout * o)),
 *   dq = scale dS k,  dk = scale dS^T q;
 * fp32 accumulation, outputs rounded to bf16 to nearest-even.
 * workspace: caller-owned, >= fa_bwd_workspace_bytes(B, H, N_q) bytes, 16-byte
 * aligned; it receives rowsum(dout * o) as float32 [B,H,N_q].
 * Outputs must not overlap inputs, each other or the workspace.  dtype must be
 * FA_DTYPE_BF16 (FA_DTYPE_F32 returns FA_ERR_UNSUPPORTED); d in {64, 128};
 * causal needs N_q <= N_kv (bottom-right alignment, as fa_fwd).  Two kernels are
 * enqueued on `stream`; every output element is summed in a fixed order, so
 * results are bitwise reproducible.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N_q);
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, int B, int H, int N_q, int N_kv, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream, fa_dtype dtype);

/*
 * Launch plans: which kernel, work-group shape and grid an entry point would use
 * for these sizes on a device with num_cu compute units (0 = the current device;
 * 256, the full MI355X, when none is visible).  The heuristics depend on the CU
 * count only through these decisions, never through the results' meaning.  Host
 * arithmetic only (no GPU call when num_cu > 0); for tests and tuning.
 *   op            FA_PLAN_FWD: fa_fwd (dtype bf16 or f32); FA_PLAN_FWD_SPLIT:
 *                 fa_fwd_split; FA_PLAN_DECODE: the split kernel of fa_decode
 *                 (N_q ignored); FA_PLAN_BWD_DQ / FA_PLAN_BWD_DKDV: the two
 *                 kernels of fa_bwd.  Split ops take num_splits (0 = automatic).
 *   out           filled on FA_OK.
 * Returns FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED for sizes the entry point rejects
 * for the same reasons (sizes < 1, d not 64 or 128, fp32 outside fa_fwd).
 */
typedef enum {
  FA_PLAN_FWD = 0,
  FA_PLAN_FWD_SPLIT = 1,
  FA_PLAN_DECODE = 2,
  FA_PLAN_BWD_DQ = 3,
  FA_PLAN_BWD_DKDV = 4
} fa_plan_op;

typedef enum {
  FA_KERNEL_BF16_4WAVE = 1,    /* bf16 forward, 4 waves x 32 query rows, two work-groups per CU */
  FA_KERNEL_BF16_8WAVE = 2,    /* bf16 forward, 8 waves x 32 query rows, one work-group per CU */
  FA_KERNEL_BF16_SPLIT = 3,    /* bf16 split-KV forward (partials + combine) */
  FA_KERNEL_F32_ROWS = 4,      /* fp32 forward, each wave walks its rows' whole key range */
  FA_KERNEL_F32_KEYSPLIT = 5,  /* fp32 forward, a 32-row work-group's waves split the keys */
  FA_KERNEL_DECODE_SPLIT = 6,  /* decode: one work-group per (b, h, split) */
  FA_KERNEL_BWD_DQ = 7,        /* backward, dQ kernel */
  FA_KERNEL_BWD_DKDV = 8       /* backward, fused dK / dV kernel */
} fa_kernel_id;

typedef struct {
  int kernel;           /* fa_kernel_id */
  int waves_per_group;  /* waves per work-group */
  int rows_per_group;   /* query rows per work-group (keys for FA_KERNEL_BWD_DKDV, 1 for decode) */
  int paired;           /* 1: causal tiles n-1-j and j share a work-group (equal work per group) */
  long long groups;     /* work-groups launched */
  int num_splits;       /* split count of the split ops, else 0 */
} fa_plan_info;

fa_status fa_plan(fa_plan_op op, int B, int H, int N_q, int N_kv, int d, int causal, fa_dtype dtype, int num_splits,
                  int num_cu, fa_plan_info* out);

/* Compute units of the current device (read once per device), 0 when no device can be queried. */
int fa_device_num_cu(void);

/* Human-readable name of a status code (static storage).  Together with fa_last_error it
 * serves the rule that an unsupported or invalid request is a visible error, never a
 * silent fallback to another code path ("Flash Attention Explained: Same Maths, Far Less
 * Memory", "The takeaway"; "FlashAttention Explained: How AI Models Process Attention
 * Faster and Use Less Memory", "Best Practices for Using FlashAttention"). */
const char* fa_status_str(fa_status s);

/* Thread-local text describing the last non-OK status returned on this thread ("" if none). */
const char* fa_last_error(void);

/* Library version string, e.g. "libfa 0.1 gfx950". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
