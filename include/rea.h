/*
 * rea.h - C ABI of librea.so: the ReAttention hot path on AMD MI355X (gfx950).
 *
 * The method (ReAttention: Training-Free Infinite Context with Finite
 * Attention Scope, arXiv 2407.15176):
 *   1. score the un-rotated queries against the pre-RoPE keys of the middle
 *      cache (everything between the first G and the last L tokens), reduce
 *      token scores to span scores and keep the top-k spans
 *      [research-map summary, "Approach"; OpenReview discussion, "Decoding
 *      Phase" pseudocode: score = query @ key[G:-L]^T, then top-k];
 *   2. concatenate global cache ++ selected spans (in original order) ++ local
 *      cache into one window [same pseudocode: key_recall / value_recall];
 *   3. apply RoPE with fresh positions 0..W-1, so the attention scope stays
 *      inside the pre-trained range [summary, "Approach"];
 *   4. run ordinary causal softmax attention over the window [pseudocode:
 *      flash_attention(query, key_recall, value_recall)].
 *
 * Readings this library takes where the pages are silent:
 *   - GQA: one selection per KV head; a token's score is the sum over the
 *     head's query group of q . k.
 *   - span score: max over the span's tokens; for a block of queries (chunked
 *     prefill) the sum over the block's queries of those maxima.
 *   - ties: the lower span index wins; selected spans are emitted ascending.
 *   - the middle is cut into spans of S tokens from its start; a shorter last
 *     span is scored over, and gathered with, its real length.
 *   - RoPE: rotate-half pairing (c, c + d/2), inverse frequency
 *     rope_theta^(-2c/d); a query takes the window position of its own key.
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates nothing and keeps no state between calls (apart from a
 *     thread-local error string).  Calls are re-entrant.  The one exception
 *     is rea_decode_step_noalloc, which works in a fixed scratch array that
 *     the library holds on each device (see there).
 *   - All argument validation happens on the host before any HIP call, so
 *     every error status below is reachable on a machine without a GPU.
 *   - Kernels are enqueued asynchronously on the caller's stream (a
 *     hipStream_t passed as void*; NULL = the null stream).  A device fault
 *     surfaces at the caller's next synchronisation.
 *   - Outputs are undefined when the return value is not REA_OK.
 *   - Sizes are in elements unless the name says bytes.
 */
#ifndef REA_H
#define REA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REA_ABI_VERSION 4

typedef enum rea_status {
    REA_OK = 0,
    REA_EINVAL = 1,        /* null pointer, struct_size mismatch, bad hyperparameter */
    REA_ESHAPE = 2,        /* inconsistent sizes (Hq % Hkv, n_q % block_q, strides, W_cap, ...) */
    REA_EDTYPE = 3,        /* dtype not REA_BF16 / REA_F32 */
    REA_EALIGN = 4,        /* a pointer or row stride is not 16-byte aligned */
    REA_EWORKSPACE = 5,    /* workspace smaller than rea_query_sizes() asks for */
    REA_ENODEVICE = 6,     /* no usable HIP device */
    REA_ELAUNCH = 7,       /* a kernel launch failed (hipGetLastError) */
    REA_EUNSUPPORTED = 8   /* valid arguments outside what the library implements */
} rea_status;

enum {
    REA_SELECT_PER_Q_HEAD = 1,
    REA_SELECT_TOKEN_SEGMENTS = 2
};

typedef enum rea_dtype {
    REA_BF16 = 0,          /* bfloat16 storage of q, K, V */
    REA_F32 = 1            /* float32 storage of q, K, V */
} rea_dtype;

/*
 * One layer's problem, batch 1.
 *
 * q      [n_q][n_q_heads][head_dim], contiguous, un-rotated.  The queries are
 *        the last n_q tokens of the cache (their K/V rows are already
 *        appended, as the pseudocode appends before scoring).
 * k, v   pre-RoPE cache: element (h, t, c) at  base[h*kv_stride_head +
 *        t*kv_stride_tok + c],  h < n_kv_heads, t < T, c < head_dim.
 *        16-byte aligned base and row stride.
 * T      valid tokens, including the n_q newest ones.
 * Query head hq reads KV head hq / (n_q_heads / n_kv_heads).
 */
typedef struct rea_problem {
    uint32_t struct_size;      /* = sizeof(rea_problem) */
    int32_t dtype;             /* rea_dtype */
    int32_t n_q;               /* >= 1 */
    int32_t n_q_heads;         /* Hq, multiple of n_kv_heads */
    int32_t n_kv_heads;        /* Hkv >= 1 */
    int32_t head_dim;          /* d: 64 or 128 */
    int64_t T;                 /* n_q <= T < 2^31 */
    const void *q;
    const void *k;
    const void *v;
    int64_t kv_stride_head;    /* >= T * kv_stride_tok */
    int64_t kv_stride_tok;     /* >= head_dim */
} rea_problem;

/*
 * Hyperparameters: global size G, span size S, number of spans k, local size
 * L [OpenReview discussion, hyperparameter list of the NIAH reply: global 32,
 * seg_size 32, num_seg 127, local 4096 on LLaMA3-8B-8K], and the number of
 * consecutive queries that share one selection (1 when decoding; a prefill
 * chunk is cut into blocks of block_q queries).  S = 1 is token-level
 * selection, the granularity of the discussion's pseudocode (topk over the
 * middle keys' scores).
 *
 * Selection flags (select_flags, a bit set):
 *   REA_SELECT_PER_Q_HEAD      select once per query head with its own
 *                              logits against its group's KV head (the
 *                              discussion's reply on eviction: selection is
 *                              redone for each attention head); without it,
 *                              once per KV head with the summed logits of the
 *                              query heads of its group.
 *   REA_SELECT_TOKEN_SEGMENTS  select the topk best single tokens instead of
 *                              spans, widen each to the S tokens
 *                              [u - (S-1)/2, u - (S-1)/2 + S) around it,
 *                              clipped to the middle, and take the union (the
 *                              discussion's InfLLM reply: the K cache is
 *                              selected directly, not cut into blocks in
 *                              advance).  Then a selection lists up to
 *                              topk * S middle-relative TOKENS (spans of one
 *                              token), sizes.n_spans counts tokens and span
 *                              scores are token scores.  H_sel = n_kv_heads or n_q_heads accordingly; every [..][H_sel][..]
 * array below is indexed by selection head, and selection head u serves query
 * heads [u * Hq / H_sel, (u + 1) * Hq / H_sel) and reads KV head
 * u * n_kv_heads / H_sel.
 *
 * Regions: G' = min(G, T), L' = min(L, T - G'), middle = [G', T - L').
 * Precondition: n_q <= L', or the middle is empty (T <= G + L).
 */
typedef struct rea_params {
    uint32_t struct_size;      /* = sizeof(rea_params) */
    int32_t G;                 /* >= 0 */
    int32_t S;                 /* >= 1 */
    int32_t topk;              /* >= 0 spans */
    int32_t L;                 /* >= 0 */
    int32_t block_q;           /* >= 1, divides n_q */
    double rope_theta;         /* > 0 */
    float softmax_scale;       /* <= 0 selects 1/sqrt(head_dim) */
    int32_t select_flags;      /* REA_SELECT_* bits, 0 for the default selection */
} rea_params;

/* Derived sizes and the workspace each entry point needs. */
typedef struct rea_sizes {
    int64_t n_blocks;          /* n_q / block_q */
    int64_t n_spans;           /* ceil((T - L' - G') / S) */
    int64_t k_sel;             /* min(topk, n_spans): spans selected per (block, H_sel head);
                                  token segments: min(topk * S, middle tokens), an upper bound */
    int64_t W_cap;             /* min(T, G' + k_sel*S + L'): the largest possible window */
    size_t ws_score_select;    /* bytes of workspace rea_score_select needs */
    size_t ws_window_attend;   /* bytes of workspace rea_window_attend needs */
    size_t ws_decode_step;     /* bytes of workspace rea_decode_step needs */
    int64_t n_sel_heads;       /* H_sel: n_kv_heads, or n_q_heads with select_per_q_head */
} rea_sizes;

/* Measurement hook of rea_decode_step_timed: hipEvent_t handles (as void*)
 * that take the start and end times of the token-scoring kernel's dispatch on
 * the call's stream (hipExtLaunchKernel).  Either may be NULL.  Events created
 * with hipEventDisableSystemFence perturb the step least. */
typedef struct rea_timing {
    void *score_begin;
    void *score_end;
} rea_timing;

int rea_abi_version(void);
const char *rea_status_string(int status);
/* Detail message of the last failing call on this thread ("" if none). */
const char *rea_last_error(void);

/* Fills *out.  Host-only: validates p and a, makes no HIP call. */
rea_status rea_query_sizes(const rea_problem *p, const rea_params *a, rea_sizes *out);

/*
 * Bytes of device workspace that suffice for every entry point below that
 * takes one (rea_score_select, rea_window_attend with W_cap = sizes.W_cap,
 * rea_decode_step): the largest of the three rea_sizes fields.  Host-only.
 * Returns (size_t)-1, a size no allocator grants, when p or a is invalid;
 * rea_last_error() then says why (rea_query_sizes returns the status).
 */
size_t rea_workspace_bytes(const rea_problem *p, const rea_params *a);

/*
 * Step 1: position-agnostic span scoring and top-k selection.
 *
 * sel          [n_blocks][H_sel][topk] int32: for block b and selection head h
 *              the selected span indices (span j covers middle tokens
 *              [G' + j*S, min(G' + (j+1)*S, T - L'))), strictly ascending,
 *              padded with -1 after n_sel entries.  May be NULL if topk == 0.
 *              Token segments: [n_blocks][H_sel][topk * S], the union's
 *              middle-relative token indices (token u is cache row G' + u).
 * n_sel        [n_blocks][H_sel] int32 = k_sel (token segments: the union's
 *              size, at most k_sel).
 * span_scores  NULL, or [n_blocks][H_sel][n_spans] double: sum over the
 *              block's queries of the span's maximum token score.
 * ws           device workspace of at least sizes.ws_score_select bytes
 *              (256-byte aligned); contents are scratch.
 *
 * Precision.  Span scores are computed in fp64: a query group's sum q_eff is
 * taken in fp64, and every product of q_eff with a key element and every sum
 * is an fp64 operation.  With bf16 inputs each product is exact (q_eff of a
 * few bf16 heads has few significant bits) and the sums are exact whenever
 * they need at most 53 significant bits, which holds unless the products of
 * one token span more than about 2^30 in magnitude; with fp32 inputs the
 * products of a group sum (g > 1) and the sums can round.  Where they round, a
 * token score lies within n * 2^-53 * sum|terms| of the exact value (n the
 * number of terms), and the selection equals the exact one unless two spans'
 * exact scores differ by less than that at the k-th boundary; these paths
 * have no guard for such near-ties.
 *
 * Blocks of 64 bf16 queries with head_dim 128 and S a multiple of 32 (the
 * MFMA path) are scored with bf16 MFMA products and fp32 sums: span_scores are
 * then approximations, each within a bound eps_j computed for its span, and
 * every span whose interval could reach across the k-th boundary is re-scored
 * in fp64 before the top-k is decided, so the selection is the one the fp64
 * scores above give.
 */
rea_status rea_score_select(const rea_problem *p, const rea_params *a,
                            int32_t *sel, int32_t *n_sel, double *span_scores,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Steps 2-3: gather the window and apply RoPE at window positions.
 *
 * sel, n_sel   as produced by rea_score_select (device).
 * k_win        [n_blocks][H_sel][W_cap][head_dim] float32: row w of the
 *              window key, rotated to position w (rows >= W untouched).
 * v_win        [n_blocks][H_sel][W_cap][head_dim], problem dtype: the
 *              window value rows, bit-exact copies of the cache rows.
 * q_rot        [n_q][n_q_heads][head_dim] float32: each query rotated to the
 *              window position of its own key, W - n_q + (query index in q).
 * W            [n_blocks][H_sel] int32 window lengths.
 * W_cap        row capacity of k_win/v_win; must be >= sizes.W_cap.
 */
rea_status rea_gather_rope(const rea_problem *p, const rea_params *a,
                           const int32_t *sel, const int32_t *n_sel,
                           float *k_win, void *v_win, float *q_rot, int32_t *W,
                           int32_t W_cap, void *stream);

/*
 * Step 4: causal softmax attention over the window.  Query i of block b sees
 * window rows w <= its position; logits are (q_rot . k_win[w]) * scale.
 * out          [n_q][n_q_heads][head_dim] float32.
 * ws           at least sizes.ws_window_attend bytes.
 */
rea_status rea_window_attend(const rea_problem *p, const rea_params *a,
                             const float *q_rot, const float *k_win, const void *v_win,
                             const int32_t *W, int32_t W_cap, float *out,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * Steps 1-4 in one call, no host synchronisation (window lengths stay on the
 * device).  The decode step of one layer when n_q == block_q == 1; any
 * n_q/block_q accepted by the three calls above is accepted here too.
 * out          [n_q][n_q_heads][head_dim] float32.
 * sel, n_sel   optional copies of the selection (NULL to skip), laid out as
 *              rea_score_select's.
 * ws           at least sizes.ws_decode_step bytes.
 */
rea_status rea_decode_step(const rea_problem *p, const rea_params *a, float *out,
                           int32_t *sel, int32_t *n_sel,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * rea_decode_step with a measurement hook: the same launches, the scoring
 * kernel's dispatch stamped into timing's events (timing may be NULL).  For
 * benchmarks; the product path is rea_decode_step.
 */
rea_status rea_decode_step_timed(const rea_problem *p, const rea_params *a, float *out,
                                 int32_t *sel, int32_t *n_sel,
                                 void *ws, size_t ws_bytes, void *stream,
                                 const rea_timing *timing);

/*
 * rea_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same kernels run on a fixed scratch
 * array of REA_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * is loaded on, until the process ends; the call itself allocates nothing.
 * The caller still passes q, K/V (in p), out and the optional sel / n_sel.
 *
 * Limit: problems whose sizes.ws_decode_step exceeds REA_NOALLOC_SCRATCH_BYTES
 * are rejected with REA_EWORKSPACE before any HIP call (16 MiB covers decode
 * steps with one selection per KV or query head up to 4M tokens of context;
 * token-level selection and large prefill chunks need rea_decode_step).
 * All calls on one device share its array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * device, on different streams or from different threads, race and must be
 * serialised by the caller.
 */
#define REA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
rea_status rea_decode_step_noalloc(const rea_problem *p, const rea_params *a, float *out,
                                   int32_t *sel, int32_t *n_sel, void *stream);

/*
 * Chunked prefill of a whole prompt (OpenReview discussion, "Prefilling
 * Phase" pseudocode: the first chunk of G + L tokens is attended in full, and
 * every later chunk is appended to the cache and attended through its own
 * top-k; the NIAH reply's settings use chunks of 512).  Every prompt token is a
 * query: p->n_q == p->T, q = [T][n_q_heads][head_dim], and the K/V cache holds
 * the whole prompt.  Chunk c covers queries [start, start + n_q) and is run as
 * one rea_decode_step with the cache cut to its first start + n_q tokens, so
 * each chunk sees exactly the tokens before and inside it.
 *
 * Plan (rea_prefill_plan): F = min(T, G + L) rounded down to a multiple of
 * block_q; if F > 0 the first chunk is [0, F) (no middle cache yet: plain
 * causal attention); then chunks of `chunk` tokens, the last one possibly
 * shorter.  A chunk whose length n is not a multiple of block_q is cut into
 * equal blocks of the largest divisor of n not above block_q.
 * Preconditions (REA_EINVAL): n_q == T, 1 <= chunk <= L, chunk a multiple of
 * block_q; every chunk must pass rea_decode_step's own checks.
 */
typedef struct rea_chunk {
    int64_t start;        /* first query (prompt token) of the chunk */
    int32_t n_q;          /* queries in the chunk */
    int32_t block_q;      /* queries per selection block within the chunk */
    int64_t first_block;  /* index of the chunk's first block among all the
                             plan's blocks (blocks numbered in plan order) */
} rea_chunk;

/* Host-only: writes up to `cap` chunks to `chunks` (may be NULL when cap is 0),
 * the total count to *n_chunks, the number of selection blocks over all
 * chunks to *n_blocks (may be NULL), and the workspace rea_prefill needs to
 * *ws_bytes (the largest of its chunk steps').  Makes no HIP call. */
rea_status rea_prefill_plan(const rea_problem *p, const rea_params *a, int32_t chunk,
                            rea_chunk *chunks, int32_t cap, int32_t *n_chunks,
                            int64_t *n_blocks, size_t *ws_bytes);

/* Runs the plan on `stream` without host synchronisation; out is
 * [T][n_q_heads][head_dim] float32.  ws as given by rea_prefill_plan.
 * sel, n_sel   NULL, or every block's selection: [n_blocks][H_sel][sel_cap]
 *              and [n_blocks][H_sel] int32 with n_blocks from the plan and
 *              sel_cap = topk (topk * S with token segments); the rows of
 *              chunk c start at block chunks[c].first_block and are laid out
 *              as rea_score_select's for that chunk's problem (span indices
 *              relative to the chunk's own middle [G', start + n_q - L')).
 *              Both or neither. */
rea_status rea_prefill(const rea_problem *p, const rea_params *a, int32_t chunk, float *out,
                       int32_t *sel, int32_t *n_sel, void *ws, size_t ws_bytes, void *stream);

/*
 * Batched decode: one decode step (one query token each) for `batch`
 * sequences that share the layer shape and the hyperparameters, in one
 * launch sequence (OpenReview discussion, the authors' decoding-throughput
 * replies: LLaMA3-8B decoding at 32K and 64K contexts with batch sizes larger
 * than full attention fits).
 *
 * p            one sequence's shape with n_q = 1 and T = the cache capacity
 *              (the largest length); p->q is [batch][n_q_heads][head_dim]
 *              (all the batch's queries); p->k, p->v are sequence 0's cache,
 *              and sequence b's cache starts b * kv_stride_seq elements later
 *              (same head and token strides).
 * a            block_q must be 1 and L >= 1; at most 8 query heads per
 *              selection head (64 for bf16 with head_dim 128), else
 *              REA_EUNSUPPORTED.
 * lengths      DEVICE array [batch] int64: sequence b has lengths[b] valid
 *              tokens, its query being token lengths[b] - 1; every region,
 *              span and window is derived from its own length.  Values are
 *              clamped to [1, p->T] on the device (never read on the host).
 * out          [batch][n_q_heads][head_dim] float32.
 * sel, n_sel   optional [batch][H_sel][topk] / [batch][H_sel] (NULL to skip).
 * ws           rea_decode_batch_workspace() bytes, 256-byte aligned.
 * Errors: as rea_decode_step, plus REA_EUNSUPPORTED for n_q or block_q != 1
 * and REA_ESHAPE for kv_stride_seq < n_kv_heads * kv_stride_head.
 */
rea_status rea_decode_batch_workspace(const rea_problem *p, const rea_params *a, int32_t batch,
                                      size_t *ws_bytes);
rea_status rea_decode_batch(const rea_problem *p, const rea_params *a, int32_t batch,
                            const int64_t *lengths, int64_t kv_stride_seq, float *out,
                            int32_t *sel, int32_t *n_sel, void *ws, size_t ws_bytes,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* REA_H */
