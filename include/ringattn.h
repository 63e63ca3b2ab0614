/*
 * ringattn.h -- C ABI of the MI355X (gfx950) ring-attention shard library.
 *
 * One GPU's share of ring attention: a local query shard Q attends to N
 * key/value sequence chunks, one non-causal softmax-attention pass per chunk,
 * and the chunk partials (output, log-sum-exp) are merged in float32.
 * Sources of the semantics:
 *   - Context-parallelism guide ("Paralelisme konteks", diffusers v0.43.0),
 *     section "Ring Attention": each GPU attends its queries to the K/V block
 *     it holds, passes the block on, and after one full turn has seen the K/V
 *     of every token.
 *   - Parallelism API page ("Paralelisme"), ContextParallelConfig:
 *     ring_degree (N chunks, N iterations), convert_to_fp32 (output and LSE
 *     kept in float32 for the merge; default True, the only mode built here),
 *     rotate_method "allgather" (every chunk is resident before the loop),
 *     ring_anything (any sequence length; uneven chunks).
 *   - Same guide, section "Ring Anything Attention" (uneven chunk lengths,
 *     inference only, no attention mask): here chunk c is either a row range
 *     of a packed K/V buffer or starts at row c * kv_chunk_stride of a
 *     padded one; keys at or past its true length are masked and never read.
 *   - Same guide, section "Perhatian Ulysses": after the all-to-all each GPU
 *     holds every token for a subset of heads; its share is full-sequence
 *     attention over those heads (ringattn_forward with one chunk).
 *
 * Conventions for every call:
 *   - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *   - Q, K, V and outputs are BSHD: [batch, seq, heads, head_dim], contiguous,
 *     head_dim innermost.  LSE is [batch, heads, q_len], float32, natural log,
 *     with the softmax scale inside: lse = ln sum_j exp(scale * q . k_j).
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them.  Q/K/V/out/workspace must be 16-byte aligned,
 *     LSE 4-byte aligned.  Chunk offsets are HOST memory, read during the call.
 *   - No call allocates device memory or synchronises.  All GPU work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     runs asynchronously.  Calls that write the same buffers on one stream
 *     are ordered; on different streams the caller orders them.
 *   - Every argument is validated before any GPU work is enqueued; on an
 *     error status nothing is launched and no buffer is written.
 *   - head_dim must be 64 or 128 (RINGATTN_EUNSUPPORTED otherwise).
 *   - Status codes are below; ringattn_last_error() gives the message of the
 *     last failing call on the calling thread.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RINGATTN_MAX_CHUNKS 128 /* largest ring degree one forward call accepts */

typedef struct ringattn_shape {
    int32_t batch;    /* B >= 1 */
    int32_t heads;    /* H >= 1 heads held by this GPU */
    int32_t head_dim; /* D: 64 or 128 */
    int32_t reserved; /* must be 0 */
    int64_t q_len;    /* Sq >= 1 local query rows */
    int64_t kv_len;   /* key/value rows: this chunk's (step) or all chunks' (forward) */
} ringattn_shape;

enum ringattn_status {
    RINGATTN_OK = 0,
    RINGATTN_EINVAL = -1,        /* bad argument: null/misaligned pointer, bad size or offsets */
    RINGATTN_EUNSUPPORTED = -2,  /* valid but not built: head_dim other than 64/128 */
    RINGATTN_EWORKSPACE = -3,    /* workspace missing or smaller than the plan needs */
    RINGATTN_EHIP = -4           /* the HIP runtime reported an error (message has it) */
};

/* Name of a status code ("RINGATTN_OK", ...); never NULL. */
const char *ringattn_status_string(int status);

/* Message describing the last failing call on this thread ("" if none).
 * The pointer stays valid until the next library call on this thread. */
const char *ringattn_last_error(void);

/* Library ABI version (incremented on any signature change). */
int32_t ringattn_abi_version(void);

/*
 * Chunk partition of a length-seq_len sequence over n_chunks ring ranks.
 * Writes offsets_out[0..n_chunks] (host memory, n_chunks + 1 entries):
 * offsets_out[0] = 0, offsets_out[n_chunks] = seq_len, chunk i is tokens
 * [offsets_out[i], offsets_out[i+1]).
 *   ring_anything = 0: plain ring attention; seq_len must divide evenly by
 *     n_chunks (guide, variant table), else RINGATTN_EINVAL.
 *   ring_anything != 0: any seq_len >= 0; the first (seq_len mod n_chunks)
 *     chunks hold one extra token, so every chunk fits the padded length
 *     ceil(seq_len / n_chunks) that Ring Anything pads to.
 * n_chunks must be in [1, RINGATTN_MAX_CHUNKS].  Pure host code.
 * Source: context parallelism guide, variant table (plain ring needs an
 * evenly divisible sequence) and section "Ring Anything Attention" (uneven
 * chunks padded to the longest); Parallelism API page,
 * ContextParallelConfig.ring_degree and ring_anything.
 */
int ringattn_chunk_offsets(int64_t seq_len, int32_t n_chunks, int32_t ring_anything,
                           int64_t *offsets_out);

/*
 * Set a float32 accumulator to the empty merge state: out_acc = 0 and
 * lse_acc = -inf (the identity of the LSE merge).  out_acc is
 * [B, q_len, H, D], lse_acc is [B, H, q_len].  shape->kv_len is ignored.
 * Source: the float32 merge state of Parallelism API page,
 * ContextParallelConfig.convert_to_fp32, before the ring's first iteration
 * (context parallelism guide, section "Ring Attention").
 */
int ringattn_acc_init(float *out_acc, float *lse_acc, const ringattn_shape *shape, void *stream);

/*
 * One ring step: attend q ([B, q_len, H, D] bf16) to one K/V chunk
 * (k_chunk, v_chunk: [B, kv_len, H, D] bf16; kv_len = shape->kv_len) with
 * softmax scale `scale`, and merge the chunk partial (its normalised output
 * and LSE) into the float32 accumulators out_acc / lse_acc in place:
 *     lse' = max(a, b) + ln(1 + exp(-|a - b|))
 *     out' = exp(a - lse') * out_acc + exp(b - lse') * out_chunk
 * with a = lse_acc, b = the chunk's LSE; where a = -inf the chunk partial is
 * copied (the old accumulator output is never multiplied).  The merge is
 * fused into the attention kernel's epilogue.  kv_len = 0 is a no-op.
 * Start from ringattn_acc_init; after all N chunks the accumulators hold the
 * shard's attention output and LSE.  scale must be finite and > 0.  One
 * workgroup sweeps each query tile over the whole chunk (no workspace);
 * ringattn_step_split below can spread the chunk's keys over several.
 * Source: context parallelism guide, section "Ring Attention" (one attention
 * pass per iteration on the K/V chunk the GPU holds, N iterations for a ring
 * of degree N); Parallelism API page, ContextParallelConfig.convert_to_fp32
 * (output and LSE in float32 for the merge).
 */
int ringattn_step(const uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk,
                  float *out_acc, float *lse_acc, float scale,
                  const ringattn_shape *shape, void *stream);

/*
 * Merge a partial (out_part [B, q_len, H, D], lse_part [B, H, q_len], float32)
 * into the accumulators in place, with the same formula as ringattn_step.
 * A partial with lse = -inf is the identity; if both are -inf the result is
 * out = 0, lse = -inf.  shape->kv_len is ignored.
 * Source: the float32 merge of chunk partials by their LSE (Parallelism API
 * page, ContextParallelConfig.convert_to_fp32; context parallelism guide,
 * section "Ring Attention").
 */
int ringattn_merge(float *out_acc, float *lse_acc, const float *out_part, const float *lse_part,
                   const ringattn_shape *shape, void *stream);

/*
 * Launch plan of ringattn_forward.
 *   n_splits: number of key/value splits -- independent partial passes over
 *     disjoint ranges of K/V tiles, merged by their LSE in split order by a
 *     merge kernel that follows the attention kernel on the stream;
 *   block_m: query rows per workgroup, 128 (4 waves, three workgroups per
 *     compute unit, 32-key tiles) or 256 (8 waves in two groups that
 *     alternate MFMA and softmax phases, 64-key tiles);
 *   workspace_bytes: device workspace the plan needs (0 when n_splits is 1):
 *     the float32 partial outputs of the splits, then their float32 LSEs
 *     (16-byte aligned).  Its contents on entry do not matter; calls that
 *     use one workspace must not overlap in time (same stream, or ordered by
 *     the caller).
 * On input n_splits and block_m are requests (0 = the library chooses from
 * the shape and the GPU's compute-unit count; n_splits > 0 is clamped to the
 * K/V tile count of the chosen kernel); on output they hold what
 * ringattn_forward will use.
 */
typedef struct ringattn_plan {
    int32_t n_splits;
    int32_t block_m;
    uint64_t workspace_bytes;
} ringattn_plan;

/*
 * The ring step of ringattn_step (same arguments, same result, the same
 * float32 LSE merge into out_acc / lse_acc) with a launch plan: the chunk's
 * keys may be split over plan->n_splits workgroups per query tile, whose
 * partials are merged by their LSE and then into the accumulator by a merge
 * kernel enqueued after the attention kernel (context parallelism guide,
 * section "Ring Attention":
 * one attention pass per chunk, overlapped with the ring's communication;
 * Parallelism API page, ContextParallelConfig.convert_to_fp32).  Plan it as
 * a one-chunk ringattn_forward: ringattn_forward_plan(shape, {0, kv_len},
 * 1, 0, &plan).  plan: NULL for the library's choice, else the requests of
 * a ringattn_plan.  workspace: as for ringattn_forward.  kv_len = 0 is a
 * no-op.
 */
int ringattn_step_split(const uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk,
                        float *out_acc, float *lse_acc, float scale, const ringattn_shape *shape,
                        const ringattn_plan *plan, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Fill *plan (see ringattn_plan) for a ringattn_forward call with these
 * arguments.  Pure host code: validates like ringattn_forward and launches
 * nothing.  Plans are deterministic for a given shape, layout and device.
 * (A launch choice of this library; the pages define no plan.)
 */
int ringattn_forward_plan(const ringattn_shape *shape, const int64_t *chunk_offsets, int32_t n_chunks,
                          int64_t kv_chunk_stride, ringattn_plan *plan);

/*
 * The whole shard in one call: q attends to all n_chunks K/V chunks and the
 * float32 result is written to out ([B, q_len, H, D]) and lse ([B, H, q_len]).
 * chunk_offsets (host, n_chunks + 1 entries) must start at 0, not decrease
 * and end at shape->kv_len; chunk c is rows [offsets[c], offsets[c+1]).
 * Where those rows live in k / v ([B, rows, H, D] bf16):
 *   kv_chunk_stride = 0: packed -- chunk c is rows offsets[c].. of k and v,
 *     which hold shape->kv_len rows per batch;
 *   kv_chunk_stride > 0: the padded all-gather buffer of Ring Anything --
 *     chunk c starts at row c * kv_chunk_stride and holds its true length
 *     offsets[c+1] - offsets[c] <= kv_chunk_stride; k and v hold
 *     n_chunks * kv_chunk_stride rows per batch and the padding rows are
 *     never read.
 * Chunks are visited in order 0..n_chunks-1 with an online softmax whose
 * running float32 (max, sum, output) state is the LSE merge of the partials
 * seen so far; with the packed layout a K/V tile may span the boundary of two
 * chunks (their rows are contiguous), with the padded layout it never does.
 * plan: NULL for the library's choice, else the requests of a
 * ringattn_plan (its workspace_bytes is ignored).  When the plan has more
 * than one split, workspace must hold the planned bytes
 * (RINGATTN_EWORKSPACE otherwise); workspace may be NULL with
 * workspace_bytes = 0 only when the plan needs none.  With kv_len = 0 the
 * result is out = 0, lse = -inf.
 * Source: context parallelism guide, section "Ring Attention" (after one
 * full turn every GPU has attended to the K/V of all tokens; with
 * rotate_method "allgather" every chunk is resident at once), section "Ring
 * Anything Attention" (the padded buffer) and section "Perhatian Ulysses"
 * (the Ulysses share is this call with one chunk); Parallelism API page,
 * ContextParallelConfig.
 */
int ringattn_forward(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const int64_t *chunk_offsets, int32_t n_chunks, int64_t kv_chunk_stride,
                     float *out, float *lse, float scale, const ringattn_shape *shape,
                     const ringattn_plan *plan, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ringattn_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid allocation):
 * the same arguments without the workspace, the same result.  The split
 * workspace of its launch plan is a fixed device array of
 * RINGATTN_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends.  With plan NULL (or n_splits 0) the library
 * chooses among the plans whose workspace fits that array; a requested plan
 * whose workspace does not fit is rejected with RINGATTN_EWORKSPACE before
 * anything is launched.  The call itself allocates nothing.  Calls on one GPU
 * share its array and need none of its contents from an earlier call:
 * calls that overlap in time on one GPU (different streams, not ordered)
 * race on it and must be avoided by the caller.
 */
#define RINGATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ringattn_forward_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const int64_t *chunk_offsets, int32_t n_chunks, int64_t kv_chunk_stride,
                             float *out, float *lse, float scale, const ringattn_shape *shape,
                             const ringattn_plan *plan, void *stream);

/*
 * The whole ring on one GPU: all n_chunks ranks of a ring over a sequence of
 * S = shape->q_len = shape->kv_len tokens.  Rank r holds query rows
 * [offsets[r], offsets[r+1]) and K/V chunk r (chunk_offsets as in
 * ringattn_forward, plain or Ring Anything).  For each rank, the output rows
 * of its shard start at the merge identity; at ring step s = 0..n_chunks-1
 * the rank attends to chunk (r + s) mod n_chunks -- the order in which a ring
 * that passes K/V blocks to the neighbouring rank delivers them -- and merges
 * that partial into its rows in float32 exactly as ringattn_step does (context
 * parallelism guide, section "Ring Attention": after one full turn of the
 * ring every rank has attended to the K/V of every token; Parallelism API
 * page, ContextParallelConfig.convert_to_fp32).
 *   q: [B, S, H, D] bf16, every rank's rows;
 *   k, v: [B, rows, H, D] bf16, packed (kv_chunk_stride = 0, rows = S) or the
 *     padded Ring Anything buffer (kv_chunk_stride > 0, rows =
 *     n_chunks * kv_chunk_stride; padding rows are never read);
 *   out: [B, S, H, D] float32, lse: [B, H, S] float32, fully written.
 * Enqueues one initialisation and, for n_chunks <= 32, one attention launch
 * per ring step covering every rank (n_chunks^2 launches above 32), on
 * `stream`; empty ranks and chunks launch nothing.  scale must be finite
 * and > 0.
 */
int ringattn_ring_sweep(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const int64_t *chunk_offsets, int32_t n_chunks, int64_t kv_chunk_stride,
                        float *out, float *lse, float scale, const ringattn_shape *shape, void *stream);

/*
 * Context-parallel layout of one rank: which tokens it holds, and which query
 * rows and heads make up its attention share, for plain ring, Ring Anything,
 * Ulysses, Ulysses Anything and Unified (ring x Ulysses) attention.
 *
 * The GPUs form a 2D grid of ring_degree x ulysses_degree; rank = r * U + u
 * with r the ring index and u the Ulysses index (a mesh whose dims are
 * ("ring", "ulysses"), row-major).  Every rank is in one Ulysses group (same
 * r) and one ring group (same u) (context parallelism guide, section
 * "Perhatian Terpadu"; Parallelism API page, ContextParallelConfig.mesh).
 *   token_begin/end: the rank's slice of the sequence before the Ulysses
 *     all-to-all: the sequence split into R*U pieces in rank order (R pieces
 *     for Ring Anything, U for Ulysses Anything), all heads;
 *   q_begin/end: its query rows after the all-to-all: ring chunk r, the union
 *     of the pieces of its Ulysses group (all S rows when R == 1);
 *   head_begin/end: its head block: block u of the H heads.
 * The share is: q rows [q_begin, q_end) and heads [head_begin, head_end)
 * attend to every token of the ring chunks (offsets from
 * ringattn_chunk_offsets(seq_len, R, ring_anything)) of the same heads.
 * Rules (guide, variant table and sections "Ulysses Anything Attention",
 * "Ring Anything Attention"; API page, ulysses_anything / ring_anything):
 *   plain: seq_len must divide by R * U and heads by U;
 *   ring_anything: R > 1 and U == 1, any seq_len; the first S mod R chunks
 *     hold one extra token;
 *   ulysses_anything: U > 1 and R == 1, any seq_len and head count; the first
 *     S mod U pieces hold one extra token and the first H mod U blocks one
 *     extra head (a block may be empty when H < U);
 *   the two "anything" modes do not combine; R <= RINGATTN_MAX_CHUNKS.
 * Violations give RINGATTN_EINVAL.  Pure host code.
 */
typedef struct ringattn_cp_config {
    int64_t seq_len;          /* S >= 0 tokens of the whole sequence */
    int32_t heads;            /* H >= 1 attention heads of the layer */
    int32_t ring_degree;      /* R >= 1 */
    int32_t ulysses_degree;   /* U >= 1 */
    int32_t ring_anything;    /* nonzero: Ring Anything */
    int32_t ulysses_anything; /* nonzero: Ulysses Anything */
    int32_t reserved;         /* must be 0 */
} ringattn_cp_config;

typedef struct ringattn_cp_share {
    int32_t ring_index;       /* r = rank / U */
    int32_t ulysses_index;    /* u = rank % U */
    int64_t token_begin, token_end;
    int64_t q_begin, q_end;
    int32_t head_begin, head_end;
} ringattn_cp_share;

int ringattn_cp_layout(const ringattn_cp_config *config, int32_t rank, ringattn_cp_share *share);

/*
 * The ring step with bf16 accumulators, the mode ContextParallelConfig's
 * convert_to_fp32 = False selects (Parallelism API page: without it the
 * output and LSE are not converted to float32 for the merge).  Built to
 * measure the error the float32 merge avoids; ringattn_step is the path.
 *   out_acc: [B, q_len, H, D] bf16, lse_acc: [B, H, q_len] bf16 (uint16_t
 *   bit patterns, 8- and 2-byte aligned).  ringattn_acc_init_bf16 sets
 *   out = 0, lse = -inf.  ringattn_step_bf16 computes the chunk partial as
 *   ringattn_step does, rounds its output and LSE to bf16 (round to nearest
 *   even), merges them with the stored state by the same formula in float32
 *   and stores the result rounded to bf16.  Same argument rules as
 *   ringattn_step; kv_len = 0 is a no-op.
 */
int ringattn_acc_init_bf16(uint16_t *out_acc, uint16_t *lse_acc, const ringattn_shape *shape, void *stream);
int ringattn_step_bf16(const uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk,
                       uint16_t *out_acc, uint16_t *lse_acc, float scale,
                       const ringattn_shape *shape, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
