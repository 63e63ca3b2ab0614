// Internal interface between the C-ABI host code (api.cpp) and the gfx950
// kernels (attn_pp.hip, attn_w3.hip, merge.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ringattn.h"

namespace ringattn {

constexpr int kMaxChunks = 128;   // == RINGATTN_MAX_CHUNKS
constexpr int kBlockN = 64;       // key/value rows per LDS tile of the 8-wave kernel
constexpr int kMaxSplits = 32;
constexpr int kMaxSweepRanks = 32;  // ranks one batched ring-step launch covers

// The K/V tiles of one forward call, chunk by chunk.  A tile never straddles
// two chunks: chunk c owns tiles [tile_start[c], tile_start[c+1]), the last of
// which may be partial (the chunk's ragged tail).
struct ChunkTable {
    int32_t n_chunks;
    int32_t n_tiles;
    int64_t row_start[kMaxChunks];      // first K/V row of chunk c (within a batch)
    int32_t len[kMaxChunks];            // true length of chunk c
    int32_t tile_start[kMaxChunks + 1];
};

enum EpilogueMode : int32_t {
    kModeFinal = 0,    // write normalised out and lse
    kModePartial = 1,  // write normalised out and lse of this split into its workspace slot
    kModeAccum = 2,    // LSE-merge into out/lse in place (ring step)
    kModeAccumBf16 = 3,  // the same with bf16 out/lse accumulators (out/lse point to uint16_t)
};

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    float *out;
    float *lse;
    int64_t q_len;
    int64_t q_pitch;           // rows per batch in the q and out buffers (>= q_len)
    int64_t lse_pitch;         // lse entries per (batch, head) (>= q_len)
    int64_t kv_rows;           // rows per batch in the k / v buffers
    int32_t batch;
    int32_t heads;
    int32_t n_qtiles;
    int32_t n_splits;
    int64_t split_out_stride;  // floats between split slots of out (partial mode)
    int64_t split_lse_stride;  // floats between split slots of lse (partial mode)
    float scale;               // softmax scale
    float scale_log2e;         // scale * log2(e), for exp2
    ChunkTable ct;
    // Batched ring step (multi-rank launches only): rank r's query rows
    // [rank_q_begin[r], +rank_q_len[r]) attend to K/V rows
    // [ct.row_start[r], +ct.len[r]); its query tiles are workgroup tiles
    // [rank_qtile_start[r], rank_qtile_start[r+1]).
    int32_t n_ranks;
    int32_t rank_qtile_start[kMaxSweepRanks + 1];
    int32_t rank_q_len[kMaxSweepRanks];
    int64_t rank_q_begin[kMaxSweepRanks];
};

struct MergeSplitsArgs {
    const float *part_out;     // [n_splits][B, Sq, H, D]
    const float *part_lse;     // [n_splits][B, H, Sq]
    float *out;
    float *lse;
    int64_t q_len;
    int32_t batch;
    int32_t heads;
    int32_t n_splits;
    int64_t split_out_stride;
    int64_t split_lse_stride;
    int32_t accum;  // 0: write the merged result to out / lse; 1: LSE-merge it into them in place
};

// 4-wave, 128-row variant (three workgroups per CU, 32-key tiles; the chunk
// table counts 32-key tiles).
// key_groups: 1 (three 4-wave workgroups per CU) or 2 (one 8-wave workgroup
// of two key groups per CU, for launches of at most one workgroup per CU)
hipError_t launch_attn_w3(const AttnArgs &a, int head_dim, int key_groups, EpilogueMode mode, bool chunked,
                          hipStream_t stream);
// 8-wave, 256-row variant; `chunked` = walk the chunk table (padded layout).
hipError_t launch_attn_pp(const AttnArgs &a, int head_dim, EpilogueMode mode, bool chunked, hipStream_t stream);
// One ring step of several ranks in one launch (8-wave kernel, in-place float32 merge).
hipError_t launch_attn_pp_multi(const AttnArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_merge_splits(const MergeSplitsArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_merge2(float *out_acc, float *lse_acc, const float *out_part, const float *lse_part,
                         int64_t q_len, int32_t batch, int32_t heads, int32_t head_dim, hipStream_t stream);
hipError_t launch_acc_init(float *out, float *lse, int64_t n_out, int64_t n_lse, hipStream_t stream);
hipError_t launch_acc_init_bf16(uint16_t *out, uint16_t *lse, int64_t n_out, int64_t n_lse, hipStream_t stream);

// Host side of the C ABI (api.cpp), for entry points defined elsewhere.
// forward_check: ringattn_forward's validation and plan with the workspace
// limited to max_ws bytes (no HIP call); forward_impl: the same call, run
// with `workspace`; report_error: set the message of ringattn_last_error().
int forward_check(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *chunk_offsets,
                  int32_t n_chunks, int64_t kv_chunk_stride, float *out, float *lse, float scale,
                  const ::ringattn_shape *shape, const ::ringattn_plan *plan, size_t max_ws,
                  size_t *ws_needed);
int forward_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *chunk_offsets,
                 int32_t n_chunks, int64_t kv_chunk_stride, float *out, float *lse, float scale,
                 const ::ringattn_shape *shape, const ::ringattn_plan *plan, void *workspace,
                 size_t workspace_bytes, size_t max_ws, hipStream_t s);
int report_error(int status, const char *message);

}  // namespace ringattn
