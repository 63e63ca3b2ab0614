// Internal interface between the C-ABI host code (api.cpp) and the gfx950
// kernels (attn_pp.hip, attn_w3.hip, merge.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ringattn {

constexpr int kMaxChunks = 128;   // == RINGATTN_MAX_CHUNKS
constexpr int kBlockN = 64;       // key/value rows per LDS tile of the 8-wave kernel
constexpr int kMaxSplits = 32;

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
};

// 4-wave, 128-row variant (three workgroups per CU, 32-key tiles; the chunk
// table counts 32-key tiles).
hipError_t launch_attn_w3(const AttnArgs &a, int head_dim, EpilogueMode mode, bool chunked, hipStream_t stream);
// 8-wave, 256-row variant; `chunked` = walk the chunk table (padded layout).
hipError_t launch_attn_pp(const AttnArgs &a, int head_dim, EpilogueMode mode, bool chunked, hipStream_t stream);
hipError_t launch_merge_splits(const MergeSplitsArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_merge2(float *out_acc, float *lse_acc, const float *out_part, const float *lse_part,
                         int64_t q_len, int32_t batch, int32_t heads, int32_t head_dim, hipStream_t stream);
hipError_t launch_acc_init(float *out, float *lse, int64_t n_out, int64_t n_lse, hipStream_t stream);
hipError_t launch_acc_init_bf16(uint16_t *out, uint16_t *lse, int64_t n_out, int64_t n_lse, hipStream_t stream);

}  // namespace ringattn
