// api.cpp -- the C ABI of include/ringattn.h: argument validation, the chunk
// partition, launch planning and kernel launches.  Validation always runs
// before any HIP call, so every error path works on a machine with no GPU.
#include "ringattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <string>

#include "kernels.h"

namespace {

using namespace ringattn;

static_assert(kMaxChunks == RINGATTN_MAX_CHUNKS, "chunk limit mismatch");

constexpr int32_t kAbiVersion = 6;

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return RINGATTN_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(RINGATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape checks shared by every entry point.  `kv_matters` is false where
// shape->kv_len is ignored.
int check_shape(const ringattn_shape *s, bool kv_matters) {
    if (!s) return fail(RINGATTN_EINVAL, "shape is NULL");
    if (s->reserved != 0) return fail(RINGATTN_EINVAL, "shape.reserved must be 0");
    if (s->batch < 1) return fail(RINGATTN_EINVAL, "batch must be >= 1 (got %d)", s->batch);
    if (s->heads < 1) return fail(RINGATTN_EINVAL, "heads must be >= 1 (got %d)", s->heads);
    if (s->q_len < 1) return fail(RINGATTN_EINVAL, "q_len must be >= 1 (got %lld)", (long long)s->q_len);
    if (kv_matters && s->kv_len < 0) return fail(RINGATTN_EINVAL, "kv_len must be >= 0");
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(RINGATTN_EUNSUPPORTED, "head_dim %d not built (64 or 128)", s->head_dim);
    // every element index must fit comfortably in int64 and grid sizes in int32
    const double elems = (double)s->batch * (double)s->q_len * s->heads * s->head_dim;
    if (elems > 4.0e18) return fail(RINGATTN_EINVAL, "tensor too large");
    return RINGATTN_OK;
}

int check_ptr(const void *p, uintptr_t align, const char *name) {
    if (!p) return fail(RINGATTN_EINVAL, "%s is NULL", name);
    if (!aligned(p, align)) return fail(RINGATTN_EINVAL, "%s is not %u-byte aligned", name, (unsigned)align);
    return RINGATTN_OK;
}

int cu_count_for_current_device() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;  // MI355X
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        cache[dev] = cus;
    }
    return cache[dev];
}

// The K/V layout of one call, as the kernels walk it.
struct Layout {
    ChunkTable ct;    // 64-key tiles (the 8-wave kernel)
    ChunkTable ct32;  // 32-key tiles (the 4-wave kernel)
    int64_t kv_rows;  // rows per batch in the k / v buffers
    bool chunked;     // tiles follow the chunk table (padded layout)
};

// The tile walk of one tile size over validated chunks.
int fill_table(const int64_t *offsets, int32_t n_chunks, int64_t stride, int64_t kv_len, bool chunked, int tile_n,
               ChunkTable *ct) {
    std::memset(ct, 0, sizeof *ct);
    if (!chunked) {
        ct->n_chunks = 1;
        ct->row_start[0] = 0;
        ct->len[0] = (int32_t)kv_len;
        ct->tile_start[0] = 0;
        ct->tile_start[1] = ct->n_tiles = (int32_t)((kv_len + tile_n - 1) / tile_n);
        return RINGATTN_OK;
    }
    ct->n_chunks = n_chunks;
    int64_t tiles = 0;
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t len = offsets[c + 1] - offsets[c];
        ct->row_start[c] = stride > 0 ? (int64_t)c * stride : offsets[c];
        ct->len[c] = (int32_t)len;
        ct->tile_start[c] = (int32_t)tiles;
        tiles += (len + tile_n - 1) / tile_n;
        if (tiles > (int64_t)INT32_MAX) return fail(RINGATTN_EINVAL, "too many K/V tiles");
    }
    ct->tile_start[n_chunks] = (int32_t)tiles;
    ct->n_tiles = (int32_t)tiles;
    return RINGATTN_OK;
}

// Validate host offsets and build the tile walk.  Packed chunks are one
// contiguous key range, so they become a single table entry and tiles may
// span chunk boundaries; the padded layout keeps one entry per chunk.
int build_layout(const int64_t *offsets, int32_t n_chunks, int64_t stride, int64_t kv_len, Layout *L) {
    if (!offsets) return fail(RINGATTN_EINVAL, "chunk_offsets is NULL");
    if (n_chunks < 1 || n_chunks > kMaxChunks)
        return fail(RINGATTN_EINVAL, "n_chunks %d outside [1, %d]", n_chunks, kMaxChunks);
    if (stride < 0) return fail(RINGATTN_EINVAL, "kv_chunk_stride must be >= 0");
    if (offsets[0] != 0) return fail(RINGATTN_EINVAL, "chunk_offsets[0] must be 0");
    if (offsets[n_chunks] != kv_len)
        return fail(RINGATTN_EINVAL, "chunk_offsets[%d] = %lld must equal kv_len %lld", n_chunks,
                    (long long)offsets[n_chunks], (long long)kv_len);
    for (int c = 0; c < n_chunks; ++c) {
        const int64_t len = offsets[c + 1] - offsets[c];
        if (len < 0) return fail(RINGATTN_EINVAL, "chunk_offsets decrease at %d", c);
        if (stride > 0 && len > stride)
            return fail(RINGATTN_EINVAL, "chunk %d length %lld exceeds kv_chunk_stride %lld", c, (long long)len,
                        (long long)stride);
        if (len > (int64_t)INT32_MAX - kBlockN) return fail(RINGATTN_EINVAL, "chunk %d too long", c);
    }
    L->chunked = stride > 0 || kv_len > (int64_t)INT32_MAX - kBlockN;
    L->kv_rows = stride > 0 ? (int64_t)n_chunks * stride : kv_len;
    int st;
    if ((st = fill_table(offsets, n_chunks, stride, kv_len, L->chunked, kBlockN, &L->ct))) return st;
    return fill_table(offsets, n_chunks, stride, kv_len, L->chunked, 32, &L->ct32);
}

struct Plan {
    int32_t block_m;
    int32_t n_qtiles;
    int32_t n_splits;
    size_t ws_bytes;
    int64_t split_out_stride;
    int64_t split_lse_stride;
    size_t lse_off;    // byte offset of the split LSE slots in the workspace
};

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Workspace of a K/V-split plan: n_splits float32 output slots, then
// n_splits float32 LSE slots (16-byte aligned).  No workspace without splits.
void plan_workspace(const ringattn_shape *s, Plan *p) {
    p->split_out_stride = (int64_t)s->batch * s->q_len * s->heads * s->head_dim;
    p->split_lse_stride = (int64_t)s->batch * s->heads * s->q_len;
    if (p->n_splits <= 1) {
        p->ws_bytes = p->lse_off = 0;
        return;
    }
    p->lse_off = align16((size_t)p->n_splits * (size_t)p->split_out_stride * 4u);
    p->ws_bytes = align16(p->lse_off + (size_t)p->n_splits * (size_t)p->split_lse_stride * 4u);
}

// Cost model of one launch, in microseconds.  Workgroups run in rounds of
// `slots` (one 8-wave workgroup or three 4-wave workgroups per CU); a
// workgroup costs its tile count times the time one tile takes (64-key
// tiles for the 8-wave kernel, 32-key tiles for the 4-wave one), plus a
// fixed start/finish cost; K/V splits add the float32 partial traffic
// (written once, read once by the merge) at HBM speed and the merge
// launch.  A 4-wave workgroup's tile time grows with the number of
// workgroups sharing its CU (1.47 us with three).  The constants are
// measured on MI355X.
double plan_cost(const ringattn_shape *s, int32_t n_tiles, int block_m, int splits) {
    const double cus = cu_count_for_current_device();
    const double slots = block_m == 256 ? cus : 3.0 * cus;
    const double n_wg = std::ceil((double)s->q_len / block_m) * s->heads * s->batch * splits;
    const double per_cu = std::min(3.0, std::ceil(n_wg / cus));
    const double tile_us = block_m == 256 ? 1.79 : 1.47 * (0.4 + 0.6 * per_cu / 3.0);
    const double fixed_us = 3.0;
    const double n_qtiles = std::ceil((double)s->q_len / block_m);
    const double base = n_qtiles * s->heads * s->batch;
    const double rounds = std::ceil(base * splits / slots);
    const double per_wg = std::ceil((double)n_tiles / splits);
    double cost = rounds * (per_wg * tile_us + fixed_us);
    if (splits > 1) {
        const double part_bytes = (double)s->batch * s->q_len * s->heads * (s->head_dim + 1) * 4.0;
        cost += (2.0 * splits * part_bytes + part_bytes) / 5.0e6 + 8.0;  // + the merge launch
    }
    return cost;
}

// Choose (or check) a launch plan.  req_*: the caller's requests (0 =
// choose).  max_ws: the largest workspace the caller can offer
// (SIZE_MAX = any); plans that need more are not chosen, and a requested
// split count whose workspace exceeds it is an error.
int make_plan(const ringattn_shape *s, const Layout &L, int32_t req_splits, int32_t req_block_m, Plan *p,
              size_t max_ws = SIZE_MAX) {
    if (req_splits < 0) return fail(RINGATTN_EINVAL, "requested n_splits must be >= 0");
    if (req_block_m != 0 && req_block_m != 128 && req_block_m != 256)
        return fail(RINGATTN_EINVAL, "block_m must be 0 (choose), 128 or 256 (got %d)", req_block_m);
    double best = 1e300;
    p->block_m = 0;
    p->n_splits = 1;
    size_t need_min = SIZE_MAX;
    for (int bm : {256, 128}) {
        if (req_block_m != 0 && bm != req_block_m) continue;
        const int32_t n_tiles = bm == 256 ? L.ct.n_tiles : L.ct32.n_tiles;
        const int32_t cap = n_tiles < 1 ? 1 : (n_tiles < kMaxSplits ? n_tiles : kMaxSplits);
        const int lo = req_splits > 0 ? (req_splits < cap ? req_splits : cap) : 1;
        const int hi = req_splits > 0 ? lo : cap;
        for (int sp = lo; sp <= hi; ++sp) {
            Plan cand;
            cand.block_m = bm;
            cand.n_splits = sp;
            cand.n_qtiles = (int32_t)std::min<int64_t>((s->q_len + bm - 1) / bm, INT32_MAX);
            plan_workspace(s, &cand);
            if (cand.ws_bytes > max_ws) {
                need_min = std::min(need_min, cand.ws_bytes);
                continue;
            }
            const double c = plan_cost(s, n_tiles, bm, sp);
            if (c < best * 0.999) {
                best = c;
                p->block_m = bm;
                p->n_splits = sp;
            }
        }
    }
    if (p->block_m == 0)
        return fail(RINGATTN_EWORKSPACE, "the requested plan needs %zu workspace bytes, more than the %zu available",
                    need_min, max_ws);
    const int64_t n_qtiles = (s->q_len + p->block_m - 1) / p->block_m;
    if (n_qtiles > INT32_MAX) return fail(RINGATTN_EINVAL, "q_len too large");
    p->n_qtiles = (int32_t)n_qtiles;
    const int64_t grid = n_qtiles * s->heads * s->batch * (int64_t)p->n_splits;
    if (grid > INT32_MAX) return fail(RINGATTN_EINVAL, "grid too large (%lld workgroups)", (long long)grid);
    plan_workspace(s, p);
    return RINGATTN_OK;
}

// Launch the planned kernel with the tile walk of its tile size.
hipError_t launch_plan(AttnArgs a, const Plan &p, const Layout &L, int head_dim, EpilogueMode mode, hipStream_t s) {
    if (p.block_m == 256) {
        a.ct = L.ct;
        return launch_attn_pp(a, head_dim, mode, L.chunked, s);
    }
    a.ct = L.ct32;
    // a launch that leaves each CU at most one workgroup runs it as two key
    // groups (8 waves) instead of one 4-wave workgroup
    const int64_t grid = (int64_t)p.n_qtiles * a.heads * a.batch * p.n_splits;
    const int key_groups = grid <= cu_count_for_current_device() ? 2 : 1;
    return launch_attn_w3(a, head_dim, key_groups, mode, L.chunked, s);
}

void fill_common(AttnArgs *a, const uint16_t *q, const uint16_t *k, const uint16_t *v, float *out, float *lse,
                 float scale, const ringattn_shape *s) {
    a->q = q;
    a->k = k;
    a->v = v;
    a->out = out;
    a->lse = lse;
    a->q_len = s->q_len;
    a->q_pitch = s->q_len;
    a->lse_pitch = s->q_len;
    a->batch = s->batch;
    a->heads = s->heads;
    a->scale = scale;
    a->scale_log2e = (float)((double)scale * 1.4426950408889634);
}

// Launch a planned attention pass over the layout L.  accum = 0: write the
// result to out / lse; accum = 1: LSE-merge it into the float32 accumulator
// out / lse in place (a ring step).  With more than one split the attention
// kernel writes the splits' partials to the workspace and a merge kernel
// combines them into out / lse.
int run_planned(const uint16_t *q, const uint16_t *k, const uint16_t *v, float *out, float *lse, float scale,
                const ringattn_shape *shape, const Layout &L, const Plan &p, void *workspace, bool accum,
                hipStream_t s) {
    AttnArgs a;
    std::memset(&a, 0, sizeof a);
    fill_common(&a, q, k, v, out, lse, scale, shape);
    a.ct = L.ct;
    a.kv_rows = L.kv_rows;
    a.n_qtiles = p.n_qtiles;
    a.n_splits = p.n_splits;
    if (p.n_splits == 1)
        return check_hip(launch_plan(a, p, L, shape->head_dim, accum ? kModeAccum : kModeFinal, s),
                         "attention launch");
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    float *part_out = reinterpret_cast<float *>(ws);
    float *part_lse = reinterpret_cast<float *>(ws + p.lse_off);
    a.out = part_out;
    a.lse = part_lse;
    a.split_out_stride = p.split_out_stride;
    a.split_lse_stride = p.split_lse_stride;
    int st;
    if ((st = check_hip(launch_plan(a, p, L, shape->head_dim, kModePartial, s), "attention launch"))) return st;
    MergeSplitsArgs m;
    m.part_out = part_out;
    m.part_lse = part_lse;
    m.out = out;
    m.lse = lse;
    m.q_len = shape->q_len;
    m.batch = shape->batch;
    m.heads = shape->heads;
    m.n_splits = p.n_splits;
    m.split_out_stride = p.split_out_stride;
    m.split_lse_stride = p.split_lse_stride;
    m.accum = accum ? 1 : 0;
    return check_hip(launch_merge_splits(m, shape->head_dim, s), "split merge launch");
}


int check_workspace(const Plan &p, void *workspace, size_t workspace_bytes) {
    if (p.n_splits <= 1) return RINGATTN_OK;
    if (!workspace || workspace_bytes < p.ws_bytes)
        return fail(RINGATTN_EWORKSPACE, "plan with %d splits needs %zu workspace bytes, got %zu", p.n_splits,
                    p.ws_bytes, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(RINGATTN_EINVAL, "workspace is not 16-byte aligned");
    return RINGATTN_OK;
}

}  // namespace

namespace ringattn {

// ringattn_forward's validation and launch plan, restricted to workspaces of
// at most max_ws bytes; host code only (no HIP call).  *ws_needed: the
// workspace bytes of the plan.
int forward_check(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *chunk_offsets,
                  int32_t n_chunks, int64_t kv_chunk_stride, float *out, float *lse, float scale,
                  const ringattn_shape *shape, const ringattn_plan *plan, size_t max_ws, size_t *ws_needed) {
    int st;
    if ((st = check_shape(shape, true))) return st;
    if ((st = check_ptr(q, 16, "q"))) return st;
    if ((st = check_ptr(out, 16, "out"))) return st;
    if ((st = check_ptr(lse, 4, "lse"))) return st;
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(RINGATTN_EINVAL, "scale must be finite and > 0");
    Layout L;
    if ((st = build_layout(chunk_offsets, n_chunks, kv_chunk_stride, shape->kv_len, &L))) return st;
    Plan p;
    if ((st = make_plan(shape, L, plan ? plan->n_splits : 0, plan ? plan->block_m : 0, &p, max_ws))) return st;
    if (L.ct.n_tiles > 0) {
        if ((st = check_ptr(k, 16, "k"))) return st;
        if ((st = check_ptr(v, 16, "v"))) return st;
    }
    *ws_needed = p.ws_bytes;
    return RINGATTN_OK;
}

// ringattn_forward with the plan restricted to workspaces of at most max_ws bytes.
int forward_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *chunk_offsets,
                 int32_t n_chunks, int64_t kv_chunk_stride, float *out, float *lse, float scale,
                 const ringattn_shape *shape, const ringattn_plan *plan, void *workspace, size_t workspace_bytes,
                 size_t max_ws, hipStream_t s) {
    int st;
    size_t need = 0;
    if ((st = forward_check(q, k, v, chunk_offsets, n_chunks, kv_chunk_stride, out, lse, scale, shape, plan, max_ws,
                            &need)))
        return st;
    Layout L;
    if ((st = build_layout(chunk_offsets, n_chunks, kv_chunk_stride, shape->kv_len, &L))) return st;
    Plan p;
    if ((st = make_plan(shape, L, plan ? plan->n_splits : 0, plan ? plan->block_m : 0, &p, max_ws))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes))) return st;
    if (L.ct.n_tiles == 0) {  // no keys at all: the empty result
        const int64_t n_out = (int64_t)shape->batch * shape->q_len * shape->heads * shape->head_dim;
        const int64_t n_lse = (int64_t)shape->batch * shape->heads * shape->q_len;
        return check_hip(launch_acc_init(out, lse, n_out, n_lse, s), "acc_init launch");
    }
    return run_planned(q, k, v, out, lse, scale, shape, L, p, workspace, false, s);
}

int report_error(int status, const char *message) { return fail(status, "%s", message); }

}  // namespace ringattn

extern "C" {

const char *ringattn_status_string(int status) {
    switch (status) {
        case RINGATTN_OK: return "RINGATTN_OK";
        case RINGATTN_EINVAL: return "RINGATTN_EINVAL";
        case RINGATTN_EUNSUPPORTED: return "RINGATTN_EUNSUPPORTED";
        case RINGATTN_EWORKSPACE: return "RINGATTN_EWORKSPACE";
        case RINGATTN_EHIP: return "RINGATTN_EHIP";
        default: return "RINGATTN_UNKNOWN_STATUS";
    }
}

const char *ringattn_last_error(void) { return g_last_error.c_str(); }

int32_t ringattn_abi_version(void) { return kAbiVersion; }

int ringattn_chunk_offsets(int64_t seq_len, int32_t n_chunks, int32_t ring_anything, int64_t *offsets_out) {
    if (!offsets_out) return fail(RINGATTN_EINVAL, "offsets_out is NULL");
    if (n_chunks < 1 || n_chunks > kMaxChunks)
        return fail(RINGATTN_EINVAL, "n_chunks %d outside [1, %d]", n_chunks, kMaxChunks);
    if (seq_len < 0) return fail(RINGATTN_EINVAL, "seq_len must be >= 0");
    const int64_t base = seq_len / n_chunks;
    const int64_t rem = seq_len % n_chunks;
    if (!ring_anything && rem != 0)
        return fail(RINGATTN_EINVAL,
                    "seq_len %lld does not divide by ring degree %d (remainder %lld); plain ring attention needs "
                    "an even split, Ring Anything does not",
                    (long long)seq_len, n_chunks, (long long)rem);
    int64_t acc = 0;
    offsets_out[0] = 0;
    for (int32_t c = 0; c < n_chunks; ++c) {
        acc += base + (c < rem ? 1 : 0);
        offsets_out[c + 1] = acc;
    }
    return ok();
}

int ringattn_acc_init(float *out_acc, float *lse_acc, const ringattn_shape *shape, void *stream) {
    int st;
    if ((st = check_shape(shape, false))) return st;
    if ((st = check_ptr(out_acc, 16, "out_acc"))) return st;
    if ((st = check_ptr(lse_acc, 4, "lse_acc"))) return st;
    const int64_t n_out = (int64_t)shape->batch * shape->q_len * shape->heads * shape->head_dim;
    const int64_t n_lse = (int64_t)shape->batch * shape->heads * shape->q_len;
    return check_hip(launch_acc_init(out_acc, lse_acc, n_out, n_lse, (hipStream_t)stream), "acc_init launch");
}

int ringattn_step(const uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk, float *out_acc,
                  float *lse_acc, float scale, const ringattn_shape *shape, void *stream) {
    const ringattn_plan one = {1, 0, 0};
    return ringattn_step_split(q, k_chunk, v_chunk, out_acc, lse_acc, scale, shape, &one, nullptr, 0, stream);
}

int ringattn_step_split(const uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk, float *out_acc,
                        float *lse_acc, float scale, const ringattn_shape *shape, const ringattn_plan *plan,
                        void *workspace, size_t workspace_bytes, void *stream) {
    int st;
    if ((st = check_shape(shape, true))) return st;
    if ((st = check_ptr(q, 16, "q"))) return st;
    if ((st = check_ptr(out_acc, 16, "out_acc"))) return st;
    if ((st = check_ptr(lse_acc, 4, "lse_acc"))) return st;
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(RINGATTN_EINVAL, "scale must be finite and > 0");
    Layout L;
    const int64_t offs[2] = {0, shape->kv_len};
    if ((st = build_layout(offs, 1, 0, shape->kv_len, &L))) return st;
    Plan p;
    if ((st = make_plan(shape, L, plan ? plan->n_splits : 0, plan ? plan->block_m : 0, &p))) return st;
    if ((st = check_workspace(p, workspace, workspace_bytes))) return st;
    if (shape->kv_len == 0) return ok();  // an empty chunk is the merge identity
    if ((st = check_ptr(k_chunk, 16, "k_chunk"))) return st;
    if ((st = check_ptr(v_chunk, 16, "v_chunk"))) return st;
    return run_planned(q, k_chunk, v_chunk, out_acc, lse_acc, scale, shape, L, p, workspace, true,
                       (hipStream_t)stream);
}

int ringattn_merge(float *out_acc, float *lse_acc, const float *out_part, const float *lse_part,
                   const ringattn_shape *shape, void *stream) {
    int st;
    if ((st = check_shape(shape, false))) return st;
    if ((st = check_ptr(out_acc, 16, "out_acc"))) return st;
    if ((st = check_ptr(lse_acc, 4, "lse_acc"))) return st;
    if ((st = check_ptr(out_part, 16, "out_part"))) return st;
    if ((st = check_ptr(lse_part, 4, "lse_part"))) return st;
    return check_hip(launch_merge2(out_acc, lse_acc, out_part, lse_part, shape->q_len, shape->batch, shape->heads,
                                   shape->head_dim, (hipStream_t)stream),
                     "merge launch");
}

int ringattn_forward_plan(const ringattn_shape *shape, const int64_t *chunk_offsets, int32_t n_chunks,
                          int64_t kv_chunk_stride, ringattn_plan *plan) {
    int st;
    if ((st = check_shape(shape, true))) return st;
    if (!plan) return fail(RINGATTN_EINVAL, "plan is NULL");
    Layout L;
    if ((st = build_layout(chunk_offsets, n_chunks, kv_chunk_stride, shape->kv_len, &L))) return st;
    Plan p;
    if ((st = make_plan(shape, L, plan->n_splits, plan->block_m, &p))) return st;
    plan->n_splits = p.n_splits;
    plan->block_m = p.block_m;
    plan->workspace_bytes = p.ws_bytes;
    return ok();
}

int ringattn_forward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *chunk_offsets,
                     int32_t n_chunks, int64_t kv_chunk_stride, float *out, float *lse, float scale,
                     const ringattn_shape *shape, const ringattn_plan *plan, void *workspace, size_t workspace_bytes,
                     void *stream) {
    return forward_impl(q, k, v, chunk_offsets, n_chunks, kv_chunk_stride, out, lse, scale, shape, plan, workspace,
                        workspace_bytes, SIZE_MAX, (hipStream_t)stream);
}

int ringattn_ring_sweep(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *chunk_offsets,
                        int32_t n_chunks, int64_t kv_chunk_stride, float *out, float *lse, float scale,
                        const ringattn_shape *shape, void *stream) {
    int st;
    if ((st = check_shape(shape, true))) return st;
    if (shape->kv_len != shape->q_len)
        return fail(RINGATTN_EINVAL, "ring sweep: q_len %lld must equal kv_len %lld (every rank's rows)",
                    (long long)shape->q_len, (long long)shape->kv_len);
    if ((st = check_ptr(q, 16, "q"))) return st;
    if ((st = check_ptr(k, 16, "k"))) return st;
    if ((st = check_ptr(v, 16, "v"))) return st;
    if ((st = check_ptr(out, 16, "out"))) return st;
    if ((st = check_ptr(lse, 4, "lse"))) return st;
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(RINGATTN_EINVAL, "scale must be finite and > 0");
    Layout L;  // validates the offsets and the padded stride
    if ((st = build_layout(chunk_offsets, n_chunks, kv_chunk_stride, shape->kv_len, &L))) return st;

    const int64_t S = shape->q_len;
    const int64_t HD = (int64_t)shape->heads * shape->head_dim;
    hipStream_t s = (hipStream_t)stream;
    const int64_t n_out = (int64_t)shape->batch * S * HD;
    const int64_t n_lse = (int64_t)shape->batch * shape->heads * S;
    if ((st = check_hip(launch_acc_init(out, lse, n_out, n_lse, s), "acc_init launch"))) return st;

    if (n_chunks <= kMaxSweepRanks) {
        // One launch per ring step s: every rank's query rows with its chunk
        // (r + s) mod N, merged into its rows in place.
        for (int step = 0; step < n_chunks; ++step) {
            AttnArgs a;
            std::memset(&a, 0, sizeof a);
            fill_common(&a, q, k, v, out, lse, scale, shape);
            a.q_pitch = S;
            a.lse_pitch = S;
            a.kv_rows = L.kv_rows;
            a.n_splits = 1;
            int nr = 0;
            int64_t tiles = 0;
            for (int r = 0; r < n_chunks; ++r) {
                const int64_t q_len = chunk_offsets[r + 1] - chunk_offsets[r];
                const int c = (r + step) % n_chunks;
                const int64_t len = chunk_offsets[c + 1] - chunk_offsets[c];
                if (q_len == 0 || len == 0) continue;  // an empty rank or chunk changes nothing
                a.rank_q_begin[nr] = chunk_offsets[r];
                a.rank_q_len[nr] = (int32_t)q_len;
                a.ct.row_start[nr] = kv_chunk_stride > 0 ? (int64_t)c * kv_chunk_stride : chunk_offsets[c];
                a.ct.len[nr] = (int32_t)len;
                tiles += (q_len + 255) / 256;
                a.rank_qtile_start[nr + 1] = (int32_t)tiles;
                ++nr;
            }
            if (nr == 0) continue;
            if (tiles * shape->heads * shape->batch > INT32_MAX) return fail(RINGATTN_EINVAL, "grid too large");
            a.n_ranks = nr;
            a.ct.n_chunks = nr;
            if ((st = check_hip(launch_attn_pp_multi(a, shape->head_dim, s), "attention launch"))) return st;
        }
        return ok();
    }
    for (int r = 0; r < n_chunks; ++r) {
        const int64_t q0 = chunk_offsets[r], q_len = chunk_offsets[r + 1] - chunk_offsets[r];
        if (q_len == 0) continue;
        for (int step = 0; step < n_chunks; ++step) {
            const int c = (r + step) % n_chunks;
            const int64_t len = chunk_offsets[c + 1] - chunk_offsets[c];
            if (len == 0) continue;  // an empty chunk is the merge identity
            const int64_t row0 = kv_chunk_stride > 0 ? (int64_t)c * kv_chunk_stride : chunk_offsets[c];
            ringattn_shape rs = *shape;
            rs.q_len = q_len;
            rs.kv_len = len;
            Layout cl;
            const int64_t offs[2] = {0, len};
            if ((st = build_layout(offs, 1, 0, len, &cl))) return st;
            Plan p;
            if ((st = make_plan(&rs, cl, 1, 0, &p))) return st;
            AttnArgs a;
            std::memset(&a, 0, sizeof a);
            fill_common(&a, q + q0 * HD, k + row0 * HD, v + row0 * HD, out + q0 * HD, lse + q0, scale, &rs);
            a.q_pitch = S;      // the rank's rows sit inside the full-sequence q / out / lse
            a.lse_pitch = S;
            a.ct = cl.ct;
            a.kv_rows = L.kv_rows;
            a.n_qtiles = p.n_qtiles;
            a.n_splits = 1;
            if ((st = check_hip(launch_plan(a, p, cl, shape->head_dim, kModeAccum, s), "attention launch")))
                return st;
        }
    }
    return ok();
}

// Piece i of n of a length-`len` range, the first len % n pieces one longer.
static void even_piece(int64_t len, int64_t n, int64_t i, int64_t *begin, int64_t *end) {
    const int64_t base = len / n, rem = len % n;
    *begin = i * base + (i < rem ? i : rem);
    *end = *begin + base + (i < rem ? 1 : 0);
}

int ringattn_cp_layout(const ringattn_cp_config *cfg, int32_t rank, ringattn_cp_share *share) {
    if (!cfg) return fail(RINGATTN_EINVAL, "config is NULL");
    if (!share) return fail(RINGATTN_EINVAL, "share is NULL");
    if (cfg->reserved != 0) return fail(RINGATTN_EINVAL, "config.reserved must be 0");
    const int64_t S = cfg->seq_len;
    const int32_t H = cfg->heads, R = cfg->ring_degree, U = cfg->ulysses_degree;
    if (S < 0) return fail(RINGATTN_EINVAL, "seq_len must be >= 0");
    if (H < 1) return fail(RINGATTN_EINVAL, "heads must be >= 1");
    if (R < 1 || R > kMaxChunks) return fail(RINGATTN_EINVAL, "ring_degree %d outside [1, %d]", R, kMaxChunks);
    if (U < 1 || U > (1 << 20)) return fail(RINGATTN_EINVAL, "ulysses_degree %d outside [1, 2^20]", U);
    const bool ra = cfg->ring_anything != 0, ua = cfg->ulysses_anything != 0;
    if (ra && ua) return fail(RINGATTN_EINVAL, "ring_anything and ulysses_anything do not combine");
    if (ra && !(R > 1 && U == 1)) return fail(RINGATTN_EINVAL, "ring_anything needs ring_degree > 1 and ulysses_degree 1");
    if (ua && !(U > 1 && R == 1)) return fail(RINGATTN_EINVAL, "ulysses_anything needs ulysses_degree > 1 and ring_degree 1");
    const int64_t world = (int64_t)R * U;
    if (rank < 0 || rank >= world) return fail(RINGATTN_EINVAL, "rank %d outside [0, %lld)", rank, (long long)world);
    if (!ra && !ua) {
        if (S % world != 0)
            return fail(RINGATTN_EINVAL, "seq_len %lld does not divide by ring_degree * ulysses_degree = %lld",
                        (long long)S, (long long)world);
        if (H % U != 0) return fail(RINGATTN_EINVAL, "heads %d do not divide by ulysses_degree %d", H, U);
    }
    ringattn_cp_share sh;
    sh.ring_index = rank / U;
    sh.ulysses_index = rank % U;
    // the sequence before the all-to-all: R*U pieces in rank order
    even_piece(S, world, rank, &sh.token_begin, &sh.token_end);
    // query rows of the share: ring chunk r
    even_piece(S, R, sh.ring_index, &sh.q_begin, &sh.q_end);
    int64_t h0, h1;
    even_piece(H, U, sh.ulysses_index, &h0, &h1);
    sh.head_begin = (int32_t)h0;
    sh.head_end = (int32_t)h1;
    *share = sh;
    return ok();
}

int ringattn_acc_init_bf16(uint16_t *out_acc, uint16_t *lse_acc, const ringattn_shape *shape, void *stream) {
    int st;
    if ((st = check_shape(shape, false))) return st;
    if ((st = check_ptr(out_acc, 8, "out_acc"))) return st;
    if ((st = check_ptr(lse_acc, 2, "lse_acc"))) return st;
    const int64_t n_out = (int64_t)shape->batch * shape->q_len * shape->heads * shape->head_dim;
    const int64_t n_lse = (int64_t)shape->batch * shape->heads * shape->q_len;
    return check_hip(launch_acc_init_bf16(out_acc, lse_acc, n_out, n_lse, (hipStream_t)stream), "acc_init launch");
}

int ringattn_step_bf16(const uint16_t *q, const uint16_t *k_chunk, const uint16_t *v_chunk, uint16_t *out_acc,
                       uint16_t *lse_acc, float scale, const ringattn_shape *shape, void *stream) {
    int st;
    if ((st = check_shape(shape, true))) return st;
    if ((st = check_ptr(q, 16, "q"))) return st;
    if ((st = check_ptr(out_acc, 8, "out_acc"))) return st;
    if ((st = check_ptr(lse_acc, 2, "lse_acc"))) return st;
    if (!(std::isfinite(scale) && scale > 0.f)) return fail(RINGATTN_EINVAL, "scale must be finite and > 0");
    if (shape->kv_len == 0) return ok();
    if ((st = check_ptr(k_chunk, 16, "k_chunk"))) return st;
    if ((st = check_ptr(v_chunk, 16, "v_chunk"))) return st;
    Layout L;
    const int64_t offs[2] = {0, shape->kv_len};
    if ((st = build_layout(offs, 1, 0, shape->kv_len, &L))) return st;
    Plan p;
    if ((st = make_plan(shape, L, 1, 0, &p))) return st;
    AttnArgs a;
    std::memset(&a, 0, sizeof a);
    fill_common(&a, q, k_chunk, v_chunk, reinterpret_cast<float *>(out_acc), reinterpret_cast<float *>(lse_acc),
                scale, shape);
    a.ct = L.ct;
    a.kv_rows = L.kv_rows;
    a.n_qtiles = p.n_qtiles;
    a.n_splits = 1;
    return check_hip(launch_plan(a, p, L, shape->head_dim, kModeAccumBf16, (hipStream_t)stream),
                     "attention launch");
}

}  // extern "C"
