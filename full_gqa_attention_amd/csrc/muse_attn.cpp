// muse_attn.cpp -- the C ABI of libmuse_attn (declared in include/muse_attn.h):
// host-side validation (fail closed, before anything is enqueued), workspace
// layout, the RoPE frequency table, and the kernel launch sequence.
#include "muse_attn.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "kernels.h"

namespace {

using muse::AttnArgs;
using muse::DecodeArgs;
using muse::PrepArgs;
using muse::VerifyArgs;

constexpr int kHeads = 32, kKvHeads = 2, kHeadDim = 128;
constexpr int kModelLayers = 52;          // "Chapter 9" 9.4: 52 blocks
constexpr int64_t kMaxPositions = 1 << 24; // positions stay exact as f32 (RoPE angle)
constexpr int32_t kMaxSeqs = 1 << 20;
constexpr size_t kAlign = 256;
constexpr float kMaxGain = 4096.0f;        // 4096 * sqrt(128) < 65504 (fp16 max)

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
size_t elem_bytes(int32_t dtype) { return dtype == MUSE_BF16 ? 2 : 4; }

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

muse_status check_layer(const muse_attn_layer* l) {
    if (!l) return MUSE_ERR_NULL;
    if (l->n_heads != kHeads || l->n_kv_heads != kKvHeads || l->head_dim != kHeadDim)
        return MUSE_ERR_SHAPE;
    if (l->dtype != MUSE_F32 && l->dtype != MUSE_BF16) return MUSE_ERR_DTYPE;
    if (l->kind == MUSE_SLIDING_ROPE) {
        if (l->window < 1 || !finite_pos(l->rope_theta)) return MUSE_ERR_LAYER;
    } else if (l->kind == MUSE_FULL_NOPE) {
        if (l->window != 0 || l->rope_theta != 0.0f) return MUSE_ERR_LAYER;
    } else {
        return MUSE_ERR_LAYER;
    }
    if (!finite_pos(l->rms_eps) || !finite_pos(l->attn_scale)) return MUSE_ERR_LAYER;
    // bf16 layers score with fp16 operands: normed rows are bounded by
    // |gain| * sqrt(128), which must stay inside fp16's range.
    if (!(std::fabs(l->q_norm_gain) <= kMaxGain) || !(std::fabs(l->k_norm_gain) <= kMaxGain))
        return MUSE_ERR_LAYER;
    // a ring cache holds a sliding layer's window ("Chapter 9" 9.7); bf16 only
    if (l->kv_ring != 0 && (l->kv_ring != 1 || l->kind != MUSE_SLIDING_ROPE || l->dtype != MUSE_BF16))
        return MUSE_ERR_LAYER;
    return MUSE_OK;
}

// Prefix positions the prefill's key copy holds per sequence: all of them on
// full layers; on sliding layers those from the window's first visible one
// rounded down to kWindowAlign.
int64_t copied_prefix(const muse_attn_layer* l, int32_t max_seq_len) {
    int64_t prefix = max_seq_len;
    const int64_t win = (int64_t)l->window - 1 + (muse::kWindowAlign - 1);
    if (l->kind == MUSE_SLIDING_ROPE && win < prefix) prefix = win;
    return prefix;
}

// Short bf16 chunks (at most kVerifyTokens new tokens, linear cache) take the
// verify kernels: split-K over the keys with every head of a KV head per
// workgroup.
bool use_verify(const muse_attn_layer* l, int32_t n_new) {
    return l->dtype == MUSE_BF16 && !l->kv_ring && n_new >= 1 && n_new <= muse::kVerifyTokens;
}

// Verify splits: about kVerifyBlocks workgroups in total, at least 16 tiles (512 keys)
// per split when the keys allow, at most 64 splits.
void verify_split(const muse_attn_layer* l, int32_t n_seq, int32_t n_new, int32_t max_seq_len,
                  int32_t* nsplit, int32_t* chunk_tiles) {
    int64_t prefix = max_seq_len;
    if (l->kind == MUSE_SLIDING_ROPE && (int64_t)l->window - 1 < prefix) prefix = (int64_t)l->window - 1;
    const int64_t bn = muse::kVerifyTile;
    const int64_t tiles = (prefix + n_new + 2 * bn - 1) / bn;   // covers any alignment of the key range
    const int64_t seqs = n_seq > 0 ? n_seq : 1;
    int64_t want = (muse::kVerifyBlocks + 2 * seqs - 1) / (2 * seqs);
    if (want > tiles / 16) want = tiles / 16;
    if (want > 64) want = 64;
    if (want < 1) want = 1;
    const int64_t ch = (tiles + want - 1) / want;
    *chunk_tiles = (int32_t)ch;
    *nsplit = (int32_t)((tiles + ch - 1) / ch);
}

// Rows the cache must hold: every position of the call, or on a ring layer
// the last min(window, positions) of them.
int64_t rows_needed(const muse_attn_layer* l, int32_t max_seq_len, int32_t n_new) {
    const int64_t need = (int64_t)max_seq_len + n_new;
    return l->kv_ring ? (need < l->window ? need : (int64_t)l->window) : need;
}

muse_status check_sizes(int32_t n_seq, int32_t n_new, int32_t max_seq_len) {
    if (n_seq < 0 || n_seq > kMaxSeqs || n_new < 0 || max_seq_len < 0) return MUSE_ERR_SHAPE;
    if ((int64_t)max_seq_len + n_new > kMaxPositions) return MUSE_ERR_SHAPE;
    if ((int64_t)n_seq * n_new > (int64_t)1 << 31) return MUSE_ERR_SHAPE;
    return MUSE_OK;
}

// Decode split: about kDecodeTargetBlocks workgroups in total, chunks a
// multiple of the 64-row tile and (when the span allows) of at least
// kDecodeMinSplitRows rows: a CU streams only a few tens of GB/s, so a short
// window is spread over many CUs, but each split also carries its first
// loads and a partial for the merge.
// The span of visible rows is at most window (sliding) or max_seq_len + 1
// (full).
void decode_split(const muse_attn_layer* l, int32_t n_seq, int32_t max_seq_len,
                  int32_t* chunk, int32_t* nsplit) {
    int64_t span = (int64_t)max_seq_len + 1;
    if (l->kind == MUSE_SLIDING_ROPE && l->window < span) span = l->window;
    const int64_t pairs = (int64_t)(n_seq > 0 ? n_seq : 1) * kKvHeads;
    const int64_t target = muse::kDecodeTargetBlocks;
    int64_t want = (target + pairs - 1) / pairs;
    const int64_t tiles = (span + muse::kDecodeTile - 1) / muse::kDecodeTile;
    const int64_t by_rows = span / muse::kDecodeMinSplitRows;
    if (want > by_rows) want = by_rows;
    if (want > tiles) want = tiles;
    if (want > muse::kMaxSplits) want = muse::kMaxSplits;
    if (want < 1) want = 1;
    int64_t ch = (span + want - 1) / want;
    ch = (ch + muse::kDecodeTile - 1) / muse::kDecodeTile * muse::kDecodeTile;
    *chunk = (int32_t)ch;
    *nsplit = (int32_t)((span + ch - 1) / ch);
}

// Prefill: on f32 layers Q-hat [S][N][32][128]; on bf16 layers (where the
// attention kernel makes Q-hat itself) the fp16 copy of the keys the chunk can
// see, [S][kq_capacity][2][128]: on full layers row = position (kq_capacity =
// max_seq_len + N), on sliding layers row = position - base with base =
// max(0, seq_len - window + 1) rounded down to kWindowAlign (kq_capacity =
// min(max_seq_len, window - 1 + kWindowAlign - 1) + N); on ring layers then a
// copy of the same rows of V, laid out alike.
// Decode: with more than one split per (sequence, KV head), the split partials
// O [S][32][nsplit][128], m and l [S][32][nsplit]; with one split, nothing.
struct WorkspaceLayout {
    size_t qhat = 0, kq = 0, vq = 0, part_o = 0, part_m = 0, part_l = 0, total = 0;
    int64_t kq_capacity = 0;
    int32_t chunk = 0, nsplit = 0;
    bool verify = false;
};

WorkspaceLayout layout_for(const muse_attn_layer* l, int32_t n_seq, int32_t n_new,
                           int32_t max_seq_len, bool decode) {
    WorkspaceLayout w;
    const size_t es = elem_bytes(l->dtype);
    size_t off = 0;
    if (!decode && use_verify(l, n_new)) {
        // short chunk: the verify partials [S][2][nsplit][16][16] x (128 + 2) floats
        w.verify = true;
        verify_split(l, n_seq, n_new, max_seq_len, &w.nsplit, &w.chunk);
        const size_t rows = (size_t)n_seq * kKvHeads * w.nsplit * (kHeads / kKvHeads) * muse::kVerifyTokens;
        w.part_o = 0;
        off = round_up(rows * kHeadDim * sizeof(float), kAlign);
        w.part_m = off;
        off += round_up(rows * sizeof(float), kAlign);
        w.part_l = off;
        off += round_up(rows * sizeof(float), kAlign);
    } else if (!decode) {
        // bf16 layers make Q-hat inside the attention kernel; f32 layers stage it
        w.qhat = 0;
        if (l->dtype != MUSE_BF16) off = round_up((size_t)n_seq * n_new * kHeads * kHeadDim * es, kAlign);
        if (l->dtype == MUSE_BF16) {
            w.kq = off;
            w.kq_capacity = copied_prefix(l, max_seq_len) + n_new;
            const size_t rows_bytes = round_up((size_t)n_seq * (size_t)w.kq_capacity * kKvHeads * kHeadDim * 2, kAlign);
            off += rows_bytes;
            if (l->kv_ring) {                          // V rows the chunk can see, out of the ring
                w.vq = off;
                off += rows_bytes;
            }
        }
    } else {
        decode_split(l, n_seq, max_seq_len, &w.chunk, &w.nsplit);
        const size_t parts = w.nsplit > 1 ? (size_t)n_seq * kHeads * w.nsplit : 0;
        w.part_o = off;
        off += round_up(parts * kHeadDim * sizeof(float), kAlign);
        w.part_m = off;
        off += round_up(parts * sizeof(float), kAlign);
        w.part_l = off;
        off += round_up(parts * sizeof(float), kAlign);
    }
    w.total = off;
    return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

void rope_table(float theta, float* out64) {
    for (int i = 0; i < kHeadDim / 2; ++i)
        out64[i] = (float)std::pow((double)theta, -(2.0 * i) / (double)kHeadDim);
}

muse_status run(const muse_attn_layer* layer, int32_t n_seq, int32_t n_new, const int32_t* seq_len,
                int32_t max_seq_len, const void* q, const void* k, const void* v, const void* gate,
                const muse_kv_cache* cache, void* out, void* workspace, size_t workspace_bytes,
                hipStream_t stream, const muse_kernel_timer* timer, bool decode) {
    muse_status st = check_layer(layer);
    if (st != MUSE_OK) return st;
    if ((st = check_sizes(n_seq, n_new, max_seq_len)) != MUSE_OK) return st;
    if (!cache) return MUSE_ERR_NULL;
    if (cache->capacity < 0) return MUSE_ERR_CAPACITY;
    if (rows_needed(layer, max_seq_len, n_new) > cache->capacity) return MUSE_ERR_CAPACITY;
    // a ring is addressed with 32-bit byte offsets
    if (layer->kv_ring && cache->capacity * (int64_t)(kKvHeads * kHeadDim * elem_bytes(layer->dtype)) > INT32_MAX)
        return MUSE_ERR_CAPACITY;
    if (n_seq == 0 || n_new == 0) return MUSE_OK;    // nothing to do
    if (!seq_len || !q || !k || !v || !gate || !out || !cache->k || !cache->v) return MUSE_ERR_NULL;
    if (timer && (!timer->start || !timer->stop)) return MUSE_ERR_NULL;
    const WorkspaceLayout wl = layout_for(layer, n_seq, n_new, max_seq_len, decode);
    if (wl.total > 0 && !workspace) return MUSE_ERR_NULL;      // a call that needs no workspace takes NULL
    const void* ptrs[] = {seq_len, q, k, v, gate, out, cache->k, cache->v, workspace};
    for (const void* p : ptrs)
        if (!aligned16(p)) return MUSE_ERR_ALIGN;
    if (workspace_bytes < wl.total) return MUSE_ERR_WORKSPACE;

    const size_t es = elem_bytes(layer->dtype);
    const size_t tok = (size_t)n_seq * n_new;
    auto R = [](const void* p, size_t n) { return Range{(uintptr_t)p, (uintptr_t)p + n}; };
    const Range r_seq = R(seq_len, (size_t)n_seq * 4);
    const Range r_q = R(q, tok * kHeads * kHeadDim * es);
    const Range r_k = R(k, tok * kKvHeads * kHeadDim * es);
    const Range r_v = R(v, tok * kKvHeads * kHeadDim * es);
    const Range r_g = R(gate, tok * kHeads * kHeadDim * es);
    const size_t cache_bytes = (size_t)n_seq * (size_t)cache->capacity * kKvHeads * kHeadDim * es;
    const Range r_ck = R(cache->k, cache_bytes);
    const Range r_cv = R(cache->v, cache_bytes);
    const Range r_out = R(out, tok * kHeads * kHeadDim * es);
    const Range r_ws = R(workspace, wl.total);
    // every written buffer (out, workspace, cache k, cache v) is disjoint from every other
    const Range all[] = {r_seq, r_q, r_k, r_v, r_g, r_ck, r_cv, r_out, r_ws};
    const int written[] = {5, 6, 7, 8};
    for (int wi : written)
        for (int j = 0; j < 9; ++j)
            if (j != wi && overlap(all[wi], all[j])) return MUSE_ERR_ALIAS;

    char* ws = (char*)workspace;
    const int dt = layer->dtype;
    const bool rope = layer->kind == MUSE_SLIDING_ROPE;
    const float scale_log2 = (float)((double)layer->attn_scale * 1.4426950408889634);

    if (decode) {
        DecodeArgs da;
        std::memset(&da, 0, sizeof da);
        da.q = q;
        da.k = k;
        da.v = v;
        da.gate = gate;
        da.out = out;
        da.cache_k = cache->k;
        da.cache_v = cache->v;
        da.capacity = cache->capacity;
        da.seq_len = seq_len;
        da.max_seq_len = max_seq_len;
        da.n_seq = n_seq;
        da.window = rope ? layer->window : 0;
        da.ring = layer->kv_ring ? cache->capacity : 0;
        da.rope = rope ? 1 : 0;
        da.eps = layer->rms_eps;
        da.q_gain = layer->q_norm_gain;
        da.k_gain = layer->k_norm_gain;
        da.scale_log2 = scale_log2;
        da.chunk = wl.chunk;
        da.nsplit = wl.nsplit;
        da.part_o = (float*)(ws + wl.part_o);
        da.part_m = (float*)(ws + wl.part_m);
        da.part_l = (float*)(ws + wl.part_l);
        if (rope) rope_table(layer->rope_theta, da.theta);
        if (timer && hipEventRecord(timer->start, stream) != hipSuccess) return MUSE_ERR_HIP;
        if (muse::launch_decode(da, dt, stream) != hipSuccess) return MUSE_ERR_HIP;
        if (timer && hipEventRecord(timer->stop, stream) != hipSuccess) return MUSE_ERR_HIP;
        if (da.nsplit > 1 && muse::launch_decode_merge(da, dt, stream) != hipSuccess) return MUSE_ERR_HIP;
        return MUSE_OK;
    }

    PrepArgs pa;
    std::memset(&pa, 0, sizeof pa);
    pa.q = q;
    pa.k = k;
    pa.v = v;
    pa.qhat = ws + wl.qhat;
    pa.cache_k = cache->k;
    pa.cache_v = cache->v;
    pa.capacity = cache->capacity;
    pa.seq_len = seq_len;
    pa.max_seq_len = max_seq_len;
    pa.n_seq = n_seq;
    pa.n_new = n_new;
    pa.rope = rope ? 1 : 0;
    pa.eps = layer->rms_eps;
    pa.q_gain = layer->q_norm_gain;
    pa.k_gain = layer->k_norm_gain;
    pa.q_scale = scale_log2;
    pa.skip_q = layer->dtype == MUSE_BF16 ? 1 : 0;
    pa.window = rope ? layer->window : 0;
    if (layer->dtype == MUSE_BF16 && !wl.verify) {
        // prefix rows the key copy holds (see copied_prefix), 64 per workgroup
        pa.kq = ws + wl.kq;
        pa.kq_capacity = wl.kq_capacity;
        pa.conv_blocks = (int32_t)((copied_prefix(layer, max_seq_len) + 63) / 64);
        pa.kq_windowed = rope ? 1 : 0;
        pa.ring = layer->kv_ring ? cache->capacity : 0;
        pa.vq = layer->kv_ring ? (void*)(ws + wl.vq) : nullptr;
    }
    if (rope) rope_table(layer->rope_theta, pa.theta);

    if (wl.verify) {
        // a short chunk: append its K-hat and V rows, then the verify kernels
        // read the keys straight from the cache (no prefix copy)
        if (muse::launch_prep(pa, dt, stream) != hipSuccess) return MUSE_ERR_HIP;
        VerifyArgs va;
        std::memset(&va, 0, sizeof va);
        va.q = q;
        va.gate = gate;
        va.out = out;
        va.cache_k = cache->k;
        va.cache_v = cache->v;
        va.capacity = cache->capacity;
        va.seq_len = seq_len;
        va.max_seq_len = max_seq_len;
        va.n_seq = n_seq;
        va.n_new = n_new;
        va.window = rope ? layer->window : 0;
        va.rope = pa.rope;
        va.eps = pa.eps;
        va.q_gain = pa.q_gain;
        va.q_scale = pa.q_scale;
        std::memcpy(va.theta, pa.theta, sizeof va.theta);
        va.nsplit = wl.nsplit;
        va.chunk_tiles = wl.chunk;
        va.part_o = (float*)(ws + wl.part_o);
        va.part_m = (float*)(ws + wl.part_m);
        va.part_l = (float*)(ws + wl.part_l);
        if (timer && hipEventRecord(timer->start, stream) != hipSuccess) return MUSE_ERR_HIP;
        if (muse::launch_verify(va, stream) != hipSuccess) return MUSE_ERR_HIP;
        if (muse::launch_verify_merge(va, stream) != hipSuccess) return MUSE_ERR_HIP;
        if (timer && hipEventRecord(timer->stop, stream) != hipSuccess) return MUSE_ERR_HIP;
        return MUSE_OK;
    }

    AttnArgs aa;
    std::memset(&aa, 0, sizeof aa);
    aa.qhat = pa.qhat;
    aa.q = q;
    aa.rope = pa.rope;
    aa.eps = pa.eps;
    aa.q_gain = pa.q_gain;
    aa.q_scale = pa.q_scale;
    std::memcpy(aa.theta, pa.theta, sizeof aa.theta);
    aa.gate = gate;
    aa.out = out;
    aa.kq = layer->dtype == MUSE_BF16 ? (const void*)(ws + wl.kq) : cache->k;
    aa.kq_capacity = layer->dtype == MUSE_BF16 ? wl.kq_capacity : cache->capacity;
    aa.cache_v = layer->kv_ring ? (const void*)(ws + wl.vq) : cache->v;
    aa.capacity = layer->kv_ring ? wl.kq_capacity : cache->capacity;
    aa.kq_windowed = pa.kq_windowed;
    aa.v_windowed = layer->kv_ring ? 1 : 0;
    aa.seq_len = seq_len;
    aa.max_seq_len = max_seq_len;
    aa.n_seq = n_seq;
    aa.n_new = n_new;
    aa.window = rope ? layer->window : 0;

    if (layer->kv_ring) {
        // the visible prefix is copied out of the ring before any new row
        // overwrites a slot it reads
        pa.phase = 1;
        if (muse::launch_prep(pa, dt, stream) != hipSuccess) return MUSE_ERR_HIP;
        pa.phase = 2;
    }
    if (muse::launch_prep(pa, dt, stream) != hipSuccess) return MUSE_ERR_HIP;
    if (timer && hipEventRecord(timer->start, stream) != hipSuccess) return MUSE_ERR_HIP;
    if (muse::launch_prefill(aa, dt, stream) != hipSuccess) return MUSE_ERR_HIP;
    if (timer && hipEventRecord(timer->stop, stream) != hipSuccess) return MUSE_ERR_HIP;
    return MUSE_OK;
}

}  // namespace

extern "C" {

muse_status muse_attn_prefill(const muse_attn_layer* layer, int32_t n_seq, int32_t n_new,
                              const int32_t* seq_len, int32_t max_seq_len,
                              const void* q, const void* k, const void* v, const void* gate,
                              const muse_kv_cache* cache, void* out,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const muse_kernel_timer* timer) {
    return run(layer, n_seq, n_new, seq_len, max_seq_len, q, k, v, gate, cache, out, workspace,
               workspace_bytes, stream, timer, false);
}

muse_status muse_attn_decode(const muse_attn_layer* layer, int32_t n_seq,
                             const int32_t* seq_len, int32_t max_seq_len,
                             const void* q, const void* k, const void* v, const void* gate,
                             const muse_kv_cache* cache, void* out,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream, const muse_kernel_timer* timer) {
    return run(layer, n_seq, 1, seq_len, max_seq_len, q, k, v, gate, cache, out, workspace,
               workspace_bytes, stream, timer, true);
}

muse_status muse_attn_decode_noalloc(const muse_attn_layer* layer, int32_t n_seq,
                                     const int32_t* seq_len, int32_t max_seq_len,
                                     const void* q, const void* k, const void* v, const void* gate,
                                     const muse_kv_cache* cache, void* out,
                                     hipStream_t stream, const muse_kernel_timer* timer) {
    muse_status st = check_layer(layer);
    if (st != MUSE_OK) return st;
    if ((st = check_sizes(n_seq, 1, max_seq_len)) != MUSE_OK) return st;
    if (layout_for(layer, n_seq, 1, max_seq_len, true).total > muse::kDecodeScratchBytes)
        return MUSE_ERR_WORKSPACE;                     // the split partials exceed the library's scratch
    void* ws = nullptr;
    if (n_seq > 0 && muse::decode_scratch(&ws) != hipSuccess) return MUSE_ERR_HIP;
    return run(layer, n_seq, 1, seq_len, max_seq_len, q, k, v, gate, cache, out, ws, muse::kDecodeScratchBytes,
               stream, timer, true);
}

muse_status muse_attn_workspace_size(const muse_attn_layer* layer, int32_t n_seq, int32_t n_new,
                                     int32_t max_seq_len, int32_t is_decode, size_t* bytes) {
    if (!bytes) return MUSE_ERR_NULL;
    muse_status st = check_layer(layer);
    if (st != MUSE_OK) return st;
    if (is_decode) n_new = 1;
    if ((st = check_sizes(n_seq, n_new, max_seq_len)) != MUSE_OK) return st;
    *bytes = layout_for(layer, n_seq, n_new, max_seq_len, is_decode != 0).total;
    return MUSE_OK;
}

muse_status muse_kv_relocate(const muse_attn_layer* layer, const muse_kv_cache* src, int32_t n_seq_src,
                             const muse_kv_cache* dst, int32_t n_seq_dst, const muse_kv_tile* tiles,
                             int32_t n_tiles, hipStream_t stream) {
    muse_status st = check_layer(layer);
    if (st != MUSE_OK) return st;
    // only position-free rows may move ("Chapter 14" 14.6)
    if (layer->kind != MUSE_FULL_NOPE || layer->rope_theta != 0.0f) return MUSE_ERR_LAYER;
    if (!src || !dst) return MUSE_ERR_NULL;
    if (n_tiles < 0 || n_seq_src < 1 || n_seq_dst < 1) return MUSE_ERR_SHAPE;
    if (n_tiles == 0) return MUSE_OK;
    if (!tiles || !src->k || !src->v || !dst->k || !dst->v) return MUSE_ERR_NULL;
    if (!aligned16(src->k) || !aligned16(src->v) || !aligned16(dst->k) || !aligned16(dst->v)) return MUSE_ERR_ALIGN;
    if (src->capacity < 0 || dst->capacity < 0) return MUSE_ERR_CAPACITY;
    const size_t row = (size_t)kKvHeads * kHeadDim * elem_bytes(layer->dtype);
    for (int32_t i = 0; i < n_tiles; ++i) {
        const muse_kv_tile& t = tiles[i];
        if (t.src_seq < 0 || t.src_seq >= n_seq_src || t.dst_seq < 0 || t.dst_seq >= n_seq_dst ||
            t.src_pos < 0 || t.dst_pos < 0 || t.n_rows < 0)
            return MUSE_ERR_SHAPE;
        if (t.src_pos > src->capacity - t.n_rows || t.dst_pos > dst->capacity - t.n_rows) return MUSE_ERR_CAPACITY;
        // byte ranges of the tile's K rows in each cache (V rows sit at the same offsets)
        const uintptr_t s0 = (uintptr_t)src->k + ((size_t)t.src_seq * (size_t)src->capacity + (size_t)t.src_pos) * row;
        const uintptr_t d0 = (uintptr_t)dst->k + ((size_t)t.dst_seq * (size_t)dst->capacity + (size_t)t.dst_pos) * row;
        const size_t n = (size_t)t.n_rows * row;
        const uintptr_t sv0 = (uintptr_t)src->v + (s0 - (uintptr_t)src->k);
        const uintptr_t dv0 = (uintptr_t)dst->v + (d0 - (uintptr_t)dst->k);
        const Range sk{s0, s0 + n}, dk{d0, d0 + n}, sv{sv0, sv0 + n}, dv{dv0, dv0 + n};
        if (n && (overlap(sk, dk) || overlap(sv, dv) || overlap(sk, dv) || overlap(sv, dk))) return MUSE_ERR_ALIAS;
    }
    // Tiles go to the device in launches of at most kRelocTiles; a launch ends
    // early where a tile reads or writes rows an earlier tile of the launch
    // writes (or writes rows it reads), so tiles apply in order.
    muse::RelocArgs ra;
    std::memset(&ra, 0, sizeof ra);
    ra.src_k = (const char*)src->k;
    ra.src_v = (const char*)src->v;
    ra.dst_k = (char*)dst->k;
    ra.dst_v = (char*)dst->v;
    Range reads[muse::kRelocTiles][2], writes[muse::kRelocTiles][2];
    auto flush = [&]() {
        const hipError_t e = muse::launch_relocate(ra, stream);
        ra.n_tiles = 0;
        ra.block0[0] = 0;
        return e;
    };
    for (int32_t i = 0; i < n_tiles; ++i) {
        const muse_kv_tile& t = tiles[i];
        if (t.n_rows == 0) continue;
        const size_t so = ((size_t)t.src_seq * (size_t)src->capacity + (size_t)t.src_pos) * row;
        const size_t dof = ((size_t)t.dst_seq * (size_t)dst->capacity + (size_t)t.dst_pos) * row;
        const size_t n = (size_t)t.n_rows * row;
        const Range rk{(uintptr_t)src->k + so, (uintptr_t)src->k + so + n}, rv{(uintptr_t)src->v + so, (uintptr_t)src->v + so + n};
        const Range wk{(uintptr_t)dst->k + dof, (uintptr_t)dst->k + dof + n}, wv{(uintptr_t)dst->v + dof, (uintptr_t)dst->v + dof + n};
        bool dep = ra.n_tiles == muse::kRelocTiles;
        for (int j = 0; j < ra.n_tiles && !dep; ++j)
            for (int x = 0; x < 2 && !dep; ++x) {
                const Range r = x ? rv : rk, w = x ? wv : wk;
                for (int y = 0; y < 2; ++y)
                    dep = dep || overlap(r, writes[j][y]) || overlap(w, writes[j][y]) || overlap(w, reads[j][y]);
            }
        if (dep && flush() != hipSuccess) return MUSE_ERR_HIP;
        const int k = ra.n_tiles;
        reads[k][0] = rk;
        reads[k][1] = rv;
        writes[k][0] = wk;
        writes[k][1] = wv;
        ra.src_off[k] = (int64_t)so;
        ra.dst_off[k] = (int64_t)dof;
        ra.bytes[k] = (int64_t)n;
        ra.block0[k + 1] = ra.block0[k] + (int32_t)((n + muse::kRelocChunk - 1) / muse::kRelocChunk);
        ra.n_tiles = k + 1;
    }
    if (ra.n_tiles && flush() != hipSuccess) return MUSE_ERR_HIP;
    return MUSE_OK;
}

muse_status muse_attn_layer_init(muse_attn_layer* layer, int32_t layer_index, int32_t dtype) {
    if (!layer) return MUSE_ERR_NULL;
    if (layer_index < 0 || layer_index >= kModelLayers) return MUSE_ERR_SHAPE;
    if (dtype != MUSE_F32 && dtype != MUSE_BF16) return MUSE_ERR_DTYPE;
    muse_attn_layer l;
    l.n_heads = kHeads;
    l.n_kv_heads = kKvHeads;
    l.head_dim = kHeadDim;
    l.kind = muse_layer_kind_for(layer_index, kModelLayers);
    l.window = l.kind == MUSE_SLIDING_ROPE ? 2048 : 0;
    l.rope_theta = l.kind == MUSE_SLIDING_ROPE ? 500000.0f : 0.0f;
    l.rms_eps = 1e-5f;
    l.q_norm_gain = 3.87f;
    l.k_norm_gain = 1.0f;
    l.attn_scale = (float)(1.0 / std::sqrt(128.0));
    l.dtype = dtype;
    l.kv_ring = 0;
    *layer = l;
    return MUSE_OK;
}

int32_t muse_layer_kind_for(int32_t layer_index, int32_t n_layers) {
    if (n_layers < 1 || layer_index < 0 || layer_index >= n_layers) return -1;
    return layer_index % 4 == 3 ? MUSE_FULL_NOPE : MUSE_SLIDING_ROPE;
}

muse_status muse_rope_theta_table(float theta, float* out_host64) {
    if (!out_host64) return MUSE_ERR_NULL;
    if (!finite_pos(theta)) return MUSE_ERR_LAYER;
    rope_table(theta, out_host64);
    return MUSE_OK;
}

muse_status muse_out_proj_workspace_size(int32_t n_tokens, size_t* bytes) {
    if (!bytes) return MUSE_ERR_NULL;
    if (n_tokens < 0 || n_tokens > kMaxPositions) return MUSE_ERR_SHAPE;
    // the f32 projection; a few tokens (at most 64) keep its 8 K slices apart
    const size_t parts = n_tokens <= 64 ? 8 : 1;
    *bytes = round_up(parts * (size_t)n_tokens * muse::kModelDim * sizeof(float), kAlign);
    return MUSE_OK;
}

muse_status muse_out_proj(int32_t n_tokens, const void* attn, const void* w, const float* gamma,
                          const void* residual, void* hidden_out, float eps,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream, const muse_kernel_timer* timer) {
    if (!attn || !w || !gamma || !residual || !hidden_out || !workspace) return MUSE_ERR_NULL;
    if (timer && (!timer->start || !timer->stop)) return MUSE_ERR_NULL;
    size_t need = 0;
    muse_status st = muse_out_proj_workspace_size(n_tokens, &need);
    if (st != MUSE_OK) return st;
    if (!finite_pos(eps)) return MUSE_ERR_LAYER;
    if (!aligned16(attn) || !aligned16(w) || !aligned16(gamma) || !aligned16(residual) || !aligned16(hidden_out) ||
        !aligned16(workspace))
        return MUSE_ERR_ALIGN;
    if (workspace_bytes < need) return MUSE_ERR_WORKSPACE;
    const size_t M = (size_t)n_tokens;
    auto range = [](const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; };
    const Range ra = range(attn, M * muse::kAttnDim * 2), rw = range(w, (size_t)muse::kModelDim * muse::kAttnDim * 2),
                rg = range(gamma, muse::kModelDim * 4), rr = range(residual, M * muse::kModelDim * 2),
                ro = range(hidden_out, M * muse::kModelDim * 2), rs = range(workspace, need);
    if (M > 0) {
        // hidden_out may be the residual itself (each element is read, then written, by one thread)
        if ((hidden_out != residual && overlap(ro, rr)) || overlap(ro, ra) || overlap(ro, rw) || overlap(ro, rg))
            return MUSE_ERR_ALIAS;
        if (overlap(rs, ra) || overlap(rs, rw) || overlap(rs, rg) || overlap(rs, rr) || overlap(rs, ro))
            return MUSE_ERR_ALIAS;
    }
    if (n_tokens == 0) return MUSE_OK;
    muse::OutProjArgs oa;
    oa.attn = attn;
    oa.w = w;
    oa.gamma = gamma;
    oa.residual = residual;
    oa.out = hidden_out;
    oa.proj = (float*)workspace;
    oa.m = n_tokens;
    oa.eps = eps;
    if (timer && hipEventRecord(timer->start, stream) != hipSuccess) return MUSE_ERR_HIP;
    if (muse::launch_out_proj_gemm(oa, stream) != hipSuccess) return MUSE_ERR_HIP;
    if (timer && hipEventRecord(timer->stop, stream) != hipSuccess) return MUSE_ERR_HIP;
    if (muse::launch_out_proj_norm(oa, stream) != hipSuccess) return MUSE_ERR_HIP;
    return MUSE_OK;
}

const char* muse_status_str(int s) {
    switch (s) {
        case MUSE_OK: return "MUSE_OK";
        case MUSE_ERR_NULL: return "MUSE_ERR_NULL: a required pointer is NULL";
        case MUSE_ERR_SHAPE: return "MUSE_ERR_SHAPE: head counts, head_dim or a size out of range";
        case MUSE_ERR_LAYER: return "MUSE_ERR_LAYER: inconsistent layer parameters";
        case MUSE_ERR_CAPACITY: return "MUSE_ERR_CAPACITY: max_seq_len + n_new exceeds the cache capacity";
        case MUSE_ERR_WORKSPACE: return "MUSE_ERR_WORKSPACE: workspace too small";
        case MUSE_ERR_DTYPE: return "MUSE_ERR_DTYPE: unsupported dtype";
        case MUSE_ERR_HIP: return "MUSE_ERR_HIP: a HIP launch or event call failed";
        case MUSE_ERR_ALIGN: return "MUSE_ERR_ALIGN: a pointer is not 16-byte aligned";
        case MUSE_ERR_ALIAS: return "MUSE_ERR_ALIAS: an output buffer overlaps another buffer";
    }
    return "unknown muse_status";
}

}  // extern "C"
