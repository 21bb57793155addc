/*
 * muse_attn.h -- C ABI of the MI355X (gfx950) attention core of one Muse
 * Glimmer text layer.
 *
 * What one call computes, for every new token t of sequence s, at position
 * p = seq_len[s] + t (pages cited by title and section):
 *   1. Per-head QK-norm: each 128-wide head slice of Q (32 heads) and K
 *      (2 heads) becomes x / sqrt(mean(x^2) + eps) * gain, with a constant
 *      gain per tensor.  ["Chapter 9 - The Muse Glimmer architecture" 9.5
 *      RMSNorm formula; "Chapter 14 - QK-norm and RoPE" 14.3]
 *   2. RoPE on sliding layers only: adjacent pairs (x[2i], x[2i+1]) rotate by
 *      the f32 angle p * theta_i, theta_i = base^(-2i/128) held as f32.
 *      Full layers are NoPE and skip this step.  [Ch 14, 14.1, 14.4.1,
 *      14.4.2, 14.5; Ch 9, 9.7]
 *   3. KV append: cache row p of KV head g receives the normed (and rotated)
 *      K and the raw V.  [Ch 14, 14.7: keys are rotated before they are stored]
 *      On a layer with kv_ring set the cache is a ring: position p lives in
 *      row p % capacity.  ["Chapter 9 - The Muse Glimmer architecture" 9.7:
 *      each sliding layer keeps a fixed 2,048-row ring, token-major]
 *   4. Causal GQA attention: query head h reads KV head h / 16; key j is
 *      visible iff j <= p and, on sliding layers, p - j < window; scores are
 *      (q . k) * attn_scale; softmax; weighted sum of V.  [Ch 9, 9.5, 9.6
 *      Figure 9.3, 9.7]
 *   5. Sigmoid output gate: out[c] = attn[c] * 1 / (1 + exp(-gate[c])) for
 *      every channel c = h * 128 + d.  [Ch 9, 9.8]
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the comment says "host".
 *   - The caller allocates and owns every buffer.  The library keeps no
 *     pointer after a call returns.
 *   - Activations, KV cache and output share one dtype (muse_dtype); all
 *     arithmetic is f32 (bf16 operands feed bf16 matrix cores, accumulating
 *     in f32).  Stores round to nearest, ties to even.
 *   - Layouts are dense, row-major, innermost dimension last:
 *       q          [n_seq][n_new][32][128]
 *       k, v       [n_seq][n_new][2][128]
 *       gate, out  [n_seq][n_new][4096]      (channel = head * 128 + dim)
 *       cache k, v [n_seq][capacity][2][128] (token-major; row = position,
 *                                             or position % capacity on a
 *                                             kv_ring layer)
 *       seq_len    int32 [n_seq]             (rows already cached)
 *     Every pointer must be 16-byte aligned.
 *   - Inputs q, k, v, gate and seq_len are read-only.  Cache rows
 *     [seq_len[s], seq_len[s] + n_new) are written; other rows are only read.
 *     On a kv_ring layer the rows written are those of the last
 *     min(n_new, capacity) new positions (earlier ones would be overwritten
 *     by later ones of the same call); the chunk's queries still see every
 *     new key in their window.
 *     seq_len is not advanced: the caller does that after the call.
 *   - out must not overlap any other buffer; workspace must not overlap any
 *     other buffer.
 *   - Calls are asynchronous on `stream` (0 = the default stream): no host
 *     synchronisation, no device-wide barrier.  Concurrent calls on different
 *     streams are safe when their buffers are disjoint.
 *   - Every argument is validated on the host BEFORE anything is enqueued;
 *     on any error nothing is enqueued and nothing is written (fail closed).
 *   - A sequence whose device-side seq_len lies outside [0, max_seq_len]
 *     (which the host cannot check) is refused on the device: its cache is
 *     not written and its output rows are filled with NaN.
 */
#ifndef MUSE_ATTN_H
#define MUSE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MUSE_OK = 0,
    MUSE_ERR_NULL = 1,      /* a required pointer is NULL                        */
    MUSE_ERR_SHAPE = 2,     /* head counts, head_dim or a size out of range      */
    MUSE_ERR_LAYER = 3,     /* kind/window/theta/eps/gain/scale inconsistent     */
    MUSE_ERR_CAPACITY = 4,  /* capacity too small (see muse_kv_cache)            */
    MUSE_ERR_WORKSPACE = 5, /* workspace_bytes below muse_attn_workspace_size    */
    MUSE_ERR_DTYPE = 6,     /* dtype is not MUSE_F32 / MUSE_BF16                 */
    MUSE_ERR_HIP = 7,       /* a HIP launch or event call failed                 */
    MUSE_ERR_ALIGN = 8,     /* a pointer is not 16-byte aligned                  */
    MUSE_ERR_ALIAS = 9      /* out or workspace overlaps another buffer          */
} muse_status;

typedef enum { MUSE_F32 = 0, MUSE_BF16 = 1 } muse_dtype;

/* Layer kinds: ["Chapter 9" 9.4 listing and Figure 9.4] */
typedef enum { MUSE_SLIDING_ROPE = 0, MUSE_FULL_NOPE = 1 } muse_layer_kind;

/* Parameters of one attention layer.  All fields are validated:
 *   n_heads, n_kv_heads, head_dim  must be 32, 2, 128 (else MUSE_ERR_SHAPE)
 *   kind        MUSE_SLIDING_ROPE or MUSE_FULL_NOPE
 *   window      sliding: >= 1 (the model uses 2048).  full: must be 0
 *   rope_theta  sliding: finite and > 0 (the model uses 500000).
 *               full: must be 0 (NoPE layers carry a zero RoPE base;
 *               "How Muse Glimmer Fits an Agent on Your Device",
 *               section "Global attention without RoPE")
 *   rms_eps     finite and > 0 (the model uses 1e-5)
 *   q_norm_gain, k_norm_gain  constant QK-norm weights (3.87 and 1.0;
 *               ["Chapter 14" 14.3]), |gain| <= 4096
 *               (bf16 layers compute Q.K with fp16 operands; normed rows
 *               are bounded by |gain| * sqrt(128), which stays below fp16's
 *               65504.  Cache K rows not written by this library must also
 *               stay below 65504 in magnitude.)
 *   attn_scale  finite and > 0 (1/sqrt(128); ["Chapter 9" 9.5])
 *   dtype       muse_dtype of activations, cache and output
 *   kv_ring     0: the cache row of position p is p.  1 (sliding bf16 layers
 *               only, else MUSE_ERR_LAYER): the cache is a ring of capacity
 *               rows and position p lives in row p % capacity, so a sliding
 *               layer needs only window rows per sequence ["Chapter 9" 9.7] */
typedef struct {
    int32_t n_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t kind;
    int32_t window;
    float rope_theta;
    float rms_eps;
    float q_norm_gain;
    float k_norm_gain;
    float attn_scale;
    int32_t dtype;
    int32_t kv_ring;
} muse_attn_layer;

/* Contiguous per-sequence KV cache: k and v are DEVICE pointers to
 * [n_seq][capacity][2][128] arrays of the layer dtype; capacity is in rows.
 * A call needs capacity >= max_seq_len + n_new, or on a kv_ring layer
 * capacity >= min(window, max_seq_len + n_new) (else MUSE_ERR_CAPACITY). */
typedef struct {
    void* k;
    void* v;
    int64_t capacity;
} muse_kv_cache;

/* Optional kernel timer.  When a call receives a non-NULL timer, `start` is
 * recorded on `stream` immediately before the call's attention kernel and
 * `stop` immediately after it (the events are the caller's, created with
 * timing enabled).  Used to measure the attention kernel alone. */
typedef struct {
    hipEvent_t start;
    hipEvent_t stop;
} muse_kernel_timer;

/*
 * Prefill: append n_new tokens per sequence and attend, causally within the
 * new chunk and over the cached prefix (chunked prefill when seq_len > 0).
 *   layer        host pointer, validated as above
 *   n_seq        >= 0 sequences;  n_new >= 0 new tokens per sequence
 *   seq_len      device int32[n_seq]: rows already cached
 *   max_seq_len  host upper bound of every seq_len[s]; sizes the grid and
 *                the capacity check (see muse_kv_cache)
 *   q, k, v, gate, out   device, layouts above
 *   cache        host pointer to the cache descriptor
 *   workspace    device scratch of at least muse_attn_workspace_size(...)
 *                bytes (contents on entry are ignored; clobbered)
 *   stream       HIP stream to enqueue on
 *   timer        optional (NULL = none)
 * n_seq == 0 or n_new == 0 is valid and enqueues nothing.
 * Short chunks (n_new <= 16 on a bf16 layer without kv_ring: the verify step
 * of speculative decoding, which scores a handful of drafted tokens against
 * a long prefix) run as split-K over the keys, every head of a KV head in one
 * workgroup, with the splits merged by a second kernel; the timer then spans
 * both kernels.  The result is the same attention within the tolerances.
 */
muse_status muse_attn_prefill(const muse_attn_layer* layer, int32_t n_seq, int32_t n_new,
                              const int32_t* seq_len, int32_t max_seq_len,
                              const void* q, const void* k, const void* v, const void* gate,
                              const muse_kv_cache* cache, void* out,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const muse_kernel_timer* timer);

/*
 * Decode: exactly one new token per sequence (n_new = 1) at position
 * seq_len[s]; the same five steps as prefill, with the attention split over
 * the cache length (split-K).  Arguments as for muse_attn_prefill with
 * n_new = 1 (q [n_seq][1][32][128], etc.).  With more than one split per
 * (sequence, KV head) the splits store their partial (max, sum, output) in
 * the workspace and a second kernel on the same stream merges them in split
 * order and applies the gate (the timer brackets the first kernel only).  The
 * workspace holds nothing between calls (contents on entry are ignored), but
 * calls that may run at the same time must not share one.  When
 * muse_attn_workspace_size reports 0 bytes (one split), workspace may be
 * NULL.
 */
muse_status muse_attn_decode(const muse_attn_layer* layer, int32_t n_seq,
                             const int32_t* seq_len, int32_t max_seq_len,
                             const void* q, const void* k, const void* v, const void* gate,
                             const muse_kv_cache* cache, void* out,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream, const muse_kernel_timer* timer);

/*
 * Decode without a caller-supplied workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same computation and kernels as
 * muse_attn_decode; the split partials go to a static device array of the
 * library, 4 MiB per GPU (every decode of up to 126 sequences fits; a call
 * whose muse_attn_workspace_size exceeds 4 MiB returns MUSE_ERR_WORKSPACE
 * and enqueues nothing).  Allocates nothing: its first call on a device (the
 * current one) looks up that device's copy of the array.  All calls on one
 * GPU share the array, so calls that may overlap on a GPU (other streams,
 * other threads) race and must not be issued.
 */
muse_status muse_attn_decode_noalloc(const muse_attn_layer* layer, int32_t n_seq,
                                     const int32_t* seq_len, int32_t max_seq_len,
                                     const void* q, const void* k, const void* v, const void* gate,
                                     const muse_kv_cache* cache, void* out,
                                     hipStream_t stream, const muse_kernel_timer* timer);

/* One tile of cache rows to relocate: rows [src_pos, src_pos + n_rows) of
 * sequence src_seq go to rows [dst_pos, dst_pos + n_rows) of sequence
 * dst_seq. */
typedef struct {
    int32_t src_seq;
    int32_t dst_seq;
    int64_t src_pos;
    int64_t dst_pos;
    int64_t n_rows;
} muse_kv_tile;

/*
 * Relocate K and V rows of a full (NoPE) layer's cache: for each of the
 * n_tiles tiles (host array, applied in order), a byte copy of the rows'
 * 1,024 bytes (bf16; 2,048 for f32) of K and of V from `src` to `dst` (which
 * may be the same cache).  A NoPE row carries no position, so the copied
 * bytes are valid at the new position without recomputation ("Chapter 14 -
 * QK-norm and RoPE" 14.6: NoPE tiles relocate by memcpy, 512-token tiles in
 * the engine; any row count is accepted here).  Fails closed:
 *   a sliding (RoPE) layer, whose rows are bound to their positions   MUSE_ERR_LAYER
 *   n_seq_src / n_seq_dst < 1, a sequence index outside them, a negative
 *   position or n_rows                                                MUSE_ERR_SHAPE
 *   rows beyond a cache's capacity                                    MUSE_ERR_CAPACITY
 *   source and destination rows of one tile overlap                   MUSE_ERR_ALIAS
 *   a NULL pointer (tiles may be NULL when n_tiles is 0)              MUSE_ERR_NULL
 *   a cache pointer not 16-byte aligned                               MUSE_ERR_ALIGN
 * Every tile is checked before the first copy is enqueued.  The copies run
 * asynchronously on `stream`, many tiles per kernel launch (a tile that reads
 * or writes rows an earlier tile writes, or writes rows it reads, starts a
 * new launch, so the result is that of applying the tiles in order);
 * n_rows == 0 tiles are skipped.
 */
muse_status muse_kv_relocate(const muse_attn_layer* layer, const muse_kv_cache* src, int32_t n_seq_src,
                             const muse_kv_cache* dst, int32_t n_seq_dst, const muse_kv_tile* tiles,
                             int32_t n_tiles, hipStream_t stream);

/* Workspace bytes a call needs (is_decode != 0 selects decode, which ignores
 * n_new).  Writes the size to *bytes (host).  Same validation as the calls. */
muse_status muse_attn_workspace_size(const muse_attn_layer* layer, int32_t n_seq, int32_t n_new,
                                     int32_t max_seq_len, int32_t is_decode, size_t* bytes);

/* Fill *layer (host) with the model's parameters for layer `layer_index`
 * (0 <= layer_index < 52): kind by the l % 4 == 3 rule, window 2048 and
 * theta 500000 on sliding layers (0 and 0 on full layers), eps 1e-5, gains
 * 3.87 / 1.0, scale 1/sqrt(128), the given dtype, and kv_ring 0.
 * ["Chapter 9" 9.4, 9.7; "Chapter 14" 14.3] */
muse_status muse_attn_layer_init(muse_attn_layer* layer, int32_t layer_index, int32_t dtype);

/* Layer kind of layer `layer_index` of an n_layers-deep model: FULL_NOPE iff
 * layer_index % 4 == 3, else SLIDING_ROPE.  Returns -1 when layer_index is
 * outside [0, n_layers) or n_layers < 1.  ["Chapter 9" 9.4 listing] */
int32_t muse_layer_kind_for(int32_t layer_index, int32_t n_layers);

/* The f32 RoPE frequency table the kernels use: out_host64[i] =
 * base^(-2i/128) rounded once to f32, i < 64 (host array of 64 floats).
 * ["Chapter 14" 14.4.1]  MUSE_ERR_LAYER unless theta is finite and > 0. */
muse_status muse_rope_theta_table(float theta, float* out_host64);

/* Static string naming a status code (never NULL).  Takes the code as an int
 * so that any value, a muse_status or not, is a valid argument; values that
 * name no status give "unknown muse_status". */
const char* muse_status_str(int status);

/* ------------------------------------------------ the block's tail (next step)
 *
 * o_proj and the post-attention norm, with the residual add ("Chapter 9 - The
 * Muse Glimmer architecture" 9.8 and 9.9, Figure 9.1): the gated attention
 * output (4,096 channels, heads concatenated, as muse_attn_* write it) is
 * projected to the model width 6,656, the projection of each token is RMS
 * normalised with its own epsilon (1e-8 in the model, unlike the other norms'
 * 1e-5) and scaled by the norm's gain, and the result is added to the
 * residual stream:
 *
 *   proj[t][n]   = sum_k attn[t][k] * w[n][k]
 *   hidden[t][n] = proj[t][n] / sqrt(mean_n proj[t][n]^2 + eps) * gamma[n]
 *                  + residual[t][n]
 *
 * Arguments (every pointer a DEVICE pointer, 16-byte aligned):
 *   n_tokens    rows of attn / residual / hidden (0 enqueues nothing)
 *   attn        bf16 [n_tokens][4096]
 *   w           bf16 [6656][4096]: row n holds output channel n's weights
 *   gamma       f32 [6656]: the norm's effective gain ("How Muse Glimmer Fits
 *               an Agent on Your Device" stores it as an offset from one; the
 *               caller passes 1 + offset)
 *   residual    bf16 [n_tokens][6656]
 *   hidden_out  bf16 [n_tokens][6656]; may be residual itself (an in-place
 *               update of the stream), must not otherwise overlap an input
 *   eps         > 0 and finite
 *   workspace   muse_out_proj_workspace_size(n_tokens) bytes or more: the f32
 *               projection; contents on entry are ignored; calls that overlap
 *               in time must not share one
 *   timer       optional: brackets the projection (GEMM) kernel
 * The projection accumulates in f32 from the bf16 operands; the norm reads
 * the f32 projection; hidden is rounded to nearest even into bf16.  Up to 64
 * tokens the projection is a kernel of this library; for more it is a
 * hipBLASLt GEMM, whose library handle the first such call on a device
 * creates (it allocates device memory: capture such calls in a graph only
 * after one eager call on that device).
 * Fails closed, before anything is enqueued: NULL pointer MUSE_ERR_NULL;
 * n_tokens < 0 or above 2^24 MUSE_ERR_SHAPE; eps not positive and finite
 * MUSE_ERR_LAYER; a misaligned pointer MUSE_ERR_ALIGN; hidden_out partly
 * overlapping residual, or overlapping attn, w, gamma or the workspace, or
 * the workspace overlapping an input MUSE_ERR_ALIAS; workspace too small
 * MUSE_ERR_WORKSPACE; a failed launch, or no hipBLASLt algorithm for the
 * shape, MUSE_ERR_HIP.  Asynchronous on stream.
 */
#define MUSE_ATTN_DIM 4096
#define MUSE_MODEL_DIM 6656
muse_status muse_out_proj(int32_t n_tokens, const void* attn, const void* w, const float* gamma,
                          const void* residual, void* hidden_out, float eps,
                          void* workspace, size_t workspace_bytes,
                          hipStream_t stream, const muse_kernel_timer* timer);

/* Workspace bytes muse_out_proj needs for n_tokens rows: n_tokens * 6656 * 4
 * (the f32 projection), 8 times that for n_tokens <= 64 (its K slices, added
 * by the norm kernel), rounded up; MUSE_ERR_SHAPE for n_tokens outside
 * [0, 2^24]. */
muse_status muse_out_proj_workspace_size(int32_t n_tokens, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* MUSE_ATTN_H */
