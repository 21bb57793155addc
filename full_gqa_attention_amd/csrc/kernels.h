// kernels.h -- argument blocks and launchers of the gfx950 kernels.  Internal
// to libmuse_attn: the public surface is include/muse_attn.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace muse {

// Kernel (a): QK-norm + RoPE + KV append, one workgroup per new token.
struct PrepArgs {
    const void* q;          // [S][N][32][128]
    const void* k;          // [S][N][2][128]
    const void* v;          // [S][N][2][128]
    void* qhat;             // workspace [S][N][32][128]: normed (and rotated) Q
    void* cache_k;          // [S][cap][2][128]
    void* cache_v;
    int64_t capacity;
    const int32_t* seq_len; // device [S]
    int32_t max_seq_len;
    int32_t n_seq;
    int32_t n_new;
    int32_t rope;           // 1: sliding layer (rotate), 0: NoPE
    int32_t skip_q;         // 1: Q-hat is made by the attention kernel (bf16 layers)
    float eps;
    float q_gain;
    float k_gain;
    float q_scale;          // attn_scale * log2(e), folded into Q-hat
    // bf16 layers: fp16 copy of the keys the attention kernel reads,
    // [S][kq_capacity][2][128] (NULL on f32 layers, which read the cache)
    void* kq;
    int64_t kq_capacity;
    int32_t window;         // 0: full; else only rows > p_first - window are copied
    int32_t conv_blocks;    // prefix-conversion workgroups per sequence
    int32_t kq_windowed;    // 1: kq (and vq) row = position - max(0, seq_len - window + 1)
    int64_t ring;           // 0: cache row = position; else cache row = position % ring
    void* vq;               // ring layers: copy of the V rows the chunk sees, laid out as kq
    int32_t phase;          // 0: prefix copy and new rows; 1: prefix copy only; 2: new rows only
    float theta[64];        // f32 RoPE frequency table
};

// Kernel (b): prefill attention over the cache with the gate epilogue.
struct AttnArgs {
    const void* qhat;       // f32 layers: workspace Q-hat [S][N][32][128], scaled by attn_scale * log2(e)
    const void* q;          // bf16 layers: raw Q [S][N][32][128] (Q-hat is made in the kernel)
    int32_t rope;           // bf16 layers: 1 on sliding layers (rotate Q)
    float eps;
    float q_gain;
    float q_scale;          // attn_scale * log2(e)
    float theta[64];        // f32 RoPE frequency table
    const void* gate;       // [S][N][4096]
    void* out;              // [S][N][4096]
    const void* kq;         // keys in the score type [S][kq_capacity][2][128]
    int64_t kq_capacity;
    const void* cache_v;    // [S][capacity][2][128]
    int64_t capacity;
    const int32_t* seq_len; // device [S]
    int32_t max_seq_len;
    int32_t n_seq;
    int32_t n_new;
    int32_t window;         // 0: full causal; else keys with p - j < window
    int32_t kq_windowed;    // 1: kq row = position - max(0, seq_len - window + 1)
    int32_t v_windowed;     // 1: cache_v row likewise (cache_v is then the V copy)
};

// Kernel (c): the decode step for one new token per sequence -- QK-norm/RoPE
// of Q and K, the KV append and split-K attention in one launch, then (with
// more than one split) the merge of the splits and the gate in a second.
struct DecodeArgs {
    const void* q;          // [S][32][128]
    const void* k;          // [S][2][128]
    const void* v;          // [S][2][128]
    const void* gate;       // [S][4096]
    void* out;              // [S][4096]
    void* cache_k;          // [S][cap][2][128]
    void* cache_v;
    int64_t capacity;
    const int32_t* seq_len; // device [S]
    int32_t max_seq_len;
    int32_t n_seq;
    int32_t window;         // 0: full causal; else keys with p - j < window
    int64_t ring;           // 0: cache row = position; else cache row = position % ring
    int32_t rope;           // 1: sliding layer (rotate), 0: NoPE
    float eps;
    float q_gain;
    float k_gain;
    float scale_log2;       // attn_scale * log2(e)
    int32_t chunk;          // keys per split
    int32_t nsplit;         // splits per (sequence, KV head)
    float* part_o;          // [S][32][nsplit][128] unnormalised partial outputs
    float* part_m;          // [S][32][nsplit] partial maxima (log2 domain)
    float* part_l;          // [S][32][nsplit] partial softmax denominators
    float theta[64];        // f32 RoPE frequency table
};

// Short bf16 chunks (at most kVerifyTokens new tokens per sequence): split-K
// attention with all 16 heads x 16 token rows of a KV head per workgroup,
// then a merge of the splits with the gate.
constexpr int kVerifyDepth = 2;     // key tiles in flight per verify workgroup (register slots)
constexpr int kVerifyBlocks = 256;  // verify workgroups a call aims for (splits = this / (2 n_seq))
constexpr int kVerifyTokens = 16;
constexpr int kVerifyTile = 32;     // keys per tile
struct VerifyArgs {
    const void* q;          // [S][N][32][128] raw Q
    const void* gate;       // [S][N][4096]
    void* out;              // [S][N][4096]
    const void* cache_k;    // [S][capacity][2][128] (the new rows already appended)
    const void* cache_v;
    int64_t capacity;
    const int32_t* seq_len; // device [S]
    int32_t max_seq_len;
    int32_t n_seq;
    int32_t n_new;          // 1 .. kVerifyTokens
    int32_t window;         // 0: full causal; else keys with p - j < window
    int32_t rope;           // 1: sliding layer (rotate Q)
    float eps;
    float q_gain;
    float q_scale;          // attn_scale * log2(e)
    float theta[64];        // f32 RoPE frequency table
    int32_t nsplit;         // key-range splits per (sequence, KV head)
    int32_t chunk_tiles;    // kVerifyTile-key tiles per split
    float* part_o;          // [S][2][nsplit][16 heads][16 tokens][128]
    float* part_m;          // [S][2][nsplit][16][16] row maxima (log2 domain)
    float* part_l;          // [S][2][nsplit][16][16] row sums
};

// Relocation of NoPE cache tiles: up to kRelocTiles tiles per launch, byte
// offsets into the K caches (the V caches use the same offsets).
constexpr int kRelocTiles = 120;
constexpr int kRelocChunk = 16 * 1024;  // bytes of K (and of V) per workgroup
struct RelocArgs {
    const char* src_k;
    const char* src_v;
    char* dst_k;
    char* dst_v;
    int32_t n_tiles;
    int32_t block0[kRelocTiles + 1];   // first workgroup of each tile; block0[n_tiles] = grid
    int64_t src_off[kRelocTiles];
    int64_t dst_off[kRelocTiles];
    int64_t bytes[kRelocTiles];
};

// Launch geometry shared by the host code and the kernels.
// The block's tail after attention: o_proj [4096 -> 6656] into an f32
// workspace, then the post-attention RMSNorm with the residual add.
constexpr int kAttnDim = 4096;
constexpr int kModelDim = 6656;
struct OutProjArgs {
    const void* attn;       // bf16 [m][4096]
    const void* w;          // bf16 [6656][4096]
    const float* gamma;     // f32 [6656]
    const void* residual;   // bf16 [m][6656]
    void* out;              // bf16 [m][6656] (may be residual itself)
    float* proj;            // f32 [m][6656] workspace
    int32_t m;              // tokens
    float eps;
};

constexpr int kPrefillBM = 128;  // query rows per prefill workgroup (4 waves x 32)
constexpr int kPrefillBN = 64;   // keys per prefill tile
constexpr int kDecodeTile = 64;  // split granularity of the decode (keys)
// The windowed key (and ring-layer V) copies of the prefill start at the
// window's first visible position rounded down to a multiple of this, so
// that every key tile the attention kernel loads (tiles start at multiples of
// their size, at most this) lies inside the copy.
constexpr int kWindowAlign = 64;
constexpr int kDecodeWaves = 4;  // waves per decode workgroup (two workgroups per CU)
constexpr int kDecodeDepth = 3;  // 16-row sub-tiles of loads in flight per decode wave
constexpr int kDecodeTargetBlocks = 256;   // decode workgroups a call aims for: one per CU
constexpr int kDecodeMinSplitRows = 64;    // rows per decode split, at least (when the span allows)
constexpr int kMaxSplits = 256;  // decode splits per (sequence, KV head), at most

int prefill_grid(int n_seq, int n_new);

hipError_t launch_prep(const PrepArgs& a, int dtype, hipStream_t stream);
hipError_t launch_prefill(const AttnArgs& a, int dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);
// Device address of the allocation-free decode's scratch on the current
// device (kDecodeScratchBytes), resolved on the first call per device.
constexpr size_t kDecodeScratchBytes = (size_t)4 << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode_merge(const DecodeArgs& a, int dtype, hipStream_t stream);   // when nsplit > 1
hipError_t launch_relocate(const RelocArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_verify_merge(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_out_proj_gemm(const OutProjArgs& a, hipStream_t stream);
hipError_t launch_out_proj_norm(const OutProjArgs& a, hipStream_t stream);

}  // namespace muse
