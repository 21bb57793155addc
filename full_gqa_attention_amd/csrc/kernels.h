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
    float eps;
    float q_gain;
    float k_gain;
    float theta[64];        // f32 RoPE frequency table
};

// Kernels (b) and (c): attention over the cache with the gate epilogue.
struct AttnArgs {
    const void* qhat;       // workspace Q-hat [S][N][32][128]
    const void* gate;       // [S][N][4096]
    void* out;              // [S][N][4096]
    const void* cache_k;    // [S][cap][2][128]
    const void* cache_v;
    int64_t capacity;
    const int32_t* seq_len; // device [S]
    int32_t max_seq_len;
    int32_t n_seq;
    int32_t n_new;
    int32_t window;         // 0: full causal; else keys with p - j < window
    float scale_log2;       // attn_scale * log2(e)
    // decode split-K
    int32_t chunk;          // keys per split
    int32_t nsplit;         // splits per (sequence, KV head)
    float* part_o;          // [S][32][nsplit][128] unnormalised partial outputs
    float* part_m;          // [S][32][nsplit] partial maxima (log2 domain)
    float* part_l;          // [S][32][nsplit] partial softmax denominators
};

// Launch geometry shared by the host code and the kernels.
constexpr int kPrefillBM = 128;  // query rows per prefill workgroup (4 waves x 32)
constexpr int kPrefillBN = 64;   // keys per prefill tile
constexpr int kDecodeTile = 64;  // keys per decode tile (4 waves x 16)

int prefill_grid(int n_seq, int n_new);

hipError_t launch_prep(const PrepArgs& a, int dtype, hipStream_t stream);
hipError_t launch_prefill(const AttnArgs& a, int dtype, hipStream_t stream);
hipError_t launch_decode(const AttnArgs& a, int dtype, hipStream_t stream);
hipError_t launch_combine(const AttnArgs& a, int dtype, hipStream_t stream);

}  // namespace muse
