// prep.hip -- kernel (a): per-head QK-norm, RoPE on sliding layers, KV append
// for a chunk of new tokens (the prefill path; decode does this inside its
// own kernel).
//
// f32 layers: one workgroup (256 threads) per new token.  A head vector of
// 128 values is handled by 16 lanes, 8 values (16 bytes, RoPE pairs
// 4i..4i+3) per lane, so one wave covers four vectors and the 36 vectors of a
// token (32 Q heads, 2 K heads, 2 V heads) take three passes of the
// workgroup.  The 64 sin/cos pairs of the token's position are computed
// once, by the first 64 threads, and shared through LDS.  bf16 layers only
// need K-hat and V here (the attention kernel makes Q-hat): one wave takes
// the four K/V vectors of four tokens in turn.
//   * QK-norm: RMS over the 128 values of one head, then the constant gain
//     ("Chapter 9 - The Muse Glimmer architecture" 9.5 RMSNorm formula;
//     "Chapter 14 - QK-norm and RoPE" 14.3: Q gain about 3.87, K gain 1).
//   * RoPE (sliding layers only): angle = f32(p) * theta_i in f32 with the
//     f32 table theta_i = base^(-2i/128); accurate sin and cos (trig.h)
//     (Ch 14, 14.4.1 table, 14.4.2 rotation, 14.5 kernel).
//   * Append: the rotated K goes to cache row p, V is copied unchanged
//     (Ch 14, 14.7: keys rotate before the store; V never rotates).
// Q-hat goes to the workspace in the score type of the attention kernel
// (fp16 on bf16 layers, f32 on f32 layers), pre-multiplied by
// attn_scale * log2(e) so that the attention kernel's scores are already in
// the log2 domain of its softmax.  On bf16 layers the attention kernel reads
// keys from an fp16 copy (converted once here rather than per tile): the new
// rows are written to it as they are appended, and extra workgroups convert
// the cached prefix rows the chunk can see.
#include "device_common.h"
#include "kernels.h"

namespace muse {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
    } else {
        const floatx4 a = *(const floatx4*)p, b = *(const floatx4*)(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&y)[8]) {
    if constexpr (sizeof(T) == 2) {
        typedef T T8 __attribute__((ext_vector_type(8)));
        T8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = from_f32<T>(y[i]);
        *(T8*)p = v;
    } else {
        floatx4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = y[i];
            b[i] = y[4 + i];
        }
        *(floatx4*)p = a;
        *(floatx4*)(p + 4) = b;
    }
}

// First position held by the fp16 key copy (and the ring layers' V copy) of
// a sequence with L cached rows: on sliding layers the window's first
// visible position rounded down to kWindowAlign, else 0.
__device__ __forceinline__ int copy_base(const PrepArgs& a, int L) {
    return a.kq_windowed ? max(0, L - a.window + 1) / kWindowAlign * kWindowAlign : 0;
}
__device__ __forceinline__ int64_t copy_row(const PrepArgs& a, int L, int64_t j) {
    return j - copy_base(a, L);
}
// Cache row of position j: j, or j % ring on a ring layer.
__device__ __forceinline__ int64_t cache_row(const PrepArgs& a, int64_t j) {
    return a.ring ? j % a.ring : j;
}

// Positions [copy_base, L) of sequence s (the ones the chunk's queries can
// see, and up to kWindowAlign - 1 before them), 64 per workgroup: bf16 cache
// -> fp16 score copy (exact for the normed keys); on ring layers V is copied
// out of the ring as well.  (Positions before the window are masked; their
// rows are copied so that every row the attention kernel loads is data.)
__device__ __forceinline__ void convert_prefix(const PrepArgs& a, int idx) {
    const int s = idx / a.conv_blocks, blk = idx % a.conv_blocks;
    const int L = a.seq_len[s];
    if (L < 0 || L > a.max_seq_len) return;
    const int r0 = copy_base(a, L) + 64 * blk;
    for (int c = threadIdx.x; c < 64 * 32; c += 256) {   // 32 chunks of 16 B per position
        const int pos = r0 + c / 32, piece = c % 32;
        if (pos >= L) break;
        const int64_t e = ((int64_t)s * a.capacity + cache_row(a, pos)) * kKvHeads * kHeadDim + piece * 8;
        const int64_t f = ((int64_t)s * a.kq_capacity + copy_row(a, L, pos)) * kKvHeads * kHeadDim + piece * 8;
        *(u32x4*)((f16_t*)a.kq + f) = k_chunk_to_score(*(const u32x4*)((const bf16_t*)a.cache_k + e), bf16_t{});
        if (a.vq) *(u32x4*)((bf16_t*)a.vq + f) = *(const u32x4*)((const bf16_t*)a.cache_v + e);
    }
}

// bf16 layers (Q-hat is made by the attention kernel): K-hat and V of
// kKvTokensPerWave tokens per wave, 16 tokens per workgroup.  Lane l holds
// the 16-byte chunk l % 16 (dims 8 (l % 16) .. + 7) of vector l / 16: K head
// 0, K head 1, V head 0, V head 1.  All of a wave's loads are issued before
// its first store (a load after a store to a buffer the compiler cannot tell
// apart would wait for it), and lane i computes (cos, sin) of RoPE pair i
// for each token, which the K lanes fetch with cross-lane reads.
constexpr int kKvTokensPerWave = 4;
__device__ __forceinline__ void prep_kv_bf16(const PrepArgs& a, int blk) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int vec = lane >> 4, sub = lane & 15;
    const int hk = vec & 1;
    const bool is_k = vec < kKvHeads;
    const int n_tok = a.n_seq * a.n_new;
    const int tok0 = (blk * 4 + wave) * kKvTokensPerWave;
    u32x4 raw[kKvTokensPerWave];
    int Ls[kKvTokensPerWave];
#pragma unroll
    for (int i = 0; i < kKvTokensPerWave; ++i) {
        const int tok = min(tok0 + i, n_tok - 1);
        const bf16_t* src = (const bf16_t*)(is_k ? a.k : a.v) + ((int64_t)tok * kKvHeads + hk) * kHeadDim + 8 * sub;
        raw[i] = *(const u32x4*)src;
        Ls[i] = a.seq_len[tok / a.n_new];
    }
    const float th = theta_of_lane<PrepArgs>(lane);
#pragma unroll
    for (int i = 0; i < kKvTokensPerWave; ++i) {
        const int tok = tok0 + i;
        if (tok >= n_tok) break;                   // uniform over the wave
        const int s = tok / a.n_new, t = tok - s * a.n_new;
        const int L = Ls[i];
        if (L < 0 || L > a.max_seq_len) continue;  // refused (the attention kernel writes NaN)
        const int64_t p = (int64_t)L + t;
        // ring layers keep only the last `ring` positions of the chunk: an
        // earlier one would share a row with a later one
        const bool to_cache = !a.ring || t >= a.n_new - a.ring;
        const int64_t row = ((int64_t)s * a.capacity + cache_row(a, p)) * kKvHeads + hk;
        const int64_t qrow = ((int64_t)s * a.kq_capacity + copy_row(a, L, p)) * kKvHeads + hk;
        if (!is_k) {                               // V: exact copy
            if (to_cache) *(u32x4*)((bf16_t*)a.cache_v + row * kHeadDim + 8 * sub) = raw[i];
            if (a.vq) *(u32x4*)((bf16_t*)a.vq + qrow * kHeadDim + 8 * sub) = raw[i];
        }
        const bf16x8 kx = __builtin_bit_cast(bf16x8, raw[i]);
        float y[8];
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[j] = (float)kx[j];
            ss += y[j] * y[j];
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);   // the 16 lanes of this head
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = (y[j] * r) * a.k_gain;
        if (a.rope) {
            float sn, cs;
            sincos_rope((float)p * th, &sn, &cs);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float c2 = __shfl(cs, 4 * sub + j, 64), s2 = __shfl(sn, 4 * sub + j, 64);
                const float y0 = y[2 * j], y1 = y[2 * j + 1];
                y[2 * j] = y0 * c2 - y1 * s2;
                y[2 * j + 1] = y0 * s2 + y1 * c2;
            }
        }
        if (is_k) {
            bf16x8 kv;
#pragma unroll
            for (int j = 0; j < 8; ++j) kv[j] = from_f32<bf16_t>(y[j]);
            const u32x4 kr = __builtin_bit_cast(u32x4, kv);
            if (to_cache) *(u32x4*)((bf16_t*)a.cache_k + row * kHeadDim + 8 * sub) = kr;
            // the score copy holds the stored values (short chunks read the cache instead)
            if (a.kq) *(u32x4*)((f16_t*)a.kq + qrow * kHeadDim + 8 * sub) = k_chunk_to_score(kr, bf16_t{});
        }
    }
}

__host__ __device__ inline int prep_kv_blocks(int n_tok) { return (n_tok + 4 * kKvTokensPerWave - 1) / (4 * kKvTokensPerWave); }

template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    typedef typename ScoreType<T>::type TQ;
    __shared__ float2 rot[64];                     // (cos, sin) of pair i at this token's position
    const int n_tok = a.n_seq * a.n_new;
    const int n_main = a.phase == 1 ? 0 : a.skip_q ? prep_kv_blocks(n_tok) : n_tok;
    if ((int)blockIdx.x >= n_main) {               // fp16 copy of visible prefix keys
        if constexpr (sizeof(T) == 2) convert_prefix(a, (int)blockIdx.x - n_main);
        return;
    }
    if constexpr (sizeof(T) == 2) {
        if (a.skip_q) {
            prep_kv_bf16(a, blockIdx.x);
            return;
        }
    }
    const int tok = blockIdx.x;                    // s * n_new + t
    const int s = tok / a.n_new;
    const int t = tok - s * a.n_new;
    const int L = a.seq_len[s];
    // Fail closed on a device-side length the host could not check: the
    // attention kernel refuses the same sequence and fills its output with NaN.
    if (L < 0 || L > a.max_seq_len) return;
    const int64_t p = (int64_t)L + t;
    const int tid = threadIdx.x;
    if (a.rope && tid < 64) {
        float sn, cs;
        rope_sincos(a.theta, tid, p, sn, cs);
        rot[tid] = make_float2(cs, sn);
    }
    __syncthreads();

    const int sub = tid & 15;                      // 8 values: dims 8*sub .. 8*sub+7
    for (int vec = (tid >> 4) + (a.skip_q ? kHeads : 0); vec < kHeads + 2 * kKvHeads; vec += 16) {
        float x[8];
        if (vec >= kHeads + kKvHeads) {            // V: exact copy
            const int g = vec - kHeads - kKvHeads;
            const T* src = (const T*)a.v + ((int64_t)tok * kKvHeads + g) * kHeadDim + 8 * sub;
            T* dst = (T*)a.cache_v + (((int64_t)s * a.capacity + cache_row(a, p)) * kKvHeads + g) * kHeadDim + 8 * sub;
            *(u32x4*)dst = *(const u32x4*)src;
            if constexpr (sizeof(T) == 4) *(u32x4*)(dst + 4) = *(const u32x4*)(src + 4);
            continue;
        }
        const bool is_q = vec < kHeads;
        const T* src = is_q ? (const T*)a.q + ((int64_t)tok * kHeads + vec) * kHeadDim
                            : (const T*)a.k + ((int64_t)tok * kKvHeads + (vec - kHeads)) * kHeadDim;
        load8(src + 8 * sub, x);
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);   // the 16 lanes of this head
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
        const float gain = is_q ? a.q_gain : a.k_gain;
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = (x[i] * r) * gain;
        if (a.rope) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float2 cs = rot[4 * sub + j];
                const float y0 = y[2 * j], y1 = y[2 * j + 1];
                y[2 * j] = y0 * cs.x - y1 * cs.y;
                y[2 * j + 1] = y0 * cs.y + y1 * cs.x;
            }
        }
        if (is_q) {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] *= a.q_scale;
            store8((TQ*)a.qhat + ((int64_t)tok * kHeads + vec) * kHeadDim + 8 * sub, y);
        } else {
            const int g = vec - kHeads;
            T* dst = (T*)a.cache_k + (((int64_t)s * a.capacity + cache_row(a, p)) * kKvHeads + g) * kHeadDim + 8 * sub;
            if constexpr (sizeof(T) == 2) {
                bf16x8 kv;
#pragma unroll
                for (int i = 0; i < 8; ++i) kv[i] = from_f32<bf16_t>(y[i]);
                const u32x4 raw = __builtin_bit_cast(u32x4, kv);
                *(u32x4*)dst = raw;
                // the score copy holds the stored values
                TQ* kq = (TQ*)a.kq + (((int64_t)s * a.kq_capacity + copy_row(a, L, p)) * kKvHeads + g) * kHeadDim + 8 * sub;
                *(u32x4*)kq = k_chunk_to_score(raw, T{});
            } else {
                store8(dst, y);
            }
        }
    }
}

hipError_t launch_prep(const PrepArgs& a, int dtype, hipStream_t stream) {
    const int n_tok = a.n_seq * a.n_new;
    const int n_main = a.phase == 1 ? 0 : a.skip_q ? prep_kv_blocks(n_tok) : n_tok;
    const int n_conv = a.phase == 2 ? 0 : a.n_seq * a.conv_blocks;
    if (n_main + n_conv == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_main + n_conv)), block(256);
    if (dtype == 1)
        hipLaunchKernelGGL(prep_kernel<bf16_t>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(prep_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
