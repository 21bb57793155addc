// prep.hip -- kernel (a): per-head QK-norm, RoPE on sliding layers, KV append.
//
// One workgroup (4 wave64s) per new token.  A head vector of 128 values is
// one wave: lane i holds the adjacent pair (x[2i], x[2i+1]), which is exactly
// RoPE pair i, so the rotation needs no data exchange and each lane computes
// its sin/cos once for all 34 vectors of the token.
//   * QK-norm: RMS over the 128 values of one head, then the constant gain
//     ("Chapter 9 - The Muse Glimmer architecture" 9.5 RMSNorm formula;
//     "Chapter 14 - QK-norm and RoPE" 14.3: Q gain about 3.87, K gain 1).
//   * RoPE (sliding layers only): angle = f32(p) * theta_i in f32 with the
//     f32 table theta_i = base^(-2i/128); accurate sincosf, no fast math
//     (Ch 14, 14.4.1 table, 14.4.2 rotation, 14.5 kernel).
//   * Append: the rotated K goes to cache row p, V is copied unchanged
//     (Ch 14, 14.7: keys rotate before the store; V never rotates).
// Q-hat goes to the workspace in the score type of the attention kernels
// (fp16 on bf16 layers, f32 on f32 layers).
#include "device_common.h"
#include "kernels.h"

namespace muse {

template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    const int tok = blockIdx.x;                    // s * n_new + t
    const int s = tok / a.n_new;
    const int t = tok - s * a.n_new;
    const int L = a.seq_len[s];
    // Fail closed on a device-side length the host could not check: the
    // attention kernels refuse the same sequence and fill its output with NaN.
    if (L < 0 || L > a.max_seq_len) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t p = (int64_t)L + t;

    float sn = 0.0f, cs = 1.0f;
    if (a.rope) {
        float th = 0.0f;
#pragma unroll
        for (int i = 0; i < 64; ++i) th = (lane == i) ? a.theta[i] : th;
        const float ang = (float)p * th;           // f32 product, as in the table's use
        sincosf(ang, &sn, &cs);
    }

    const T* q = (const T*)a.q;
    const T* k = (const T*)a.k;
    const T* v = (const T*)a.v;
    typedef typename ScoreType<T>::type TQ;
    TQ* qhat = (TQ*)a.qhat;
    T* ck = (T*)a.cache_k;
    T* cv = (T*)a.cache_v;

    for (int vec = wave; vec < kHeads + 2 * kKvHeads; vec += 4) {
        const T* src;
        T* dst = nullptr;
        TQ* qdst = nullptr;
        float gain = 1.0f;
        bool norm = true;
        if (vec < kHeads) {
            const int64_t off = ((int64_t)tok * kHeads + vec) * kHeadDim;
            src = q + off;
            qdst = qhat + off;
            gain = a.q_gain;
        } else if (vec < kHeads + kKvHeads) {
            const int g = vec - kHeads;
            src = k + ((int64_t)tok * kKvHeads + g) * kHeadDim;
            dst = ck + (((int64_t)s * a.capacity + p) * kKvHeads + g) * kHeadDim;
            gain = a.k_gain;
        } else {
            const int g = vec - kHeads - kKvHeads;
            src = v + ((int64_t)tok * kKvHeads + g) * kHeadDim;
            dst = cv + (((int64_t)s * a.capacity + p) * kKvHeads + g) * kHeadDim;
            norm = false;
        }
        const T r0 = src[2 * lane];
        const T r1 = src[2 * lane + 1];
        if (!norm) {                               // V: exact copy
            dst[2 * lane] = r0;
            dst[2 * lane + 1] = r1;
            continue;
        }
        const float x0 = to_f32(r0), x1 = to_f32(r1);
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
        float y0 = (x0 * r) * gain;
        float y1 = (x1 * r) * gain;
        if (a.rope) {
            const float z0 = y0 * cs - y1 * sn;
            const float z1 = y0 * sn + y1 * cs;
            y0 = z0;
            y1 = z1;
        }
        if (qdst) {
            qdst[2 * lane] = from_f32<TQ>(y0);
            qdst[2 * lane + 1] = from_f32<TQ>(y1);
        } else {
            dst[2 * lane] = from_f32<T>(y0);
            dst[2 * lane + 1] = from_f32<T>(y1);
        }
    }
}

hipError_t launch_prep(const PrepArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * a.n_new)), block(256);
    if (dtype == 1)
        hipLaunchKernelGGL(prep_kernel<bf16_t>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(prep_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
