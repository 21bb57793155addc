// decode.hip -- kernel (c): split-K decode attention for one new token per
// sequence, and the combine kernel that merges the splits and applies the
// sigmoid gate.
//
// The step is bound by reading the cache: 1,024 bytes of K and V per visible
// row per sequence ("Chapter 9 - The Muse Glimmer architecture" 9.5, 9.6),
// shared by the 16 query heads of each KV head (Ch 9, Figure 9.3).  So one
// workgroup owns one (sequence, KV head, split) and computes all 16 heads
// from a single pass over its rows: scores are a 16-keys x 16-heads MFMA
// tile (S^T = K Q^T, fp16 16x16x32 on bf16 layers with K converted as it is
// staged), P.V a second MFMA (O^T = V^T P^T, bf16 16x16x16) whose B operand is the score tile as it sits in registers.
// Rows stream through LDS in 64-row tiles with 16-byte coalesced loads; the
// next tile is fetched into registers while the current one is computed.
// Within a wave the row max over 16 keys needs two lane exchanges (xor 16,
// 32); the 4 waves of a workgroup merge their (max, sum, O) in LDS and the
// workgroup writes one partial per head.  Visible rows are [p - W + 1, p] on
// sliding layers and [0, p] on full layers (Ch 9, 9.7), with p = seq_len.
#include "device_common.h"
#include "kernels.h"

namespace muse {

template <typename T>
__global__ __launch_bounds__(256) void decode_kernel(AttnArgs a) {
    typedef typename ScoreType<T>::type TQ;         // Q.K^T operand type
    using MW = Mma16Wide<TQ>;
    using MN = Mma16Narrow<T>;
    constexpr int D = kHeadDim, BT = kDecodeTile;
    constexpr int LDK = D + 16 / (int)sizeof(T);
    static_assert(sizeof(TQ) == sizeof(T), "K staging keeps the row size");
    constexpr int KW = MW::KPL, KN = MN::KPL;
    constexpr int NSTQ = D / (4 * KW);                 // K-steps of Q.K
    constexpr int NSTP = 4 / KN;                       // K-steps of P.V (16 keys)
    constexpr int CPR = D * (int)sizeof(T) / 16;       // 16-byte chunks per row
    constexpr int NCH = BT * CPR;
    constexpr int PER_THREAD = NCH / 256;
    static_assert(NCH % 256 == 0, "tile chunks must divide the workgroup");
    // LDS: K and V tiles; reused at the end for the 4-wave merge
    constexpr int TILE_ELEMS = BT * LDK;
    constexpr int MERGE_FLOATS = 4 * kHeadsPerKv * (D + 2);
    constexpr int LDS_BYTES = (2 * TILE_ELEMS * (int)sizeof(T) > MERGE_FLOATS * 4)
                                  ? 2 * TILE_ELEMS * (int)sizeof(T) : MERGE_FLOATS * 4;
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    TQ* Ks = (TQ*)lds;
    T* Vs = (T*)(Ks + TILE_ELEMS);

    const int b = blockIdx.x;
    const int c = b % a.nsplit;
    const int sg = b / a.nsplit;
    const int s = sg >> 1, g = sg & 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int L = a.seq_len[s];
    const int W = a.window;

    const int64_t p = L;
    const int64_t lo = (W > 0) ? max((int64_t)0, p - W + 1) : 0;
    const int64_t cs = lo + (int64_t)c * a.chunk;
    const int64_t ce = min(cs + (int64_t)a.chunk, p + 1);     // exclusive

    const int64_t pbase = ((int64_t)s * kHeads + g * kHeadsPerKv) * a.nsplit + c;  // head 16g, split c
    if (L < 0 || L > a.max_seq_len || cs >= ce) {
        // empty split (or a refused sequence): a neutral partial
        for (int i = tid; i < kHeadsPerKv * D; i += 256) {
            const int hh = i / D, d = i % D;
            a.part_o[(pbase + (int64_t)hh * a.nsplit) * D + d] = 0.0f;
        }
        if (tid < kHeadsPerKv) {
            a.part_m[pbase + (int64_t)tid * a.nsplit] = kNegInf;
            a.part_l[pbase + (int64_t)tid * a.nsplit] = 0.0f;
        }
        return;
    }

    // Q-hat of head 16g + l16 as the B operand of S^T = K Q^T
    typename MW::Frag qf[NSTQ];
    {
        const TQ* qrow = (const TQ*)a.qhat + ((int64_t)s * kHeads + g * kHeadsPerKv + l16) * D;
#pragma unroll
        for (int st = 0; st < NSTQ; ++st) qf[st] = *(const typename MW::Frag*)(qrow + 4 * KW * st + KW * q4);
    }

    const char* gk = (const char*)a.cache_k;
    const char* gv = (const char*)a.cache_v;
    const int ntiles = (int)((ce - cs + BT - 1) / BT);
    uint4 kr[PER_THREAD], vr[PER_THREAD];
    auto fetch = [&](int it) {
        const int64_t j0 = cs + (int64_t)it * BT;
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const int cidx = tid + 256 * u;
            const int r = cidx / CPR, cc = cidx % CPR;
            const int64_t jj = j0 + r;
            kr[u] = uint4{0, 0, 0, 0};
            vr[u] = uint4{0, 0, 0, 0};
            if (jj < ce) {
                const int64_t off = ((((int64_t)s * a.capacity + jj) * kKvHeads + g) * D) * (int64_t)sizeof(T) + cc * 16;
                kr[u] = *(const uint4*)(gk + off);
                vr[u] = *(const uint4*)(gv + off);
            }
        }
    };

    floatx4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{};
    float m_run = kNegInf, l_run = 0.0f;

    fetch(0);
    for (int it = 0; it < ntiles; ++it) {
        const int64_t j0 = cs + (int64_t)it * BT;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const int cidx = tid + 256 * u;
            const int r = cidx / CPR, cc = cidx % CPR;
            *(uint4*)((char*)Ks + (r * LDK) * (int)sizeof(TQ) + cc * 16) = k_chunk_to_score(kr[u], T{});
            *(uint4*)((char*)Vs + (r * LDK) * (int)sizeof(T) + cc * 16) = vr[u];
        }
        __syncthreads();
        if (it + 1 < ntiles) fetch(it + 1);

        // this wave's 16 keys: rows 16*wave .. +15 of the tile
        const int64_t jw = j0 + 16 * wave;
        if (jw >= ce) continue;
        floatx4 sc = floatx4{};
#pragma unroll
        for (int st = 0; st < NSTQ; ++st) {
            const typename MW::Frag kf =
                *(const typename MW::Frag*)(Ks + (16 * wave + l16) * LDK + 4 * KW * st + KW * q4);
            sc = MW::mma(kf, qf[st], sc);
        }
        // sc[i]: key jw + 4*q4 + i, head 16g + l16
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = sc[i] * a.scale_log2;
            if (jw + 4 * q4 + i >= ce) x = kNegInf;
            sc[i] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);            // finite: key jw is visible
        const float alpha = fast_exp2(m_run - m_new);
        float rs = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = fast_exp2(sc[i] - m_new);
            rs += sc[i];
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;

#pragma unroll
        for (int st = 0; st < NSTP; ++st) {
            typename MN::Frag pf;
#pragma unroll
            for (int t = 0; t < KN; ++t) frag_set(pf, t, sc[st * KN + t]);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                typename MN::Frag vf;
#pragma unroll
                for (int t = 0; t < KN; ++t)
                    frag_set_raw(vf, t, Vs[(16 * wave + 4 * q4 + st * KN + t) * LDK + 16 * dt + l16]);
                o[dt] = MN::mma(vf, pf, o[dt]);
            }
        }
    }

    // ---- merge the 4 waves: LDS holds per wave [16 heads][128 + 2] floats
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    __syncthreads();
    float* mg = (float*)lds;
    float* mw = mg + (wave * kHeadsPerKv + l16) * (D + 2);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mw[16 * dt + 4 * q4 + i] = o[dt][i];
    if (q4 == 0) {
        mw[D] = m_run;
        mw[D + 1] = l_run;
    }
    __syncthreads();
    for (int i = tid; i < kHeadsPerKv * D; i += 256) {
        const int hh = i / D, d = i % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, mg[(w * kHeadsPerKv + hh) * (D + 2) + D]);
        float acc = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float* row = mg + (w * kHeadsPerKv + hh) * (D + 2);
            const float e = (row[D] == kNegInf) ? 0.0f : fast_exp2(row[D] - M);
            acc += row[d] * e;
            den += row[D + 1] * e;
        }
        const int64_t pi = pbase + (int64_t)hh * a.nsplit;
        a.part_o[pi * D + d] = acc;
        if (d == 0) {
            a.part_m[pi] = M;
            a.part_l[pi] = den;
        }
    }
}

// Merge the splits of one (sequence, head): m = max m_c, l = sum l_c 2^(m_c - m),
// o = sum o_c 2^(m_c - m) / l, then out = o * sigma(gate).
template <typename T>
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
    const int sh = blockIdx.x;                         // s * 32 + h
    const int s = sh / kHeads;
    const int d = threadIdx.x;
    const int L = a.seq_len[s];
    const int64_t obase = (int64_t)sh * kHeadDim;      // n_new == 1
    T* out = (T*)a.out;
    if (L < 0 || L > a.max_seq_len) {
        out[obase + d] = from_f32<T>(__builtin_nanf(""));
        return;
    }
    const int64_t pb = (int64_t)sh * a.nsplit;
    float M = kNegInf;
    for (int c = 0; c < a.nsplit; ++c) M = fmaxf(M, a.part_m[pb + c]);
    float acc = 0.0f, den = 0.0f;
    for (int c = 0; c < a.nsplit; ++c) {
        const float mc = a.part_m[pb + c];
        const float e = (mc == kNegInf) ? 0.0f : fast_exp2(mc - M);
        acc += a.part_o[(pb + c) * kHeadDim + d] * e;
        den += a.part_l[pb + c] * e;
    }
    const float gv = to_f32(((const T*)a.gate)[obase + d]);
    out[obase + d] = from_f32<T>(acc / den * sigmoid(gv));
}

hipError_t launch_decode(const AttnArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kKvHeads * a.nsplit)), block(256);
    if (dtype == 1)
        hipLaunchKernelGGL(decode_kernel<bf16_t>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(decode_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kHeads)), block(128);
    if (dtype == 1)
        hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
