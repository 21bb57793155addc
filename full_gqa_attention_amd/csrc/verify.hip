// verify.hip -- bf16 chunks of at most kVerifyTokens new tokens per
// sequence (the multi-token verify step of speculative decoding): the same
// attention as the prefill (causal within the chunk, over the cached prefix;
// "Chapter 9 - The Muse Glimmer architecture" 9.5-9.8), laid out for a long
// prefix and few queries.
//
// A workgroup owns one (sequence, KV head, split of the key range) and all
// 16 query heads of the KV head for every new token: wave w holds heads 2w
// and 2w + 1, 16 token rows each, as the 32 rows of its MFMA tiles, so each
// staged K/V tile feeds 16 heads x 16 tokens and the matrix cores see full
// tiles even for one token.  (The prefill kernel's rows are tokens of one
// head: a 16-token chunk would leave half of them empty and read every K/V
// row once per 8 heads.)  Keys are read from the bf16 cache and converted to
// fp16 while staged (no prefix copy for a handful of queries).  The softmax
// keeps a running row maximum (online; the chunk is short, so the O rescale
// is cheap).  Each split writes (max, sum, O) per row; a second kernel
// merges the splits in fixed order and applies the gate.
//
// The new rows' Q-hat is made here from the raw Q (QK-norm with gain, RoPE on
// sliding layers at the row's position; "Chapter 14 - QK-norm and RoPE"
// 14.3-14.5); the prep kernel has already appended the new K-hat and V.
#include "device_common.h"
#include "kernels.h"

namespace muse {

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void verify_kernel(VerifyArgs a) {
    typedef bf16_t T;
    typedef f16_t TQ;
    using MQ = Mma32<TQ>;
    using MP = Mma32<T>;
    using FragQ = MQ::Frag;
    using FragP = MP::Frag;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    constexpr int D = kHeadDim, BN = 32, NT = 512, ES = 2;
    constexpr int LDK = D + 8, LDV = D + 32;           // conflict-free b128 / transposing reads
    constexpr int NST = D / (2 * MQ::KPL);             // K-steps of Q.K (8)
    constexpr int CPR = D * ES / 16;                   // 16-byte chunks per row (16)
    static_assert(BN * CPR == NT, "one chunk of K and one of V per thread per tile");
    __shared__ __attribute__((aligned(16))) TQ Ks[2][BN * LDK];
    __shared__ __attribute__((aligned(16))) T Vs[2][BN * LDV];
    __shared__ float2 rot[kVerifyTokens][kHeadDim / 2 + 1];

    const int b = blockIdx.x;
    const int c = b % a.nsplit;
    const int sg = b / a.nsplit;
    const int s = sg >> 1, g = sg & 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, gl = lane >> 5;
    const int t = l32 & 15;                            // this lane's row: token t ...
    const int hg = 2 * wave + (l32 >> 4);              // ... of head 16g + hg
    const int h = g * kHeadsPerKv + hg;
    const int N = a.n_new;
    const int L = a.seq_len[s];
    if (L < 0 || L > a.max_seq_len) return;            // the merge writes NaN for it
    const int W = a.window;
    const int p = L + t;                               // the row's position (rows t >= N are padding)

    // keys of the chunk: [lo, hi); split c takes tiles [tile0 + c * chunk_tiles, ...)
    const int lo = W > 0 ? max(0, L - W + 1) : 0;
    const int hi = L + N;
    const int tile_first = lo / BN + c * a.chunk_tiles;
    const int tile_last = min(tile_first + a.chunk_tiles, (hi - 1) / BN + 1) - 1;   // inclusive
    const int ntiles = tile_last - tile_first + 1;     // may be <= 0: an empty split

    // ---- Q-hat of this lane's row (B operand of S^T = K Q^T; the row's other
    // 64 values sit in lane l ^ 32)
    if (a.rope) {
        float th = 0.0f;                               // theta[lane] without indexing the argument block
#pragma unroll
        for (int i = 0; i < 64; ++i) th = (lane == i) ? a.theta[i] : th;
        for (int tt = wave; tt < kVerifyTokens; tt += NT / 64) {
            float sn, cs;
            sincosf((float)(L + tt) * th, &sn, &cs);
            rot[tt][lane] = make_float2(cs, sn);
        }
        __syncthreads();
    }
    FragQ qf[NST];
    {
        const T* qrow = (const T*)a.q + (((int64_t)s * N + min(t, N - 1)) * kHeads + h) * D;
        float x[NST][8];
        float ss = 0.0f;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const bf16x8 raw = *(const bf16x8*)(qrow + 2 * MQ::KPL * st + MQ::KPL * gl);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[st][j] = (float)raw[j];
                ss += x[st][j] * x[st][j];
            }
        }
        ss = sum_halves(ss);
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) y[j] = (x[st][j] * r) * a.q_gain;
            if (a.rope) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {          // pair (dims 2i, 2i+1), i = 8 st + 4 gl + j
                    const float2 cz = rot[t][8 * st + 4 * gl + j];
                    const float y0 = y[2 * j], y1 = y[2 * j + 1];
                    y[2 * j] = y0 * cz.x - y1 * cz.y;
                    y[2 * j + 1] = y0 * cz.y + y1 * cz.x;
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) qf[st][j] = (TQ)(t < N ? y[j] * a.q_scale : 0.0f);
        }
    }

    // ---- tile staging: key row r_t, 16-byte chunk c_t of K (converted to
    // fp16) and of V.  Rows past the last position are clamped to it (masked
    // later, like every key outside a row's window).
    const int r_t = tid / CPR, c_t = tid % CPR;
    constexpr int64_t ROW = (int64_t)kKvHeads * D * ES;
    const char* kbase = (const char*)a.cache_k + (((int64_t)s * a.capacity) * kKvHeads + g) * D * ES + c_t * 16;
    const char* vbase = (const char*)a.cache_v + (((int64_t)s * a.capacity) * kKvHeads + g) * D * ES + c_t * 16;
    u32x4 kr, vr;
    auto load = [&](int tile) __attribute__((always_inline)) {
        const int64_t off = (int64_t)min(tile * BN + r_t, hi - 1) * ROW;
        kr = *(const u32x4*)(kbase + off);
        vr = *(const u32x4*)(vbase + off);
    };
    auto store = [&](int bufi) __attribute__((always_inline)) {
        *(u32x4*)((char*)Ks[bufi] + (r_t * LDK + c_t * 8) * 2) = k_chunk_to_score(kr, T{});
        *(u32x4*)((char*)Vs[bufi] + (r_t * LDV + c_t * 8) * 2) = vr;
    };

    floatx16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = floatx16{};
    float m_run = kNegInf, l_run = 0.0f;
    const unsigned wlim = W > 0 ? (unsigned)W : 0x7fffffffu;

    if (ntiles > 0) {
        load(tile_first);
        store(0);
        load(min(tile_first + 1, tile_last));
        __syncthreads();
    }
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        const int j0 = (tile_first + it) * BN;
        // S^T: keys j0 .. j0 + 31 x this wave's 32 rows
        floatx16 sc = floatx16{};
        const TQ* Kc = Ks[cur];
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const FragQ kf = *(const FragQ*)(Kc + l32 * LDK + 2 * MQ::KPL * st + MQ::KPL * gl);
            sc = MQ::mma(kf, qf[st], sc);
        }
        store(cur ^ 1);                                // the next tile (free since the last barrier)
        load(min(tile_first + it + 2, tile_last));     // past the end: harmless repeats
        // item i of this lane: key j0 + 8 (i / 4) + 4 gl + i % 4 of row (t, hg)
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = j0 + 8 * (i / 4) + 4 * gl + (i % 4);
            const float x = ((unsigned)(p - j) < wlim) ? sc[i] : kNegInf;
            sc[i] = x;
            mx = fmaxf(mx, x);
        }
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx);
        // a row with no visible key yet keeps m = -inf and P = 0
        const float alpha = m_new == kNegInf ? 1.0f : fast_exp2(m_run - m_new);
        const float sub = m_new == kNegInf ? 0.0f : m_new;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
        l_run *= alpha;
        // P = exp2(S - m) in bf16; l += those P; O^T += V^T P^T
        const T* Vc = Vs[cur];
#pragma unroll
        for (int st = 0; st < 2; ++st) {               // 16 keys per K-step
            FragP pf;
#pragma unroll
            for (int j = 0; j < MP::KPL; ++j) frag_set(pf, j, fast_exp2(sc[8 * st + j] - sub));
            const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
            float acc = l_run;
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), one, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), one, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), one, acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), one, acc, false);
            l_run = acc;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                // transposing reads of V rows kb + i/4 (+ 8), as in the prefill kernel
                typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
                const int kb = 16 * st + 4 * gl;
                const int i16 = lane & 15;
                const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
                const T* src0 = Vc + (kb + (i16 >> 2)) * LDV + col;
                const T* src1 = src0 + 8 * LDV;
                const shortx4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_shortx4*)(__attribute__((address_space(3))) void*)src0);
                const shortx4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_shortx4*)(__attribute__((address_space(3))) void*)src1);
                const FragP vf = __builtin_bit_cast(FragP, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
                o[dt] = MP::mma(vf, pf, o[dt]);
            }
        }
        __syncthreads();
    }

    // ---- this split's partial of the row: (m, l, O), O^T item i of lane l is
    // dim 32 dt + 8 (i / 4) + 4 gl + i % 4
    const float l_tot = sum_halves(l_run);
    const int64_t pr = (((int64_t)sg * a.nsplit + c) * kHeadsPerKv + hg) * kVerifyTokens + t;   // partial row
    float* po = a.part_o + pr * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
            floatx4 v4;
#pragma unroll
            for (int x = 0; x < 4; ++x) v4[x] = o[dt][4 * ig + x];
            *(floatx4*)(po + 32 * dt + 8 * ig + 4 * gl) = v4;
        }
    if (gl == 0) {
        a.part_m[pr] = m_run;
        a.part_l[pr] = l_tot;
    }
}

// Merge the splits of each (sequence, head, token) row in split order and
// apply the gate: one 64-lane wave per row, two dims per lane.
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);        // (s * 32 + h) * N + t
    const int lane = threadIdx.x & 63;
    const int N = a.n_new;
    if (row >= a.n_seq * kHeads * N) return;
    const int t = row % N, h = (row / N) % kHeads, s = row / (N * kHeads);
    const int g = h / kHeadsPerKv, hg = h % kHeadsPerKv;
    const int64_t obase = (((int64_t)s * N + t) * kHeads + h) * kHeadDim;
    bf16_t* out = (bf16_t*)a.out + obase;
    const int L = a.seq_len[s];
    if (L < 0 || L > a.max_seq_len) {
        out[2 * lane] = out[2 * lane + 1] = from_f32<bf16_t>(__builtin_nanf(""));
        return;
    }
    const bf16_t* gate = (const bf16_t*)a.gate + obase;
    const float g0 = sigmoid(to_f32(gate[2 * lane])), g1 = sigmoid(to_f32(gate[2 * lane + 1]));
    auto prow = [&](int c) { return (((int64_t)(s * kKvHeads + g) * a.nsplit + c) * kHeadsPerKv + hg) * kVerifyTokens + t; };
    float M = kNegInf;
    for (int c = 0; c < a.nsplit; ++c) M = fmaxf(M, a.part_m[prow(c)]);
    float den = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c = 0; c < a.nsplit; ++c) {
        const int64_t r = prow(c);
        const float m = a.part_m[r];
        if (m == kNegInf) continue;                    // a split with no visible key for this row
        const float e = fast_exp2(m - M);
        den += a.part_l[r] * e;
        const float2 v = *(const float2*)(a.part_o + r * kHeadDim + 2 * lane);
        o0 += v.x * e;
        o1 += v.y * e;
    }
    const float inv = 1.0f / den;
    out[2 * lane] = from_f32<bf16_t>(o0 * inv * g0);
    out[2 * lane + 1] = from_f32<bf16_t>(o1 * inv * g1);
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kKvHeads * a.nsplit)), block(512);
    hipLaunchKernelGGL(verify_kernel, grid, block, 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipSuccess;
}

hipError_t launch_verify_merge(const VerifyArgs& a, hipStream_t stream) {
    const int rows = a.n_seq * kHeads * a.n_new;
    hipLaunchKernelGGL(verify_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
