// prefill.hip -- kernel (b): causal / sliding-window GQA attention over the
// KV cache for a chunk of new tokens, with the sigmoid gate fused into the
// epilogue.  Flash-style: the score matrix is never stored; softmax is online
// in the log2 domain (scores pre-multiplied by attn_scale * log2 e).
//
// Math (pages cited by title and section):
//   key j is visible to the query at position p iff j <= p and, on sliding
//   layers, p - j < window ("Chapter 9 - The Muse Glimmer architecture" 9.7);
//   query head h reads KV head h / 16 (Ch 9, Figure 9.3); score = q.k *
//   attn_scale (Ch 9, 9.5); out = softmax-weighted V times sigma(gate)
//   (Ch 9, 9.8).
//
// Shape of the work: one workgroup = 128 query rows of one head (4 waves x
// 32 rows).  KV tiles of 64 keys are staged in LDS and shared by the 4 waves.
// Each wave computes S^T = K Q^T on 32x32 MFMA tiles (fp16 32x32x16 on bf16
// layers, with K converted to fp16 as it is staged; f32 32x32x2 on f32
// layers), so a lane holds one query's scores: the row max
// and sum need one exchange with lane l ^ 32 only.  P.V is computed as O^T =
// V^T P^T, reusing the score registers directly as the B operand (the key
// order inside a K-step is permuted identically in P and V).
// Window-aware tile skipping: only tiles intersecting [p_lo - W + 1, p_hi]
// are visited; masks are applied only on tiles that straddle a boundary.
// Workgroups are numbered so that the 16 heads sharing one KV head and one
// query block land on the same XCD (round-robin dispatch over 8 XCDs), so
// their K/V tiles are served by that XCD's L2; heavy (late) query blocks are
// dispatched first.
#include "device_common.h"
#include "kernels.h"

namespace muse {

int prefill_grid(int n_seq, int n_new) {
    const int nqb = (n_new + kPrefillBM - 1) / kPrefillBM;
    const int units = n_seq * kKvHeads * nqb;          // (q-block, seq, kv head)
    return ((units + 7) / 8) * 8 * kHeadsPerKv;
}

template <typename T>
__global__ __launch_bounds__(256) void prefill_kernel(AttnArgs a) {
    typedef typename ScoreType<T>::type TQ;         // Q.K^T operand type
    using MQ = Mma32<TQ>;
    using MP = Mma32<T>;                               // P.V in the storage type
    using FragQ = typename MQ::Frag;
    using FragP = typename MP::Frag;
    constexpr int KPLQ = MQ::KPL, KPLP = MP::KPL;
    constexpr int BM = kPrefillBM, BN = kPrefillBN, D = kHeadDim;
    constexpr int LDK = D + 16 / (int)sizeof(TQ);     // padded LDS rows (elements)
    constexpr int LDV = D + 16 / (int)sizeof(T);
    constexpr int NST = D / (2 * KPLQ);                // K-steps of Q.K
    constexpr int NSTP = BN / (2 * KPLP);              // K-steps of P.V
    static_assert(sizeof(TQ) == sizeof(T), "K staging keeps the row size");
    __shared__ __attribute__((aligned(16))) TQ Ks[BN * LDK];
    __shared__ __attribute__((aligned(16))) T Vs[BN * LDV];

    // ---- work item: 16 heads of one (q-block, seq, kv head) per XCD
    const int nqb = (a.n_new + BM - 1) / BM;
    const int b = blockIdx.x;
    const int unit = (b >> 7) * 8 + (b & 7);
    const int hj = (b >> 3) & 15;
    const int per_qb = a.n_seq * kKvHeads;
    if (unit >= per_qb * nqb) return;
    const int qb = nqb - 1 - unit / per_qb;            // heavy blocks first
    const int s = (unit % per_qb) >> 1;
    const int g = (unit % per_qb) & 1;
    const int h = g * kHeadsPerKv + hj;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, gl = lane >> 5;
    const int q0 = qb * BM;
    const int N = a.n_new;
    const int L = a.seq_len[s];

    T* out = (T*)a.out;
    if (L < 0 || L > a.max_seq_len) {                  // refused on the device
        const int rows = min(BM, N - q0);
        for (int i = tid; i < rows * D; i += 256) {
            const int t = q0 + i / D;
            out[(((int64_t)s * N + t) * kHeads + h) * D + (i % D)] = from_f32<T>(__builtin_nanf(""));
        }
        return;
    }

    const int tq = q0 + wave * 32 + l32;               // this lane's query (new-token index)
    const int64_t pq = (int64_t)L + tq;                // its position
    const int tw0 = q0 + wave * 32;
    const int tw1 = min(tw0 + 31, N - 1);
    const bool wave_live = tw0 < N;
    const int64_t pw0 = (int64_t)L + tw0, pw1 = (int64_t)L + tw1;
    const int W = a.window;

    // ---- Q-hat fragments (B operand of S^T = K Q^T), held for the whole loop
    FragQ qf[NST];
    {
        const TQ* qrow = (const TQ*)a.qhat + (((int64_t)s * N + tq) * kHeads + h) * D;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if (tq < N)
                qf[st] = *(const FragQ*)(qrow + 2 * KPLQ * st + KPLQ * gl);
            else
                qf[st] = FragQ{};
        }
    }

    // ---- keys this block can see
    const int tb1 = min(q0 + BM - 1, N - 1);
    const int64_t P0 = (int64_t)L + q0, P1 = (int64_t)L + tb1;
    int64_t kv_lo = 0;
    if (W > 0) kv_lo = max((int64_t)0, P0 - W + 1);
    const int64_t kv_hi = P1;
    const int64_t kv_end = (int64_t)L + N;             // rows present in the cache
    const int64_t tile_lo = kv_lo / BN, tile_hi = kv_hi / BN;

    const char* gk = (const char*)a.cache_k;
    const char* gv = (const char*)a.cache_v;
    constexpr int CPR = D * (int)sizeof(T) / 16;       // 16-byte chunks per row
    constexpr int NCH = BN * CPR;

    floatx16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = floatx16{};
    float m_run = kNegInf, l_run = 0.0f;

    for (int64_t tile = tile_lo; tile <= tile_hi; ++tile) {
        const int64_t j0 = tile * BN;
        __syncthreads();
        for (int c = tid; c < NCH; c += 256) {
            const int r = c / CPR, cc = c % CPR;
            const int64_t jj = j0 + r;
            uint4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
            if (jj >= kv_lo && jj < kv_end) {
                const int64_t off = ((((int64_t)s * a.capacity + jj) * kKvHeads + g) * D) * (int64_t)sizeof(T) + cc * 16;
                kx = *(const uint4*)(gk + off);
                vx = *(const uint4*)(gv + off);
            }
            *(uint4*)((char*)Ks + (r * LDK) * (int)sizeof(TQ) + cc * 16) = k_chunk_to_score(kx, T{});
            *(uint4*)((char*)Vs + (r * LDV) * (int)sizeof(T) + cc * 16) = vx;
        }
        __syncthreads();
        if (!wave_live) continue;
        const bool any = (j0 <= pw1) && (W == 0 || pw0 - (j0 + BN - 1) < W);
        if (!any) continue;
        const bool need_mask = (j0 + BN - 1 > pw0) || (W > 0 && pw1 - j0 >= W);

        // S^T tiles: keys 32kt..32kt+31 x this wave's 32 queries
        floatx16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            sacc[kt] = floatx16{};
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                const FragQ kf = *(const FragQ*)(Ks + (32 * kt + l32) * LDK + 2 * KPLQ * st + KPLQ * gl);
                sacc[kt] = MQ::mma(kf, qf[st], sacc[kt]);
            }
        }

        // online softmax for query l32 (its other 32 keys sit in lane l ^ 32)
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = sacc[kt][i] * a.scale_log2;
                if (need_mask) {
                    const int64_t jj = j0 + 32 * kt + 8 * (i / 4) + 4 * gl + (i % 4);
                    if (jj > pq || (W > 0 && pq - jj >= W)) x = kNegInf;
                }
                sacc[kt][i] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float rs = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = fast_exp2(sacc[kt][i] - m_use);
                sacc[kt][i] = pv;
                rs += pv;
            }
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;

        // O^T += V^T P^T over the 64 keys of the tile
#pragma unroll
        for (int st = 0; st < NSTP; ++st) {
            FragP pf;
#pragma unroll
            for (int t = 0; t < KPLP; ++t) {
                const int I = st * KPLP + t;
                frag_set(pf, t, sacc[I / 16][I % 16]);
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                FragP vf;
#pragma unroll
                for (int t = 0; t < KPLP; ++t) {
                    const int I = st * KPLP + t;
                    const int key = 32 * (I / 16) + 8 * ((I % 16) / 4) + 4 * gl + (I % 4);
                    frag_set_raw(vf, t, Vs[key * LDV + 32 * dt + l32]);
                }
                o[dt] = MP::mma(vf, pf, o[dt]);
            }
        }
    }

    // ---- epilogue: normalise, gate, store (lane: 4 consecutive dims per item group)
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (!wave_live || tq >= N) return;
    const float inv = 1.0f / l_tot;
    const int64_t base = (((int64_t)s * N + tq) * kHeads + h) * D;
    const T* gate = (const T*)a.gate + base;
    T* dst = out + base;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
            const int d0 = 32 * dt + 8 * ig + 4 * gl;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float gv = to_f32(gate[d0 + x]);
                dst[d0 + x] = from_f32<T>(o[dt][4 * ig + x] * inv * sigmoid(gv));
            }
        }
    }
}

hipError_t launch_prefill(const AttnArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)prefill_grid(a.n_seq, a.n_new)), block(256);
    if (dtype == 1)
        hipLaunchKernelGGL(prefill_kernel<bf16_t>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
