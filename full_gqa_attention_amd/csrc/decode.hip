// decode.hip -- kernel (c): the whole decode step (one new token per
// sequence) in a single launch: QK-norm and RoPE of the new Q and K, the KV
// append, split-K attention over the cache, the merge of the splits and the
// sigmoid gate.
//
// The step is bound by reading the cache: 1,024 bytes of K and V per visible
// row per sequence ("Chapter 9 - The Muse Glimmer architecture" 9.5, 9.6),
// shared by the 16 query heads of each KV head (Ch 9, Figure 9.3).  One
// workgroup owns one (sequence, KV head, split) and computes all 16 heads in
// a single pass over its rows.
//
// Streaming: each of the 8 waves owns every eighth 16-row sub-tile of the split and
// keeps DEPTH sub-tiles of loads in flight in registers; there is no
// workgroup barrier inside the loop, so the waves of a CU overlap freely.
//   * K rows go through a wave-private LDS buffer into the A-operand layout of
//     a 16x16x32 MFMA (16 rows x 16 heads per tile, S^T = K Q^T).  On bf16 layers Q-hat is
//     split into bf16 hi + lo parts (two MFMAs), which scores with about 16
//     significant bits and takes the stored bf16 keys as they are.
//   * V rows are written to a wave-private LDS buffer and read back with the
//     transposing LDS load (ds_read_b64_tr_b16), which delivers the A operand
//     of O^T = V^T P^T (16x16x16 MFMA) directly; P^T is the score tile as it
//     sits in registers.
//   * Online softmax in the log2 domain; the row max over 16 keys needs two
//     lane exchanges (xor 16, 32).
//
// Before the loop each workgroup computes Q-hat of its 16 heads from the raw
// Q (norm, gain, RoPE on sliding layers: "Chapter 14 - QK-norm and RoPE"
// 14.3-14.5).  The workgroup whose split holds position p also normalises and
// rotates the new K, stores K-hat and V to cache row p (Ch 14, 14.7) and
// substitutes that row in its registers.
//
// After the loop the waves merge in LDS; each split writes a partial (max,
// sum, O); the last split of a (sequence, KV head) to arrive merges all of
// them and applies the gate (Ch 9, 9.8).  Arrivals are counted in a 64-bit
// word holding (call tag, count): a word carrying another call's tag counts
// as zero, so the workspace needs no clearing; the merging split resets the
// count.  Splits that would cover no row of a shorter sequence exit at once.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

#ifndef MUSE_DECODE_WAVES
#define MUSE_DECODE_WAVES 2        // waves per SIMD the register budget targets
#endif
#ifndef MUSE_DECODE_DEPTH
#define MUSE_DECODE_DEPTH 3        // 16-row sub-tiles in flight per wave
#endif

namespace muse {

// Split partials cross workgroups (and XCDs): written and read with
// agent-scope atomic accesses, which are coherent per access.
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float observe(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T> struct DecodeTraits;
// bf16: K in registers in MFMA layout (4 x 16 B per lane), V row-major (4 x 16 B)
// bf16: K and V rows loaded alike (4 rows x 256 B per load instruction) and
// staged in LDS; K is read back in the A-operand layout of the 16x16x32 MFMA
template <> struct DecodeTraits<bf16_t> {
    static constexpr int KREG = 4, VREG = 4;
    static constexpr int LDV = kHeadDim + 16;          // V row stride in LDS (elements)
    static constexpr int LDKW = kHeadDim + 8;          // K row stride in LDS: b128 reads conflict-free
};
// f32 (parity path): K and V both row-major through LDS (8 x 16 B each)
template <> struct DecodeTraits<float> {
    static constexpr int KREG = 8, VREG = 8;
    static constexpr int LDV = kHeadDim + 4;
    static constexpr int LDKW = kHeadDim + 4;
};

template <typename T>
struct SubTile {
    u32x4 k[DecodeTraits<T>::KREG];
    u32x4 v[DecodeTraits<T>::VREG];
};

template <typename T, int DEPTH>
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(MUSE_DECODE_WAVES, MUSE_DECODE_WAVES)))
void decode_kernel(DecodeArgs a) {
    using Tr = DecodeTraits<T>;
    constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
    constexpr int D = kHeadDim, HG = kHeadsPerKv, SUB = 16;
    constexpr int LDV = Tr::LDV, LDKW = Tr::LDKW, LDQ = D + 4;
    constexpr int ES = (int)sizeof(T);
    constexpr int WAVE_V = SUB * LDV * ES, WAVE_K = SUB * LDKW * ES;
    constexpr int NW = kDecodeWaves, NT = 64 * NW;
    constexpr int LOOP_BYTES = NW * (WAVE_V + WAVE_K) + HG * LDQ * 4;
    constexpr int MERGE_BYTES = NW * HG * (D + 2) * 4 + HG * kMaxSplits * 4;
    constexpr int LDS_BYTES = LOOP_BYTES > MERGE_BYTES ? LOOP_BYTES : MERGE_BYTES;
    // per-wave V (and f32 K) buffers and the f32 Q-hat; the 4-wave merge after the loop
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    __shared__ __attribute__((aligned(16))) T knew[D];    // new key row p (stored values)
    __shared__ __attribute__((aligned(16))) T vnew[D];    // new value row p
    __shared__ int last_flag;

    const int b = blockIdx.x;
    const int c = b % a.nsplit;
    const int sg = b / a.nsplit;
    const int s = sg >> 1, g = sg & 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int L = a.seq_len[s];
    const int W = a.window;
    const int64_t obase = ((int64_t)s * kHeads + g * HG) * D;     // out/gate/q of head 16g

    if (L < 0 || L > a.max_seq_len) {                  // refused on the device
        if (c == 0)
            for (int i = tid; i < HG * D; i += NT) ((T*)a.out)[obase + i] = from_f32<T>(__builtin_nanf(""));
        return;
    }
    const int64_t p = L;
    const int64_t lo = (W > 0) ? max((int64_t)0, p - W + 1) : 0;
    const int64_t cs = lo + (int64_t)c * a.chunk;
    if (cs > p) return;                                // split beyond this sequence's rows
    const int64_t ce = min(cs + (int64_t)a.chunk, p + 1);   // exclusive
    const int n_live = (int)((p - lo) / a.chunk) + 1;       // splits with rows
    const bool owns_p = (ce == p + 1);
    const int n_sub = (int)((ce - cs + SUB - 1) / SUB);
    const int my_cnt = n_sub > wave ? (n_sub - wave + NW - 1) / NW : 0;  // sub-tiles wave, wave+NW, ...

    char* wave_lds = lds + wave * (WAVE_V + WAVE_K);
    T* Vw = (T*)wave_lds;
    T* Kw = (T*)(wave_lds + WAVE_V);
    float* Qf = (float*)(lds + NW * (WAVE_V + WAVE_K));

    // ---- loads of one 16-row sub-tile.  Every lane always loads (a load
    // skipped by some waves would make the compiler wait for all of them):
    // rows past the split are clamped to its last row ce - 1, whose score is
    // masked to P = 0 later; a lane whose (clamped) row is p gets the new
    // K/V row from LDS instead of the cache row being written.
    const int64_t row_stride = (int64_t)kKvHeads * D * ES;          // bytes per position
    const char* gk = (const char*)a.cache_k + ((int64_t)s * a.capacity * kKvHeads + g) * D * ES;
    const char* gv = (const char*)a.cache_v + ((int64_t)s * a.capacity * kKvHeads + g) * D * ES;
    auto clamp_row = [&](int64_t j) __attribute__((always_inline)) { return j < ce ? j : ce - 1; };
    auto issue = [&](SubTile<T>& t, int k) __attribute__((always_inline)) {
        const int64_t j0 = cs + (int64_t)SUB * (wave + NW * k);
        if constexpr (kBf16) {
            // K and V: rows 4u + lane/16, 16-B chunk lane%16 (whole 256-B rows per
            // 16 lanes; loading K straight into the MFMA layout, 64 B from each of
            // 16 rows per instruction, streams far slower)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t jv = clamp_row(j0 + 4 * u + q4);
                t.k[u] = __builtin_nontemporal_load((const u32x4*)(gk + jv * row_stride + l16 * 16));
                t.v[u] = __builtin_nontemporal_load((const u32x4*)(gv + jv * row_stride + l16 * 16));
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {              // rows 2u + lane/32, 16-B chunk lane%32
                const int64_t jj = clamp_row(j0 + 2 * u + (lane >> 5));
                t.k[u] = __builtin_nontemporal_load((const u32x4*)(gk + jj * row_stride + (lane & 31) * 16));
                t.v[u] = __builtin_nontemporal_load((const u32x4*)(gv + jj * row_stride + (lane & 31) * 16));
            }
        }
    };

    // pipeline stages as named variables (an indexed array of them ends up in scratch)
    static_assert(DEPTH >= 1 && DEPTH <= 8, "pipeline depth 1..8");
    SubTile<T> b0, b1, b2, b3, b4, b5, b6, b7;
    // (sub-tiles past the wave's share load clamped rows and are never processed)
    issue(b0, 0);
    if constexpr (DEPTH > 1) issue(b1, 1);
    if constexpr (DEPTH > 2) issue(b2, 2);
    if constexpr (DEPTH > 3) issue(b3, 3);
    if constexpr (DEPTH > 4) issue(b4, 4);
    if constexpr (DEPTH > 5) issue(b5, 5);
    if constexpr (DEPTH > 6) issue(b6, 6);
    if constexpr (DEPTH > 7) issue(b7, 7);

    // ---- prologue: Q-hat of the 16 heads (f32 in LDS); the owner of p also
    // makes the new K/V row
    {
        float sn = 0.0f, cs_ = 1.0f;
        if (a.rope) rope_sincos(a.theta, lane, p, sn, cs_);
        const T* q = (const T*)a.q + obase;
#pragma unroll
        for (int i = 0; i < HG / NW; ++i) {
            const int hh = wave * (HG / NW) + i;
            float y0, y1;
            norm_rope_pair(to_f32(q[hh * D + 2 * lane]), to_f32(q[hh * D + 2 * lane + 1]), a.eps,
                           a.q_gain, a.rope, sn, cs_, y0, y1);
            Qf[hh * LDQ + 2 * lane] = y0;
            Qf[hh * LDQ + 2 * lane + 1] = y1;
        }
        if (owns_p && wave == 0) {
            const T* kr = (const T*)a.k + ((int64_t)s * kKvHeads + g) * D;
            float y0, y1;
            norm_rope_pair(to_f32(kr[2 * lane]), to_f32(kr[2 * lane + 1]), a.eps, a.k_gain, a.rope,
                           sn, cs_, y0, y1);
            const T k0 = from_f32<T>(y0), k1 = from_f32<T>(y1);
            T* dst = (T*)a.cache_k + (((int64_t)s * a.capacity + p) * kKvHeads + g) * D;
            dst[2 * lane] = k0;
            dst[2 * lane + 1] = k1;
            knew[2 * lane] = k0;
            knew[2 * lane + 1] = k1;
        }
        if (owns_p && wave == 1) {
            const T* vr = (const T*)a.v + ((int64_t)s * kKvHeads + g) * D;
            T* dst = (T*)a.cache_v + (((int64_t)s * a.capacity + p) * kKvHeads + g) * D;
            const T v0 = vr[2 * lane], v1 = vr[2 * lane + 1];
            dst[2 * lane] = v0;
            dst[2 * lane + 1] = v1;
            vnew[2 * lane] = v0;
            vnew[2 * lane + 1] = v1;
        }
    }
    __syncthreads();

    // Q-hat as the B operand of S^T = K Q^T: lane holds head l16, k-group q4
    constexpr int NSTQ = kBf16 ? 4 : 32;               // 16x16x32 bf16 / 16x16x4 f32 steps
    using MW = Mma16Wide<T>;
    using MN = Mma16Narrow<T>;
    typename MW::Frag qhi[NSTQ], qlo[kBf16 ? NSTQ : 1];
    {
        const float* qrow = Qf + l16 * LDQ;
        if constexpr (kBf16) {
#pragma unroll
            for (int st = 0; st < NSTQ; ++st) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float x = qrow[32 * st + 8 * q4 + t];
                    const bf16_t hi = (bf16_t)x;
                    qhi[st][t] = hi;
                    qlo[st][t] = (bf16_t)(x - (float)hi);
                }
            }
        } else {
#pragma unroll
            for (int st = 0; st < NSTQ; ++st) qhi[st] = qrow[4 * st + q4];
        }
    }

    floatx4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{};
    float m_run = kNegInf, l_run = 0.0f;

    auto process = [&](SubTile<T>& t, int k) __attribute__((always_inline)) {
        const int64_t j0 = cs + (int64_t)SUB * (wave + NW * k);
        // ---- scores S^T[key j0 + 4*q4 + i][head l16]
        floatx4 sc = floatx4{};
        if constexpr (kBf16) {
            // stage K and V rows (row p from the new row), then K back in the A layout
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * u + q4;
                u32x4 kraw = t.k[u], vraw = t.v[u];
                if (clamp_row(j0 + r) == p) {
                    kraw = *(const u32x4*)(knew + l16 * 8);
                    vraw = *(const u32x4*)(vnew + l16 * 8);
                }
                *(u32x4*)(Kw + r * LDKW + l16 * 8) = kraw;
                *(u32x4*)(Vw + r * LDV + l16 * 8) = vraw;
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 kf = *(const bf16x8*)(Kw + l16 * LDKW + 8 * q4 + 32 * st);
                sc = MW::mma(kf, qhi[st], sc);
                sc = MW::mma(kf, qlo[st], sc);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 2 * u + (lane >> 5);
                u32x4 kraw = t.k[u], vraw = t.v[u];
                if (clamp_row(j0 + r) == p) {
                    kraw = *(const u32x4*)(knew + (lane & 31) * 4);
                    vraw = *(const u32x4*)(vnew + (lane & 31) * 4);
                }
                *(u32x4*)(Kw + r * LDKW + (lane & 31) * 4) = kraw;
                *(u32x4*)(Vw + r * LDV + (lane & 31) * 4) = vraw;
            }
#pragma unroll
            for (int st = 0; st < NSTQ; ++st) sc = MW::mma(Kw[l16 * LDKW + 4 * st + q4], qhi[st], sc);
        }
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = sc[i] * a.scale_log2;
            if (j0 + 4 * q4 + i >= ce) x = kNegInf;
            sc[i] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);            // finite: key j0 is visible
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

        // ---- O^T += V^T P^T
        if constexpr (kBf16) {
            typename MN::Frag pf;
#pragma unroll
            for (int i = 0; i < 4; ++i) frag_set(pf, i, sc[i]);
            // source lane i of each 16-lane group q4 points at V row 4*q4 + i/4,
            // columns 4*(i%4) .. +3 of the 16-column block dt
            typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
            const int vrow = 4 * q4 + (l16 >> 2);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const T* src = Vw + vrow * LDV + 16 * dt + 4 * (l16 & 3);
                const shortx4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_shortx4*)(__attribute__((address_space(3))) void*)src);
                o[dt] = MN::mma(vf, pf, o[dt]);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) {           // 16x16x4 f32: key 4*q4 + st
                const float pf = sc[st];
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    o[dt] = MN::mma(Vw[(4 * q4 + st) * LDV + 16 * dt + l16], pf, o[dt]);
            }
        }
    };

    // the same number of loads in every stage keeps the compiler's load
    // counting exact (it waits for one stage's loads, not for all)
    auto stage = [&](SubTile<T>& t, int k) __attribute__((always_inline)) {
        if (k < my_cnt) process(t, k);
        issue(t, k + DEPTH);
    };
    for (int k0 = 0; k0 < my_cnt; k0 += DEPTH) {
        stage(b0, k0);
        if constexpr (DEPTH > 1) stage(b1, k0 + 1);
        if constexpr (DEPTH > 2) stage(b2, k0 + 2);
        if constexpr (DEPTH > 3) stage(b3, k0 + 3);
        if constexpr (DEPTH > 4) stage(b4, k0 + 4);
        if constexpr (DEPTH > 5) stage(b5, k0 + 5);
        if constexpr (DEPTH > 6) stage(b6, k0 + 6);
        if constexpr (DEPTH > 7) stage(b7, k0 + 7);
    }

    // ---- merge the waves: LDS holds per wave [16 heads][128 + 2] floats
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    __syncthreads();
    float* mg = (float*)lds;
    float* mw = mg + (wave * HG + l16) * (D + 2);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mw[16 * dt + 4 * q4 + i] = o[dt][i];
    if (q4 == 0) {
        mw[D] = m_run;
        mw[D + 1] = l_run;
    }
    __syncthreads();
    const T* gate = (const T*)a.gate + obase;
    T* out = (T*)a.out + obase;
    // this split's partial for (head hh, dim d) from the waves' rows in LDS
    auto split_partial = [&](int hh, int d, float& M, float& den) __attribute__((always_inline)) {
        M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mg[(w * HG + hh) * (D + 2) + D]);
        float acc = 0.0f;
        den = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float* row = mg + (w * HG + hh) * (D + 2);
            const float e = (row[D] == kNegInf) ? 0.0f : fast_exp2(row[D] - M);
            acc += row[d] * e;
            den += row[D + 1] * e;
        }
        return acc;
    };
    if (n_live == 1) {                                 // the only split: finish here
        for (int i = tid; i < HG * D; i += NT) {
            float M, den;
            const float acc = split_partial(i / D, i % D, M, den);
            out[i] = from_f32<T>(acc / den * sigmoid(to_f32(gate[i])));
        }
        return;
    }

    // ---- several splits.  Each split first counts its arrival: the last one
    // merges, and it does not publish its own partial.  The others publish
    // (m, l, O) with agent-coherent stores, wait for them to complete, then
    // set their ready word to this call's tag; the merging split waits for
    // those words (every other split has already arrived, so they are
    // running) and reads the partials with agent-coherent loads.  No
    // agent-scope fence is used: on this GPU one writes back / invalidates
    // the whole L2 of an XCD, which costs more than the attention itself.
    // Thread -> (head hh, DPT consecutive dims) in the final merge; its gate
    // values are read now, so that the merging split does not wait for them.
    constexpr int TPH = NT / HG, DPT = D / TPH;        // threads per head, dims per thread
    const int hh = tid / TPH, d0 = (tid % TPH) * DPT;
    float gsig[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) gsig[x] = sigmoid(to_f32(gate[hh * D + d0 + x]));
    if (tid == 0) {
        // count this split's arrival on a tagged word (tag << 32 | count); true
        // for the arrival that completes n, which resets the word for a replay
        // with the same tag.  The first attempt assumes it completes n: right
        // for the split whose merge ends the call, one round trip saved.
        auto arrive = [&](unsigned long long* word, int n) {
            unsigned long long old = ((unsigned long long)a.tag << 32) | (unsigned int)(n - 1);
            unsigned int arrived = 0;
            for (;;) {                                 // retries only on contention
                const unsigned int cnt = ((unsigned int)(old >> 32) == a.tag) ? (unsigned int)old : 0u;
                const unsigned long long want = ((unsigned long long)a.tag << 32) | (cnt + 1);
                if (__hip_atomic_compare_exchange_strong(word, &old, want, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                    arrived = cnt + 1;
                    break;
                }
            }
            const bool done = arrived == (unsigned int)n;
            if (done)
                __hip_atomic_store(word, (unsigned long long)a.tag << 32, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            return done;
        };
        // Many splits arriving on one word serialise on its compare-and-swap, so
        // they count in groups of kArriveGroup first; the last of each group then
        // arrives on the (sequence, KV head) word.
        unsigned long long* words = a.arrivals + (int64_t)(s * kKvHeads + g) * kArriveWords;
        const int n_grps = (n_live + kArriveGroup - 1) / kArriveGroup;
        bool last = true;
        if (n_grps > 1) {
            const int grp = c / kArriveGroup;
            last = arrive(words + 1 + grp, min(kArriveGroup, n_live - grp * kArriveGroup));
        }
        if (last) last = arrive(words, n_grps > 1 ? n_grps : n_live);
        last_flag = last;
    }
    __syncthreads();
    unsigned int* ready = a.ready + (int64_t)(s * kKvHeads + g) * a.nsplit;
    const int64_t pbase = ((int64_t)s * kHeads + g * HG) * a.nsplit + c;   // head 16g, split c
    if (!last_flag) {
        for (int i = tid; i < HG * D; i += NT) {
            const int h2 = i / D, d = i % D;
            float M, den;
            const float acc = split_partial(h2, d, M, den);
            const int64_t pi = pbase + (int64_t)h2 * a.nsplit;
            publish(a.part_o + pi * D + d, acc);
            if (d == 0) {
                publish(a.part_m + pi, M);
                publish(a.part_l + pi, den);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);                 // the partial is stored before it is marked ready
        __syncthreads();
        if (tid == 0) __hip_atomic_store(ready + c, a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ---- the merging split: wait (bounded) for the other splits' partials
    if (tid == 0) last_flag = 1;                       // reused below as "all ready"
    __syncthreads();
    for (int cc = tid; cc < n_live; cc += NT) {
        if (cc == c) continue;
        int spins = 0;
        while (__hip_atomic_load(ready + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.tag) {
            if (++spins > kDecodeReadySpins) {
                last_flag = 0;                         // give up: the output becomes NaN
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        // consumed: cleared for the next call or graph replay
        __hip_atomic_store(ready + cc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_flag) {
#pragma unroll
        for (int x = 0; x < DPT; ++x) out[hh * D + d0 + x] = from_f32<T>(__builtin_nanf(""));
        return;
    }

    // ---- merge (the result does not depend on which split merges).
    // Phase 1: thread (head hh, lane k of the head's TPH threads) reads (m, l)
    // of splits k, k + TPH, ... in one round of loads; the head's maximum and
    // denominator come from a reduction over those TPH lanes (one wave half),
    // and each split's weight exp2(m_c - M) goes to LDS.
    static_assert(TPH == 32, "one head per half wave in the merge");
    float* wts = (float*)lds + NW * HG * (D + 2);      // [16 heads][kMaxSplits] after the wave rows
    const int k = tid % TPH;
    const int64_t hb = ((int64_t)s * kHeads + g * HG + hh) * a.nsplit;
    float own_m, own_l, own_o[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) own_o[x] = split_partial(hh, d0 + x, own_m, own_l);
    float pm[kMaxSplits / TPH], pl[kMaxSplits / TPH];
    float M = kNegInf;
#pragma unroll
    for (int j = 0; j < kMaxSplits / TPH; ++j) {
        const int cc = k + TPH * j;
        pm[j] = kNegInf;
        pl[j] = 0.0f;
        if (cc == c) {
            pm[j] = own_m;
            pl[j] = own_l;
        } else if (cc < n_live) {
            pm[j] = observe(a.part_m + hb + cc);
            pl[j] = observe(a.part_l + hb + cc);
        }
        M = fmaxf(M, pm[j]);
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));   // within the half wave
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxSplits / TPH; ++j) {
        const int cc = k + TPH * j;
        const float e = fast_exp2(pm[j] - M);          // 0 past n_live
        if (cc < n_live) wts[hh * kMaxSplits + cc] = e;
        den += pl[j] * e;
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
    __syncthreads();
    // Phase 2: O = sum_c w_c O_c over the splits, eight splits per round of loads
    float acc[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) acc[x] = 0.0f;
    for (int c0 = 0; c0 < n_live; c0 += 8) {
        float po[8][DPT];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cc = c0 + j;
#pragma unroll
            for (int x = 0; x < DPT; ++x) po[j][x] = 0.0f;
            if (cc == c) {
#pragma unroll
                for (int x = 0; x < DPT; ++x) po[j][x] = own_o[x];
            } else if (cc < n_live) {
#pragma unroll
                for (int x = 0; x < DPT; ++x) po[j][x] = observe(a.part_o + (hb + cc) * D + d0 + x);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cc = c0 + j;
            const float e = cc < n_live ? wts[hh * kMaxSplits + cc] : 0.0f;
#pragma unroll
            for (int x = 0; x < DPT; ++x) acc[x] += po[j][x] * e;
        }
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int x = 0; x < DPT; ++x) out[hh * D + d0 + x] = from_f32<T>(acc[x] * inv * gsig[x]);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kKvHeads * a.nsplit)), block(64 * kDecodeWaves);
    if (dtype == 1)
        hipLaunchKernelGGL((decode_kernel<bf16_t, MUSE_DECODE_DEPTH>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<float, 2>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
