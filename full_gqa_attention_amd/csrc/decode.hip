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
// Before the loop each wave computes Q-hat of the 16 heads from the raw Q
// itself, in the B-operand layout it needs (norm, gain, RoPE on sliding
// layers: "Chapter 14 - QK-norm and RoPE" 14.3-14.5), with no workgroup
// barrier; it also makes the new K row (K-hat, rounded as stored) in the
// chunk layout of its sub-tiles, for the lanes whose row is position p.  The
// workgroup whose split holds p stores K-hat and V to cache row p (Ch 14,
// 14.7).
//
// After the loop the waves merge in LDS; each split writes a partial (max,
// sum, O); the splits' partials are merged in two levels (groups of
// consecutive splits, then the groups) by the last split to arrive at each,
// and the final merge applies the gate (Ch 9, 9.8).  Arrivals are counted in
// 64-bit words holding (call tag, count): a word carrying another call's tag
// counts as zero, so the workspace needs no clearing; the merging split
// resets the count.  Splits that would cover no row of a shorter sequence
// exit at once.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"



namespace muse {


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
__global__ __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_kernel(DecodeArgs a) {
    using Tr = DecodeTraits<T>;
    constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
    constexpr int D = kHeadDim, HG = kHeadsPerKv, SUB = 16;
    constexpr int LDV = Tr::LDV, LDKW = Tr::LDKW;
    constexpr int ES = (int)sizeof(T);
    constexpr int WAVE_V = SUB * LDV * ES, WAVE_K = SUB * LDKW * ES;
    constexpr int NW = kDecodeWaves, NT = 64 * NW;
    constexpr int LOOP_BYTES = NW * (WAVE_V + WAVE_K);
    constexpr int MERGE_BYTES = NW * HG * (D + 2) * 4;
    constexpr int LDS_BYTES = LOOP_BYTES > MERGE_BYTES ? LOOP_BYTES : MERGE_BYTES;
    // per-wave K and V buffers; the waves' partials after the loop
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    __shared__ int last_flag;

    const int b = blockIdx.x;
    const int c = b % a.nsplit;
    const int sg = b / a.nsplit;
    const int s = sg >> 1, g = sg & 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int64_t obase = ((int64_t)s * kHeads + g * HG) * D;     // out/gate/q of head 16g
    // ---- first the small loads, which do not depend on the sequence's
    // length (they go out before seq_len is read) and do not queue behind
    // the cache stream: the raw Q of the 16 heads in the B-operand layout of
    // S^T = K Q^T (lane: head l16, k-group q4), the new K and V rows in the
    // chunk layout of a cache sub-tile (every wave loads them; rows equal to
    // p take them), and the gate values this thread applies at the end.
    u32x4 qv[4];                                       // bf16: dims 32 st + 8 q4 .. + 7
    float qf32[kBf16 ? 1 : 32];                        // f32: dims 4 st + q4
    {
        const T* qh = (const T*)a.q + obase + (int64_t)l16 * D;
        if constexpr (kBf16) {
#pragma unroll
            for (int st = 0; st < 4; ++st) qv[st] = *(const u32x4*)(qh + 32 * st + 8 * q4);
        } else {
#pragma unroll
            for (int st = 0; st < 32; ++st) qf32[st] = to_f32(qh[4 * st + q4]);
        }
    }
    const int nch = kBf16 ? l16 : (lane & 31);         // 16-B chunk of a row this lane holds
    const int64_t new_off = ((int64_t)s * kKvHeads + g) * D * ES + 16 * nch;
    const u32x4 kn_raw = *(const u32x4*)((const char*)a.k + new_off);
    u32x4 vnew_c = *(const u32x4*)((const char*)a.v + new_off);
    // thread -> (head hh, DPT consecutive dims) after the loop
    constexpr int TPH = NT / HG, DPT = D / TPH;        // threads per head, dims per thread
    static_assert(TPH == 32 && DPT == 4, "a head per half wave, 4 dims per thread");
    const int hh = tid / TPH, d0 = (tid % TPH) * DPT;
    constexpr int GREG = DPT * ES / 16 > 0 ? DPT * ES / 16 : 1;   // 16-B loads of gate values
    u32x4 graw[GREG];
    if constexpr (kBf16) {
        const uint2 g2 = *(const uint2*)((const char*)a.gate + (obase + hh * D + d0) * ES);
        graw[0] = u32x4{g2.x, g2.y, 0u, 0u};
    } else {
        graw[0] = *(const u32x4*)((const char*)a.gate + (obase + hh * D + d0) * ES);
    }
    // this lane's RoPE frequency (pair = lane), loaded with the loads above
    const float th = theta_of_lane<DecodeArgs>(lane);
    // The exits below use those loads too (an empty asm that takes them):
    // otherwise the compiler moves the loads past the exits, behind the wait
    // for seq_len, and the two round trips no longer overlap.
    auto hold_loads = [&]() __attribute__((always_inline)) {
        if constexpr (kBf16) asm volatile("" :: "v"(qv[0]), "v"(qv[1]), "v"(qv[2]), "v"(qv[3]));
        else asm volatile("" :: "v"(qf32[0]));
        asm volatile("" :: "v"(kn_raw), "v"(vnew_c), "v"(graw[0]), "v"(th));
    };
    const int L = a.seq_len[s];
    const int W = a.window;

    if (L < 0 || L > a.max_seq_len) {                  // refused on the device
        hold_loads();
        if (c == 0)
            for (int i = tid; i < HG * D; i += NT) ((T*)a.out)[obase + i] = from_f32<T>(__builtin_nanf(""));
        return;
    }
    const int64_t p = L;
    const int64_t lo = (W > 0) ? max((int64_t)0, p - W + 1) : 0;
    const int64_t cs = lo + (int64_t)c * a.chunk;
    if (cs > p) {                                      // split beyond this sequence's rows
        hold_loads();
        return;
    }
    const int64_t ce = min(cs + (int64_t)a.chunk, p + 1);   // exclusive
    const int n_live = (int)((p - lo) / a.chunk) + 1;       // splits with rows
    const bool owns_p = (ce == p + 1);
    const int n_sub = (int)((ce - cs + SUB - 1) / SUB);
    const int my_cnt = n_sub > wave ? (n_sub - wave + NW - 1) / NW : 0;  // sub-tiles wave, wave+NW, ...

    char* wave_lds = lds + wave * (WAVE_V + WAVE_K);
    T* Vw = (T*)wave_lds;
    T* Kw = (T*)(wave_lds + WAVE_V);

    auto gate_sig = [&](int x) __attribute__((always_inline)) {     // sigmoid of gate value d0 + x
        float gv;
        if constexpr (kBf16) {
            const unsigned w = graw[0][x / 2];
            gv = __uint_as_float((x % 2) ? (w & 0xffff0000u) : (w << 16));
        } else {
            gv = __uint_as_float(graw[0][x]);
        }
        return sigmoid(gv);
    };

    // ---- loads of one 16-row sub-tile.  Every lane always loads (a load
    // skipped by some waves would make the compiler wait for all of them):
    // rows past the split are clamped to its last row ce - 1, whose score is
    // masked to P = 0 later; a lane whose (clamped) row is p gets the new
    // K/V row from LDS instead of the cache row being written.
    const int64_t row_stride = (int64_t)kKvHeads * D * ES;          // bytes per position
    const char* gk = (const char*)a.cache_k + ((int64_t)s * a.capacity * kKvHeads + g) * D * ES;
    const char* gv = (const char*)a.cache_v + ((int64_t)s * a.capacity * kKvHeads + g) * D * ES;
    auto clamp_row = [&](int64_t j) __attribute__((always_inline)) { return j < ce ? j : ce - 1; };
    // cache row of position j: j, or j % ring on a ring layer, where the
    // split's positions [cs, ce) (at most `ring` of them) wrap at most once
    const int64_t row_cs = a.ring ? cs % a.ring : cs;
    const int64_t wrap = a.ring ? a.ring : INT64_MAX;
    auto cache_row = [&](int64_t j) __attribute__((always_inline)) {
        const int64_t r = row_cs + (j - cs);
        return r >= wrap ? r - wrap : r;
    };
    auto issue = [&](SubTile<T>& t, int k) __attribute__((always_inline)) {
        const int64_t j0 = cs + (int64_t)SUB * (wave + NW * k);
        if constexpr (kBf16) {
            // K and V: rows 4u + lane/16, 16-B chunk lane%16 (whole 256-B rows per
            // 16 lanes; loading K straight into the MFMA layout, 64 B from each of
            // 16 rows per instruction, streams far slower)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t jv = cache_row(clamp_row(j0 + 4 * u + q4));
                t.k[u] = __builtin_nontemporal_load((const u32x4*)(gk + jv * row_stride + l16 * 16));
                t.v[u] = __builtin_nontemporal_load((const u32x4*)(gv + jv * row_stride + l16 * 16));
            }
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {              // rows 2u + lane/32, 16-B chunk lane%32
                const int64_t jj = cache_row(clamp_row(j0 + 2 * u + (lane >> 5)));
                t.k[u] = __builtin_nontemporal_load((const u32x4*)(gk + jj * row_stride + (lane & 31) * 16));
                t.v[u] = __builtin_nontemporal_load((const u32x4*)(gv + jj * row_stride + (lane & 31) * 16));
            }
        }
    };

    // pipeline stages as named variables (an indexed array of them ends up in scratch)
    static_assert(DEPTH >= 1 && DEPTH <= 8, "pipeline depth 1..8");
    SubTile<T> b0, b1, b2, b3, b4, b5, b6, b7;
    // The first DEPTH sub-tiles' loads go out as soon as the rows are known,
    // so that they are under way while Q-hat is made (sub-tiles past the
    // wave's share load clamped rows and are never processed).
    issue(b0, 0);
    if constexpr (DEPTH > 1) issue(b1, 1);
    if constexpr (DEPTH > 2) issue(b2, 2);
    if constexpr (DEPTH > 3) issue(b3, 3);
    if constexpr (DEPTH > 4) issue(b4, 4);
    if constexpr (DEPTH > 5) issue(b5, 5);
    if constexpr (DEPTH > 6) issue(b6, 6);
    if constexpr (DEPTH > 7) issue(b7, 7);

    // ---- Q-hat and the new K row, wave by wave (no workgroup barrier): RMS
    // norm with gain, then RoPE on sliding layers ("Chapter 14 - QK-norm and
    // RoPE" 14.3-14.5).  Lane i computes (cos, sin) of pair i into a table in
    // the wave's own LDS (its V buffer, unused until the loop); lanes read the
    // pairs they hold from there, several per LDS read.
    float2* rot = (float2*)Vw;
    if (a.rope) {
        float sn, cs_;
        sincos_rope((float)p * th, &sn, &cs_);
        rot[lane] = make_float2(cs_, sn);
    }
    auto rotate = [&](float& y0, float& y1, int pair) __attribute__((always_inline)) {
        const float2 cz = rot[pair];
        const float c2 = cz.x, s2 = cz.y;
        const float z0 = y0 * c2 - y1 * s2;
        const float z1 = y0 * s2 + y1 * c2;
        y0 = z0;
        y1 = z1;
    };
    auto bf16_at = [](const u32x4& v, int t) __attribute__((always_inline)) {
        const unsigned w = v[t / 2];
        return __uint_as_float((t % 2) ? (w & 0xffff0000u) : (w << 16));
    };
    constexpr int NSTQ = kBf16 ? 4 : 32;               // 16x16x32 bf16 / 16x16x4 f32 steps
    using MW = Mma16Wide<T>;
    using MN = Mma16Narrow<T>;
    typename MW::Frag qhi[NSTQ], qlo[kBf16 ? NSTQ : 1];
    {
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = kBf16 ? bf16_at(qv[i / 8], i % 8) : qf32[kBf16 ? 0 : i];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) ss += x[i] * x[i];
        ss = sum_halves(sum_rows16(ss));               // the head's other k-groups (lanes ^ 16, ^ 32)
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = (x[i] * r) * a.q_gain;
        if constexpr (kBf16) {
            if (a.rope) {
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) rotate(x[8 * st + 2 * j], x[8 * st + 2 * j + 1], 16 * st + 4 * q4 + j);
            }
#pragma unroll
            for (int st = 0; st < NSTQ; ++st) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float xv = x[8 * st + t];
                    const bf16_t hi = (bf16_t)xv;
                    qhi[st][t] = hi;
                    qlo[st][t] = (bf16_t)(xv - (float)hi);
                }
            }
        } else {
            if (a.rope) {                              // dim 4 st + q4; its pair partner sits in lane ^ 16
#pragma unroll
                for (int st = 0; st < 32; ++st) {
                    const float other = __shfl_xor(x[st], 16, 64);
                    float y0 = (q4 & 1) ? other : x[st], y1 = (q4 & 1) ? x[st] : other;
                    rotate(y0, y1, 2 * st + (q4 >> 1));
                    x[st] = (q4 & 1) ? y1 : y0;
                }
            }
#pragma unroll
            for (int st = 0; st < NSTQ; ++st) qhi[st] = x[st];
        }
    }
    // the new K row as it is stored (K-hat rounded to the cache type), in the
    // lane's chunk; the owner of p writes both rows to the cache
    u32x4 knew_c;
    {
        constexpr int NV = 16 / ES;                    // values per chunk
        float x[NV];
#pragma unroll
        for (int t = 0; t < NV; ++t) x[t] = kBf16 ? bf16_at(kn_raw, t) : __uint_as_float(kn_raw[t % 4]);
        float ss = 0.0f;
#pragma unroll
        for (int t = 0; t < NV; ++t) ss += x[t] * x[t];
#pragma unroll
        for (int o2 = 1; o2 < (kBf16 ? 16 : 32); o2 <<= 1) ss += __shfl_xor(ss, o2, 64);   // the row's chunks
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
        for (int t = 0; t < NV; ++t) x[t] = (x[t] * r) * a.k_gain;
        if (a.rope) {
#pragma unroll
            for (int j = 0; j < NV / 2; ++j) rotate(x[2 * j], x[2 * j + 1], (NV / 2) * nch + j);
        }
        if constexpr (kBf16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned lo16 = __builtin_bit_cast(unsigned short, from_f32<bf16_t>(x[2 * j]));
                const unsigned hi16 = __builtin_bit_cast(unsigned short, from_f32<bf16_t>(x[2 * j + 1]));
                knew_c[j] = lo16 | (hi16 << 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) knew_c[j] = __float_as_uint(x[kBf16 ? 0 : j]);
        }
    }
    if (owns_p && wave == 0 && (kBf16 ? q4 == 0 : lane < 32)) {
        const int64_t row_off = (((int64_t)s * a.capacity + cache_row(p)) * kKvHeads + g) * D * ES + 16 * nch;
        *(u32x4*)((char*)a.cache_k + row_off) = knew_c;
        *(u32x4*)((char*)a.cache_v + row_off) = vnew_c;
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
                    kraw = knew_c;
                    vraw = vnew_c;
                }
                *(u32x4*)(Kw + r * LDKW + l16 * 8) = kraw;
                *(u32x4*)(Vw + r * LDV + l16 * 8) = vraw;
            }
            // hi and lo parts in two accumulation chains (half the dependent
            // MFMA latency), added at the end
            floatx4 sl = floatx4{};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8 kf = *(const bf16x8*)(Kw + l16 * LDKW + 8 * q4 + 32 * st);
                sc = MW::mma(kf, qhi[st], sc);
                sl = MW::mma(kf, qlo[st], sl);
            }
            sc += sl;
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = 2 * u + (lane >> 5);
                u32x4 kraw = t.k[u], vraw = t.v[u];
                if (clamp_row(j0 + r) == p) {
                    kraw = knew_c;
                    vraw = vnew_c;
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
        mx = max_halves(max_rows16(mx));                 // lanes ^ 16 and ^ 32 hold the head's other keys
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
    l_run = sum_halves(sum_rows16(l_run));
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
    T* out = (T*)a.out + obase;
    // this split's partial for (head h2, dim d) from the waves' rows in LDS
    auto split_partial = [&](int h2, int d, float& M, float& den) __attribute__((always_inline)) {
        M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mg[(w * HG + h2) * (D + 2) + D]);
        float acc = 0.0f;
        den = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float* row = mg + (w * HG + h2) * (D + 2);
            const float e = (row[D] == kNegInf) ? 0.0f : fast_exp2(row[D] - M);
            acc += row[d] * e;
            den += row[D + 1] * e;
        }
        return acc;
    };
    float own_m, own_l, own_o[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) own_o[x] = split_partial(hh, d0 + x, own_m, own_l);
    if (n_live == 1) {                                 // the only split: finish here
        const float inv = 1.0f / own_l;
#pragma unroll
        for (int x = 0; x < DPT; ++x) out[hh * D + d0 + x] = from_f32<T>(own_o[x] * inv * gate_sig(x));
        return;
    }

    // ---- several splits, merged in two levels: the splits of a (sequence,
    // KV head) form groups of kArriveGroup consecutive splits.  Each split
    // first counts its arrival on its group's word; the last of a group (the
    // group merger) then counts on the (sequence, KV head) word, and the last
    // there is the final merger.  A split that merges does not publish its
    // own partial.  The others
    // publish (m, l, O) with agent-coherent stores, wait for them to
    // complete, then set their ready word to this call's tag; a merger waits
    // for those words (every split it waits for has already arrived, so it is
    // running) and reads the partials with agent-coherent loads.  A group
    // merger that is not final publishes its group's merged partial in the
    // slot of the group's first split (already consumed) and sets the group's
    // ready word.  No agent-scope fence is used: on this GPU one writes back /
    // invalidates the whole L2 of an XCD, which costs more than the attention
    // itself.  Every merge runs in fixed order with a merger's own partial
    // taken from registers (bit-equal to what it would have published), so
    // the output does not depend on which splits merge.
    constexpr int G = kArriveGroup;
    const int n_grps = (n_live + G - 1) / G;
    const int grp = c / G, c0 = grp * G, gsize = min(G, n_live - c0);
    if (tid == 0) {
        // count this split's arrival (arrive_tagged: the first attempt assumes
        // it completes n, right for the split whose merge ends the call)
        auto arrive = [&](unsigned long long* word, int n) { return arrive_tagged(word, a.tag, n); };
        unsigned long long* words = a.arrivals + (int64_t)(s * kKvHeads + g) * kArriveWords;   // pair, then groups
        int role = 0;                                  // 0 publish, 1 group merger, 2 final merger
        if (n_grps == 1) role = arrive(words, n_live) ? 2 : 0;
        else if (arrive(words + 1 + grp, gsize)) role = arrive(words, n_grps) ? 2 : 1;
        last_flag = role;
    }
    __syncthreads();
    const int role = last_flag;
    unsigned int* ready = a.ready + (int64_t)(s * kKvHeads + g) * kReadyWords;   // splits, then groups
    // the partials of this KV head's 16 query heads: O [16][nsplit][128], (m, l) [16][nsplit]
    float* po = a.part_o + ((int64_t)s * kHeads + g * HG) * a.nsplit * D;
    const __amdgpu_buffer_rsrc_t rs_o = partial_rsrc(po, (uint32_t)(HG * a.nsplit * D * 4));
    const int64_t ml_head = ((int64_t)s * kHeads + g * HG + hh) * a.nsplit;   // (m, l) of head hh, slot 0
    auto publish_partial = [&](int slot, float m, float l, const float (&o)[DPT]) __attribute__((always_inline)) {
        const int off = ((hh * a.nsplit + slot) * D + d0) * 4;            // bytes
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])},
            rs_o, off, 0, kCoherent);
        if (d0 == 0) {
            publish(a.part_m + ml_head + slot, m);
            publish(a.part_l + ml_head + slot, l);
        }
        __builtin_amdgcn_s_waitcnt(0);                 // the partial is stored before it is marked ready
        __syncthreads();
    };
    if (role == 0) {
        publish_partial(c, own_m, own_l, own_o);
        if (tid == 0) __hip_atomic_store(ready + c, a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // wait (bounded) for ready words first .. first + n - 1 except entry own,
    // clearing each for the next call or graph replay; false on a time-out
    __shared__ int ready_ok[2];
    auto wait_ready = [&](int first, int n, int own, int flag) __attribute__((always_inline)) {
        if (tid == 0) ready_ok[flag] = 1;
        __syncthreads();
        for (int j = tid; j < n; j += NT) {
            if (j == own) continue;
            int spins = 0;
            while (__hip_atomic_load(ready + first + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.tag) {
                if (++spins > kDecodeReadySpins) {
                    ready_ok[flag] = 0;                // give up: the output becomes NaN
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            __hip_atomic_store(ready + first + j, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        return ready_ok[flag] != 0;
    };
    // Merge n <= 16 partials in slot order first, first + stride, ...; entry
    // own comes from (om, ol, oo).  Lane k of the head's TPH reads entry k's
    // (m, l); the maximum and the denominator are reductions over those
    // lanes; then every thread sums its DPT dims of the n O rows, all loads
    // of one merge in flight together.
    constexpr int ME = 16;                             // merge entries at most
    static_assert(G <= ME && kMaxSplits / G <= ME && ME <= TPH, "one merge entry per lane");
    auto merge = [&](int first, int stride, int n, int own, float om, float ol, const float (&oo)[DPT],
                     float& m_out, float& l_out, float (&acc)[DPT]) __attribute__((always_inline)) {
        // the O rows first, so that one round trip covers these loads and the (m, l) below
        u32x4 raw[ME];
#pragma unroll
        for (int j = 0; j < ME; ++j) {
            if (j < n) {                               // n is uniform over the workgroup
                const int off = ((hh * a.nsplit + first + stride * j) * D + d0) * 4;
                raw[j] = __builtin_amdgcn_raw_buffer_load_b128(rs_o, off, 0, kCoherent);
            }
        }
        const int k = tid % TPH;
        float mk = kNegInf, lk = 0.0f;
        if (k == own) {
            mk = om;
            lk = ol;
        } else if (k < n) {
            mk = observe(a.part_m + ml_head + first + stride * k);
            lk = observe(a.part_l + ml_head + first + stride * k);
        }
        float M = mk;
#pragma unroll
        for (int o2 = TPH / 2; o2 >= 1; o2 >>= 1) M = fmaxf(M, __shfl_xor(M, o2, 64));
        const float e = k < n ? fast_exp2(mk - M) : 0.0f;
        float den = lk * e;
#pragma unroll
        for (int o2 = TPH / 2; o2 >= 1; o2 >>= 1) den += __shfl_xor(den, o2, 64);
#pragma unroll
        for (int x = 0; x < DPT; ++x) acc[x] = 0.0f;
#pragma unroll
        for (int j = 0; j < ME; ++j) {
            const float w = __shfl(e, (lane & ~(TPH - 1)) | j, 64);    // entry j's weight (0 past n)
            if (j < n) {
#pragma unroll
                for (int x = 0; x < DPT; ++x) {
                    const float v = (j == own) ? oo[x] : __uint_as_float(raw[j][x]);
                    acc[x] += v * w;
                }
            }
        }
        m_out = M;
        l_out = den;
    };

    // ---- a merger: first its group
    float gm, gl, go[DPT];
    const bool ok = wait_ready(c0, gsize, c - c0, 0);
    merge(c0, 1, gsize, c - c0, own_m, own_l, own_o, gm, gl, go);
    if (!ok) {
        gm = gl = __builtin_nanf("");
#pragma unroll
        for (int x = 0; x < DPT; ++x) go[x] = __builtin_nanf("");
    }
    if (role == 1) {                                   // publish the group's partial
        publish_partial(c0, gm, gl, go);
        if (tid == 0) __hip_atomic_store(ready + kMaxSplits + grp, a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    float fl = gl, fo[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) fo[x] = go[x];
    if (n_grps > 1) {                                  // the final merger: then the groups' partials
        const bool ok2 = wait_ready(kMaxSplits, n_grps, grp, 1);
        float fm;
        merge(0, G, n_grps, grp, gm, gl, go, fm, fl, fo);
        if (!ok2) fl = __builtin_nanf("");
    }
    const float inv = 1.0f / fl;
#pragma unroll
    for (int x = 0; x < DPT; ++x) out[hh * D + d0 + x] = from_f32<T>(fo[x] * inv * gate_sig(x));
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kKvHeads * a.nsplit)), block(64 * kDecodeWaves);
    if (dtype == 1)
        hipLaunchKernelGGL((decode_kernel<bf16_t, kDecodeDepth>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<float, 2>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
