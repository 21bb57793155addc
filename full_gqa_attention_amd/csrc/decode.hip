// decode.hip -- kernel (c): the decode step (one new token per sequence):
// QK-norm and RoPE of the new Q and K, the KV append and split-K attention
// over the cache in one launch (decode_kernel), then, when a sequence's keys
// are split over several workgroups, the merge of the splits with the sigmoid
// gate in a second (decode_merge_kernel).
//
// The step is bound by reading the cache: 1,024 bytes of K and V per visible
// row per sequence ("Chapter 9 - The Muse Glimmer architecture" 9.5, 9.6),
// shared by the 16 query heads of each KV head (Ch 9, Figure 9.3).  One
// workgroup owns one (sequence, KV head, split) and computes all 16 heads in
// a single pass over its rows.
//
// A CU streams only a few tens of GB/s on its own, so a short key range (a
// 2,048-row window) is spread over many small splits, and every step a
// workgroup takes before its first loads return is latency: the prologue is
// kept short.
//   * Q-hat (norm, gain, RoPE: "Chapter 14 - QK-norm and RoPE" 14.3-14.5) is
//     made once per workgroup, each wave normalising 16 / NW of the heads, and
//     handed to every wave through LDS as the B operand of S^T = K Q^T.  On
//     bf16 layers it is split into bf16 hi + lo parts (two MFMAs), which
//     scores with about 16 significant bits against the stored bf16 keys.
//   * Cache rows are read with buffer loads from a per-workgroup base and
//     32-bit offsets (K and V share the offsets), 16 lanes per 256-byte row.
//   * Each wave streams every NW-th 16-row sub-tile with DEPTH sub-tiles of
//     loads in flight in registers and no workgroup barrier in the loop.  K
//     rows go through a wave-private LDS buffer into the A-operand layout of
//     a 16x16x32 MFMA; V rows are read back with the transposing LDS load
//     (ds_read_b64_tr_b16), the A operand of O^T = V^T P^T (16x16x16 MFMA),
//     P^T being the score tile as it sits in registers.
//   * Online softmax in the log2 domain; the running output is rescaled only
//     when some row's maximum grows.
//   * The new K row (K-hat, rounded as stored) and V row are made and used
//     only by the wave whose sub-tile holds position p; that wave stores them
//     to cache row p (Ch 14, 14.7: keys rotate before they are stored).
//
// After the loop the waves merge in LDS into the split's partial (max, sum,
// O).  A sequence with one split applies the gate (Ch 9, 9.8) and stores the
// output; otherwise each split stores its partial and decode_merge_kernel,
// the next launch on the stream, merges the splits in split order.  Splits
// that would cover no row of a shorter sequence exit at once.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

// Profiling build only (-DMUSE_DECODE_TIMELINE, libmuse_attn_timeline.so):
// every split and merge workgroup records when it reaches each phase of its
// work (s_memrealtime, a 100 MHz clock common to the whole GPU), for
// muse_decode_timeline_read.  The stamps wait for what they name (the data
// of a phase, the completion of the final stores); nothing else changes.  In
// the regular build the macros are empty.
#ifdef MUSE_DECODE_TIMELINE
#include "muse_attn_timeline.h"
#define MUSE_TL_STAMP(var) const unsigned long long var = __builtin_amdgcn_s_memrealtime()
#define MUSE_TL_HOLD(...) asm volatile("" ::__VA_ARGS__)
#define MUSE_TL_DRAIN() __builtin_amdgcn_s_waitcnt(0)
#else
#define MUSE_TL_STAMP(var)
#define MUSE_TL_HOLD(...)
#define MUSE_TL_DRAIN()
#endif

namespace muse {

#ifdef MUSE_DECODE_TIMELINE
__device__ unsigned long long decode_tl_split[MUSE_TL_SPLIT_WORKGROUPS * MUSE_TL_SPLIT_SLOTS];
__device__ unsigned long long decode_tl_merge[MUSE_TL_MERGE_WORKGROUPS * MUSE_TL_MERGE_SLOTS];
#endif

template <typename T> struct DecodeTraits;
// bf16: K and V rows loaded alike, 4 rows x 256 B per load instruction (16
// lanes per row), staged in LDS; K is read back in the A-operand layout of
// the 16x16x32 MFMA
template <> struct DecodeTraits<bf16_t> {
    static constexpr int KREG = 4, VREG = 4;           // 16-byte loads of K (and V) per lane per sub-tile
    static constexpr int RPL = 4;                      // rows per load instruction
    static constexpr int LDV = kHeadDim + 16;          // V row stride in LDS (elements)
    static constexpr int LDKW = kHeadDim + 8;          // K row stride in LDS: b128 reads conflict-free
    static constexpr int LDQ = kHeadDim + 8;           // Q-hat row stride in LDS
};
// f32 (parity path): 2 rows x 512 B per load instruction
template <> struct DecodeTraits<float> {
    static constexpr int KREG = 8, VREG = 8;
    static constexpr int RPL = 2;
    static constexpr int LDV = kHeadDim + 4;
    static constexpr int LDKW = kHeadDim + 4;
    static constexpr int LDQ = kHeadDim + 4;
};

template <typename T>
struct SubTile {
    u32x4 k[DecodeTraits<T>::KREG];
    u32x4 v[DecodeTraits<T>::VREG];
};

// Buffer resource over `bytes` from `base` (raw, untyped dword access); a
// load beyond it returns zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t decode_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
constexpr int kNontemporal = 2;                        // nt cache policy of a buffer load

// Sum over each aligned group of 16 lanes (DPP within a row).  Every step
// adds a lane's value to its partner's, partners pairing up both ways (quad
// neighbours, then the two quads of each half row by row_half_mirror, then
// the two halves by row_mirror), so every lane of the group ends with the
// same bits.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
    return x;
}
// Sum over each aligned group of N lanes, N in {16, 32, 64}.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x = row16_sum(x);
    if constexpr (N >= 32) x = sum_rows16(x);
    if constexpr (N >= 64) x = sum_halves(x);
    return x;
}
// Maximum over the whole wave, by the same partner steps.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
    return max_halves(max_rows16(x));
}

template <typename T, int DEPTH, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_kernel(DecodeArgs a) {
    using Tr = DecodeTraits<T>;
    constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
    constexpr int D = kHeadDim, HG = kHeadsPerKv, SUB = 16;
    constexpr int LDV = Tr::LDV, LDKW = Tr::LDKW, LDQ = Tr::LDQ, RPL = Tr::RPL;
    constexpr int ES = (int)sizeof(T);
    constexpr int WAVE_V = SUB * LDV * ES, WAVE_K = SUB * LDKW * ES;
    constexpr int NT = 64 * NW;
    constexpr int LOOP_BYTES = NW * (WAVE_V + WAVE_K);
    constexpr int MERGE_BYTES = NW * HG * (D + 2) * 4;
    constexpr int LDS_BYTES = LOOP_BYTES > MERGE_BYTES ? LOOP_BYTES : MERGE_BYTES;
    static_assert(HG % NW == 0, "each wave normalises the same number of heads");
    // per-wave K and V buffers in the loop; the waves' partials after it
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    // Q-hat of the 16 heads (bf16: hi and lo parts; f32: the values)
    __shared__ __attribute__((aligned(16))) T qs_hi[HG * LDQ];
    __shared__ __attribute__((aligned(16))) T qs_lo[kBf16 ? HG * LDQ : 4];
    __shared__ float2 rot_all[NW][kHeadDim / 2];       // per-wave (cos, sin) of the 64 RoPE pairs

    // workgroup b takes pair b mod (2 n_seq) and split b / (2 n_seq): with
    // dispatch round-robin over the 8 XCDs, all splits of a pair share an
    // XCD when the pair count is a multiple of 8 (so does the pair's merge)
    MUSE_TL_STAMP(tl0);
    const int b = blockIdx.x;
    const int npair = 2 * a.n_seq;
    const int c = b / npair;
    const int sg = b % npair;
    const int s = sg >> 1, g = sg & 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int64_t obase = ((int64_t)s * kHeads + g * HG) * D;     // out/gate/q of head 16g

    // ---- loads that do not depend on the sequence's length go out first:
    // the lane's RoPE frequency (pair = lane) before Q, so that the (cos, sin)
    // table, which does not need Q, is made while Q is on its way.
    const float th = theta_of_lane<DecodeArgs>(lane);
    // This wave's share of the raw Q: HPW heads, LPH lanes per head, DPL
    // consecutive dims per lane.
    constexpr int HPW = HG / NW, LPH = 64 / HPW, DPL = D / LPH;
    constexpr int QREG = DPL * ES / 16 > 0 ? DPL * ES / 16 : 1;   // 16-byte loads of raw Q
    const int qh = wave * HPW + lane / LPH;            // head within the KV group
    const int qd0 = (lane % LPH) * DPL;                // its first dim
    u32x4 qraw[QREG];
    {
        const char* qp = (const char*)a.q + (obase + qh * D + qd0) * ES;
        if constexpr (DPL * ES == 8) {
            const uint2 q2 = *(const uint2*)qp;
            qraw[0] = u32x4{q2.x, q2.y, 0u, 0u};
        } else {
#pragma unroll
            for (int i = 0; i < QREG; ++i) qraw[i] = *(const u32x4*)(qp + 16 * i);
        }
    }
    // the new K and V rows in the chunk layout of a cache sub-tile (lane: the
    // 16-byte chunk nch of a row); only the split holding p uses them
    const int nch = kBf16 ? l16 : (lane & 31);
    const int64_t new_off = ((int64_t)s * kKvHeads + g) * D * ES + 16 * nch;
    const u32x4 kn_raw = *(const u32x4*)((const char*)a.k + new_off);
    const u32x4 vnew_c = *(const u32x4*)((const char*)a.v + new_off);
    // thread -> (head hh, DPT consecutive dims) after the loop
    constexpr int TPH = NT / HG, DPT = D / TPH;        // threads per head, dims per thread
    static_assert((TPH == 32 && DPT == 4) || (TPH == 16 && DPT == 8), "4 or 8 dims per thread");
    const int hh = tid / TPH, d0 = (tid % TPH) * DPT;
    constexpr int GREG = DPT * ES / 16 > 0 ? DPT * ES / 16 : 1;   // 16-byte loads of gate values
    u32x4 graw[GREG];
    auto load_gate = [&]() __attribute__((always_inline)) {
        const char* gp = (const char*)a.gate + (obase + hh * D + d0) * ES;
        if constexpr (DPT * ES == 8) {
            const uint2 g2 = *(const uint2*)gp;
            graw[0] = u32x4{g2.x, g2.y, 0u, 0u};
        } else {
#pragma unroll
            for (int i = 0; i < GREG; ++i) graw[i] = *(const u32x4*)(gp + 16 * i);
        }
    };
    // with one split per sequence this workgroup applies the gate (else the
    // merge kernel does, or a short sequence's only live split loads it late)
    if (a.nsplit == 1) load_gate();
    // The exits below use those loads too (an empty asm that takes them):
    // otherwise the compiler moves the loads past the exits, behind the wait
    // for seq_len, and the two round trips no longer overlap.
    auto hold_loads = [&]() __attribute__((always_inline)) {
        asm volatile("" :: "v"(qraw[0]), "v"(kn_raw), "v"(vnew_c), "v"(th));
    };
    const int L = a.seq_len[s];
    const int W = a.window;

    if (L < 0 || L > a.max_seq_len) {                  // refused on the device
        hold_loads();
        if (c == 0)
            for (int i = tid; i < HG * D; i += NT) ((T*)a.out)[obase + i] = from_f32<T>(__builtin_nanf(""));
        return;
    }
    // positions are below 2^24 (checked on the host): 32-bit arithmetic
    const int p = L;
    MUSE_TL_HOLD("s"(p));
    MUSE_TL_STAMP(tl1);
    const int lo = (W > 0) ? max(0, p - W + 1) : 0;
    const int cs = lo + c * a.chunk;
    if (cs > p) {                                      // split beyond this sequence's rows
        hold_loads();
        return;
    }
    const int ce = min(cs + a.chunk, p + 1);           // exclusive
    const int n_live = (p - lo) / a.chunk + 1;         // splits with rows
    const bool owns_p = (ce == p + 1);
    const int n_sub = (ce - cs + SUB - 1) / SUB;
    const int my_cnt = n_sub > wave ? (n_sub - wave + NW - 1) / NW : 0;  // sub-tiles wave, wave+NW, ...

    char* wave_lds = lds + wave * (WAVE_V + WAVE_K);
    T* Vw = (T*)wave_lds;
    T* Kw = (T*)(wave_lds + WAVE_V);

    auto gate_sig = [&](int x) __attribute__((always_inline)) {     // sigmoid of gate value d0 + x
        float gv;
        if constexpr (kBf16) {
            const unsigned w = graw[x / 8][(x % 8) / 2];
            gv = __uint_as_float((x % 2) ? (w & 0xffff0000u) : (w << 16));
        } else {
            gv = __uint_as_float(graw[x / 4][x % 4]);
        }
        return sigmoid(gv);
    };

    // ---- cache rows: one buffer resource over the split's rows (linear
    // cache: from row cs; ring: the whole ring, position j in row j % ring,
    // the split's positions wrapping at most once).  K and V share offsets.
    constexpr int ROW = kKvHeads * D * ES;             // bytes per position
    const bool ring = a.ring != 0;
    const int ringn = (int)a.ring;
    const int row_cs = ring ? cs % ringn : 0;
    const int64_t rbase = ring ? 0 : cs;
    const uint32_t extent = (uint32_t)(ring ? (int64_t)ringn * ROW : (int64_t)(ce - cs) * ROW);
    const int64_t base_off = ((int64_t)s * a.capacity + rbase) * ROW + (int64_t)g * D * ES;
    const __amdgpu_buffer_rsrc_t rs_k = decode_rsrc((const char*)a.cache_k + base_off, extent);
    const __amdgpu_buffer_rsrc_t rs_v = decode_rsrc((const char*)a.cache_v + base_off, extent);
    auto row_bytes = [&](int j) __attribute__((always_inline)) {  // offset of position j's row
        int r = j - cs;
        if (ring) {
            r += row_cs;
            r = r >= ringn ? r - ringn : r;
        }
        return (uint32_t)r * (uint32_t)ROW;
    };
    // ---- loads of one 16-row sub-tile.  Every lane always loads (a load
    // skipped by some waves would make the compiler wait for all of them):
    // rows past the split are clamped to its last row ce - 1, whose score is
    // masked to P = 0 later.
    const int rl = lane / (64 / RPL);                  // row of the lane within a load
    const uint32_t lane_col = 16u * (uint32_t)(lane % (64 / RPL));
    auto issue = [&](SubTile<T>& t, int k) __attribute__((always_inline)) {
        const int j0 = cs + SUB * (wave + NW * k);
#pragma unroll
        for (int u = 0; u < Tr::KREG; ++u) {
            const uint32_t off = row_bytes(min(j0 + RPL * u + rl, ce - 1)) + lane_col;
            t.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rs_k, off, 0, kNontemporal);
            t.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs_v, off, 0, kNontemporal);
        }
    };

    // pipeline stages as named variables (an indexed array of them ends up in scratch)
    static_assert(DEPTH >= 1 && DEPTH <= 4, "pipeline depth 1..4");
    SubTile<T> b0, b1, b2, b3;
    // The first DEPTH sub-tiles' loads go out as soon as the rows are known,
    // so that they are under way while Q-hat is made (sub-tiles past the
    // wave's share load clamped rows and are never processed).
    issue(b0, 0);
    if constexpr (DEPTH > 1) issue(b1, 1);
    if constexpr (DEPTH > 2) issue(b2, 2);
    if constexpr (DEPTH > 3) issue(b3, 3);

    // ---- (cos, sin) of the 64 pairs at position p in the wave's own table,
    // then Q-hat of the wave's HPW heads: RMS norm with gain, RoPE on sliding
    // layers ("Chapter 14 - QK-norm and RoPE" 14.3-14.5)
    MUSE_TL_HOLD("v"(qraw[0]));
    MUSE_TL_STAMP(tl2);
    float2* rot = rot_all[wave];
    if (a.rope) {
        float sn, cs_;
        sincos_rope((float)p * th, &sn, &cs_);
        rot[lane] = make_float2(cs_, sn);
    }
    auto rotate = [&](float& y0, float& y1, int pair) __attribute__((always_inline)) {
        const float2 cz = rot[pair];
        const float z0 = y0 * cz.x - y1 * cz.y;
        const float z1 = y0 * cz.y + y1 * cz.x;
        y0 = z0;
        y1 = z1;
    };
    auto elem = [](const u32x4* v, int t) __attribute__((always_inline)) {   // value t of a raw chunk run
        if constexpr (kBf16) {
            const unsigned w = v[t / 8][(t % 8) / 2];
            return __uint_as_float((t % 2) ? (w & 0xffff0000u) : (w << 16));
        } else {
            return __uint_as_float(v[t / 4][t % 4]);
        }
    };
    {
        float x[DPL];
        float ss = 0.0f;
#pragma unroll
        for (int t = 0; t < DPL; ++t) {
            x[t] = elem(qraw, t);
            ss += x[t] * x[t];
        }
        ss = group_sum<LPH>(ss);
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + a.eps);   // v_rsq_f32, ~1 ulp
#pragma unroll
        for (int t = 0; t < DPL; ++t) x[t] = (x[t] * r) * a.q_gain;
        if (a.rope) {
#pragma unroll
            for (int j = 0; j < DPL / 2; ++j) rotate(x[2 * j], x[2 * j + 1], qd0 / 2 + j);
        }
        T hv[DPL], lv[DPL];
#pragma unroll
        for (int t = 0; t < DPL; ++t) {
            hv[t] = from_f32<T>(x[t]);
            lv[t] = kBf16 ? from_f32<T>(x[t] - to_f32(hv[t])) : hv[t];
        }
        __builtin_memcpy(qs_hi + qh * LDQ + qd0, hv, sizeof hv);   // one vector store each
        if constexpr (kBf16) __builtin_memcpy(qs_lo + qh * LDQ + qd0, lv, sizeof lv);
    }
    __syncthreads();
    MUSE_TL_STAMP(tl3);
    constexpr int NSTQ = kBf16 ? 4 : 32;               // 16x16x32 bf16 / 16x16x4 f32 steps
    using MW = Mma16Wide<T>;
    using MN = Mma16Narrow<T>;
    // B operand of S^T = K Q^T: lane (head l16, k-group q4)
    typename MW::Frag qhi[NSTQ], qlo[kBf16 ? NSTQ : 1];
#pragma unroll
    for (int st = 0; st < NSTQ; ++st) {
        if constexpr (kBf16) {
            qhi[st] = *(const bf16x8*)(qs_hi + l16 * LDQ + 32 * st + 8 * q4);
            qlo[st] = *(const bf16x8*)(qs_lo + l16 * LDQ + 32 * st + 8 * q4);
        } else {
            qhi[st] = qs_hi[l16 * LDQ + 4 * st + q4];
        }
    }

    // the new K row as it is stored (K-hat rounded to the cache type), in the
    // lane's chunk; made by the wave whose sub-tile holds p, which also stores
    // both new rows to cache row p
    auto new_k_row = [&]() __attribute__((always_inline)) {
        constexpr int NV = 16 / ES;                    // values per chunk
        float x[NV];
#pragma unroll
        for (int t = 0; t < NV; ++t) x[t] = elem(&kn_raw, t);
        float ss = 0.0f;
#pragma unroll
        for (int t = 0; t < NV; ++t) ss += x[t] * x[t];
        ss = group_sum<kBf16 ? 16 : 32>(ss);           // the row's chunks
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + a.eps);   // v_rsq_f32, ~1 ulp
#pragma unroll
        for (int t = 0; t < NV; ++t) x[t] = (x[t] * r) * a.k_gain;
        if (a.rope) {
#pragma unroll
            for (int j = 0; j < NV / 2; ++j) rotate(x[2 * j], x[2 * j + 1], (NV / 2) * nch + j);
        }
        u32x4 kc;
        if constexpr (kBf16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned lo16 = __builtin_bit_cast(unsigned short, from_f32<bf16_t>(x[2 * j]));
                const unsigned hi16 = __builtin_bit_cast(unsigned short, from_f32<bf16_t>(x[2 * j + 1]));
                kc[j] = lo16 | (hi16 << 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) kc[j] = __float_as_uint(x[kBf16 ? 0 : j]);
        }
        return kc;
    };

    floatx4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{};
    float m_run = kNegInf, l_run = 0.0f;

    auto process = [&](SubTile<T>& t, int k) __attribute__((always_inline)) {
        const int j0 = cs + SUB * (wave + NW * k);
        if (owns_p && j0 + SUB > p) {                  // the sub-tile holding p (wave-uniform)
            asm volatile("");                          // keep this a branch
            const u32x4 knew_c = new_k_row();
            if (rl == 0) {                             // one copy of the row's chunks
                const int64_t row_off = (((int64_t)s * a.capacity + (ring ? p % ringn : p)) * kKvHeads + g) * D * ES +
                                        16 * nch;
                *(u32x4*)((char*)a.cache_k + row_off) = knew_c;
                *(u32x4*)((char*)a.cache_v + row_off) = vnew_c;
            }
#pragma unroll
            for (int u = 0; u < Tr::KREG; ++u) {
                if (min(j0 + RPL * u + rl, ce - 1) == p) {
                    t.k[u] = knew_c;
                    t.v[u] = vnew_c;
                }
            }
        }
        // ---- scores S^T[key j0 + 4*q4 + i][head l16]
        floatx4 sc = floatx4{};
        if constexpr (kBf16) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * u + q4;
                *(u32x4*)(Kw + r * LDKW + l16 * 8) = t.k[u];
                *(u32x4*)(Vw + r * LDV + l16 * 8) = t.v[u];
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
                *(u32x4*)(Kw + r * LDKW + (lane & 31) * 4) = t.k[u];
                *(u32x4*)(Vw + r * LDV + (lane & 31) * 4) = t.v[u];
            }
#pragma unroll
            for (int st = 0; st < NSTQ; ++st) sc = MW::mma(Kw[l16 * LDKW + 4 * st + q4], qhi[st], sc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] *= a.scale_log2;
        if (j0 + SUB > ce) {                           // the split's last, partial sub-tile
            asm volatile("");
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (j0 + 4 * q4 + i >= ce) sc[i] = kNegInf;
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mx = max_halves(max_rows16(mx));               // lanes ^ 16 and ^ 32 hold the head's other keys
        if (__ballot(mx > m_run) != 0) {               // some row's maximum grows: rescale
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first sub-tile
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
            m_run = m_new;
        }
        float rs = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = fast_exp2(sc[i] - m_run);
            rs += sc[i];
        }
        l_run += rs;

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
    if (my_cnt <= DEPTH) {                             // every sub-tile of the wave is in flight already
        if (my_cnt > 0) process(b0, 0);
        if constexpr (DEPTH > 1) if (my_cnt > 1) process(b1, 1);
        if constexpr (DEPTH > 2) if (my_cnt > 2) process(b2, 2);
        if constexpr (DEPTH > 3) if (my_cnt > 3) process(b3, 3);
    } else {
        for (int k0 = 0; k0 < my_cnt; k0 += DEPTH) {
            stage(b0, k0);
            if constexpr (DEPTH > 1) stage(b1, k0 + 1);
            if constexpr (DEPTH > 2) stage(b2, k0 + 2);
            if constexpr (DEPTH > 3) stage(b3, k0 + 3);
        }
    }

    // ---- merge the waves: LDS holds per wave [16 heads][128 + 2] floats
    MUSE_TL_HOLD("v"(o[0]), "v"(o[D / 16 - 1]));
    MUSE_TL_STAMP(tl4);
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
    // this split's partial for (head hh, dim d) from the waves' rows in LDS
    // (a wave without sub-tiles holds m = -inf, l = 0, O = 0)
    float own_m = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) own_m = fmaxf(own_m, mg[(w * HG + hh) * (D + 2) + D]);
    float own_l = 0.0f, own_o[DPT];
#pragma unroll
    for (int x = 0; x < DPT; ++x) own_o[x] = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float* row = mg + (w * HG + hh) * (D + 2);
        const float e = (row[D] == kNegInf) ? 0.0f : fast_exp2(row[D] - own_m);
        own_l += row[D + 1] * e;
#pragma unroll
        for (int x = 0; x < DPT; ++x) own_o[x] += row[d0 + x] * e;
    }
    MUSE_TL_HOLD("v"(own_l), "v"(own_o[0]));
    MUSE_TL_STAMP(tl5);
#ifdef MUSE_DECODE_TIMELINE
    auto tl_record = [&]() __attribute__((always_inline)) {
        MUSE_TL_DRAIN();
        MUSE_TL_STAMP(tl6);
        if (tid == 0 && b < MUSE_TL_SPLIT_WORKGROUPS) {
            unsigned long long* d = decode_tl_split + (size_t)b * MUSE_TL_SPLIT_SLOTS;
            d[0] = tl0; d[1] = tl1; d[2] = tl2; d[3] = tl3; d[4] = tl4; d[5] = tl5; d[6] = tl6;
            d[7] = (unsigned long long)my_cnt;
        }
    };
#endif
    if (n_live == 1) {                                 // the only split: finish here
        if (a.nsplit > 1) load_gate();                 // a short sequence of a split call
        T* out = (T*)a.out + obase;
        const float inv = 1.0f / own_l;
#pragma unroll
        for (int x = 0; x < DPT; ++x) out[hh * D + d0 + x] = from_f32<T>(own_o[x] * inv * gate_sig(x));
#ifdef MUSE_DECODE_TIMELINE
        tl_record();
#endif
        return;
    }
    // ---- several splits: store this split's partial (m, l, O) for the merge
    // kernel that follows in stream order (the kernel boundary orders these
    // plain stores before its reads)
    const int64_t head_row = ((int64_t)s * kHeads + g * HG + hh) * a.nsplit + c;   // (head, split)
#pragma unroll
    for (int x = 0; x < DPT; x += 4)
        *(floatx4*)(a.part_o + head_row * D + d0 + x) = floatx4{own_o[x], own_o[x + 1], own_o[x + 2], own_o[x + 3]};
    if (d0 == 0) {
        a.part_m[head_row] = own_m;
        a.part_l[head_row] = own_l;
    }
#ifdef MUSE_DECODE_TIMELINE
    tl_record();
#endif
}

// ---- the merge of the split partials: one wave per (sequence, query head)
// and workgroup.  Lane (h, q) = (lane / 32, lane % 32) holds dims
// 4q .. 4q + 3 of the splits j with j % 2 == h, so one 16-byte load per lane
// and split pair brings in 32 splits' O rows at once.  With M the largest
// partial maximum, split j weighs w_j = 2^(m_j - M); the output is
// sum_j w_j O_j / sum_j w_j l_j, times sigma(gate) ("Chapter 9 - The Muse
// Glimmer architecture" 9.8): the softmax over the union of the splits' keys,
// an exact reformulation.  Every load (the partials of the first 32 slots,
// the gate, seq_len) goes out at once, so up to 32 splits cost one memory
// round trip; slots at or past the sequence's live splits are read but not
// used.  Lane j holds split j's (m, l) (and j + 64, ...); the reductions leave
// the same bits in every lane, each half adds its O rows in split order and
// the two halves are then added, so the result does not depend on how the
// split workgroups were scheduled.
constexpr int kMergeWaves = 1;                         // heads per merge workgroup (one wave: its loads use a CU of their own)
constexpr int kMergeBatch = 16;                        // O rows in flight per lane: 32 splits per round trip
template <typename T>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(DecodeArgs a) {
    MUSE_TL_STAMP(tm0);
    constexpr int D = kHeadDim, B = kMergeBatch, R = kMaxSplits / 64;
    static_assert(kMaxSplits % 64 == 0 && kHeads % kMergeWaves == 0, "whole lanes and workgroups");
    static_assert(D == 4 * 32, "32 lanes of 4 dims cover a head");
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, dq = 4 * (lane & 31);
    // workgroup b takes head q (of the pair's 16) of pair b mod (2 n_seq), q = b / (2 n_seq)
    // (the XCD of that pair's splits)
    const int npair = 2 * a.n_seq;
    const int mpair = blockIdx.x % npair, mq = blockIdx.x / npair;
    const int sh = (mpair >> 1) * kHeads + (mpair & 1) * kHeadsPerKv + kMergeWaves * mq + (threadIdx.x >> 6);   // (sequence, head)
    const int s = sh / kHeads;
    const int nsplit = a.nsplit;
    const int64_t row0 = (int64_t)sh * nsplit;
    const float* po = a.part_o + row0 * D + dq;
    // (m, l) of slots lane, lane + 64, ...
    float mj[R], lj[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = lane + 64 * r;
        mj[r] = j < nsplit ? a.part_m[row0 + j] : kNegInf;
        lj[r] = j < nsplit ? a.part_l[row0 + j] : 0.0f;
    }
    // the O rows of slots h, h + 2, ..., h + 2 (B - 1)
    floatx4 ov[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
        const int j = 2 * i + h;
        ov[i] = j < nsplit ? *(const floatx4*)(po + (int64_t)j * D) : floatx4{};
    }
    const int64_t obase = (int64_t)sh * D + dq;
    float gv[4];
    if constexpr (std::is_same<T, bf16_t>::value) {
        const uint2 w = *(const uint2*)((const bf16_t*)a.gate + obase);
        gv[0] = __uint_as_float(w.x << 16);
        gv[1] = __uint_as_float(w.x & 0xffff0000u);
        gv[2] = __uint_as_float(w.y << 16);
        gv[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
        const floatx4 g4 = *(const floatx4*)((const float*)a.gate + obase);
#pragma unroll
        for (int x = 0; x < 4; ++x) gv[x] = g4[x];
    }
    const int L = a.seq_len[s];
    T* out = (T*)a.out + obase;
    auto store4 = [&](const float (&v)[4]) __attribute__((always_inline)) {   // dims dq .. dq + 3, from half 0
        if (h != 0) return;
        if constexpr (std::is_same<T, bf16_t>::value) {
            unsigned w[2];
#pragma unroll
            for (int x = 0; x < 2; ++x)
                w[x] = (unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(v[2 * x])) |
                       ((unsigned)__builtin_bit_cast(unsigned short, from_f32<bf16_t>(v[2 * x + 1])) << 16);
            *(uint2*)out = make_uint2(w[0], w[1]);
        } else {
            *(floatx4*)out = floatx4{v[0], v[1], v[2], v[3]};
        }
    };
    if (L < 0 || L > a.max_seq_len) {                  // refused on the device
        const float nan = __builtin_nanf("");
        store4({nan, nan, nan, nan});
        return;
    }
    const int lo = (a.window > 0) ? max(0, L - a.window + 1) : 0;
    const int n = (L - lo) / a.chunk + 1;              // live splits
    if (n == 1) return;                                // that split stored the output itself
    float M = kNegInf;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (lane + 64 * r < n) M = fmaxf(M, mj[r]);
    M = wave_max(M);
    MUSE_TL_HOLD("v"(ov[0]), "v"(ov[B - 1]), "v"(M));
    MUSE_TL_STAMP(tm1);
    float wj[R], den = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {                      // slots past n hold stale bytes: selected out, not weighted
        const bool live = lane + 64 * r < n;
        wj[r] = live ? fast_exp2(mj[r] - M) : 0.0f;
        den += live ? lj[r] * wj[r] : 0.0f;
    }
    den = group_sum<64>(den);
    floatx4 acc = floatx4{};
    for (int jb = 0; jb < n; jb += 2 * B) {
        if (jb > 0) {                                  // later batches
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const int j = jb + 2 * i + h;
                ov[i] = j < nsplit ? *(const floatx4*)(po + (int64_t)j * D) : floatx4{};
            }
        }
        // the batch's 32 weights sit in lanes jb % 64 .. jb % 64 + 31 of wj[jb / 64]
        float wb = wj[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
            if (jb / 64 == r) wb = wj[r];
        const int lb = jb % 64;
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int j0 = jb + 2 * i;                 // the pair's even split (wave-uniform)
            if (j0 < n) {
                const float we = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wb), lb + 2 * i));
                const float wo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wb), lb + 2 * i + 1));
                const bool live = j0 + h < n;          // split j0 + 1 may be past the live ones
                const floatx4 c = ov[i] * (h ? wo : we);
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[x] += live ? c[x] : 0.0f;
            }
        }
    }
    const float inv = 1.0f / den;
    float res[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) res[x] = sum_halves(acc[x]) * inv * sigmoid(gv[x]);
    store4(res);
#ifdef MUSE_DECODE_TIMELINE
    MUSE_TL_DRAIN();
    MUSE_TL_STAMP(tm2);
    if (threadIdx.x == 0 && blockIdx.x < MUSE_TL_MERGE_WORKGROUPS) {
        unsigned long long* d = decode_tl_merge + (size_t)blockIdx.x * MUSE_TL_MERGE_SLOTS;
        d[0] = tm0; d[1] = tm1; d[2] = tm2; d[3] = (unsigned long long)n;
    }
#endif
}

// The allocation-free decode's scratch: split partials in a file-scope
// device array (each GPU the library runs on holds its own copy until the
// process ends).  Host code never passes `scratch` itself to a kernel (on the
// host the name is only a stand-in): its device address is resolved once per
// device with hipGetSymbolAddress and that address is used.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {                            // first call on this device, which is current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

#ifdef MUSE_DECODE_TIMELINE
static hipError_t decode_timeline_read(uint64_t* split, size_t split_count, uint64_t* merge, size_t merge_count,
                                int32_t clear) {
    const size_t ns = (size_t)MUSE_TL_SPLIT_WORKGROUPS * MUSE_TL_SPLIT_SLOTS;
    const size_t nm = (size_t)MUSE_TL_MERGE_WORKGROUPS * MUSE_TL_MERGE_SLOTS;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess && split)
        e = hipMemcpyFromSymbol(split, HIP_SYMBOL(decode_tl_split), (split_count < ns ? split_count : ns) * 8, 0,
                                hipMemcpyDeviceToHost);
    if (e == hipSuccess && merge)
        e = hipMemcpyFromSymbol(merge, HIP_SYMBOL(decode_tl_merge), (merge_count < nm ? merge_count : nm) * 8, 0,
                                hipMemcpyDeviceToHost);
    if (e == hipSuccess && clear) {
        void* ps = nullptr;
        void* pm = nullptr;
        e = hipGetSymbolAddress(&ps, HIP_SYMBOL(decode_tl_split));
        if (e == hipSuccess) e = hipGetSymbolAddress(&pm, HIP_SYMBOL(decode_tl_merge));
        if (e == hipSuccess) e = hipMemset(ps, 0, ns * 8);
        if (e == hipSuccess) e = hipMemset(pm, 0, nm * 8);
        if (e == hipSuccess) e = hipDeviceSynchronize();
    }
    return e;
}
#endif

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kKvHeads * a.nsplit)), block(64 * kDecodeWaves);
    if (dtype == 1)
        hipLaunchKernelGGL((decode_kernel<bf16_t, kDecodeDepth, kDecodeWaves>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<float, 2, kDecodeWaves>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kHeads / kMergeWaves)), block(64 * kMergeWaves);
    if (dtype == 1)
        hipLaunchKernelGGL(decode_merge_kernel<bf16_t>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(decode_merge_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse

#ifdef MUSE_DECODE_TIMELINE
extern "C" int muse_decode_timeline_read(uint64_t* split_host, size_t split_count, uint64_t* merge_host,
                                         size_t merge_count, int32_t clear) {
    return muse::decode_timeline_read(split_host, split_count, merge_host, merge_count, clear) == hipSuccess ? 0 : 7;
}
#endif
