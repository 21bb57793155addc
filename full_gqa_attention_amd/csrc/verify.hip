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
// fp16 while staged (no prefix copy for a handful of queries); DEP tiles of
// loads wait in registers ahead of the tile in use.  The softmax takes a
// fixed per-row reference (no running maximum, no O rescale), with an exact
// recomputation if that overflows.  Each split writes (reference, sum, O)
// per row; a second kernel merges the splits in fixed order and applies the
// gate.
//
// The new rows' Q-hat is made here from the raw Q (QK-norm with gain, RoPE on
// sliding layers at the row's position; "Chapter 14 - QK-norm and RoPE"
// 14.3-14.5); the prep kernel has already appended the new K-hat and V.
#include "device_common.h"
#include "kernels.h"

namespace muse {

template <int DEP>
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

    // workgroup b takes pair b mod (2 n_seq) and split b / (2 n_seq): with
    // dispatch round-robin over the 8 XCDs, all splits of a pair share an
    // XCD when the pair count is a multiple of 8 (so do the pair's merges)
    const int b = blockIdx.x;
    const int npair = 2 * a.n_seq;
    const int c = b / npair;
    const int sg = b % npair;
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
        const float th = theta_of_lane<VerifyArgs>(lane);
        for (int tt = wave; tt < kVerifyTokens; tt += NT / 64) {
            float sn, cs;
            sincos_rope((float)(L + tt) * th, &sn, &cs);
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
    // later, like every key outside a row's window).  Tile k of the split
    // waits in register slot k % DEP, DEP tiles ahead of the one in use.
    // Each cached row is read by one workgroup: nontemporal loads.
    const int r_t = tid / CPR, c_t = tid % CPR;
    constexpr int64_t ROW = (int64_t)kKvHeads * D * ES;
    const char* kbase = (const char*)a.cache_k + (((int64_t)s * a.capacity) * kKvHeads + g) * D * ES + c_t * 16;
    const char* vbase = (const char*)a.cache_v + (((int64_t)s * a.capacity) * kKvHeads + g) * D * ES + c_t * 16;
    u32x4 kr[DEP], vr[DEP];
    auto load = [&](int slot, int k) __attribute__((always_inline)) {
        const int64_t off = (int64_t)min(min(tile_first + k, tile_last) * BN + r_t, hi - 1) * ROW;
        kr[slot] = __builtin_nontemporal_load((const u32x4*)(kbase + off));
        vr[slot] = __builtin_nontemporal_load((const u32x4*)(vbase + off));
    };
    auto store = [&](int slot, int bufi, bool with_v) __attribute__((always_inline)) {
        *(u32x4*)((char*)Ks[bufi] + (r_t * LDK + c_t * 8) * 2) = k_chunk_to_score(kr[slot], T{});
        if (with_v) *(u32x4*)((char*)Vs[bufi] + (r_t * LDV + c_t * 8) * 2) = vr[slot];
    };

    // ---- softmax reference.  Each row's reference is fixed at the maximum of
    // the first tile of the split in which it sees a key and then never
    // moves, so the tile loop keeps no running maximum and rescales nothing:
    // P = exp2(s - ref) may exceed 1, and softmax does not depend on the
    // reference.  The Q.K MFMAs start from -ref.  The one failure, an
    // overflow of P, l or O to inf, is checked at the end; then the split is
    // computed again with each row's exact maximum from a Q.K-only sweep.
    const unsigned wlim = W > 0 ? (unsigned)W : 0x7fffffffu;
    const int P0 = L, P1 = L + kVerifyTokens - 1;      // lowest and highest row position
    auto apply_mask = [&](floatx16& sc, int j0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {                 // item i: key j0 + 8 (i / 4) + 4 gl + i % 4
            const int j = j0 + 8 * (i / 4) + 4 * gl + (i % 4);
            sc[i] = ((unsigned)(p - j) < wlim) ? sc[i] : kNegInf;
        }
    };
    auto row_max = [&](const floatx16& v) __attribute__((always_inline)) {
        float m4[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int i = 4; i < 16; ++i) m4[i % 4] = fmaxf(m4[i % 4], v[i]);
        return max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    };
    auto qk = [&](const TQ* Kc, floatx16 init) __attribute__((always_inline)) {
        floatx16 sc = init;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const FragQ kf = *(const FragQ*)(Kc + l32 * LDK + 2 * MQ::KPL * st + MQ::KPL * gl);
            sc = MQ::mma(kf, qf[st], sc);
        }
        return sc;
    };
    float ref = kNegInf;
    floatx16 nref = floatx16{};                        // -ref broadcast (0 while unset)
    floatx16 o[4];
    float l_run = 0.0f;

    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            // exact row maxima: Q.K over the same tiles, no P.V
            float mx = kNegInf;
            load(0, 0);
            store(0, 0, false);
            __syncthreads();
            for (int it = 0; it < ntiles; ++it) {
                load(0, it + 1);                       // past the end: a harmless repeat
                floatx16 sc = qk(Ks[it & 1], floatx16{});
                apply_mask(sc, (tile_first + it) * BN);
                mx = fmaxf(mx, row_max(sc));
                store(0, (it + 1) & 1, false);
                __syncthreads();
            }
            ref = mx;
#pragma unroll
            for (int i = 0; i < 16; ++i) nref[i] = ref == kNegInf ? 0.0f : -ref;
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = floatx16{};
        l_run = 0.0f;

        if (ntiles > 0) {
#pragma unroll
            for (int d = 0; d < DEP; ++d) load(d, d);
            store(0, 0, true);
            load(0, DEP);
            __syncthreads();
        }
        // one tile: S^T = K Q^T (from -ref), mask on boundary tiles, P = exp2,
        // l and O^T += V^T P^T; stages tile it + 1 (slot sn) and refills the slot
        auto step = [&](int it, int sn) __attribute__((always_inline)) {
            const int cur = it & 1;
            const int j0 = (tile_first + it) * BN;
            floatx16 sc = qk(Ks[cur], nref);
            store(sn, cur ^ 1, true);                  // that buffer is free since the last barrier
            load(sn, it + 1 + DEP);
            if ((j0 + BN - 1 > P0) || (W > 0 && P1 - j0 >= W)) {   // uniform over the workgroup
                asm volatile("");                      // keep this a branch
                apply_mask(sc, j0);
            }
            if (__ballot(ref == kNegInf) != 0) {       // rows still without a reference
                asm volatile("");
                const bool unset = ref == kNegInf;
                const float m = row_max(sc);
                if (unset && m > kNegInf) ref = m;
                const float r = (unset && ref != kNegInf) ? ref : 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sc[i] -= r;
                    nref[i] = ref == kNegInf ? 0.0f : -ref;
                }
            }
            const T* Vc = Vs[cur];
#pragma unroll
            for (int st = 0; st < 2; ++st) {           // 16 keys per K-step
                FragP pf;
#pragma unroll
                for (int j = 0; j < MP::KPL; ++j) frag_set(pf, j, fast_exp2(sc[8 * st + j]));
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
        };
        // whole groups of DEP tiles, then the rest: an early exit inside the
        // loop body would join the loop's back edge, and the compiler would
        // then wait for every load in flight at the top of each group
        int it0 = 0;
        for (; it0 + DEP <= ntiles; it0 += DEP) {
#pragma unroll
            for (int u = 0; u < DEP; ++u) step(it0 + u, (u + 1) % DEP);
        }
#pragma unroll
        for (int u = 0; u < DEP - 1; ++u) {
            if (it0 + u >= ntiles) break;
            step(it0 + u, (u + 1) % DEP);
        }

        // Drain the loads still in flight (repeats of the last tile).  Without
        // this the compiler, joining this point to the next pass's loop head,
        // takes the tail's loads for the newest ones there and waits for all
        // loads at the top of every group of tiles.
        __builtin_amdgcn_s_waitcnt(0x0f70);            // vmcnt(0)
        // an overflow anywhere shows up as a non-finite l or O
        float chk = l_run;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) chk += o[dt][i];
        if (!__syncthreads_or(!__builtin_isfinite(chk))) break;
    }

    // ---- this split's partial of the row: (ref, l, O) with O and l relative
    // to exp2(s - ref); O^T item i of lane l is dim 32 dt + 8 (i / 4) + 4 gl + i % 4
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
        a.part_m[pr] = ref;
        a.part_l[pr] = l_tot;
    }
}

// Merge the splits of each (sequence, token, head) row in split order and
// apply the gate.  A workgroup takes one (sequence, token, KV head): 16 heads
// x 16 threads, 8 dims per thread, so the gate reads and output stores of a
// workgroup are one contiguous 4 KB run.  The splits are read MC at a time,
// every load of a group issued before any is used (one memory round trip
// when nsplit <= MC); groups combine with a running reference.
template <int MC>
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyArgs a) {
    const int tid = threadIdx.x, hg = tid >> 4, dq = tid & 15;
    const int blk = blockIdx.x;                        // t * (2 n_seq) + 2 s + g: the XCD of the pair's splits
    const int npair = 2 * a.n_seq;
    const int N = a.n_new;
    const int g = (blk % npair) & 1, s = (blk % npair) >> 1, t = blk / npair;
    const int st = s * N + t;
    const int h = g * kHeadsPerKv + hg;
    const int64_t obase = ((int64_t)st * kHeads + h) * kHeadDim + 8 * dq;
    const u32x4 graw = *(const u32x4*)((const bf16_t*)a.gate + obase);
    const int L = a.seq_len[s];
    u32x4* dst = (u32x4*)((bf16_t*)a.out + obase);
    if (L < 0 || L > a.max_seq_len) {
        bf16x8 nan8;
#pragma unroll
        for (int x = 0; x < 8; ++x) nan8[x] = from_f32<bf16_t>(__builtin_nanf(""));
        *dst = __builtin_bit_cast(u32x4, nan8);
        return;
    }
    const int64_t row0 = (((int64_t)(s * kKvHeads + g) * a.nsplit) * kHeadsPerKv + hg) * kVerifyTokens + t;
    constexpr int64_t CSTRIDE = (int64_t)kHeadsPerKv * kVerifyTokens;   // partial rows between splits
    // Each split's (m, l) holds l = sum of exp2(s - m) over its keys, so
    // m + log2(l) is the log2 of its total weight.  The largest of those is
    // the reference, which keeps every scaled l at most 1 (a split's m is
    // its reference, not its maximum).
    float M = kNegInf, den = 0.0f, acc[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = 0.0f;
    for (int c0 = 0; c0 < a.nsplit; c0 += MC) {
        float mv[MC], lv[MC];
        floatx4 ov[MC][2];
#pragma unroll
        for (int c = 0; c < MC; ++c) {
            const int64_t r = row0 + (int64_t)min(c0 + c, a.nsplit - 1) * CSTRIDE;
            mv[c] = a.part_m[r];
            lv[c] = a.part_l[r];
            ov[c][0] = *(const floatx4*)(a.part_o + r * kHeadDim + 8 * dq);
            ov[c][1] = *(const floatx4*)(a.part_o + r * kHeadDim + 8 * dq + 4);
        }
        float mc = kNegInf;
#pragma unroll
        for (int c = 0; c < MC; ++c)
            if (c0 + c < a.nsplit && mv[c] != kNegInf) mc = fmaxf(mc, mv[c] + log2f(lv[c]));
        const float mn = fmaxf(M, mc);
        if (mn == kNegInf) continue;                   // no visible key yet
        const float rs = M == kNegInf ? 0.0f : fast_exp2(M - mn);
        den *= rs;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] *= rs;
#pragma unroll
        for (int c = 0; c < MC; ++c) {
            if (c0 + c >= a.nsplit || mv[c] == kNegInf) continue;   // a split with no visible key for this row
            const float e = fast_exp2(mv[c] - mn);
            den += lv[c] * e;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                acc[x] += ov[c][0][x] * e;
                acc[4 + x] += ov[c][1][x] * e;
            }
        }
        M = mn;
    }
    const float inv = 1.0f / den;                      // a row always sees its own key: den > 0
    const bf16x8 gv = __builtin_bit_cast(bf16x8, graw);
    bf16x8 y;
#pragma unroll
    for (int x = 0; x < 8; ++x) y[x] = from_f32<bf16_t>(acc[x] * inv * sigmoid((float)gv[x]));
    *dst = __builtin_bit_cast(u32x4, y);
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * kKvHeads * a.nsplit)), block(512);
    hipLaunchKernelGGL(verify_kernel<kVerifyDepth>, grid, block, 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipSuccess;
}

hipError_t launch_verify_merge(const VerifyArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.n_seq * a.n_new * kKvHeads)), block(256);
    if (a.nsplit <= 2)
        hipLaunchKernelGGL(verify_merge_kernel<2>, grid, block, 0, stream, a);
    else if (a.nsplit <= 4)
        hipLaunchKernelGGL(verify_merge_kernel<4>, grid, block, 0, stream, a);
    else if (a.nsplit <= 8)
        hipLaunchKernelGGL(verify_merge_kernel<8>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(verify_merge_kernel<16>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
