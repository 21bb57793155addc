// prefill.hip -- kernel (b): causal / sliding-window GQA attention over the
// KV cache for a chunk of new tokens, with the sigmoid gate fused into the
// epilogue.  Flash-style: the score matrix is never stored; softmax is online
// in the log2 domain (Q-hat arrives pre-multiplied by attn_scale * log2 e).
//
// Math (pages cited by title and section):
//   key j is visible to the query at position p iff j <= p and, on sliding
//   layers, p - j < window ("Chapter 9 - The Muse Glimmer architecture" 9.7);
//   query head h reads KV head h / 16 (Ch 9, Figure 9.3); score = q.k *
//   attn_scale (Ch 9, 9.5); out = softmax-weighted V times sigma(gate)
//   (Ch 9, 9.8).
//
// Two kernels share the scheme below.  prefill_kernel (f32 layers): one
// workgroup = 128 query rows of one head (4 waves x 32 rows), 64-key tiles,
// online softmax whose reference moves lazily.  prefill_group_kernel (bf16
// layers, further down): one workgroup = 8 heads of one KV group over the same
// 32 query rows, 32-key tiles, a fixed per-row softmax reference.
//
// Each wave computes S^T = K Q^T on 32x32 MFMA tiles (fp16 32x32x16 on bf16
// layers, reading the fp16 key copy the prep kernel made; f32 32x32x2 on f32
// layers), so a lane holds one query's scores: the row max and sum need one
// exchange with lane l ^ 32 only.  P.V is computed as O^T = V^T P^T: the
// score registers are the B operand as they are (the key order inside a
// K-step is permuted identically in P and V), and the V^T A operand comes
// from the transposing LDS load (ds_read_b64_tr_b16), two per MFMA.
// K/V tiles are double-buffered in LDS with the next tile's loads in flight
// during the compute (one barrier per tile).  Window-aware tile skipping:
// only tiles intersecting [p_lo - W + 1, p_hi] are visited; masks are applied
// only on tiles that straddle a boundary.  Workgroups are numbered so that the
// 16 heads sharing one KV head and one query block land on the same XCD
// (round-robin dispatch over 8 XCDs), so their K/V tiles are served by that
// XCD's L2; heavy (late) query blocks are dispatched first.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

// bf16 layers: 32-row query groups per wave, waves (heads of one KV group)
// per workgroup, 32-key halves per K/V tile
constexpr int kGroupQG = 1, kGroupWPB = 8, kGroupKT = 1;

namespace muse {

int prefill_grid(int n_seq, int n_new) {
    const int nqb = (n_new + kPrefillBM - 1) / kPrefillBM;
    const int units = n_seq * kKvHeads * nqb;          // (q-block, seq, kv head)
    return ((units + 7) / 8) * 8 * kHeadsPerKv;
}

template <typename T> struct PrefillTraits;
template <> struct PrefillTraits<bf16_t> {
    static constexpr int LDK = kHeadDim + 8;           // 272-byte K rows: b128 reads conflict-free
    static constexpr int LDV = kHeadDim + 32;          // 320-byte V rows: transposing reads conflict-free
    static constexpr int WAVES = 2;
};
template <> struct PrefillTraits<float> {
    static constexpr int LDK = kHeadDim + 4;
    static constexpr int LDV = kHeadDim + 4;
    static constexpr int WAVES = 1;
};

template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PrefillTraits<T>::WAVES)))
void prefill_kernel(AttnArgs a) {
    typedef typename ScoreType<T>::type TQ;         // Q.K^T operand type
    constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
    using MQ = Mma32<TQ>;
    using MP = Mma32<T>;                               // P.V in the storage type
    using FragQ = typename MQ::Frag;
    using FragP = typename MP::Frag;
    constexpr int KPLQ = MQ::KPL, KPLP = MP::KPL;
    constexpr int BM = kPrefillBM, BN = kPrefillBN, D = kHeadDim;
    constexpr int LDK = PrefillTraits<T>::LDK, LDV = PrefillTraits<T>::LDV;
    constexpr int NST = D / (2 * KPLQ);                // K-steps of Q.K
    constexpr int NSTP = BN / (2 * KPLP);              // K-steps of P.V
    constexpr int ES = (int)sizeof(T);
    static_assert(sizeof(TQ) == sizeof(T), "K staging keeps the row size");
    constexpr int CPR = D * ES / 16;                   // 16-byte chunks per row
    constexpr int NCH = BN * CPR / 256;                // chunks per thread per tile
    __shared__ __attribute__((aligned(16))) TQ Ks[2][BN * LDK];
    __shared__ __attribute__((aligned(16))) T Vs[2][BN * LDV];

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

    // positions fit in int32 (the host bounds them by 2^24)
    const int tq = q0 + wave * 32 + l32;               // this lane's query (new-token index)
    const int pq = L + tq;                             // its position
    const int tw0 = q0 + wave * 32;
    const int tw1 = min(tw0 + 31, N - 1);
    const bool wave_live = tw0 < N;
    const int pw0 = L + tw0, pw1 = L + tw1;
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
    const int P0 = L + q0, P1 = L + tb1;
    const int kv_lo = (W > 0) ? max(0, P0 - W + 1) : 0;
    const int kv_end = L + N;                          // rows present in the cache
    const int tile_lo = kv_lo / BN, tile_hi = P1 / BN;
    const int ntiles = tile_hi - tile_lo + 1;

    constexpr int64_t ROW = (int64_t)kKvHeads * D * ES;   // bytes per position
    constexpr int RSTEP = 256 / CPR;                       // tile rows per chunk step
    // this thread's chunk: row tid / CPR (+ RSTEP * u), 16-byte column tid % CPR
    const int r_t = tid / CPR, c_t = tid % CPR;
    const char* kbase = (const char*)a.kq + (((int64_t)s * a.kq_capacity) * kKvHeads + g) * D * ES +
                        r_t * ROW + c_t * 16;
    const char* vbase = (const char*)a.cache_v + (((int64_t)s * a.capacity) * kKvHeads + g) * D * ES +
                        r_t * ROW + c_t * 16;
    u32x4 kreg[NCH], vreg[NCH];
    auto load_tile = [&](int tile) __attribute__((always_inline)) {
        const int j0 = tile * BN;
        const char* kp = kbase + (int64_t)j0 * ROW;
        const char* vp = vbase + (int64_t)j0 * ROW;
        if (j0 >= kv_lo && j0 + BN <= kv_end) {           // interior tile: every row present
#pragma unroll
            for (int u = 0; u < NCH; ++u) {
                kreg[u] = *(const u32x4*)(kp + u * RSTEP * ROW);
                vreg[u] = *(const u32x4*)(vp + u * RSTEP * ROW);
            }
        } else {
            asm volatile("");                              // keep this a branch
#pragma unroll
            for (int u = 0; u < NCH; ++u) {
                const int jj = j0 + r_t + u * RSTEP;
                const bool in = jj >= kv_lo && jj < kv_end;
                kreg[u] = in ? *(const u32x4*)(kp + u * RSTEP * ROW) : u32x4{0, 0, 0, 0};
                vreg[u] = in ? *(const u32x4*)(vp + u * RSTEP * ROW) : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int bufi) __attribute__((always_inline)) {
        char* kd = (char*)Ks[bufi] + r_t * LDK * ES + c_t * 16;
        char* vd = (char*)Vs[bufi] + r_t * LDV * ES + c_t * 16;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            *(u32x4*)(kd + u * RSTEP * LDK * ES) = kreg[u];
            *(u32x4*)(vd + u * RSTEP * LDV * ES) = vreg[u];
        }
    };

    floatx16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = floatx16{};
    float m_run = kNegInf, l_run = 0.0f;

    load_tile(tile_lo);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        const int j0 = (tile_lo + it) * BN;
        if (it + 1 < ntiles) load_tile(tile_lo + it + 1);   // in flight during the compute
        const bool any = wave_live && (j0 <= pw1) && (W == 0 || pw0 - (j0 + BN - 1) < W);
        if (any) {
            const bool need_mask = (j0 + BN - 1 > pw0) || (W > 0 && pw1 - j0 >= W);
            const TQ* Kc = Ks[cur];
            const T* Vc = Vs[cur];

            // S^T tiles: keys 32kt..32kt+31 x this wave's 32 queries (log2 domain)
            floatx16 sacc[2] = {floatx16{}, floatx16{}};
#pragma unroll
            for (int st = 0; st < NST; ++st) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const FragQ kf = *(const FragQ*)(Kc + (32 * kt + l32) * LDK + 2 * KPLQ * st + KPLQ * gl);
                    sacc[kt] = MQ::mma(kf, qf[st], sacc[kt]);
                }
            }

            // online softmax for query l32 (its other 32 keys sit in lane l ^ 32).
            // Scores are relative to a per-row reference m_run; the reference
            // moves only when a row's maximum exceeds it by more than 2^8 (so
            // P <= 256) -- the common tile takes exp2 of the scores as they are.
            if (need_mask) {
                asm volatile("");                          // keep this a branch
                const unsigned wlim = W > 0 ? (unsigned)W : 0x7fffffffu;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int jj = j0 + 32 * kt + 8 * (i / 4) + 4 * gl + (i % 4);
                        sacc[kt][i] = ((unsigned)(pq - jj) < wlim) ? sacc[kt][i] : kNegInf;
                    }
                }
            }
            // four independent max chains (short dependency chains), then the
            // partner half of the row
            float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) m4[i % 4] = fmaxf(m4[i % 4], sacc[kt][i]);
            const float mx = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
            // a row (re)starts its reference at its first visible scores, or when
            // its max exceeds the reference by more than 8 (log2 units)
            const bool fresh = (m_run == kNegInf);
            const bool grow = fresh ? (mx > kNegInf) : (mx - m_run > 8.0f);
            if (__ballot(grow) != 0) {
                asm volatile("");                          // keep this a branch
                const float m_new = grow ? mx : m_run;
                const float alpha = fresh ? 1.0f : fast_exp2(m_run - m_new);   // 1 unless grown
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
                m_run = m_new;
            }
            const float ref = (m_run == kNegInf) ? 0.0f : m_run;   // rows with nothing visible stay -inf
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kt][i] -= ref;
            float r4[4] = {0.0f, 0.0f, 0.0f, 0.0f};          // four partial row sums
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = fast_exp2(sacc[kt][i]);
                    sacc[kt][i] = pv;
                    r4[i % 4] += pv;
                }
            }
            l_run += (r4[0] + r4[1]) + (r4[2] + r4[3]);

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
                    if constexpr (kBf16) {
                        // item t of lane group gl is key kb + 8*(t/4) + t%4 with
                        // kb = 32(st/2) + 16(st%2) + 4gl; each run of 4 keys is one
                        // transposing read: source lane i of a 16-lane group points at
                        // row kb + 8r + i/4, columns 32dt + 16*(group%2) + 4*(i%4)..+3
                        typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
                        const int kb = 32 * (st / 2) + 16 * (st % 2) + 4 * gl;
                        const int i16 = lane & 15;
                        const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
                        const T* src0 = Vc + (kb + (i16 >> 2)) * LDV + col;
                        const T* src1 = src0 + 8 * LDV;
                        const shortx4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_shortx4*)(__attribute__((address_space(3))) void*)src0);
                        const shortx4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_shortx4*)(__attribute__((address_space(3))) void*)src1);
                        typedef short shortx8 __attribute__((ext_vector_type(8)));
                        const shortx8 both = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
                        vf = __builtin_bit_cast(FragP, both);
                    } else {
#pragma unroll
                        for (int t = 0; t < KPLP; ++t) {
                            const int I = st * KPLP + t;
                            const int key = 32 * (I / 16) + 8 * ((I % 16) / 4) + 4 * gl + (I % 4);
                            frag_set_raw(vf, t, Vc[key * LDV + 32 * dt + l32]);
                        }
                    }
                    o[dt] = MP::mma(vf, pf, o[dt]);
                }
            }
        }
        if (it + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: normalise, gate, store (lane: 4 consecutive dims per item
    // group).  The gate values are all read before the first output store, so
    // that no read waits behind a store it might alias.
    const float l_tot = sum_halves(l_run);
    if (!wave_live || tq >= N) return;
    const float inv = 1.0f / l_tot;
    const int64_t base = (((int64_t)s * N + tq) * kHeads + h) * D;
    const T* gate = (const T*)a.gate + base;
    T* dst = out + base;
    float gv[4][4][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig)
#pragma unroll
            for (int x = 0; x < 4; ++x) gv[dt][ig][x] = to_f32(gate[32 * dt + 8 * ig + 4 * gl + x]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
            const int d0 = 32 * dt + 8 * ig + 4 * gl;
#pragma unroll
            for (int x = 0; x < 4; ++x) dst[d0 + x] = from_f32<T>(o[dt][4 * ig + x] * inv * sigmoid(gv[dt][ig][x]));
        }
    }
}

// ---- bf16 layers: heads of one KV group per workgroup, one head per wave,
// all waves over the same query rows, so tile ranges and masks are uniform
// across the workgroup and each K/V tile staged in LDS serves every wave.
// The build uses 8 heads x 32 rows per workgroup with 32-key tiles (QG = 1,
// WPB = 8, KT = 1, no software pipelining): one workgroup of two waves per
// SIMD on each CU; each staged tile serves 8 waves, one 16-byte chunk of K
// and one of V per thread.  That measured about 8% faster than two
// workgroups of 4 heads per CU.  64 rows per wave (QG = 2) halves the LDS
// reads per flop but needs one wave per SIMD, and measured slower, as did
// the pipelined loop.
//
// Softmax reference.  Each row's reference is fixed at the maximum of the
// first 32-key half-tile in which it sees a key, and never moves: later
// exponentials are exp2(s - ref) with s - ref possibly > 0.  Softmax is
// invariant to the reference (O and l carry the same factor), the maximum
// key has P >= 1 so nothing underflows that matters, and the only failure is
// an overflow to inf in P, l or O -- checked at the end.  Under QK-norm the
// scores are bounded by |q-hat| |k-hat|, so this does not happen with the
// model's gains; if it does, the workgroup recomputes its rows with the
// exact row maxima from a Q.K-only pass (then P <= 1).  A fixed reference
// removes the running maximum and the O rescale from the tile loop, and lets
// the Q.K MFMAs start from -ref instead of 0, so no subtraction is left
// either.  Row sums are taken from the bf16 P values that enter the P.V
// product (v_dot2 against (1, 1)).
// One direct load: every lane fetches 16 bytes at `src` (its own address) and
// the active lanes' pieces land at the LDS address `dst` + 16 x lane (`dst`
// uniform).  Issued as inline asm, so the compiler neither counts it nor
// guards LDS accesses with waits for it (the builtin made the RoPE table
// wait for every load in flight): the caller waits (s_waitcnt vmcnt) before
// it reads that LDS.  M0 holds the LDS address, with a wait state before the
// load; nothing else in this file's kernels uses M0 (checked in their gfx950
// assembly: no s_movrel/v_movrel, GWS, LDS-direct or s_sendmsg), so the
// clobber loses nothing.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, void* dst) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int QG> struct GroupTraits {
    static constexpr int WAVES = QG == 1 ? 2 : 1;      // waves per SIMD the registers allow
};

int prefill_grid_group(int n_seq, int n_new, int rows_per_wave, int heads_per_block) {
    const int nqb = (n_new + rows_per_wave - 1) / rows_per_wave;
    const int units = n_seq * kKvHeads * nqb;          // (q-block, seq, kv head)
    return ((units + 7) / 8) * 8 * (kHeadsPerKv / heads_per_block);
}

// QG: 32-row query groups per wave; WPB: waves (= heads of one KV group) per
// workgroup; KT: 32-key halves per K/V tile
template <int QG, int WPB, int KT>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(GroupTraits<QG>::WAVES)))
void prefill_group_kernel(AttnArgs a) {
    typedef bf16_t T;
    typedef f16_t TQ;
    using MQ = Mma32<TQ>;
    using MP = Mma32<T>;
    using FragQ = MQ::Frag;
    using FragP = MP::Frag;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    constexpr int BMW = 32 * QG, BN = 32 * KT, D = kHeadDim;
    constexpr int LDK = D + 8, LDV = D + 32;           // conflict-free b128 / transposing reads
    constexpr int NST = D / (2 * MQ::KPL);             // K-steps of Q.K (8)
    constexpr int ES = 2;
    constexpr int CPR = D * ES / 16;                   // 16-byte chunks per row
    constexpr int NT = 64 * WPB;                       // threads per block
    constexpr int HQ = kHeadsPerKv / WPB;              // blocks per (q-block, seq, kv head)
    constexpr int NCH = BN * CPR / NT;                 // chunks per thread per tile
    __shared__ __attribute__((aligned(16))) TQ Ks[2][BN * LDK];
    __shared__ __attribute__((aligned(16))) T Vs[2][BN * LDV];
    constexpr int LDE = D + 8;                         // epilogue rows: 272 bytes = 17 slots of 16 bytes
    static_assert(QG == 1, "the epilogue buffer holds one 32-row group per wave");
    __shared__ __attribute__((aligned(16))) T ebuf[WPB][32 * LDE];

    // ---- work item: block b runs head group (b >> 3) % HQ of unit (b >> 3) / HQ * 8 + (b & 7),
    // so the workgroups of a unit (its 16 heads) share an XCD
    const int nqb = (a.n_new + BMW - 1) / BMW;
    const int b = blockIdx.x;
    const int hq = (b >> 3) % HQ;
    const int unit = (b >> 3) / HQ * 8 + (b & 7);
    const int per_qb = a.n_seq * kKvHeads;
    if (unit >= per_qb * nqb) return;
    const int qb = nqb - 1 - unit / per_qb;            // heavy blocks first
    const int s = (unit % per_qb) >> 1;
    const int g = (unit % per_qb) & 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, gl = lane >> 5;
    const int h = g * kHeadsPerKv + hq * WPB + wave;
    const int q0 = qb * BMW;
    const int N = a.n_new;
    const int L = a.seq_len[s];

    T* out = (T*)a.out;
    if (L < 0 || L > a.max_seq_len) {                  // refused on the device
        const int rows = min(BMW, N - q0);
        for (int i = lane; i < rows * D; i += 64) {
            const int t = q0 + i / D;
            out[(((int64_t)s * N + t) * kHeads + h) * D + (i % D)] = from_f32<T>(__builtin_nanf(""));
        }
        return;
    }

    // ---- keys the workgroup can see (positions fit in int32: bounded by 2^24)
    const int W = a.window;
    const int P0 = L + q0, P1 = L + min(q0 + BMW - 1, N - 1);
    const int kv_lo = (W > 0) ? max(0, P0 - W + 1) : 0;
    const int kv_end = L + N;
    const int tile_lo = kv_lo / BN, tile_hi = P1 / BN;
    const int ntiles = tile_hi - tile_lo + 1;
    const int pq0 = L + q0 + l32;                      // position of this lane's row in group 0

    constexpr int64_t ROW = (int64_t)kKvHeads * D * ES;
    constexpr int RSTEP = NT / CPR;
    const int r_t = tid / CPR, c_t = tid % CPR;
    // rows of the K copy (and of V on ring layers) start on sliding layers at
    // the window's first visible position rounded down to kWindowAlign; every
    // tile read here starts at or past that (tiles start at multiples of BN,
    // which divides kWindowAlign)
    static_assert(kWindowAlign % BN == 0, "key tiles start inside the windowed copy");
    const int64_t win0 = W > 0 ? max(0, L - W + 1) / kWindowAlign * kWindowAlign : 0;
    const char* kbase = (const char*)a.kq + ((((int64_t)s * a.kq_capacity) - (a.kq_windowed ? win0 : 0)) * kKvHeads + g) * D * ES + c_t * 16;
    const char* vbase = (const char*)a.cache_v + ((((int64_t)s * a.capacity) - (a.v_windowed ? win0 : 0)) * kKvHeads + g) * D * ES + c_t * 16;
    // ---- Q-hat of the wave's rows (B operand of S^T = K Q^T), made here from the
    // raw Q: QK-norm with gain ("Chapter 9 - The Muse Glimmer architecture" 9.5;
    // "Chapter 14 - QK-norm and RoPE" 14.3), RoPE on sliding layers (Ch 14,
    // 14.4-14.5: angle f32(p) * theta_i in f32, accurate sin and cos), then
    // attn_scale * log2(e), rounded to fp16.  Each (row, head) is made by
    // exactly one wave, so this costs no more than a separate pass and saves
    // writing Q-hat to HBM and reading it back.  The workgroup's rows share one
    // (cos, sin) table in LDS.
    __shared__ float2 rot[BMW][kHeadDim / 2 + 1];       // padded: rows start 2 banks apart
    // The epilogue's gate rows (32 rows x 256 bytes of head h) go straight to
    // the wave's epilogue buffer first of all, so the epilogue does not wait
    // for them.  They are requested before every load the compiler counts:
    // vector loads complete in issue order, so the compiler's waits (which do
    // not know of these) still wait exactly for what they name.
    // Slot k (16 bytes) of the buffer is row k / 17, chunk k % 17; chunk 16 is
    // the row's padding and takes a copy of chunk 15.  Nine loads of 64 slots
    // cover the 544 slots; the last one only with lanes 0-31.
    {
        const char* grow = (const char*)a.gate + ((int64_t)s * N * kHeads + h) * D * ES;
        char* eb0 = (char*)ebuf[wave];
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            const int slot = 64 * j + lane, r = slot / 17, c = min(slot % 17, 15);
            const int t = min(q0 + r, N - 1);
            if (j < 8 || lane < 32)
                lds_dma16(grow + (int64_t)t * kHeads * D * ES + 16 * c, eb0 + 1024 * j);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // This lane's RoPE frequency is requested next, then the raw Q rows and
    // the first K/V tile, all before the (cos, sin) table is built: the table
    // waits for the frequency alone, and the Q and tile round trips overlap it.
    // (Requested after them, the frequency made the table wait for every load
    // in flight: 3.4 us per sliding workgroup instead of 0.6.)
    const float th = a.rope ? theta_of_lane<AttnArgs>(lane) : 0.0f;
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 qraw[QG][NST];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int tq = q0 + 32 * qg + l32;
        const bf16_t* qrow = (const bf16_t*)a.q + (((int64_t)s * N + min(tq, N - 1)) * kHeads + h) * D;
#pragma unroll
        for (int st = 0; st < NST; ++st) qraw[qg][st] = *(const bf16x8*)(qrow + 2 * MQ::KPL * st + MQ::KPL * gl);
    }
    u32x4 ka0[NCH], va0[NCH];                          // the loop's first K/V tile
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int64_t off = (int64_t)min(tile_lo * BN + r_t + u * RSTEP, kv_end - 1) * ROW;
        ka0[u] = *(const u32x4*)(kbase + off);
        va0[u] = *(const u32x4*)(vbase + off);
    }
    if (a.rope) {
        for (int row = wave; row < BMW; row += WPB) {
            float sn, cs;
            sincos_rope((float)((int64_t)L + q0 + row) * th, &sn, &cs);
            rot[row][lane] = make_float2(cs, sn);
        }
        __syncthreads();
    }
    FragQ qf[QG][NST];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int tq = q0 + 32 * qg + l32;
        float x[NST][8];
        float ss = 0.0f;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                x[st][t] = (float)qraw[qg][st][t];
                ss += x[st][t] * x[st][t];
            }
        }
        ss = sum_halves(ss);                           // the row's other 64 values sit in lane l ^ 32
        const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            float y[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) y[t] = (x[st][t] * r) * a.q_gain;
            if (a.rope) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {          // pair (dims 2i, 2i+1), i = 8 st + 4 gl + j
                    const float2 c = rot[32 * qg + l32][8 * st + 4 * gl + j];
                    const float y0 = y[2 * j], y1 = y[2 * j + 1];
                    y[2 * j] = y0 * c.x - y1 * c.y;
                    y[2 * j + 1] = y0 * c.y + y1 * c.x;
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) qf[qg][st][t] = (TQ)(tq < N ? y[t] * a.q_scale : 0.0f);
        }
    }

    u32x4 kreg[NCH], vreg[NCH];
    // Tile rows into registers.  Rows past the last cached position are
    // clamped to it (in-bounds, finite data): every key there lies after
    // every query of the workgroup, so the mask gives it P = 0.  Rows before
    // the window start are real cache rows and are masked the same way.  No
    // branch here: a zero-fill path would make the compiler wait for all
    // loads where the two paths meet.
    auto load_tile = [&](int tile, bool with_v) __attribute__((always_inline)) {
        const int j0 = tile * BN;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int64_t off = (int64_t)min(j0 + r_t + u * RSTEP, kv_end - 1) * ROW;
            kreg[u] = *(const u32x4*)(kbase + off);
            if (with_v) vreg[u] = *(const u32x4*)(vbase + off);
        }
    };
    auto store_tile = [&](int bufi, bool with_v) __attribute__((always_inline)) {
        char* kd = (char*)Ks[bufi] + r_t * LDK * ES + c_t * 16;
        char* vd = (char*)Vs[bufi] + r_t * LDV * ES + c_t * 16;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            *(u32x4*)(kd + u * RSTEP * LDK * ES) = kreg[u];
            if (with_v) *(u32x4*)(vd + u * RSTEP * LDV * ES) = vreg[u];
        }
    };

    // S^T halves (keys 32kt..32kt+31 x the wave's row groups), started at c0
    auto qk = [&](floatx16 (&sc)[KT][QG], const TQ* Kc, const floatx16 (&c0)[QG]) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) sc[kt][qg] = c0[qg];
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                const FragQ kf = *(const FragQ*)(Kc + (32 * kt + l32) * LDK + 2 * MQ::KPL * st + MQ::KPL * gl);
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) sc[kt][qg] = MQ::mma(kf, qf[qg][st], sc[kt][qg]);
            }
        }
    };
    // key 32kt + 8(i/4) + 4gl + i%4 of the tile at j0 is visible to row (qg, l32)
    // iff 0 <= p - key < W (W = infinity on full layers)
    auto apply_mask = [&](floatx16 (&sc)[KT][QG], int j0) __attribute__((always_inline)) {
        const unsigned wlim = W > 0 ? (unsigned)W : 0x7fffffffu;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int jj = j0 + 32 * kt + 8 * (i / 4) + 4 * gl + (i % 4);
                    sc[kt][qg][i] = ((unsigned)(pq0 + 32 * qg - jj) < wlim) ? sc[kt][qg][i] : kNegInf;
                }
    };
    auto row_max = [&](const floatx16& v) __attribute__((always_inline)) {
        float m4[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
        for (int i = 4; i < 16; ++i) m4[i % 4] = fmaxf(m4[i % 4], v[i]);
        return max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    };

    float ref[QG];                                     // row references; -inf until set
    floatx16 nref[QG];                                 // -ref broadcast (0 while unset)
    floatx16 o[4][QG];                                 // O^T tiles [dims 32dt..][row group]
    float l_run[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        ref[qg] = kNegInf;
        nref[qg] = floatx16{};
    }
    auto set_nref = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            const float v = ref[qg] == kNegInf ? 0.0f : -ref[qg];
#pragma unroll
            for (int i = 0; i < 16; ++i) nref[qg][i] = v;
        }
    };

    auto record_unset = [&](bool (&unset)[QG]) __attribute__((always_inline)) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) unset[qg] = ref[qg] == kNegInf;
    };
    // mask of a boundary tile; rows still without a reference take the maximum
    // of their first visible half (their scores were computed from 0, not -ref)
    auto fix_tile = [&](floatx16 (&sc)[KT][QG], int j0, const bool (&unset)[QG]) __attribute__((always_inline)) {
        const bool masked = (j0 + BN - 1 > P0) || (W > 0 && P1 - j0 >= W);
        if (masked) {
            asm volatile("");                              // keep this a branch
            apply_mask(sc, j0);
        }
        bool any_unset = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) any_unset = any_unset || unset[qg];
        if (__ballot(any_unset) != 0) {
            asm volatile("");                              // keep this a branch
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) {
                    const float m = row_max(sc[kt][qg]);
                    if (ref[qg] == kNegInf && m > kNegInf) ref[qg] = m;
                    const float r = (unset[qg] && ref[qg] != kNegInf) ? ref[qg] : 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) sc[kt][qg][i] -= r;
                }
            set_nref();
        }
    };
    // P = exp2(S - ref) in bf16; l += sum of those P; O^T += V^T P^T
    auto softmax_pv = [&](floatx16 (&sc)[KT][QG], const T* Vc) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < 2 * KT; ++st) {              // 16 keys per K-step
            FragP pf[QG];
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
                for (int t = 0; t < MP::KPL; ++t) frag_set(pf[qg], t, fast_exp2(sc[st / 2][qg][8 * (st % 2) + t]));
                const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
                float acc = l_run[qg];
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qg], pf[qg], 0, 1), one, acc, false);
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qg], pf[qg], 2, 3), one, acc, false);
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qg], pf[qg], 4, 5), one, acc, false);
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[qg], pf[qg], 6, 7), one, acc, false);
                l_run[qg] = acc;
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                // item t of lane group gl is key kb + 8*(t/4) + t%4 with
                // kb = 32(st/2) + 16(st%2) + 4gl; each run of 4 keys is one
                // transposing read: source lane i of a 16-lane group points at
                // row kb + 8r + i/4, columns 32dt + 16*(group%2) + 4*(i%4)..+3
                typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
                const int kb = 32 * (st / 2) + 16 * (st % 2) + 4 * gl;
                const int i16 = lane & 15;
                const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
                const T* src0 = Vc + (kb + (i16 >> 2)) * LDV + col;
                const T* src1 = src0 + 8 * LDV;
                const shortx4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_shortx4*)(__attribute__((address_space(3))) void*)src0);
                const shortx4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_shortx4*)(__attribute__((address_space(3))) void*)src1);
                const FragP vf = __builtin_bit_cast(FragP, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) o[dt][qg] = MP::mma(vf, pf[qg], o[dt][qg]);
            }
        }
    };

    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            // exact row maxima from a Q.K-only sweep over the same tiles
            float mx[QG];
            floatx16 zero[QG];
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                mx[qg] = kNegInf;
                zero[qg] = floatx16{};
            }
            load_tile(tile_lo, false);
            store_tile(0, false);
            __syncthreads();
            for (int it = 0; it < ntiles; ++it) {
                const int cur = it & 1;
                const int j0 = (tile_lo + it) * BN;
                load_tile(min(tile_lo + it + 1, tile_hi), false);   // the last one is a harmless repeat
                floatx16 sc[KT][QG];
                qk(sc, Ks[cur], zero);
                apply_mask(sc, j0);
#pragma unroll
                for (int qg = 0; qg < QG; ++qg)
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) mx[qg] = fmaxf(mx[qg], row_max(sc[kt][qg]));
                store_tile(cur ^ 1, false);
                __syncthreads();
            }
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) ref[qg] = mx[qg];
            set_nref();
        }
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt][qg] = floatx16{};
            l_run[qg] = 0.0f;
        }

        // loads run two tiles ahead, alternating between two register sets
        u32x4 ka[NCH], va[NCH], kb2[NCH], vb2[NCH];
        auto ld2 = [&](u32x4 (&kr)[NCH], u32x4 (&vr)[NCH], int tile) __attribute__((always_inline)) {
            const int j0 = tile * BN;
#pragma unroll
            for (int u = 0; u < NCH; ++u) {
                const int64_t off = (int64_t)min(j0 + r_t + u * RSTEP, kv_end - 1) * ROW;
                kr[u] = *(const u32x4*)(kbase + off);
                vr[u] = *(const u32x4*)(vbase + off);
            }
        };
        auto st2 = [&](const u32x4 (&kr)[NCH], const u32x4 (&vr)[NCH], int bufi) __attribute__((always_inline)) {
            char* kd = (char*)Ks[bufi] + r_t * LDK * ES + c_t * 16;
            char* vd = (char*)Vs[bufi] + r_t * LDV * ES + c_t * 16;
#pragma unroll
            for (int u = 0; u < NCH; ++u) {
                *(u32x4*)(kd + u * RSTEP * LDK * ES) = kr[u];
                *(u32x4*)(vd + u * RSTEP * LDV * ES) = vr[u];
            }
        };
        if (pass == 0) {                               // loaded before Q-hat
#pragma unroll
            for (int u = 0; u < NCH; ++u) {
                ka[u] = ka0[u];
                va[u] = va0[u];
            }
        } else {
            ld2(ka, va, tile_lo);
        }
        st2(ka, va, 0);
        ld2(kb2, vb2, min(tile_lo + 1, tile_hi));
        __syncthreads();
        auto step = [&](int it, u32x4 (&kn)[NCH], u32x4 (&vn)[NCH], u32x4 (&kf)[NCH], u32x4 (&vf)[NCH])
            __attribute__((always_inline)) {
            // kn/vn hold tile it+1 (loaded one iteration ago); kf/vf take tile it+2
            const int cur = it & 1;
            ld2(kf, vf, min(tile_lo + it + 2, tile_hi));
            __builtin_amdgcn_sched_barrier(0);
            bool unset[QG];
            record_unset(unset);
            floatx16 sc[KT][QG];
            qk(sc, Ks[cur], nref);
            st2(kn, vn, cur ^ 1);                          // that buffer is free since the last barrier
            fix_tile(sc, (tile_lo + it) * BN, unset);
            softmax_pv(sc, Vs[cur]);
            __syncthreads();
        };
        for (int it = 0; it < ntiles; it += 2) {
            step(it, kb2, vb2, ka, va);
            if (it + 1 < ntiles) step(it + 1, ka, va, kb2, vb2);
        }

        // an overflow anywhere shows up as a non-finite l or O
        float chk = 0.0f;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) chk += l_run[qg];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
#pragma unroll
                for (int i = 0; i < 16; ++i) chk += o[dt][qg][i];
        if (!__syncthreads_or(!__builtin_isfinite(chk))) break;
    }

    // ---- epilogue: normalise, gate, store.  The wave's 32-row x 128 tile goes
    // through its own LDS buffer: the gate rows are loaded whole (16 lanes per
    // 256-byte row), read back in the accumulator layout, combined with O and
    // written back in place, then stored as whole rows.  (Straight from the
    // accumulator layout every load and store instruction touched 32 rows, 16
    // bytes in each.)  Only this wave touches its buffer, and a wave's LDS
    // accesses complete in order, so the phases need no barrier; the wave
    // barriers keep the compiler from moving accesses across phases.
    T* eb = ebuf[wave];
    const int er = lane >> 4, ec = lane & 15;          // whole-row phases: row 4u + er, 16-byte chunk ec
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int t0 = q0 + 32 * qg;
        __builtin_amdgcn_s_waitcnt(0);                 // the gate rows loaded into eb at the start
        __builtin_amdgcn_wave_barrier();
        const float inv = 1.0f / sum_halves(l_run[qg]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                // dims 32 dt + 8 ig + 4 gl .. + 3 of row l32
                T* e = eb + l32 * LDE + 32 * dt + 8 * ig + 4 * gl;
                const uint2 g2 = *(const uint2*)e;
                unsigned packed[2];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const unsigned w = x < 2 ? g2.x : g2.y;
                    const float gv = __uint_as_float((x & 1) ? (w & 0xffff0000u) : (w << 16));
                    const T y = from_f32<T>(o[dt][qg][4 * ig + x] * inv * sigmoid(gv));
                    const unsigned u16 = __builtin_bit_cast(unsigned short, y);
                    if (x & 1) packed[x / 2] |= u16 << 16;
                    else packed[x / 2] = u16;
                }
                *(uint2*)e = make_uint2(packed[0], packed[1]);
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = t0 + 4 * u + er;
            const u32x4 v = *(const u32x4*)(eb + (4 * u + er) * LDE + 8 * ec);
            if (t < N) *(u32x4*)(out + (((int64_t)s * N + t) * kHeads + h) * D + 8 * ec) = v;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

hipError_t launch_prefill(const AttnArgs& a, int dtype, hipStream_t stream) {
    if (dtype == 1)
        hipLaunchKernelGGL((prefill_group_kernel<kGroupQG, kGroupWPB, kGroupKT>),
                           dim3((unsigned)prefill_grid_group(a.n_seq, a.n_new, 32 * kGroupQG, kGroupWPB)),
                           dim3(64 * kGroupWPB), 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_kernel<float>, dim3((unsigned)prefill_grid(a.n_seq, a.n_new)), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace muse
