// outproj.hip -- the attention block's tail after the gate ("Chapter 9 - The
// Muse Glimmer architecture" 9.8 and 9.9, Figure 9.1): o_proj maps the 4,096
// gated attention channels of each token to the model width 6,656, the
// post-attention RMSNorm (its own epsilon, 1e-8 in the model) scales each
// token's projection, and the result joins the residual stream.
//
// Two kernels.  The projection is a plain GEMM, proj = attn . W^T, on
// v_mfma_f32_32x32x16_bf16 with f32 accumulation, written in f32 to the
// workspace.  The norm needs a whole 6,656-wide row, which no GEMM tile holds,
// so a second, memory-bound kernel takes one row per workgroup: sum of
// squares, 1 / sqrt(mean + eps), times the gain, plus the residual, rounded
// once to bf16.
#include "device_common.h"
#include "kernels.h"

namespace muse {

// ---- GEMM: a workgroup computes a kOpBM x kOpBN tile of proj with 8 waves
// (kOpWM along the tokens x kOpWN along the channels, each 32 kOpTM x 32 kOpTN:
// kOpTM x kOpTN MFMA tiles).  256 x 256 tiles of 64 x 128 per wave (4 x 2
// waves) measured 15% faster than 256 x 128 tiles of 64 x 64: each operand
// read from LDS feeds more MFMAs.
// K advances 64 at a time through two LDS buffers; global loads run two
// k-steps ahead in alternating register sets.  Both operands are K-contiguous
// (attn rows and W rows), so every MFMA operand is one 16-byte LDS read.
#ifndef MUSE_OP_TM
#define MUSE_OP_TM 2
#endif
#ifndef MUSE_OP_TN
#define MUSE_OP_TN 4
#endif
#ifndef MUSE_OP_WM
#define MUSE_OP_WM 4
#endif
constexpr int kOpTM = MUSE_OP_TM, kOpTN = MUSE_OP_TN, kOpWM = MUSE_OP_WM, kOpWN = 8 / kOpWM;
constexpr int kOpBM = 32 * kOpTM * kOpWM, kOpBN = 32 * kOpTN * kOpWN, kOpBK = 64;
constexpr int kOpLds = kOpBK + 8;                      // 144-byte rows: b128 reads conflict-free
constexpr int kOpThreads = 512;
constexpr int kOpAChunks = kOpBM * kOpBK * 2 / 16 / kOpThreads;   // 16-byte chunks per thread (4)
constexpr int kOpBChunks = kOpBN * kOpBK * 2 / 16 / kOpThreads;   // (2)
static_assert(kModelDim % kOpBN == 0 && kAttnDim % kOpBK == 0, "tile sizes divide the shapes");

__global__ __launch_bounds__(kOpThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void out_proj_gemm_kernel(OutProjArgs a) {
    using MP = Mma32<bf16_t>;
    constexpr int K = kAttnDim, N = kModelDim, NK = K / kOpBK;
    __shared__ __attribute__((aligned(16))) bf16_t As[2][kOpBM * kOpLds];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kOpBN * kOpLds];

    const int nblk = N / kOpBN;
    const int nb = blockIdx.x % nblk, mb = blockIdx.x / nblk;   // the channel blocks of a token block run together
    const int m0 = mb * kOpBM, n0 = nb * kOpBN;
    const int M = a.m;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, gl = lane >> 5;
    const int wm = wave / kOpWN, wn = wave % kOpWN;

    // staging: chunk c = tid + 512 u is row c / 8, 16-byte piece c % 8 of a 64-wide k slice
    const bf16_t* A = (const bf16_t*)a.attn;
    const bf16_t* B = (const bf16_t*)a.w;
    auto load = [&](u32x4 (&ra)[kOpAChunks], u32x4 (&rb)[kOpBChunks], int ks) __attribute__((always_inline)) {
        const int k0 = min(ks, NK - 1) * kOpBK;                  // past the end: harmless repeats
#pragma unroll
        for (int u = 0; u < kOpAChunks; ++u) {
            const int c = tid + kOpThreads * u, r = c >> 3, p = c & 7;
            const int row = min(m0 + r, M - 1);                  // rows past the last token repeat it
            ra[u] = *(const u32x4*)(A + (int64_t)row * K + k0 + 8 * p);
        }
#pragma unroll
        for (int u = 0; u < kOpBChunks; ++u) {
            const int c = tid + kOpThreads * u, r = c >> 3, p = c & 7;
            rb[u] = *(const u32x4*)(B + (int64_t)(n0 + r) * K + k0 + 8 * p);
        }
    };
    auto store = [&](const u32x4 (&ra)[kOpAChunks], const u32x4 (&rb)[kOpBChunks], int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kOpAChunks; ++u) {
            const int c = tid + kOpThreads * u, r = c >> 3, p = c & 7;
            *(u32x4*)(As[buf] + r * kOpLds + 8 * p) = ra[u];
        }
#pragma unroll
        for (int u = 0; u < kOpBChunks; ++u) {
            const int c = tid + kOpThreads * u, r = c >> 3, p = c & 7;
            *(u32x4*)(Bs[buf] + r * kOpLds + 8 * p) = rb[u];
        }
    };

    floatx16 acc[kOpTM][kOpTN];
#pragma unroll
    for (int i = 0; i < kOpTM; ++i)
#pragma unroll
        for (int j = 0; j < kOpTN; ++j) acc[i][j] = floatx16{};
    // C[m][n] += A[m][k] W[n][k]: lane (l32, gl) gives A row l32 and W row l32
    // (the B column), k = 8 gl .. 8 gl + 7 of each 16-wide step
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const bf16_t* Ab = As[buf] + (32 * kOpTM * wm + l32) * kOpLds + 8 * gl;
        const bf16_t* Bb = Bs[buf] + (32 * kOpTN * wn + l32) * kOpLds + 8 * gl;
#pragma unroll
        for (int kk = 0; kk < kOpBK / 16; ++kk) {
            bf16x8 af[kOpTM], bfr[kOpTN];
#pragma unroll
            for (int i = 0; i < kOpTM; ++i) af[i] = *(const bf16x8*)(Ab + 32 * i * kOpLds + 16 * kk);
#pragma unroll
            for (int j = 0; j < kOpTN; ++j) bfr[j] = *(const bf16x8*)(Bb + 32 * j * kOpLds + 16 * kk);
#pragma unroll
            for (int i = 0; i < kOpTM; ++i)
#pragma unroll
                for (int j = 0; j < kOpTN; ++j) acc[i][j] = MP::mma(af[i], bfr[j], acc[i][j]);
        }
    };

    u32x4 ra0[kOpAChunks], rb0[kOpBChunks], ra1[kOpAChunks], rb1[kOpBChunks];
    load(ra0, rb0, 0);
    store(ra0, rb0, 0);
    load(ra1, rb1, 1);
    __syncthreads();
    // step ks: buffer ks & 1 holds k-slice ks, (rn, bn) holds slice ks + 1,
    // (rf, bf) receives slice ks + 2
    auto step = [&](int ks, u32x4 (&rn)[kOpAChunks], u32x4 (&bn)[kOpBChunks],
                    u32x4 (&rf)[kOpAChunks], u32x4 (&bf)[kOpBChunks]) __attribute__((always_inline)) {
        load(rf, bf, ks + 2);
        compute(ks & 1);
        store(rn, bn, (ks + 1) & 1);                   // free since the last barrier
        __syncthreads();
    };
    static_assert(NK % 2 == 0, "k-steps come in pairs");
    for (int ks = 0; ks < NK; ks += 2) {
        step(ks, ra1, rb1, ra0, rb0);
        step(ks + 1, ra0, rb0, ra1, rb1);
    }

    // ---- proj rows m0 + 32 (kOpTM wm + i) + 8 (e / 4) + 4 gl + e % 4, channel
    // n0 + 32 (kOpTN wn + j) + l32: 32 lanes store 128 contiguous bytes per item
#pragma unroll
    for (int i = 0; i < kOpTM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + 32 * (kOpTM * wm + i) + 8 * (e / 4) + 4 * gl + (e % 4);
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < kOpTN; ++j) a.proj[(int64_t)m * N + n0 + 32 * (kOpTN * wn + j) + l32] = acc[i][j][e];
        }
}

// ---- GEMM for a few tokens (a decode step: at most 64).  Reading W's 54.5
// MB is the whole cost, so every CU must stream an equal share with as much
// of it in flight as it can hold.  The product is cut into 8 slices of K (512
// each) x 32 blocks of 208 channels: 256 workgroups, one per CU, each reading
// 208 KB of W.  A block is 13 groups of 16 channels; wave v takes groups v
// and v + 8 (waves 5-7 only the first) and requests every W load of its
// groups at once, straight into the layout of the 16 x 16 x 32 MFMA (lane
// (l16, g4): 16 bytes of row n + l16 at k + 8 g4 of each 32-wide step).  The
// attn slice (all tokens x 512; rows past the last token repeat it) is
// requested before W and staged in LDS while W streams in.  A workgroup
// writes its slice's partial product; the norm kernel adds the 8 slices in
// slice order (the sum does not depend on timing).
constexpr int kSkinnyMaxM = 64;
constexpr int kSkinnySlices = 8, kSkinnyK = kAttnDim / kSkinnySlices;    // 512
constexpr int kSkinnyBlocks = 32, kSkinnyCh = kModelDim / kSkinnyBlocks;  // 208 channels
constexpr int kSkinnyGroups = kSkinnyCh / 16;                             // 13
constexpr int kSkinnyLds = kSkinnyK + 8;                // 1,040-byte rows: b128 reads conflict-free
static_assert(kSkinnyCh * kSkinnyBlocks == kModelDim && kSkinnyCh % 16 == 0 && kSkinnyGroups > 8 &&
                  kSkinnyGroups <= 16,
              "skinny tiling");

// MT tiles of 16 tokens x NG groups of 16 channels (the wave's first group,
// and the one 8 groups on) x one K slice.
template <int MT, int NG>
__device__ __forceinline__ void skinny_wave(const OutProjArgs& a, bf16_t* As, int ks, int blk, int wave, int lane) {
    using MP = Mma16Wide<bf16_t>;
    constexpr int KS = kSkinnyK / 32;                   // 32-wide k steps
    constexpr int CPR = kSkinnyK / 8;                   // 16-byte chunks per attn row
    constexpr int STAGE = 16 * MT * CPR / 512;          // chunks per thread
    static_assert(16 * MT * CPR % 512 == 0, "staging split");
    const int tid = 64 * wave + lane, l16 = lane & 15, g4 = lane >> 4;
    const int k0 = ks * kSkinnyK, M = a.m;
    const bf16_t* attn = (const bf16_t*)a.attn;
    u32x4 st[STAGE];
#pragma unroll
    for (int s = 0; s < STAGE; ++s) {
        const int c = tid + 512 * s, r = c / CPR, p = c % CPR;
        st[s] = *(const u32x4*)(attn + (int64_t)min(r, M - 1) * kAttnDim + k0 + 8 * p);
    }
    __builtin_amdgcn_sched_barrier(0);                  // attn first: its wait leaves W in flight
    const int n = blk * kSkinnyCh + 16 * wave;
    const bf16_t* wp = (const bf16_t*)a.w + (int64_t)(n + l16) * kAttnDim + k0 + 8 * g4;
    bf16x8 bw[KS][NG];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int g = 0; g < NG; ++g) bw[s][g] = *(const bf16x8*)(wp + (int64_t)g * 128 * kAttnDim + 32 * s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < STAGE; ++s) {
        const int c = tid + 512 * s, r = c / CPR, p = c % CPR;
        *(u32x4*)(As + r * kSkinnyLds + 8 * p) = st[s];
    }
    __syncthreads();
    floatx4 acc[NG][MT];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[g][i] = floatx4{};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const bf16x8 af = *(const bf16x8*)(As + (16 * i + l16) * kSkinnyLds + 32 * s + 8 * g4);
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g][i] = MP::mma(af, bw[s][g], acc[g][i]);
        }
    // partial of slice ks: token 16 i + 4 g4 + e, channel n + 128 g + l16
    float* part = a.proj + (int64_t)ks * M * kModelDim + n + l16;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 16 * i + 4 * g4 + e;
                if (m < M) part[(int64_t)m * kModelDim + 128 * g] = acc[g][i][e];
            }
}

template <int MT>
__global__ __launch_bounds__(512) void out_proj_skinny_kernel(OutProjArgs a) {
    __shared__ __attribute__((aligned(16))) bf16_t As[16 * MT * kSkinnyLds];
    // blockIdx = 64 q + 8 r + x: slice r, block 8 q + x.  Consecutive
    // workgroups go to the 8 XCDs in turn, so XCD x holds blocks x, x + 8, ...
    // with all 8 slices of each: its L2 sees every part of W's rows, and a
    // block's partials are written within one XCD.
    static_assert(kSkinnySlices == 8 && kSkinnyBlocks == 32, "block mapping");
    const int ks = (blockIdx.x >> 3) & 7, blk = ((blockIdx.x >> 6) << 3) | (blockIdx.x & 7);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // wave-uniform: each path reaches the workgroup barrier once
    if (wave + 8 < kSkinnyGroups)
        skinny_wave<MT, 2>(a, As, ks, blk, wave, lane);
    else
        skinny_wave<MT, 1>(a, As, ks, blk, wave, lane);
}

// ---- post-attention RMSNorm + residual: one token row per workgroup, 4
// channels per thread and step (6,656 = 1,664 groups of 4).  NPARTS K slices
// of the projection (a few tokens) are added in slice order, all their loads
// in flight together; those rows get 1,024 threads so that the loads of a
// thread stay few.
constexpr int kNormGroups = kModelDim / 4;

template <int NPARTS, int THREADS>
__global__ __launch_bounds__(THREADS) void out_proj_norm_kernel(OutProjArgs a) {
    constexpr int PER = (kNormGroups + THREADS - 1) / THREADS;
    // a long batch's projection, residual and output are each touched once:
    // nontemporal (the few-token slices were just written and are read cached)
    constexpr bool kStream = NPARTS == 1;
    __shared__ float red[THREADS / 64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float* prow = a.proj + (int64_t)t * kModelDim;
    const int64_t pstride = (int64_t)a.m * kModelDim;  // between K slices
    floatx4 x[PER];
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int gidx = min(tid + THREADS * u, kNormGroups - 1);
        floatx4 part[NPARTS];
#pragma unroll
        for (int q = 0; q < NPARTS; ++q) {
            const floatx4* src = (const floatx4*)(prow + q * pstride + 4 * gidx);
            part[q] = kStream ? __builtin_nontemporal_load(src) : *src;
        }
        x[u] = part[0];
#pragma unroll
        for (int q = 1; q < NPARTS; ++q) x[u] += part[q];
        if (tid + THREADS * u >= kNormGroups) x[u] = floatx4{};
        ss += x[u][0] * x[u][0] + x[u][1] * x[u][1] + x[u][2] * x[u][2] + x[u][3] * x[u][3];
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) tot += red[w];
    const float inv = 1.0f / sqrtf(tot * (1.0f / kModelDim) + a.eps);
    const bf16_t* res = (const bf16_t*)a.residual + (int64_t)t * kModelDim;
    bf16_t* out = (bf16_t*)a.out + (int64_t)t * kModelDim;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int gidx = tid + THREADS * u;
        if (gidx >= kNormGroups) break;
        const floatx4 g = *(const floatx4*)(a.gamma + 4 * gidx);
        const unsigned long long* rsrc = (const unsigned long long*)(res + 4 * gidx);
        const unsigned long long r64 = kStream ? __builtin_nontemporal_load(rsrc) : *rsrc;
        const uint2 rr = make_uint2((unsigned)r64, (unsigned)(r64 >> 32));
        const float r4[4] = {__uint_as_float(rr.x << 16), __uint_as_float(rr.x & 0xffff0000u),
                             __uint_as_float(rr.y << 16), __uint_as_float(rr.y & 0xffff0000u)};
        unsigned packed[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const unsigned u16 = __builtin_bit_cast(unsigned short, from_f32<bf16_t>(x[u][c] * inv * g[c] + r4[c]));
            if (c & 1) packed[c / 2] |= u16 << 16;
            else packed[c / 2] = u16;
        }
        const unsigned long long o64 = (unsigned long long)packed[0] | ((unsigned long long)packed[1] << 32);
        if (kStream) __builtin_nontemporal_store(o64, (unsigned long long*)(out + 4 * gidx));
        else *(unsigned long long*)(out + 4 * gidx) = o64;
    }
}

hipError_t launch_out_proj_gemm(const OutProjArgs& a, hipStream_t stream) {
    if (a.m <= kSkinnyMaxM) {
        const dim3 sgrid(kSkinnySlices * kSkinnyBlocks), sblock(512);
        switch ((a.m + 15) / 16) {
        case 1: hipLaunchKernelGGL(out_proj_skinny_kernel<1>, sgrid, sblock, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(out_proj_skinny_kernel<2>, sgrid, sblock, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(out_proj_skinny_kernel<3>, sgrid, sblock, 0, stream, a); break;
        default: hipLaunchKernelGGL(out_proj_skinny_kernel<4>, sgrid, sblock, 0, stream, a); break;
        }
        return hipGetLastError();
    }
    const int64_t mblk = (a.m + kOpBM - 1) / kOpBM;
    hipLaunchKernelGGL(out_proj_gemm_kernel, dim3((unsigned)(mblk * (kModelDim / kOpBN))), dim3(kOpThreads), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_out_proj_norm(const OutProjArgs& a, hipStream_t stream) {
    if (a.m <= kSkinnyMaxM)
        hipLaunchKernelGGL((out_proj_norm_kernel<kSkinnySlices, 1024>), dim3((unsigned)a.m), dim3(1024), 0, stream, a);
    else
        hipLaunchKernelGGL((out_proj_norm_kernel<1, 256>), dim3((unsigned)a.m), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
