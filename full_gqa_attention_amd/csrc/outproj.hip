// outproj.hip -- the attention block's tail after the gate ("Chapter 9 - The
// Muse Glimmer architecture" 9.8 and 9.9, Figure 9.1): o_proj maps the 4,096
// gated attention channels of each token to the model width 6,656, the
// post-attention RMSNorm (its own epsilon, 1e-8 in the model) scales each
// token's projection, and the result joins the residual stream.
//
// Two steps.  The projection is a plain GEMM, proj = attn . W^T, with f32
// accumulation, written in f32 to the workspace: for a few tokens (a decode
// step) a kernel of this file that streams W across every CU, for more tokens
// hipBLASLt.  The norm needs a whole 6,656-wide row, which no GEMM tile holds,
// so a second, memory-bound kernel takes one row per workgroup: sum of
// squares, 1 / sqrt(mean + eps), times the gain, plus the residual, rounded
// once to bf16.
#include <map>
#include <mutex>

#include <hipblaslt/hipblaslt.h>

#include "device_common.h"
#include "kernels.h"

namespace muse {

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

// ---- the projection of more tokens through hipBLASLt.  Column-major, as the
// library sees it: D (f32 6656 x m, ld 6656; proj row-major [m][6656]) =
// op(A) x B with A = W read as 4096 x 6656 (ld 4096) and op(A) its transpose,
// B = attn read as 4096 x m (ld 4096).  One library handle per device, made on
// the first such call there (it allocates: capture graphs only after one
// eager call).  The algorithm is the library's heuristic choice among those
// that need no workspace (the call passes none: an algorithm that wanted one
// wrote through the missing buffer), kept per token count, so repeated calls
// run the same kernels and give the same bits.
namespace {
struct BlasDevice {
    hipblasLtHandle_t handle = nullptr;
    std::map<int32_t, hipblasLtMatmulAlgo_t> algo;
};
std::mutex g_blas_mu;
std::map<int, BlasDevice> g_blas;

hipError_t launch_out_proj_blas(const OutProjArgs& a, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorUnknown;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    BlasDevice& bd = g_blas[dev];
    if (!bd.handle && hipblasLtCreate(&bd.handle) != HIPBLAS_STATUS_SUCCESS) {
        bd.handle = nullptr;
        return hipErrorUnknown;
    }
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    hipError_t err = hipErrorUnknown;
    const hipblasOperation_t opA = HIPBLAS_OP_T, opB = HIPBLAS_OP_N;
    const float alpha = 1.0f, beta = 0.0f;
    const auto ok = [](hipblasStatus_t st) { return st == HIPBLAS_STATUS_SUCCESS; };
    do {
        if (!ok(hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F)) ||
            !ok(hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opA, sizeof(opA))) ||
            !ok(hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opB, sizeof(opB))))
            break;
        if (!ok(hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, kAttnDim, kModelDim, kAttnDim)) ||
            !ok(hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, kAttnDim, (uint64_t)a.m, kAttnDim)) ||
            !ok(hipblasLtMatrixLayoutCreate(&lc, HIP_R_32F, kModelDim, (uint64_t)a.m, kModelDim)))
            break;
        auto it = bd.algo.find(a.m);
        if (it == bd.algo.end()) {
            const uint64_t no_workspace = 0;
            if (!ok(hipblasLtMatmulPreferenceCreate(&pref)) ||
                !ok(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                          &no_workspace, sizeof(no_workspace))))
                break;
            hipblasLtMatmulHeuristicResult_t res[8];
            int n = 0;
            if (!ok(hipblasLtMatmulAlgoGetHeuristic(bd.handle, desc, la, lb, lc, lc, pref, 8, res, &n))) break;
            int pick = -1;
            for (int i = 0; i < n && pick < 0; ++i)
                if (ok(res[i].state) && res[i].workspaceSize == 0) pick = i;
            if (pick < 0) break;
            it = bd.algo.emplace(a.m, res[pick].algo).first;
        }
        if (!ok(hipblasLtMatmul(bd.handle, desc, &alpha, a.w, la, a.attn, lb, &beta, a.proj, lc, a.proj, lc,
                                &it->second, nullptr, 0, stream)))
            break;
        err = hipSuccess;
    } while (false);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (lc) hipblasLtMatrixLayoutDestroy(lc);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (desc) hipblasLtMatmulDescDestroy(desc);
    return err;
}
}  // namespace

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
    return launch_out_proj_blas(a, stream);
}

hipError_t launch_out_proj_norm(const OutProjArgs& a, hipStream_t stream) {
    if (a.m <= kSkinnyMaxM)
        hipLaunchKernelGGL((out_proj_norm_kernel<kSkinnySlices, 1024>), dim3((unsigned)a.m), dim3(1024), 0, stream, a);
    else
        hipLaunchKernelGGL((out_proj_norm_kernel<1, 256>), dim3((unsigned)a.m), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
