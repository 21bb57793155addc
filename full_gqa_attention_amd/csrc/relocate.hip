// relocate.hip -- byte copy of NoPE cache tiles (K and V) between positions,
// sequences or caches, many tiles in one launch.  A full (NoPE) layer's rows
// carry no position, so a copied row is valid at its new position ("Chapter
// 14 - QK-norm and RoPE" 14.6: NoPE tiles relocate by memcpy).
//
// Each workgroup copies one kRelocChunk-byte piece of one tile, in K and in
// V; a tile's pieces are workgroups block0[t] .. block0[t + 1] - 1.  The host
// splits the tile list into launches so that no tile of a launch reads or
// writes rows another tile of the same launch writes: tiles apply in order.
#include "device_common.h"
#include "kernels.h"

namespace muse {

__global__ __launch_bounds__(256) void relocate_kernel(RelocArgs a) {
    const int b = blockIdx.x;
    int t = 0;
    while (t + 1 < a.n_tiles && b >= a.block0[t + 1]) ++t;     // at most kRelocTiles steps
    const int64_t piece = (int64_t)(b - a.block0[t]) * kRelocChunk;
    const int64_t n = min((int64_t)kRelocChunk, a.bytes[t] - piece);   // bytes of this piece, a multiple of 16
    const char* sk = a.src_k + a.src_off[t] + piece;
    const char* sv = a.src_v + a.src_off[t] + piece;
    char* dk = a.dst_k + a.dst_off[t] + piece;
    char* dv = a.dst_v + a.dst_off[t] + piece;
    // every load before the first store: a load after a store the compiler
    // cannot tell apart from it would wait for the store
    constexpr int PER = kRelocChunk / (256 * 16);
    u32x4 x[PER], y[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int64_t i = ((int64_t)u * 256 + threadIdx.x) * 16;
        if (i < n) {
            x[u] = __builtin_nontemporal_load((const u32x4*)(sk + i));
            y[u] = __builtin_nontemporal_load((const u32x4*)(sv + i));
        }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int64_t i = ((int64_t)u * 256 + threadIdx.x) * 16;
        if (i < n) {
            __builtin_nontemporal_store(x[u], (u32x4*)(dk + i));
            __builtin_nontemporal_store(y[u], (u32x4*)(dv + i));
        }
    }
}

hipError_t launch_relocate(const RelocArgs& a, hipStream_t stream) {
    if (a.n_tiles == 0 || a.block0[a.n_tiles] == 0) return hipSuccess;
    hipLaunchKernelGGL(relocate_kernel, dim3((unsigned)a.block0[a.n_tiles]), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace muse
