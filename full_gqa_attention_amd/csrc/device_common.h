// device_common.h -- small device-side helpers shared by the gfx950 kernels:
// storage types, conversions, wave reductions and MFMA wrappers.
#pragma once
#include <cstddef>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "trig.h"

namespace muse {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16 raw bytes
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kHeads = 32;      // query heads
constexpr int kKvHeads = 2;     // KV heads
constexpr int kHeadDim = 128;   // head_dim
constexpr int kHeadsPerKv = 16; // query heads served by one KV head

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// f32 -> bf16 rounds to nearest, ties to even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }

// Operand type of the Q.K^T products.  bf16 layers score in fp16: Q-hat keeps
// 3 more mantissa bits than bf16 (its rounding is the dominant error of the
// bf16 path), and a bf16 K row converts to fp16 exactly while its entries
// stay inside fp16's normal range; normed keys are bounded by
// |k_gain| * sqrt(128), which the host keeps far below 65504.  P.V stays in
// the storage type (V is raw and unbounded).
template <typename T> struct ScoreType;
template <> struct ScoreType<bf16_t> { typedef f16_t type; };
template <> struct ScoreType<float> { typedef float type; };

// 16 bytes of storage-type K -> 16 bytes of score-type K (bf16 -> fp16;
// f32 unchanged).
__device__ __forceinline__ u32x4 k_chunk_to_score(u32x4 x, bf16_t) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, x);
    f16x8 h;
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = (f16_t)(float)b[t];
    return __builtin_bit_cast(u32x4, h);
}
__device__ __forceinline__ u32x4 k_chunk_to_score(u32x4 x, float) { return x; }

// The value of x held by lane l ^ 32, paired with this lane's own: after
// v_permlane32_swap of x with itself, one of the two results is x of this
// lane and the other x of lane l ^ 32 (which is which depends on the half),
// so a symmetric combination of the pair is the same in lanes l and l ^ 32.
struct HalfPair { float a, b; };
__device__ __forceinline__ HalfPair halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return HalfPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// v_permlane16_swap of x with itself: the two results are x of this lane
// and of lane l ^ 16 (in an order that depends on the lane), so again a
// symmetric combination is the same in both lanes.
__device__ __forceinline__ HalfPair rows16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return HalfPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_rows16(float x) {
    const HalfPair p = rows16(x);
    return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float sum_rows16(float x) {
    const HalfPair p = rows16(x);
    return p.a + p.b;
}
__device__ __forceinline__ float max_halves(float x) {
    const HalfPair p = halves(x);
    return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float sum_halves(float x) {
    const HalfPair p = halves(x);
    return p.a + p.b;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// 2^x on the hardware exp unit (v_exp_f32).  Softmax works in the log2
// domain: scores are pre-multiplied by scale * log2(e).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sigma(g) = 1 / (1 + e^-g), with the hardware reciprocal (about 1 ulp; an
// IEEE division costs a dozen instructions per value, and the prefill
// epilogue evaluates 4,096 of these per token).  For g below about -88,
// e^-g overflows to inf and the reciprocal gives 0, the correct limit.
__device__ __forceinline__ float sigmoid(float g) {
    return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-g * 1.4426950408889634f));
}

constexpr float kNegInf = -__builtin_huge_valf();

// ----------------------------------------------------- QK-norm and RoPE
// One head vector of 128 values per wave: lane i holds the adjacent pair
// (x[2i], x[2i+1]), which is RoPE pair i.

// theta[lane] of a kernel whose only argument is the struct Args (so the
// struct sits at the start of the kernel's argument block): one vector load
// at the table's offset.  Selecting it out of the scalar copies of the
// arguments takes 64 selects and several dependent scalar-load round trips.
template <typename Args>
__device__ __forceinline__ float theta_of_lane(int lane) {
    typedef const __attribute__((address_space(4))) char* KArg;
    return *((const __attribute__((address_space(4))) float*)(
                 (KArg)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(Args, theta)) + lane);
}

// sin/cos of the f32 angle f32(p) * theta[lane] (accurate: trig.h).  The
// table sits in kernel arguments; the unrolled select keeps every access at
// a constant index.
__device__ __forceinline__ void rope_sincos(const float (&theta)[64], int lane, int64_t p,
                                            float& sn, float& cs) {
    float th = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) th = (lane == i) ? theta[i] : th;
    const float ang = (float)p * th;
    sincos_rope(ang, &sn, &cs);
}

// RMS-normalise the wave's 128-vector, scale by gain, then (rope) rotate the
// lane's pair by the angle whose sin/cos are given.
__device__ __forceinline__ void norm_rope_pair(float x0, float x1, float eps, float gain, bool rope,
                                               float sn, float cs, float& y0, float& y1) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float r = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
    y0 = (x0 * r) * gain;
    y1 = (x1 * r) * gain;
    if (rope) {
        const float z0 = y0 * cs - y1 * sn;
        const float z1 = y0 * sn + y1 * cs;
        y0 = z0;
        y1 = z1;
    }
}

// ---------------------------------------------------------------- MFMA
// 32x32 tiles (prefill).  Operand layout for C = A * B (A: 32 x K, B: K x 32):
// lane l holds A[l % 32][KPL * (l / 32) + t] and B[KPL * (l / 32) + t][l % 32]
// for t < KPL; the f32 result has C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32]
// in item i of lane l.
template <typename T> struct Mma32;
template <> struct Mma32<bf16_t> {
    static constexpr int KPL = 8;          // v_mfma_f32_32x32x16_bf16
    typedef bf16x8 Frag;
    static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma32<f16_t> {
    static constexpr int KPL = 8;          // v_mfma_f32_32x32x16_f16
    typedef f16x8 Frag;
    static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma32<float> {
    static constexpr int KPL = 1;          // v_mfma_f32_32x32x2_f32
    typedef float Frag;
    static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// 16x16 tiles (decode).  lane l holds A[l % 16][KPL * (l / 16) + t] and
// B[KPL * (l / 16) + t][l % 16]; C[4 * (l / 16) + i][l % 16] is item i.
// "Wide" is the long-K instruction (Q.K over head_dim), "Narrow" the K = 16
// (bf16) / K = 4 (f32) one used for P.V over 16 keys.
template <typename T> struct Mma16Wide;
template <> struct Mma16Wide<bf16_t> {
    static constexpr int KPL = 8;          // v_mfma_f32_16x16x32_bf16
    typedef bf16x8 Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma16Wide<f16_t> {
    static constexpr int KPL = 8;          // v_mfma_f32_16x16x32_f16
    typedef f16x8 Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma16Wide<float> {
    static constexpr int KPL = 1;          // v_mfma_f32_16x16x4_f32
    typedef float Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};
template <typename T> struct Mma16Narrow;
template <> struct Mma16Narrow<bf16_t> {
    static constexpr int KPL = 4;          // v_mfma_f32_16x16x16_bf16
    typedef shortx4 Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma16Narrow<float> {
    static constexpr int KPL = 1;          // v_mfma_f32_16x16x4_f32
    typedef float Frag;
    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// Element t of a fragment (t is a compile-time constant after unrolling).
__device__ __forceinline__ void frag_set(bf16x8& f, int t, float v) { f[t] = (bf16_t)v; }
__device__ __forceinline__ void frag_set(float& f, int, float v) { f = v; }
__device__ __forceinline__ void frag_set(shortx4& f, int t, float v) {
    bf16_t b = (bf16_t)v;
    f[t] = __builtin_bit_cast(short, b);
}
__device__ __forceinline__ void frag_set_raw(bf16x8& f, int t, bf16_t v) { f[t] = v; }
__device__ __forceinline__ void frag_set_raw(float& f, int, float v) { f = v; }
__device__ __forceinline__ void frag_set_raw(shortx4& f, int t, bf16_t v) {
    f[t] = __builtin_bit_cast(short, v);
}

}  // namespace muse
