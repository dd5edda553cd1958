// Device helpers shared by the partial-state and tree-merge kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef TA_STREAM_NT
#define TA_STREAM_NT 1
#endif

namespace ta {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Exact widening of a packed pair of bfloat16 values (low half = first element).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Streaming 16-byte load: each K/V byte is read once, so the load carries the
// nontemporal hint and does not displace reusable lines from the caches.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
#if TA_STREAM_NT
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
#else
    return *p;
#endif
}

// 2^x on the hardware exponential unit; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane moves inside one 16-lane DPP row (gfx9 DPP controls).
enum : int {
    kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,  // lane i <-> 7 - i inside each 8-lane half row
    kDppMirror = 0x140,      // lane i <-> 15 - i inside each 16-lane row
};

template <int Ctrl>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of L consecutive lanes (L in {8, 16, 32}); every lane
// of the group receives the group total. The pairings xor1, xor2, half-mirror,
// mirror each join two disjoint halves of a growing aligned group, so after
// log2(L) steps each lane holds the sum over its whole group.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L == 8 || L == 16 || L == 32, "group size");
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    x += dpp_mov<kDppHalfMirror>(x);
    if constexpr (L >= 16) x += dpp_mov<kDppMirror>(x);
    if constexpr (L >= 32) x += __shfl_xor(x, 16, kWave);
    return x;
}

// The page's merge operator on states kept in base 2: state (o, l, m) stands for
// o = sum 2^(s_j - m) v_j and l = sum 2^(s_j - m) with s_j in log2 units.
// An empty state is (0, 0, -inf); when both inputs are empty the result stays empty
// (the reference point is taken as 0 so that no -inf - -inf is formed).
struct Rescale {
    float a, b, m;
};
__device__ __forceinline__ Rescale merge_factors(float ma, float mb) {
    const float m = fmaxf(ma, mb);
    const float ref = (m == -INFINITY) ? 0.0f : m;
    return {exp2_fast(ma - ref), exp2_fast(mb - ref), m};
}

}  // namespace ta
