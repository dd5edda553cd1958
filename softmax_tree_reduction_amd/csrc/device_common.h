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

// The value of lane (this lane XOR K). K = 1, 2: quad permutes; K = 4: row_ror:N
// gives lane i the value of lane (i - N) mod 16, so lanes whose bit 2 is clear read
// lane i + 4 through row_ror:12 and the others lane i - 4 through row_ror:4, each
// half written under its bank mask (a bank is 4 lanes); K = 8: row_ror:8 inside
// the 16-lane row; K = 16: across rows through v_permlane16_swap (see xor_lanes).
template <int K>
__device__ __forceinline__ float lane_xor(float x) {
    if constexpr (K == 1) {
        return dpp_mov<kDppXor1>(x);
    } else if constexpr (K == 2) {
        return dpp_mov<kDppXor2>(x);
    } else if constexpr (K == 4) {
        int t = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x12C, 0xF, 0x5, false);
        t = __builtin_amdgcn_update_dpp(t, __float_as_int(x), 0x124, 0xF, 0xA, false);
        return __int_as_float(t);
    } else if constexpr (K == 8) {
        return dpp_mov<0x128>(x);
    } else {
        static_assert(K == 16, "lane_xor");
        const unsigned u = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float(((__lane_id() >> 4) & 1u) ? r[0] : r[1]);
    }
}

// The value lane (lane ^ off) holds, for off in {8, 16, 32} without any LDS traffic:
// 8 through DPP row_ror:8 inside the 16-lane row, 16 and 32 through gfx950's row
// and half swaps (v_permlane16_swap_b32, v_permlane32_swap_b32). Given two copies
// of x, a swap's first result holds every even row's (lower half's) values in both
// rows (halves) of a pair and the second every odd row's (upper half's), so each
// lane takes its partner's from the other parity. Other offsets use the ordinary
// shuffle.
__device__ __forceinline__ float xor_lanes(float x, int off) {
    if (off == 8) return lane_xor<8>(x);
    if (off == 16) return lane_xor<16>(x);
    if (off == 32) {
        const unsigned u = __float_as_uint(x);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float((__lane_id() >> 5) ? r[0] : r[1]);
    }
    return __shfl_xor(x, off, 64);
}

// Lane K of each aligned group of L lanes (L in {8, 16, 32}, K < 8), for every lane
// of the group. L = 16 and 32 use row_newbcast (each 16-lane row takes its own lane
// K; in a 32-lane group both rows hold the same value wherever this is used). L = 8
// broadcasts each half row separately under bank masks.
template <int K, int L>
__device__ __forceinline__ float group_bcast(float x) {
    static_assert(K < 8, "lane");
    if constexpr (L == 8) {
        int t = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xF, 0x3, false);
        t = __builtin_amdgcn_update_dpp(t, __float_as_int(x), 0x158 + K, 0xF, 0xC, false);
        return __int_as_float(t);
    } else {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + K, 0xF, 0xF, true));
    }
}

// Sum of per-head partial dot products over one row's L lanes (L in {8, 16, 32}),
// scattered by head. On entry d[r] is this lane's partial for head r ^ (lane & (G-1))
// (the caller loads q in that lane-dependent order). Head bit b pairs lane with lane
// XOR 2^b: each lane keeps the registers whose bit b is clear and adds its partner's
// register with bit b set, which holds the same head, so no select is needed. The
// remaining lane bits are summed in full: rotations by 2^b inside the 16-lane row
// (their offsets cover every lane with the same low bits), or XOR partners where
// the group is 8 lanes wide. On return d[0] is the full dot product for head
// (lane & (G-1)), the same in every lane of the row that holds that head.
template <int G, int L>
__device__ __forceinline__ void row_reduce_scatter(float (&d)[G]) {
    static_assert(L == 8 || L == 16 || L == 32, "row size");
    static_assert(G <= L, "heads per row");
    if constexpr (G >= 2) {
#pragma unroll
        for (int r = 0; r < G; r += 2) d[r] += lane_xor<1>(d[r + 1]);
    }
    if constexpr (G >= 4) {
#pragma unroll
        for (int r = 0; r < G; r += 4) d[r] += lane_xor<2>(d[r + 2]);
    }
    if constexpr (G >= 8) {
        d[0] += lane_xor<4>(d[4]);
    }
    if constexpr (L == 8) {
        if constexpr (G <= 1) d[0] += lane_xor<1>(d[0]);
        if constexpr (G <= 2) d[0] += lane_xor<2>(d[0]);
        if constexpr (G <= 4) d[0] += lane_xor<4>(d[0]);
    } else {
        if constexpr (G <= 1) d[0] += dpp_mov<0x121>(d[0]);  // row_ror:1
        if constexpr (G <= 2) d[0] += dpp_mov<0x122>(d[0]);  // row_ror:2
        if constexpr (G <= 4) d[0] += dpp_mov<0x124>(d[0]);  // row_ror:4
        d[0] += dpp_mov<0x128>(d[0]);                        // row_ror:8
        if constexpr (L == 32) d[0] += lane_xor<16>(d[0]);
    }
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
