// The binary merge tree over the stored partial states of one (sequence, head)
// row, run by one workgroup of the merge kernel.
//
// Sections "Core Innovation 1" step 3 and "Core Innovation 2" of "Tree Attention
// Guide: Topology-Aware LLM Decoding": partial states are merged pairwise up a tree
// with m = max(m_A, m_B), alpha = exp(m_A - m), beta = exp(m_B - m),
// l = alpha l_A + beta l_B, o = alpha o_A + beta o_B. The tree is fixed: at level
// t, node i merges node i + 2^t when i is a multiple of 2^(t+1); a node without a
// partner passes up unchanged. A stored partial (o_i, lse_i) enters as the page's
// tuple (o_i, 1, lse_i); lse_i = -inf is the empty state (0, 0, -inf).
//
// Layout: the d channels are split into float4 columns, CG = d / 4 threads per
// leaf row (one coalesced read per row); the S = NT / CG slots each take R
// consecutive leaves and run the lowest log2(R) levels in registers, then the
// slots run the remaining log2(S) levels, by lane shuffles between slots of one
// wave and through LDS between waves. Merging with an empty state
// returns the other operand bit for bit, so padding the leaf count up to S * R
// leaves the tree, and every result, unchanged.
#pragma once

#include "device_common.h"

namespace ta {

struct MState {
    float4 o;
    float l;
    float m;  // natural-log units
};

__device__ __forceinline__ MState merge_states(const MState& A, const MState& B) {
    const float m = fmaxf(A.m, B.m);
    const float ref = (m == -INFINITY) ? 0.0f : m;
    const float a = exp2_fast((A.m - ref) * kLog2e);
    const float b = exp2_fast((B.m - ref) * kLog2e);
    MState r;
    r.m = m;
    r.l = a * A.l + b * B.l;
    r.o.x = a * A.o.x + b * B.o.x;
    r.o.y = a * A.o.y + b * B.o.y;
    r.o.z = a * A.o.z + b * B.o.z;
    r.o.w = a * A.o.w + b * B.o.w;
    return r;
}

template <int D, int NT>
struct MergeSmem {
    static constexpr int CG = D / 4;
    static constexpr int S = NT / CG;
    float4 o[S][CG];
    float l[S];
    float m[S];
};

// The R leaves one thread reads for one row (lse_i and its float4 column of o_i).
template <int R>
struct Leaves {
    float lse[R];
    float4 o[R];
};

// Issues the loads of this thread's leaves of one row: leaves [first, first + S*R)
// are split into S slots of R consecutive leaves; leaves at or past `valid` are not
// read.
template <int D, int R, int NT>
__device__ __forceinline__ Leaves<R> load_leaves(const float* po, int64_t po_sp, const float* pl, int64_t pl_sp,
                                                 int first, int valid) {
    constexpr int CG = D / 4;
    const int cg = threadIdx.x % CG;
    const int base = first + (int)(threadIdx.x / CG) * R;
    Leaves<R> lv;
    if constexpr (R % 4 == 0) {
        // Every leaf of the workgroup holds data and the lse are contiguous and 16-byte
        // aligned (the same decision in every lane): one 64-bit product per thread, then
        // wave-uniform leaf strides, and the lse of 4 consecutive leaves in one load.
        constexpr int S = NT / CG;
        if (first + S * R <= valid && pl_sp == 1 && (reinterpret_cast<uintptr_t>(pl + first) & 15u) == 0) {
            const float* op = po + (int64_t)base * po_sp + 4 * cg;
            const float* lp = pl + base;
#pragma unroll
            for (int r = 0; r < R; r += 4) {
                const float4 v = *reinterpret_cast<const float4*>(lp + r);
                lv.lse[r] = v.x;
                lv.lse[r + 1] = v.y;
                lv.lse[r + 2] = v.z;
                lv.lse[r + 3] = v.w;
            }
#pragma unroll
            for (int r = 0; r < R; ++r) lv.o[r] = *reinterpret_cast<const float4*>(op + (int64_t)r * po_sp);
            return lv;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = base + r;
        lv.lse[r] = -INFINITY;
        lv.o[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < valid) {
            lv.lse[r] = pl[(int64_t)i * pl_sp];
            lv.o[r] = *reinterpret_cast<const float4*>(po + (int64_t)i * po_sp + 4 * cg);
        }
    }
    return lv;
}

// Runs the tree over the leaves loaded by load_leaves. Every thread of the workgroup
// must call it; on return threads of slot 0 (tid < CG) hold the root state of their
// column. Ends with a barrier, so the LDS can be reused right after.
template <int D, int R, int NT>
__device__ __forceinline__ MState reduce_leaves(const Leaves<R>& lv, MergeSmem<D, NT>& sm) {
    constexpr int CG = D / 4;
    constexpr int S = NT / CG;
    static_assert(S * CG == NT && (S & (S - 1)) == 0, "slots");
    const int cg = threadIdx.x % CG;
    const int slot = threadIdx.x / CG;
    MState leaf[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool full = lv.lse[r] != -INFINITY;
        leaf[r].o = full ? lv.o[r] : make_float4(0.f, 0.f, 0.f, 0.f);
        leaf[r].l = full ? 1.0f : 0.0f;
        leaf[r].m = lv.lse[r];
    }
    // lowest levels, in registers: strides 1, 2, ..., R/2
#pragma unroll
    for (int stride = 1; stride < R; stride <<= 1) {
#pragma unroll
        for (int r = 0; r < R; r += 2 * stride) leaf[r] = merge_states(leaf[r], leaf[r + stride]);
    }
    MState st = leaf[0];
    // remaining levels across slots: slot s merges slot s + t when s is a multiple of 2t.
    // Levels whose two slots share a wave exchange states between lanes t * CG apart
    // (16 or 32: row and half swaps, no LDS); the others go through LDS. (Every lane
    // merges; only the lower slot of each pair goes on.)
    constexpr int kSlotsPerWave = kWave / CG < S ? kWave / CG : S;
#pragma unroll
    for (int t = 1; t < kSlotsPerWave; t <<= 1) {
        MState other;
        other.o.x = xor_lanes(st.o.x, t * CG);
        other.o.y = xor_lanes(st.o.y, t * CG);
        other.o.z = xor_lanes(st.o.z, t * CG);
        other.o.w = xor_lanes(st.o.w, t * CG);
        other.l = xor_lanes(st.l, t * CG);
        other.m = xor_lanes(st.m, t * CG);
        st = merge_states(st, other);
    }
#pragma unroll
    for (int t = kSlotsPerWave; t < S; t <<= 1) {
        if ((slot & (2 * t - 1)) == t) {
            sm.o[slot][cg] = st.o;
            if (cg == 0) {
                sm.l[slot] = st.l;
                sm.m[slot] = st.m;
            }
        }
        __syncthreads();
        if ((slot & (2 * t - 1)) == 0) {
            MState other;
            other.o = sm.o[slot + t][cg];
            other.l = sm.l[slot + t];
            other.m = sm.m[slot + t];
            st = merge_states(st, other);
        }
        __syncthreads();
    }
    return st;
}

// The tree over leaves [first, first + S*R) of one row.
template <int D, int R, int NT>
__device__ __forceinline__ MState tree_merge_row(const float* po, int64_t po_sp, const float* pl, int64_t pl_sp,
                                                 int first, int valid, MergeSmem<D, NT>& sm) {
    return reduce_leaves<D, R, NT>(load_leaves<D, R, NT>(po, po_sp, pl, pl_sp, first, valid), sm);
}

// Root normalisation (end of "Core Innovation 2"): O = o / l, lse = m + ln l.
// An empty root gives O = 0 and lse = -inf. Called by one thread per float4 column
// cg of the row (by default the threads of slot 0, whose index is the column).
__device__ __forceinline__ void write_root(const MState& st, float* out_row, float* lse_ptr,
                                           int cg = threadIdx.x) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = -INFINITY;
    if (st.l > 0.0f) {
        const float inv = 1.0f / st.l;
        o.x = st.o.x * inv; o.y = st.o.y * inv; o.z = st.o.z * inv; o.w = st.o.w * inv;
        lse = st.m + __log2f(st.l) * kLn2;
    }
    *reinterpret_cast<float4*>(out_row + 4 * cg) = o;
    if (cg == 0 && lse_ptr) *lse_ptr = lse;
}

}  // namespace ta
