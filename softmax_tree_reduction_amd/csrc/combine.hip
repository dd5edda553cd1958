// Tree merge of partial states for gfx950.
//
// Section "Core Innovation 1" step 3 of "Tree Attention Guide: Topology-Aware LLM
// Decoding" reduces the partial states up a tree of depth ceil(log_k P); section
// "Core Innovation 2" gives the merge applied at each node:
//   m = max(m_A, m_B), alpha = exp(m_A - m), beta = exp(m_B - m),
//   l = alpha l_A + beta l_B, o = alpha o_A + beta o_B,
// and the normalisation O = o / l at the root. Here k = 2 and the tree is fixed:
// at level t, node i merges node i + 2^t whenever i is a multiple of 2^(t+1).
//
// A stored partial is normalised, (o_i, lse_i); it enters the tree as the page's
// tuple (o_i, 1, lse_i), which is the same state. A leaf with lse_i = -inf is
// the empty state (0, 0, -inf).
//
// One workgroup of 256 threads merges up to S * R leaves of one (sequence, head)
// row: the d channels are split into float4 columns (CG = d / 4 threads per
// leaf row, so a leaf row is one coalesced read) and the S = 256 / CG slots each
// take R consecutive leaves. A slot first runs the lowest log2(R) levels of the
// tree in registers over its R leaves, then the slots run the remaining log2(S)
// levels through LDS. Rows with more leaves than one workgroup takes are merged
// in several passes over aligned groups of leaves, which is the same tree.
#include "device_common.h"
#include "kernels.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxR = 16;

struct State {
    float4 o;
    float l;
    float m;  // natural-log units
};

__device__ __forceinline__ State merge(const State& A, const State& B) {
    const float m = fmaxf(A.m, B.m);
    const float ref = (m == -INFINITY) ? 0.0f : m;
    const float a = exp2_fast((A.m - ref) * kLog2e);
    const float b = exp2_fast((B.m - ref) * kLog2e);
    State r;
    r.m = m;
    r.l = a * A.l + b * B.l;
    r.o.x = a * A.o.x + b * B.o.x;
    r.o.y = a * A.o.y + b * B.o.y;
    r.o.z = a * A.o.z + b * B.o.z;
    r.o.w = a * A.o.w + b * B.o.w;
    return r;
}

__device__ __forceinline__ State empty_state() {
    return {make_float4(0.f, 0.f, 0.f, 0.f), 0.0f, -INFINITY};
}

template <int D, int R>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
    constexpr int CG = D / 4;          // threads per leaf row
    constexpr int S = kThreads / CG;   // slots
    constexpr int SPAN = S * R;        // leaves per workgroup
    static_assert(S * CG == kThreads && (S & (S - 1)) == 0, "slots");

    __shared__ float4 sm_o[S][CG];
    __shared__ float sm_l[S];
    __shared__ float sm_m[S];

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int grp = blockIdx.z;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int slot = tid / CG;

    // number of leaves that can hold tokens in this row
    int valid = p.n_parts;
    if (p.seqlens) {
        int n = p.seqlens[b];
        n = n < 0 ? 0 : (n > p.N ? p.N : n);
        const int pb = (int)(((int64_t)n + p.chunk - 1) / p.chunk);
        valid = pb < valid ? pb : valid;
    }

    const float* po = p.po + (int64_t)b * p.po_sb + (int64_t)h * p.po_sh;
    const float* pl = p.plse + (int64_t)b * p.pl_sb + (int64_t)h * p.pl_sh;
    const int first = grp * SPAN + slot * R;

    // load this slot's R leaves
    State leaf[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = first + r;
        leaf[r] = empty_state();
        if (i < valid) {
            const float lse = pl[(int64_t)i * p.pl_sp];
            if (lse != -INFINITY) {
                leaf[r].o = *reinterpret_cast<const float4*>(po + (int64_t)i * p.po_sp + 4 * cg);
                leaf[r].l = 1.0f;
                leaf[r].m = lse;
            }
        }
    }
    // lowest levels of the tree, in registers: stride 1, 2, ..., R/2
#pragma unroll
    for (int stride = 1; stride < R; stride <<= 1) {
#pragma unroll
        for (int r = 0; r < R; r += 2 * stride) leaf[r] = merge(leaf[r], leaf[r + stride]);
    }
    State st = leaf[0];

    // remaining levels across slots: slot s merges slot s + t when s is a multiple of 2t
#pragma unroll
    for (int t = 1; t < S; t <<= 1) {
        if ((slot & (2 * t - 1)) == t) {
            sm_o[slot][cg] = st.o;
            if (cg == 0) {
                sm_l[slot] = st.l;
                sm_m[slot] = st.m;
            }
        }
        __syncthreads();
        if ((slot & (2 * t - 1)) == 0) {
            State other;
            other.o = sm_o[slot + t][cg];
            other.l = sm_l[slot + t];
            other.m = sm_m[slot + t];
            st = merge(st, other);
        }
        __syncthreads();
    }

    if (slot == 0) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float lse = -INFINITY;
        if (st.l > 0.0f) {
            const float inv = 1.0f / st.l;
            o.x = st.o.x * inv; o.y = st.o.y * inv; o.z = st.o.z * inv; o.w = st.o.w * inv;
            lse = st.m + __log2f(st.l) * kLn2;
        }
        float* out = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + (int64_t)grp * p.out_sg;
        *reinterpret_cast<float4*>(out + 4 * cg) = o;
        if (cg == 0 && p.lse) p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)grp * p.lse_sg] = lse;
    }
}

template <int D>
hipError_t launch_d(const CombineParams& p, int B, int H, int n_groups, int leaves, hipStream_t stream) {
    constexpr int S = kThreads / (D / 4);
    dim3 grid(H, B, n_groups);
    const int r = (leaves + S - 1) / S;
    if (r <= 1) hipLaunchKernelGGL((combine_kernel<D, 1>), grid, dim3(kThreads), 0, stream, p);
    else if (r <= 2) hipLaunchKernelGGL((combine_kernel<D, 2>), grid, dim3(kThreads), 0, stream, p);
    else if (r <= 4) hipLaunchKernelGGL((combine_kernel<D, 4>), grid, dim3(kThreads), 0, stream, p);
    else if (r <= 8) hipLaunchKernelGGL((combine_kernel<D, 8>), grid, dim3(kThreads), 0, stream, p);
    else if (r <= kMaxR) hipLaunchKernelGGL((combine_kernel<D, kMaxR>), grid, dim3(kThreads), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int combine_max_leaves(int d) { return (kThreads / (d / 4)) * kMaxR; }

hipError_t launch_combine_pass(const CombineParams& p, int d, int B, int H, int n_groups,
                               int leaves_per_group, hipStream_t stream) {
    if (d == 128) return launch_d<128>(p, B, H, n_groups, leaves_per_group, stream);
    if (d == 64) return launch_d<64>(p, B, H, n_groups, leaves_per_group, stream);
    return hipErrorInvalidValue;
}

}  // namespace ta
