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
// row with the tree of merge_tree.h. Rows with more leaves than one workgroup
// takes are merged in several passes over aligned groups of leaves, which is the
// same tree.
#include "kernels.h"
#include "merge_tree.h"

namespace ta {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxR = 16;

template <int D, int R>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
    constexpr int S = kThreads / (D / 4);
    constexpr int SPAN = S * R;  // leaves per workgroup
    __shared__ MergeSmem<D, kThreads> sm;

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int grp = blockIdx.z;

    // leaves that can hold tokens in this row
    int valid = p.n_parts;
    if (p.seqlens) {
        int n = p.seqlens[b];
        n = n < 0 ? 0 : (n > p.N ? p.N : n);
        const int pb = (int)(((int64_t)n + p.chunk - 1) / p.chunk);
        valid = pb < valid ? pb : valid;
    }
    const float* po = p.po + (int64_t)b * p.po_sb + (int64_t)h * p.po_sh;
    const float* pl = p.plse + (int64_t)b * p.pl_sb + (int64_t)h * p.pl_sh;
    const MState st = tree_merge_row<D, R, kThreads>(po, p.po_sp, pl, p.pl_sp, grp * SPAN, valid, sm);
    if (threadIdx.x < D / 4) {
        float* out = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + (int64_t)grp * p.out_sg;
        float* lse = p.lse ? p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)grp * p.lse_sg : nullptr;
        write_root(st, out, lse);
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
