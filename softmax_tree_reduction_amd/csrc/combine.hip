// Merges of partial states for gfx950.
//
// Section "Core Innovation 1" step 3 of "Tree Attention Guide: Topology-Aware LLM
// Decoding" reduces the partial states up a tree of depth ceil(log_k P); section
// "Core Innovation 2" gives the merge applied at each node:
//   m = max(m_A, m_B), alpha = exp(m_A - m), beta = exp(m_B - m),
//   l = alpha l_A + beta l_B, o = alpha o_A + beta o_B,
// and the normalisation O = o / l at the root.
//
// A stored partial is normalised, (o_i, lse_i); it enters the tree as the page's
// tuple (o_i, 1, lse_i), which is the same state. A leaf with lse_i = -inf is
// the empty state (0, 0, -inf).
//
// Three kernels:
//  - combine_kernel: the binary tree (k = 2), fixed: at level t, node i merges
//    node i + 2^t whenever i is a multiple of 2^(t+1). One workgroup of 256
//    threads merges up to S * R leaves of one (sequence, head) row with the tree
//    of merge_tree.h. This is the merge of the decode path.
//  - combine_k_kernel: the same page's tree at a branching factor 2 <= K <= 16.
//  - chain_kernel: the states folded one after another, the order of a ring: the
//    baseline the tree is measured against.
// Rows with more leaves than one workgroup of a tree kernel takes are merged in
// several passes over aligned groups of leaves, each group a whole subtree, which
// is the same tree.
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
        const int pb = (int)(((unsigned)n + (unsigned)p.chunk - 1u) / (unsigned)p.chunk);  // n <= N <= INT32_MAX - chunk
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

// The tree of arity K (2 <= K <= 16) over up to `span` (a power of K) leaves of
// one row ("Core Innovation 1" step 3: depth ceil(log_K P)). At each level the
// nodes are taken in aligned groups of K consecutive nodes and each group merges
// left to right into its first node; nodes past the end of the row are empty
// states, which leave every merge bit for bit unchanged.
//
// Level 1 runs in registers: each (group, column) item reads the K leaves of its
// group and merges them (groups wholly past the end of the row are skipped: they
// are empty); a thread takes its items in batches of about 16 leaves,
// every load of a batch issued before its first merge. The span / K level-1
// nodes then go through LDS (sized to the launch), one level per barrier pair:
// every (parent, column) item reads its K children, then writes the parent.
constexpr int kKaryNodes = 64;     // most level-1 nodes of one workgroup
constexpr int kKaryBatchLoads = 16;  // leaves per thread in flight in level 1

template <int D, int K>
__global__ __launch_bounds__(kThreads) void combine_k_kernel(CombineParams p, int span) {
    constexpr int CG = D / 4;
    constexpr int kBatch = kKaryBatchLoads / K > 1 ? kKaryBatchLoads / K : 1;  // items per batch
    constexpr int kItemsL = kKaryNodes / 2 * CG / kThreads;                  // widest LDS level per thread
    extern __shared__ float4 kary_lds[];

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int grp = blockIdx.z;
    const int tid = threadIdx.x;

    int valid = p.n_parts;
    if (p.seqlens) {
        int n = p.seqlens[b];
        n = n < 0 ? 0 : (n > p.N ? p.N : n);
        const int pb = (int)(((unsigned)n + (unsigned)p.chunk - 1u) / (unsigned)p.chunk);  // n <= N <= INT32_MAX - chunk
        valid = pb < valid ? pb : valid;
    }
    const int first = grp * span;
    const int nodes = span / K;  // level-1 nodes
    // level-1 nodes holding at least one leaf of the row; the rest are empty
    // states, and skipping them skips identity merges only
    const int live = valid <= first ? 0 : ((valid - first + K - 1) / K < nodes ? (valid - first + K - 1) / K : nodes);
    float4* sm_o = kary_lds;                                         // [nodes][CG]
    float* sm_l = reinterpret_cast<float*>(kary_lds + nodes * CG);   // [nodes][CG]
    float* sm_m = sm_l + nodes * CG;                                 // [nodes][CG]
    const float* po = p.po + (int64_t)b * p.po_sb + (int64_t)h * p.po_sh;
    const float* pl = p.plse + (int64_t)b * p.pl_sb + (int64_t)h * p.pl_sh;

    // level 1: leaves enter as the page's tuples (o_i, 1, lse_i), or (0, 0, -inf)
#pragma unroll 1
    for (int base = 0; base < live * CG; base += kBatch * kThreads) {
        float lse[kBatch][K];
        float4 o[kBatch][K];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = base + tid + k * kThreads;
            const int leaf0 = first + (i / CG) * K, c = i % CG;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                lse[k][j] = -INFINITY;
                o[k][j] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (i < live * CG && leaf0 + j < valid) {
                    lse[k][j] = pl[(int64_t)(leaf0 + j) * p.pl_sp];
                    o[k][j] = *reinterpret_cast<const float4*>(po + (int64_t)(leaf0 + j) * p.po_sp + 4 * c);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = base + tid + k * kThreads;
            if (i < live * CG) {
                auto leaf = [&](int j) {
                    const bool full = lse[k][j] != -INFINITY;
                    return MState{full ? o[k][j] : make_float4(0.f, 0.f, 0.f, 0.f), full ? 1.0f : 0.0f, lse[k][j]};
                };
                MState st = leaf(0);
#pragma unroll
                for (int j = 1; j < K; ++j) st = merge_states(st, leaf(j));
                sm_o[i] = st.o;  // i = node * CG + column
                sm_l[i] = st.l;
                sm_m[i] = st.m;
            }
        }
    }
    __syncthreads();
    // levels 2 and up, in LDS (strides in level-1 nodes)
    for (int stride = 1; stride < live; stride *= K) {
        const int parents = (live + stride * K - 1) / (stride * K);
        MState st[kItemsL];
#pragma unroll
        for (int k = 0; k < kItemsL; ++k) {
            const int i = tid + k * kThreads;
            if (i < parents * CG) {
                const int at = (i / CG) * stride * K * CG + i % CG;  // first child, this column
                st[k] = {sm_o[at], sm_l[at], sm_m[at]};
#pragma unroll
                for (int j = 1; j < K; ++j) {
                    const int child = at + j * stride * CG;
                    if (child < live * CG) st[k] = merge_states(st[k], MState{sm_o[child], sm_l[child], sm_m[child]});
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kItemsL; ++k) {
            const int i = tid + k * kThreads;
            if (i < parents * CG) {
                const int at = (i / CG) * stride * K * CG + i % CG;
                sm_o[at] = st[k].o;
                sm_l[at] = st[k].l;
                sm_m[at] = st[k].m;
            }
        }
        __syncthreads();
    }
    if (tid < CG) {
        MState root{make_float4(0.f, 0.f, 0.f, 0.f), 0.0f, -INFINITY};
        if (live > 0) root = {sm_o[tid], sm_l[tid], sm_m[tid]};
        float* out = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + (int64_t)grp * p.out_sg;
        float* lse_out = p.lse ? p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)grp * p.lse_sg : nullptr;
        write_root(root, out, lse_out);
    }
}

// Largest power of K whose level-1 nodes (span / K) fit kKaryNodes.
template <int K>
int kary_span() {
    int span = K;
    while (span <= kKaryNodes) span *= K;  // span * K has span level-1 nodes
    return span;
}

template <int D, int K>
hipError_t launch_kary(const CombineParams& p, int B, int H, int n_groups, int span, hipStream_t stream) {
    if (span < K || span > kary_span<K>() || span % K) return hipErrorInvalidValue;
    const size_t lds = (size_t)(span / K) * (D / 4) * (sizeof(float4) + 2 * sizeof(float));
    hipLaunchKernelGGL((combine_k_kernel<D, K>), dim3(H, B, n_groups), dim3(kThreads), lds, stream, p, span);
    return hipGetLastError();
}

template <int D, int K = 2>
hipError_t dispatch_kary(int arity, const CombineParams& p, int B, int H, int n_groups, int span, hipStream_t stream) {
    if (arity == K) return launch_kary<D, K>(p, B, H, n_groups, span, stream);
    if constexpr (K < 16) return dispatch_kary<D, K + 1>(arity, p, B, H, n_groups, span, stream);
    return hipErrorInvalidValue;
}

template <int K = 2>
int span_kary(int arity) {
    if (arity == K) return kary_span<K>();
    if constexpr (K < 16) return span_kary<K + 1>(arity);
    return 0;
}

// The order in which a ring of P workers accumulates ([guide] "The Flaw of Ring
// Attention During Autoregressive Decoding": P - 1 sequential hops): the running
// state takes in one partial state per step, ((s_0 (+) s_1) (+) s_2) (+) ..., a
// chain of P - 1 dependent merges against the tree's ceil(log2 P) levels. It is
// the baseline the tree is measured against.
// One thread per (row, float4 column), kThreads / (D / 4) rows of one sequence per
// workgroup; the loads of the next batch of leaves are issued before the current
// batch is merged. Leaves past the end of the row are empty states, which leave
// the running state bit for bit unchanged.
template <int D>
__global__ __launch_bounds__(kThreads) void chain_kernel(CombineParams p, int H) {
    constexpr int CG = D / 4;
    constexpr int kRows = kThreads / CG;
    constexpr int kBatch = 8;
    const int h = blockIdx.x * kRows + (int)threadIdx.x / CG;
    const int b = blockIdx.y;
    const int c = threadIdx.x % CG;
    if (h >= H) return;  // no barrier below
    const int valid = p.n_parts;
    const float* po = p.po + (int64_t)b * p.po_sb + (int64_t)h * p.po_sh + 4 * c;
    const float* pl = p.plse + (int64_t)b * p.pl_sb + (int64_t)h * p.pl_sh;

    float lse_n[kBatch];
    float4 o_n[kBatch];
    auto load = [&](int base) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            lse_n[j] = -INFINITY;
            o_n[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (base + j < valid) {
                lse_n[j] = pl[(int64_t)(base + j) * p.pl_sp];
                o_n[j] = *reinterpret_cast<const float4*>(po + (int64_t)(base + j) * p.po_sp);
            }
        }
    };
    MState st{make_float4(0.f, 0.f, 0.f, 0.f), 0.0f, -INFINITY};
    load(0);
    for (int base = 0; base < valid; base += kBatch) {
        float lse_c[kBatch];
        float4 o_c[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            lse_c[j] = lse_n[j];
            o_c[j] = o_n[j];
        }
        load(base + kBatch);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const bool full = lse_c[j] != -INFINITY;
            const MState leaf{full ? o_c[j] : make_float4(0.f, 0.f, 0.f, 0.f), full ? 1.0f : 0.0f, lse_c[j]};
            st = (base == 0 && j == 0) ? leaf : merge_states(st, leaf);
        }
    }
    float* out = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh;
    float* lse = p.lse ? p.lse + (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh : nullptr;
    write_root(st, out, lse, c);
}

}  // namespace

hipError_t launch_combine_chain(const CombineParams& p, int d, int B, int H, hipStream_t stream) {
    if (d == 128) {
        hipLaunchKernelGGL(chain_kernel<128>, dim3((H + 7) / 8, B), dim3(kThreads), 0, stream, p, H);
    } else if (d == 64) {
        hipLaunchKernelGGL(chain_kernel<64>, dim3((H + 15) / 16, B), dim3(kThreads), 0, stream, p, H);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int combine_max_leaves(int d) { return (kThreads / (d / 4)) * kMaxR; }

int combine_k_span(int d, int arity) {
    return d == 128 || d == 64 ? span_kary(arity) : 0;
}

hipError_t launch_combine_k_pass(const CombineParams& p, int d, int arity, int B, int H, int n_groups, int span,
                                 hipStream_t stream) {
    if (d == 128) return dispatch_kary<128>(arity, p, B, H, n_groups, span, stream);
    if (d == 64) return dispatch_kary<64>(arity, p, B, H, n_groups, span, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_combine_pass(const CombineParams& p, int d, int B, int H, int n_groups,
                               int leaves_per_group, hipStream_t stream) {
    if (d == 128) return launch_d<128>(p, B, H, n_groups, leaves_per_group, stream);
    if (d == 64) return launch_d<64>(p, B, H, n_groups, leaves_per_group, stream);
    return hipErrorInvalidValue;
}

}  // namespace ta
