// Launch parameters and launchers of the two kernels behind the C ABI.
// Host-side code only includes this header; the kernels live in partial.hip and
// combine.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta {

enum class Dtype : int { F32 = 0, BF16 = 1 };

// Split-KV partial states: one workgroup per (chunk, group of heads sharing a KV head, sequence).
struct PartialParams {
    const void* q;             // [B, Hq, d]
    const void* k;             // [B, Hkv, N, d]
    const void* v;             // [B, Hkv, N, d]
    const int32_t* seqlens;    // [B] or nullptr
    float* po;                 // [B, Hq, P, d]
    float* plse;               // [B, Hq, P]
    int64_t q_sb, q_sh;        // element strides of q (batch, head)
    int64_t k_sb, k_sh, k_st;  // element strides of K (batch, kv head, token)
    int64_t v_sb, v_sh, v_st;
    int64_t po_sb, po_sh, po_sp;
    int64_t pl_sb, pl_sh, pl_sp;
    int32_t N;                 // cache capacity per sequence
    int32_t chunk;             // tokens per partial state
    int32_t group;             // query heads per KV head (Hq / Hkv)
    float scale_log2;          // log2(e) / sqrt(d)
    // 1: a chunk past its sequence's end writes the empty state (0, -inf). 0: it
    // writes nothing, for callers whose merge reads only the chunks that hold tokens.
    int32_t empty_states;
    // 1: the states are written with nontemporal stores (set by the launcher).
    int32_t stream_states;
};

// Tree merge of partial states: one workgroup per (head, sequence, group of leaves).
struct CombineParams {
    const float* po;           // [B, H, P, d]
    const float* plse;         // [B, H, P]
    int64_t po_sb, po_sh, po_sp;
    int64_t pl_sb, pl_sh, pl_sp;
    int32_t n_parts;           // leaves per row at this pass
    // ragged decode: leaves past ceil(seqlens[b] / chunk) are empty and are not read
    const int32_t* seqlens;    // [B] or nullptr
    int32_t chunk;
    int32_t N;
    // output: one state per (b, h, leaf group); the final pass has a single group
    float* out;                // [B, H, groups, d]
    float* lse;                // [B, H, groups] or nullptr
    int64_t out_sb, out_sh, out_sg;
    int64_t lse_sb, lse_sh, lse_sg;
};

// Leaves one workgroup of the merge kernel can take for head dimension d.
int combine_max_leaves(int d);

hipError_t launch_partial(const PartialParams& p, Dtype dt, int d, int heads_per_wg, int B, int Hq,
                          int n_chunks, hipStream_t stream);

// The sequential (ring-order) merge of the leading p.n_parts states of every row,
// one pass, no workspace; p.seqlens is not read.
hipError_t launch_combine_chain(const CombineParams& p, int d, int B, int H, hipStream_t stream);

// The read-bandwidth probe: streams n16 16-byte items from buf, in a launch shape
// chosen from the size and the device's `cus` compute units.
hipError_t launch_stream_read(const void* buf, int64_t n16, uint32_t* sink, int cus, hipStream_t stream);

// Leaves per workgroup of the arity-K merge: the largest power of K it takes.
int combine_k_span(int d, int arity);

// One pass of the arity-K merge tree over `n_parts` leaves per row, in groups of
// `span` (a power of K) consecutive leaves. Writes one normalised state per group.
hipError_t launch_combine_k_pass(const CombineParams& p, int d, int arity, int B, int H, int n_groups, int span,
                                 hipStream_t stream);

// One pass of the merge tree over `n_parts` leaves per row, in groups of up to
// combine_max_leaves(d) consecutive leaves. Writes one normalised state per group.
hipError_t launch_combine_pass(const CombineParams& p, int d, int B, int H, int n_groups,
                               int leaves_per_group, hipStream_t stream);

}  // namespace ta
