/*
 * tree_attn.h - C ABI of the single-GPU Tree Attention decode path (gfx950).
 *
 * What is computed. One decode step of exact softmax attention: for every
 * sequence b and query head h, a single query q[b,h,:] attends to the first
 * n_b keys and values of its KV head,
 *
 *     s_j = q . K_j / sqrt(d),   out = sum_j softmax(s)_j V_j,   lse = ln sum_j exp(s_j),
 *
 * ("Tree Attention Guide: Topology-Aware LLM Decoding", section "Core
 * Innovation 2: Mathematical Formulation of Online Softmax on Trees", the
 * softmax with a global maximum; the 1/sqrt(d) scale is the one the same
 * page's worker listing applies to its scores). The keys are cut into chunks
 * of `chunk` tokens. Each chunk yields a partial state (running max m, sum of
 * exponentials l, weighted value sum o), as in section "Core Innovation 1",
 * step 2 of that page; the partial states are merged by the page's merge
 * operator (m = max, rescale by exp(m_A - m) and exp(m_B - m), add) as a
 * binary tree of depth ceil(log2 P) (section "Core Innovation 1", step 3),
 * and the root is normalised, O = o / l (end of "Core Innovation 2").
 *
 * Conventions shared by every entry point:
 *  - Tensors are passed as host-side ta_tensor descriptors whose `data`
 *    points to device memory on the current HIP device (it may be NULL for a
 *    tensor with no elements, which is never accessed). The descriptors are
 *    read during the call only; the library keeps no pointer after it returns.
 *    The caller owns every tensor.
 *  - Strides are in elements, never negative. In q, k, v, out and partial_o the
 *    last dimension (the head dimension d) must be contiguous (stride 1) and
 *    every row start 16-byte aligned; lse and partial_lse take any strides.
 *  - Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 *  - The log-sum-exp is a natural logarithm. A sequence with no tokens (and a
 *    partial state of an empty chunk) has out = 0 and lse = -inf.
 *  - A partial state is stored normalised: o_i = o / l (the softmax-weighted
 *    mean of V over the chunk) and lse_i = m + ln l. This is the same state as
 *    the page's (o, l, m): (o_i, 1, lse_i) merges exactly like it.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without waiting for it. Inputs must stay
 *    valid and unmodified until the stream reaches the work.
 *  - Outputs must not alias inputs.
 *  - Results are bitwise reproducible for the same inputs, shapes and chunk
 *    (fixed reduction order, no atomics).
 *
 * Errors: a negative return code means nothing was enqueued (argument
 * validation happens before any launch) or, for TA_ERR_HIP, that the HIP
 * runtime refused an allocation or a launch. ta_last_error() returns a
 * message for the most recent non-zero return on the calling thread.
 * Faults during execution surface on the stream, as for any HIP kernel.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TA_MAX_DIMS 4

typedef enum ta_dtype {
    TA_F32 = 0,   /* IEEE binary32 */
    TA_BF16 = 1   /* bfloat16: the upper 16 bits of a binary32 */
} ta_dtype;

typedef struct ta_tensor {
    void* data;                    /* device pointer */
    int32_t dtype;                 /* ta_dtype */
    int32_t ndim;                  /* number of used entries in shape/stride */
    int64_t shape[TA_MAX_DIMS];
    int64_t stride[TA_MAX_DIMS];   /* in elements */
} ta_tensor;

enum {
    TA_OK = 0,
    TA_ERR_NULL = -1,         /* a required pointer or descriptor is NULL */
    TA_ERR_SHAPE = -2,        /* wrong ndim, or shapes that do not agree */
    TA_ERR_DTYPE = -3,        /* unsupported or mismatched dtype */
    TA_ERR_STRIDE = -4,       /* d not contiguous, or a row not 16-byte aligned */
    TA_ERR_ARG = -5,          /* chunk < 1, n_parts out of range, ... */
    TA_ERR_UNSUPPORTED = -6,  /* a head dimension or size the library has no kernel for */
    TA_ERR_HIP = -7           /* the HIP runtime returned an error */
};

/*
 * ta_decode - one decode step: partial states per chunk, tree merge, output.
 *
 *   q        [B, Hq, d]      bf16 or f32 (the query of every head)
 *   k, v     [B, Hkv, N, d]  same dtype as q; N is the cache capacity per sequence
 *   seqlens  device int32[B], the number of valid tokens of each sequence
 *            (0 <= n_b <= N; values outside are clamped to that range), or
 *            NULL for n_b = N. Keys and values at or past n_b are never read.
 *   out      [B, Hq, d]      f32, the attention output
 *   lse      [B, Hq]         f32, natural-log log-sum-exp of the logits, or NULL
 *   chunk    tokens per partial state, >= 1
 *
 * Supported: d in {64, 128}; Hq a multiple of Hkv; B <= 65535; Hq <= 65535;
 * a token stride of k and v below 256 MiB; P = ceil(N / chunk) <= 65535 * 128
 * (d = 128) or 65535 * 256 (d = 64), the states one merge pass takes
 * (TA_ERR_UNSUPPORTED beyond any of these).
 * Needs about Hq * P * (d + 1) * 4 bytes of device workspace per sequence
 * (P = ceil(N / chunk)). The library keeps one workspace buffer per (device,
 * stream), allocated with hipMallocAsync on that stream the first time it is
 * needed and grown when a call needs more; it is held until the process ends.
 * Host threads may call concurrently, on the same stream or on different
 * ones: a call holds its stream's buffer from its first launch until it
 * returns, so the kernels of concurrent calls on one stream are enqueued back
 * to back (in an unspecified order) and never read each other's partial
 * states. While the stream is being captured into a graph the workspace is
 * allocated and released inside the captured work instead.
 */
int ta_decode(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v,
              const int32_t* seqlens, const ta_tensor* out, const ta_tensor* lse,
              int32_t chunk, void* stream);

/*
 * ta_decode_noalloc - ta_decode for callers that cannot allocate device memory
 * (code under graph capture, serving loops or harnesses that forbid hipMalloc).
 *
 * Arguments, semantics, supported sizes and results are those of ta_decode,
 * bit for bit (the same kernels run). The partial states and the merge's
 * scratch live in one static device array of 64 MiB (67108864 bytes) held by
 * every device the library runs on, from the library's first use on it until
 * the process ends, instead of in library workspace. The call allocates and
 * frees nothing. A step needs about B * Hq * P * (d + 1) * 4 bytes of it
 * (P = ceil(N / chunk)); a call needing more than 64 MiB returns
 * TA_ERR_UNSUPPORTED before any launch. Nothing in the array needs clearing
 * between calls: every state a call reads it has written first.
 * Every call on one device uses the same array: two calls whose work can
 * overlap on the device (on different streams with no ordering between them)
 * race and give wrong results. Calls from several host threads on one stream
 * are serialised by the library and do not race.
 */
int ta_decode_noalloc(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v,
                      const int32_t* seqlens, const ta_tensor* out, const ta_tensor* lse,
                      int32_t chunk, void* stream);

/*
 * ta_combine - merge n_parts partial states per row by the binary tree, then
 * normalise ("Core Innovation 1" step 3 and "Core Innovation 2" of the page).
 *
 *   partial_o    [B, H, P, d] f32 (normalised partial outputs o_i)
 *   partial_lse  [B, H, P]    f32 (natural-log lse_i; -inf marks an empty state,
 *                whose o_i is then ignored)
 *   n_parts      number of leading states to merge, 0 <= n_parts <= P
 *                (0 gives out = 0, lse = -inf)
 *   out          [B, H, d] f32;  lse [B, H] f32 or NULL
 *
 * Leaf i covers the i-th state; level t of the tree merges node i with node
 * i + 2^t for every i that is a multiple of 2^(t+1) (a node without a partner
 * passes up unchanged), giving ceil(log2 n_parts) levels.
 * Supported: d in {64, 128}; n_parts <= 65535 * 128 (d = 128) or 65535 * 256
 * (d = 64). n_parts above 128 (d = 128) or 256 (d = 64) runs the same tree in
 * several launches and takes workspace as ta_decode does.
 */
int ta_combine(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts,
               const ta_tensor* out, const ta_tensor* lse, void* stream);

/*
 * ta_combine_k - ta_combine with a tree of branching factor `arity` (the page's
 * k, "Core Innovation 1" step 3: ceil(log_k n_parts) levels).
 *
 *   arity        2 <= arity <= 16; other arguments as for ta_combine.
 *
 * At each level the nodes are taken in aligned groups of `arity` consecutive
 * nodes; each group merges left to right into its first node, and a group cut
 * short by the end of the row merges the nodes it has. Arity 2 is the tree of
 * ta_combine. One launch merges up to arity^j leaves per row, the largest
 * power with arity^(j-1) <= 64 (81 to 512 leaves); longer rows run the same tree in
 * several launches, one per aligned group of that many leaves and then over
 * the group roots, and take workspace as ta_decode does; at most 65535 such
 * groups per row. Errors: TA_ERR_ARG for an arity outside [2, 16], otherwise
 * as ta_combine.
 */
int ta_combine_k(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts, int32_t arity,
                 const ta_tensor* out, const ta_tensor* lse, void* stream);

/*
 * ta_combine_chain - the same merge in the order a ring of workers accumulates
 * it ("The Flaw of Ring Attention During Autoregressive Decoding" in the guide
 * page: P - 1 sequential hops): out = ((s_0 + s_1) + s_2) + ... + s_{n_parts-1}
 * under the merge operator, a chain of n_parts - 1 dependent merges where the
 * tree has ceil(log2 n_parts) levels. A baseline for the tree, not a faster
 * path. Arguments as for ta_combine; one launch for any n_parts, no workspace.
 */
int ta_combine_chain(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts,
                     const ta_tensor* out, const ta_tensor* lse, void* stream);

/*
 * ta_partial - the per-chunk partial states alone (the first half of ta_decode).
 *
 * Arguments as for ta_decode, with the outputs
 *   partial_o    [B, Hq, P, d] f32, P >= ceil(N / chunk)
 *   partial_lse  [B, Hq, P]    f32
 * Chunk i of sequence b covers tokens [i*chunk, min((i+1)*chunk, n_b)); a
 * chunk with no tokens gets o_i = 0 and lse_i = -inf. Entries i >= ceil(N/chunk)
 * are not written, except that an empty cache (N = 0) writes the empty state
 * to entry 0 of every row when P >= 1 (the one state ta_decode merges then).
 * ta_combine over these states (ceil(N/chunk) of them, or 1 when N = 0)
 * equals ta_decode bit for bit. Allocates nothing.
 */
int ta_partial(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v,
               const int32_t* seqlens, const ta_tensor* partial_o, const ta_tensor* partial_lse,
               int32_t chunk, void* stream);

/*
 * ta_stream_read - measurement utility, not part of the decode path: reads
 * `bytes` bytes of device memory at `buf` once, with 16-byte nontemporal loads
 * (the width and cache policy of the partial kernel's K and V loads), and
 * computes nothing from them.
 * Timing it gives the device's practical read ceiling for this access. Buffers
 * of up to 256 KiB per compute unit are read by one round of workgroups of
 * 32 KiB each (every load in flight at once); larger ones by one workgroup per
 * compute unit, each streaming one contiguous slice.
 *
 *   buf     device pointer, 16-byte aligned; bytes >= 0, a multiple of 16
 *   sink    device pointer to one uint32 that the probe may overwrite
 *   stream  hipStream_t (NULL = default stream); asynchronous
 *
 * Returns TA_ERR_NULL or TA_ERR_ARG (size or alignment) without launching,
 * TA_ERR_HIP on a launch failure, with the message in ta_last_error.
 */
int ta_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * ta_suggest_chunk - a chunk for ta_decode or ta_partial that gives the partial
 * kernel about one workgroup per compute unit, which measured fastest on
 * batches whose sequences all hold n tokens: the largest power of two, at
 * least 64 and at most n, for which
 *     batch x head groups x ceil(n / chunk) >= compute units,
 * where head groups = q_heads / (the largest of 8, 4, 2, 1 dividing
 * q_heads / kv_heads). In ragged batches the short sequences leave such a grid
 * partly idle, and a smaller chunk does better. The chunk is the merge tree's
 * leaf, so the choice changes the rounding of the result, never its meaning.
 *
 *   batch, q_heads, kv_heads, n   as in ta_decode (n: tokens per sequence)
 *   compute_units                 > 0, or 0 for the current device's count
 *
 * Returns the chunk (>= 64), or TA_ERR_ARG for a size below 1 or q_heads not a
 * multiple of kv_heads, or TA_ERR_HIP when the device cannot be queried, with
 * the message in ta_last_error. Launches nothing.
 */
int32_t ta_suggest_chunk(int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t n, int32_t compute_units);

/* Message for the last non-zero return on this thread ("" if none). Never NULL. */
const char* ta_last_error(void);

/* ABI version, currently 1. */
int ta_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
