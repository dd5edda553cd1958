// Split-KV partial-state kernel for gfx950.
//
// Computes, for one chunk of the KV cache and the G query heads that share its
// KV head, the partial state of section "Core Innovation 1" step 2 of "Tree
// Attention Guide: Topology-Aware LLM Decoding": the maximum logit m, the sum of
// exponentials l = sum exp(s_j - m) and the weighted sum o = sum exp(s_j - m) V_j,
// with s_j = q . K_j / sqrt(d). It writes the state normalised, (o / l, m + ln l).
//
// Layout of the work (one workgroup = one chunk x one head group x one sequence):
//  - A K or V row of d elements is 256 bytes for bf16 d = 128 (or f32 d = 64). A
//    wave reads it as 16-byte segments, one per lane, so SEGS = row / 16 lanes hold
//    one row and a wave-wide load covers RG = 64 / SEGS consecutive rows (1 KB,
//    fully coalesced). Each lane keeps its segment of q for every head of the group.
//  - Per token, each lane forms the partial dot products of its segment with the G
//    query segments (bf16 pairs through v_dot2_f32_bf16), and a DPP reduce-scatter
//    inside the SEGS-lane row sums them by head: each lane ends with the logit of
//    one head (lane mod G) for its tokens.
//  - The running max, the rescale of the accumulators and the exponentials follow
//    the page's merge operator, once per block of TPL tokens per lane, in base 2
//    (exp(x) = 2^(x log2 e), the log2 e folded into the logit scale); each lane
//    exponentiates only its own head's logits.
//  - V rows arrive in the same lane layout, so each lane accumulates the G heads
//    for its own 16-byte slice of channels, each token's weight broadcast from a
//    lane that holds its head.
//  - The K/V rows of one block are in flight while the previous block is computed
//    (two register buffers per lane). The GQA group shares every byte read: each
//    K/V element is loaded once and used by all G heads.
//  - Each wave walks the chunk in blocks of RG x TPL tokens, interleaved with the
//    other waves (4 per workgroup, 8 when the grid has fewer workgroups than the
//    device has compute units). At the end the row groups of a wave, then the
//    waves, are merged with the same operator (shuffles, then LDS) and the state
//    is written.
//  - A chunk past its sequence's end does no work. Its empty state, when the
//    caller reads it, is written by the row's non-empty workgroups. Grids of many
//    rounds of workgroups write the states with nontemporal stores, and ragged ones
//    among them run two workgroups per CU instead of three.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

// Launch shape: waves per workgroup, tokens per lane per block, blocks in the register ring.
// TA_PARTIAL_WAVES is the workgroup size of grids that fill the device; grids with
// fewer workgroups than compute units take TA_PARTIAL_WAVES_SMALL waves each.
#ifndef TA_PARTIAL_WAVES
#define TA_PARTIAL_WAVES 4
#endif
#ifndef TA_PARTIAL_WAVES_SMALL
#define TA_PARTIAL_WAVES_SMALL 8
#endif
#ifndef TA_PARTIAL_TPL
#define TA_PARTIAL_TPL 4
#endif
#ifndef TA_PARTIAL_NBUF
#define TA_PARTIAL_NBUF 2
#endif

namespace ta {
namespace {

// Most chunks one workgroup of the several-chunks kernel streams. Its LDS holds one
// set of wave states per chunk until the end, slots x 4 waves x GT x D floats: 128 KiB
// at 16 slots with GT = 4 (d = 128), of the 160 KiB a CU has. Workgroups of 8 heads
// do not take several chunks: that kernel needs 256 VGPRs and spills into AGPRs, and
// measured 19-22% slower than the per-chunk grid on GQA 8:1 shapes where it applied
// (64 query heads, 8 KV heads; 320k-768k tokens, chunks 2048-8192, 3 and 5 chunks
// per workgroup, d = 64 and 128).
template <int GT>
constexpr int max_chunks_per_wg() { return GT <= 4 ? 16 : 0; }

// Shortest stream (tokens per workgroup) for which a workgroup takes several chunks.
constexpr int64_t kMultiMinTokens = 8192;

// LDS a launch of the per-chunk kernel reserves beyond its own, unused, so that at
// most two workgroups share a CU (with the kernel's own 8 KiB at GT = 4 and d = 128,
// two take 137 KiB of the CU's 160 KiB, three would need 205). Ragged grids of many
// rounds (seqlens given, more than 8 workgroups per CU on the grid) streamed
// 0.2-1.1% faster with two resident workgroups than with the three the registers
// allow (bf16, d = 128, GQA 4:1: batches of 2 to 64 sequences, chunks 512 to 4096),
// and never slower.
constexpr unsigned kTwoPerCuLds = 60u << 10;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Storage;
template <>
struct Storage<uint16_t> {  // bfloat16 bits
    static constexpr int kElems = 8;
};
template <>
struct Storage<float> {
    static constexpr int kElems = 4;
};

// Partial dot product of one 16-byte segment of q with one of K.
template <typename T>
__device__ __forceinline__ float seg_dot(const uint4& qs, const uint4& ks);

template <>
__device__ __forceinline__ float seg_dot<uint16_t>(const uint4& qs, const uint4& ks) {
    // the first pair in the three-operand form with a zero accumulator (the compiler's
    // choice, the accumulating two-operand form, needs a separate zeroing move)
    float acc;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(qs.x), "v"(ks.x));
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qs.y), __builtin_bit_cast(bf16x2, ks.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qs.z), __builtin_bit_cast(bf16x2, ks.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qs.w), __builtin_bit_cast(bf16x2, ks.w), acc, false);
    return acc;
}

template <>
__device__ __forceinline__ float seg_dot<float>(const uint4& qs, const uint4& ks) {
    float acc = __uint_as_float(qs.x) * __uint_as_float(ks.x);
    acc = fmaf(__uint_as_float(qs.y), __uint_as_float(ks.y), acc);
    acc = fmaf(__uint_as_float(qs.z), __uint_as_float(ks.z), acc);
    acc = fmaf(__uint_as_float(qs.w), __uint_as_float(ks.w), acc);
    return acc;
}

// Widen one 16-byte segment of V to float.
template <typename T>
__device__ __forceinline__ void seg_widen(const uint4& s, float (&f)[Storage<T>::kElems]);

template <>
__device__ __forceinline__ void seg_widen<uint16_t>(const uint4& s, float (&f)[8]) {
    f[0] = bf16_lo(s.x); f[1] = bf16_hi(s.x);
    f[2] = bf16_lo(s.y); f[3] = bf16_hi(s.y);
    f[4] = bf16_lo(s.z); f[5] = bf16_hi(s.z);
    f[6] = bf16_lo(s.w); f[7] = bf16_hi(s.w);
}

template <>
__device__ __forceinline__ void seg_widen<float>(const uint4& s, float (&f)[4]) {
    f[0] = __uint_as_float(s.x); f[1] = __uint_as_float(s.y);
    f[2] = __uint_as_float(s.z); f[3] = __uint_as_float(s.w);
}

// One wave-wide load of 16-byte segments through a buffer resource whose base is the
// load's first row (wave-uniform, in scalar registers) and whose range is the `span`
// bytes the load covers; `off` is this lane's offset from that row. The address sum
// happens in the load unit: a global load would need a 64-bit vector add per lane
// first, because the compiler folds the lane offset into a per-lane pointer. A lane
// offset past the span would read zeros instead of other memory. Nontemporal, like
// load_stream. The fourth word of the resource, 0x00020000, is the gfx9 family's
// setting for untyped 32-bit data.
__device__ __forceinline__ uint4 load_rows(const char* row0, uint32_t span, uint32_t off) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row0), (short)0, (int)span, 0x00020000);
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, TA_STREAM_NT ? 2 : 0);
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ const uint4* row_ptr(const char* base, int64_t row, int64_t row_bytes) {
    return reinterpret_cast<const uint4*>(base + row * row_bytes);
}

// Writes one head's 16-byte slice of o and, from the lane of slice 0, its lse.
// Nontemporal stores when `stream` is set: in grids of many rounds of workgroups
// most states are written while other workgroups are still streaming K and V, and
// ordinary write-back stores then cost the stream more than the bytes they carry.
__device__ __forceinline__ void store_state(float* o_ptr, float* lse_ptr, float4 o, float lse, bool first,
                                            bool stream) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    if (stream) {
        const f32x4 v = {o.x, o.y, o.z, o.w};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o_ptr));
        if (first) __builtin_nontemporal_store(lse, lse_ptr);
    } else {
        *reinterpret_cast<float4*>(o_ptr) = o;
        if (first) *lse_ptr = lse;
    }
}

// The partial state of tokens [c0, c1) (c0 < c1) for the GT heads from h0, written to
// po / pl (already offset to this sequence, head h0 and chunk).
// MULTI: [c0, c1) is instead nc (<= max_chunks_per_wg) consecutive whole chunks of
// p.chunk tokens, each a whole number of rounds of NW blocks. Each wave walks all of
// them in one stream; at the end of each chunk it leaves its part of that chunk's
// state in LDS and streams on, with no barrier. After the last chunk the workgroup
// merges the waves' parts of every chunk and writes chunk j's state to po + j * p.po_sp,
// pl + j * p.pl_sp. Every wave takes the same blocks of each chunk, in the same order,
// as it would for that chunk alone, and the merges are the same, so the states are
// the same bits.
template <typename T, int D, int GT, int NW, int TPL, int NBUF, bool MULTI = false>
__device__ __forceinline__ void chunk_state(const PartialParams& p, int b, int h0, int g, int64_t c0, int64_t c1,
                                            float* po, float* pl, int nc = 1) {
    constexpr int E = Storage<T>::kElems;  // elements per 16-byte segment
    constexpr int SEGS = D / E;            // lanes per row
    constexpr int RG = kWave / SEGS;       // rows per wave-wide load
    constexpr int BT = RG * TPL;           // tokens per wave block
    static_assert(SEGS >= 8 && SEGS <= 32 && RG * SEGS == kWave, "row layout");

    constexpr int SLOTS = MULTI ? max_chunks_per_wg<GT>() : 1;  // chunks whose wave states wait in LDS
    __shared__ float sm_acc[SLOTS][NW][GT][D];
    __shared__ float sm_m[SLOTS][NW][GT];
    __shared__ float sm_l[SLOTS][NW][GT];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int seg = lane % SEGS;
    const int rg = lane / SEGS;

    // the value held by the lanes of this row whose head is h (lane h of the row)
    auto bcast_head = [](float x, int h) -> float {
        if constexpr (GT == 1) return x;
        switch (h) {
            case 0: return group_bcast<0, SEGS>(x);
            case 1: return group_bcast<1, SEGS>(x);
            case 2: return group_bcast<2, SEGS>(x);
            case 3: return group_bcast<3, SEGS>(x);
            case 4: return group_bcast<4, SEGS>(x);
            case 5: return group_bcast<5, SEGS>(x);
            case 6: return group_bcast<6, SEGS>(x);
            default: return group_bcast<7, SEGS>(x);
        }
    };

    // this lane's 16-byte segment of q for each head of the group, register r holding
    // head r ^ (lane & (GT - 1)) (the order row_reduce_scatter expects)
    uint4 qs[GT];
    {
        const char* qb = reinterpret_cast<const char*>(p.q) + ((int64_t)b * p.q_sb + (int64_t)h0 * p.q_sh) * (int64_t)sizeof(T);
#pragma unroll
        for (int r = 0; r < GT; ++r) {
            const int h = r ^ (lane & (GT - 1));
            qs[r] = *reinterpret_cast<const uint4*>(qb + (int64_t)h * p.q_sh * (int64_t)sizeof(T) + seg * 16);
        }
    }

    // Row addresses: a wave-uniform base (scalar registers) for each row of a block plus
    // this lane's 32-bit offset inside its row group (row stride x row-group index +
    // 16-byte segment). Full blocks load through buffer resources built on that base
    // (load_rows), so the address sum happens in the load unit and a full block costs
    // no per-lane address arithmetic.
    const int64_t ks_bytes = p.k_st * (int64_t)sizeof(T);
    const int64_t vs_bytes = p.v_st * (int64_t)sizeof(T);
    const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)b * p.k_sb + (int64_t)g * p.k_sh) * (int64_t)sizeof(T);
    const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)b * p.v_sb + (int64_t)g * p.v_sh) * (int64_t)sizeof(T);
    const uint32_t koff = (uint32_t)(rg * ks_bytes) + (uint32_t)(seg * 16);
    const uint32_t voff = (uint32_t)(rg * vs_bytes) + (uint32_t)(seg * 16);
    // bytes one wave-wide load spans from its first row: RG rows of the tensor's stride
    // (below 2 GiB, as the token stride is below 256 MiB)
    const uint32_t k_span = (uint32_t)((RG - 1) * ks_bytes) + (uint32_t)(D * sizeof(T));
    const uint32_t v_span = (uint32_t)((RG - 1) * vs_bytes) + (uint32_t)(D * sizeof(T));

    // Running state of this lane's row group. The lane keeps the running max and sum
    // of head (lane & (GT - 1)) (every lane of the row holding that head keeps the same
    // values) and the weighted V sums of all GT heads for its own channels.
    float m_own = -INFINITY, l_own = 0.0f, acc[GT][E];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;

    const int64_t last = c1 - 1;
    // A full block (t0 wave-uniform): uniform row bases plus this lane's offset.
    auto load_full = [&](int64_t t0, uint4 (&kb)[TPL], uint4 (&vb)[TPL]) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const char* kr = kbase + (t0 + j * RG) * ks_bytes;
            const char* vr = vbase + (t0 + j * RG) * vs_bytes;
            kb[j] = load_rows(kr, k_span, koff);
            vb[j] = load_rows(vr, v_span, voff);
        }
    };
    // The chunk's last, partial block: rows past its end are clamped to its last row
    // (always valid memory) and weighted 0.
    auto load_tail = [&](int64_t t0, uint4 (&kb)[TPL], uint4 (&vb)[TPL]) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            int64_t t = t0 + j * RG + rg;
            t = t < last ? t : last;
            kb[j] = load_stream(row_ptr(kbase + seg * 16, t, ks_bytes));
            vb[j] = load_stream(row_ptr(vbase + seg * 16, t, vs_bytes));
        }
    };

    // One block: the logits of the lane's TPL tokens for its own head, the page's
    // merge of the block into the running state (skipped when no lane's maximum
    // grew, when every rescale factor is exactly 1), then the weighted V sums of
    // all GT heads, each token's weight broadcast from a lane that holds its head.
    const float c = p.scale_log2;
    auto compute_block = [&](auto masked, int64_t t0, const uint4 (&kb)[TPL], const uint4 (&vb)[TPL]) {
        float sj[TPL];  // raw q.k of token j for the lane's head
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            float d[GT];
#pragma unroll
            for (int r = 0; r < GT; ++r) d[r] = seg_dot<T>(qs[r], kb[j]);
            row_reduce_scatter<GT, SEGS>(d);
            sj[j] = d[0];
        }
        if constexpr (decltype(masked)::value) {  // tokens past the chunk's end weigh 0
#pragma unroll
            for (int j = 0; j < TPL; ++j)
                if (t0 + j * RG + rg > last) sj[j] = -INFINITY;
        }
        float bm = sj[0];
#pragma unroll
        for (int j = 1; j < TPL; ++j) bm = fmaxf(bm, sj[j]);
        const float mn = fmaxf(m_own, bm * c);  // c > 0: the max of the scaled logits
        if (__builtin_amdgcn_ballot_w64(mn > m_own)) {
            const float alpha = exp2_fast(m_own - ((mn == -INFINITY) ? 0.0f : mn));
            l_own *= alpha;
            m_own = mn;
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                const float ah = bcast_head(alpha, h);
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] *= ah;
            }
        }
        const float nref = (m_own == -INFINITY) ? 0.0f : -m_own;
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            sj[j] = exp2_fast(fmaf(sj[j], c, nref));  // the weight 2^(s c - m)
            l_own += sj[j];
        }
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            float vf[E];
            seg_widen<T>(vb[j], vf);
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                const float pw = bcast_head(sj[j], h);
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pw, vf[e], acc[h][e]);
            }
        }
    };

    // The end of a chunk, in two halves. park: this wave merges its row groups (lanes
    // that hold the same channels) with the page's operator, leaves the result in LDS
    // slot `slot` and starts a fresh state; no other wave is waited for. finish: after
    // one barrier, the waves' states of each slot are merged and written, normalised,
    // to (po_j, pl_j).
    auto park = [&](int slot) {
        // every head's running max and sum, in every lane of the row
        float m[GT], l[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            m[h] = bcast_head(m_own, h);
            l[h] = bcast_head(l_own, h);
        }

        // merge the row groups of this wave (lanes that hold the same channels)
#pragma unroll
        for (int off = SEGS; off < kWave; off <<= 1) {
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                const float mo = xor_lanes(m[h], off);
                const float lo = xor_lanes(l[h], off);
                const Rescale r = merge_factors(m[h], mo);
                l[h] = r.a * l[h] + r.b * lo;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float ao = xor_lanes(acc[h][e], off);
                    acc[h][e] = r.a * acc[h][e] + r.b * ao;
                }
                m[h] = r.m;
            }
        }

        // and leave it in LDS for the merge across the waves
        if (rg == 0) {
#pragma unroll
            for (int h = 0; h < GT; ++h) {
#pragma unroll
                for (int e = 0; e < E; ++e) sm_acc[slot][wave][h][seg * E + e] = acc[h][e];
                if (seg == 0) {
                    sm_m[slot][wave][h] = m[h];
                    sm_l[slot][wave][h] = l[h];
                }
            }
        }
        m_own = -INFINITY;
        l_own = 0.0f;
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    };
    auto finish = [&](int slot, float* po_j, float* pl_j) {
        for (int i = tid; i < GT * (D / 4); i += NW * kWave) {
            const int h = i / (D / 4), c4 = i % (D / 4);
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[slot][w][h]);
            const float ref = (M == -INFINITY) ? 0.0f : M;
            float L = 0.0f;
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = exp2_fast(sm_m[slot][w][h] - ref);
                L += f * sm_l[slot][w][h];
                o.x += f * sm_acc[slot][w][h][4 * c4 + 0];
                o.y += f * sm_acc[slot][w][h][4 * c4 + 1];
                o.z += f * sm_acc[slot][w][h][4 * c4 + 2];
                o.w += f * sm_acc[slot][w][h][4 * c4 + 3];
            }
            float lse = -INFINITY;
            if (L > 0.0f) {
                const float inv = 1.0f / L;
                o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
                lse = (M + __log2f(L)) * kLn2;
            } else {
                o = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            store_state(po_j + (int64_t)h * p.po_sh + 4 * c4, pl_j + (int64_t)h * p.pl_sh, o, lse, c4 == 0,
                        p.stream_states != 0);
        }
    };

    // Full blocks, interleaved over the waves, through a ring of NBUF register
    // buffers: blocks blk+NW, ..., blk+(NBUF-1)NW are in flight while block blk is
    // computed. Then the partial last block, if any, by the wave it falls to.
    // The loop runs in two phases. While every prefetch of a turn of the ring lies
    // inside the range, the loads are issued unconditionally, so the compiler's
    // count of loads in flight stays exact and block blk waits for its own loads
    // only. A prefetch under a branch would merge that count with the branch's
    // not-taken side, and each block would then also wait for the prefetch just
    // issued, leaving the memory latency of every turn exposed. The at most
    // 2 NBUF - 2 blocks per wave left after the steady turns run as straight-line
    // code per case (with NBUF = 2: one or two blocks), or through the branch form
    // for other ring depths.
    // The several-chunks kernel for bf16 with d = 128 runs the branch form
    // throughout: there the workgroup streams 8192 tokens or more alone on its CU,
    // and that form measured 0.7-1.5% faster (1M and 4 x 512k tokens), while the
    // steady form measured faster everywhere else (the per-chunk kernel, and
    // d = 64, whose blocks take twice the arithmetic per byte).
    const int64_t nfull = (c1 - c0) / BT;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int64_t per_chunk = MULTI ? nfull / nc / NW : 0;  // blocks of one chunk per wave
    int64_t done = 0;
    int cur = 0;
    auto after_block = [&]() {
        if constexpr (MULTI) {
            if (++done == per_chunk) {  // this wave's last block of chunk cur
                park(cur);
                done = 0;
                ++cur;
            }
        }
    };
    {
        uint4 kb[NBUF][TPL], vb[NBUF][TPL];
        int64_t blk = wave_u;
#pragma unroll
        for (int s = 0; s < NBUF - 1; ++s)
            if (blk + s * NW < nfull) load_full(c0 + (blk + s * NW) * BT, kb[s], vb[s]);
        // steady turns: the last prefetch of the turn, block blk + (2 NBUF - 2) NW, exists
        constexpr bool kSteady = !MULTI || !(std::is_same<T, uint16_t>::value && D == 128);
        while (kSteady && blk + (2 * NBUF - 2) * NW < nfull) {
#pragma unroll
            for (int s = 0; s < NBUF; ++s) {
                load_full(c0 + (blk + (NBUF - 1) * NW) * BT, kb[(s + NBUF - 1) % NBUF], vb[(s + NBUF - 1) % NBUF]);
                compute_block(std::false_type{}, c0 + blk * BT, kb[s], vb[s]);
                blk += NW;
                after_block();
            }
        }
        if constexpr (kSteady && NBUF == 2) {
            // The ring holds block blk; one or two blocks are left. Each path issues
            // its loads unconditionally, so the waits stay exact here too.
            if (blk + NW < nfull) {
                load_full(c0 + (blk + NW) * BT, kb[1], vb[1]);
                compute_block(std::false_type{}, c0 + blk * BT, kb[0], vb[0]);
                after_block();
                compute_block(std::false_type{}, c0 + (blk + NW) * BT, kb[1], vb[1]);
                after_block();
            } else if (blk < nfull) {
                compute_block(std::false_type{}, c0 + blk * BT, kb[0], vb[0]);
                after_block();
            }
            blk = nfull;  // every full block of this wave is done
        }
        bool more = blk < nfull;
        while (more) {
#pragma unroll
            for (int s = 0; s < NBUF; ++s) {
                if (more) {
                    const int64_t pre = blk + (NBUF - 1) * NW;
                    if (pre < nfull) load_full(c0 + pre * BT, kb[(s + NBUF - 1) % NBUF], vb[(s + NBUF - 1) % NBUF]);
                    compute_block(std::false_type{}, c0 + blk * BT, kb[s], vb[s]);
                    blk += NW;
                    more = blk < nfull;
                    after_block();
                }
            }
        }
        if constexpr (!MULTI) {
            if (c0 + nfull * BT < c1 && nfull % NW == wave_u) {
                load_tail(c0 + nfull * BT, kb[0], vb[0]);
                compute_block(std::true_type{}, c0 + nfull * BT, kb[0], vb[0]);
            }
        }
    }
    if constexpr (!MULTI) park(0);
    __syncthreads();
    for (int j = 0; j < (MULTI ? nc : 1); ++j) finish(j, po + (int64_t)j * p.po_sp, pl + (int64_t)j * p.pl_sp);
}

// The empty state (o = 0, lse = -inf) of GT heads of one chunk.
template <int D, int GT, int NW>
__device__ __forceinline__ void write_empty(float* po, float* pl, const PartialParams& p) {
    for (int i = threadIdx.x; i < GT * (D / 4); i += NW * kWave) {
        const int h = i / (D / 4), c4 = i % (D / 4);
        store_state(po + (int64_t)h * p.po_sh + 4 * c4, pl + (int64_t)h * p.pl_sh, make_float4(0.f, 0.f, 0.f, 0.f),
                    -INFINITY, c4 == 0, p.stream_states != 0);
    }
}

// Most sequences a ragged grid may have for the compacted order below: one per lane
// of a wave.
constexpr int kCompactMaxBatch = kWave;

// The (chunk, head group, sequence) item of workgroup L in the compacted order of a
// ragged grid (P chunks, HG head groups, B <= 64 sequences): the items that hold
// tokens, sequence by sequence, head group by head group, chunk by chunk, take
// workgroups 0 .. total - 1 in that order. The workgroups after them take, in order,
// every (chunk, head group) item of the sequences without tokens; the others get
// none (`valid` false). `n` is the item's clamped sequence length. Every value is
// wave-uniform: lane i reads sequence i's length and the wave scans the chunk counts.
struct Item {
    bool valid;
    int chunk, hg, b, n;
};
__device__ __forceinline__ Item compact_item(const PartialParams& p, uint64_t L, int P, int HG, int B) {
    const int lane = threadIdx.x % kWave;
    int nl = 0;
    if (lane < B) {
        nl = p.seqlens[lane];
        nl = nl < 0 ? 0 : (nl > p.N ? p.N : nl);
    }
    const int nbl = (int)(((unsigned)nl + (unsigned)p.chunk - 1u) / (unsigned)p.chunk);
    int incl = nbl;  // chunks holding tokens in sequences 0 .. lane
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    const uint64_t total = (uint64_t)__builtin_amdgcn_readlane(incl, kWave - 1) * (uint64_t)HG;
    Item it{false, 0, 0, 0, 0};
    if (L < total) {
        const uint64_t past = __ballot((uint64_t)incl * HG > L);  // sequences ending after item L
        const int b = __ffsll((unsigned long long)past) - 1;
        const int nb = __builtin_amdgcn_readlane(nbl, b);
        const uint64_t off = L - (uint64_t)(__builtin_amdgcn_readlane(incl, b) - nb) * HG;
        it = Item{true, (int)(off % (uint64_t)nb), (int)(off / (uint64_t)nb), b, __builtin_amdgcn_readlane(nl, b)};
    } else {
        const uint64_t empty = __ballot(lane < B && nl == 0);  // sequences without tokens
        const uint64_t i = L - total, per_seq = (uint64_t)P * HG;
        const uint64_t k = i / per_seq;  // the k-th of them
        if (k < (uint64_t)__popcll(empty)) {
            const bool kth = ((empty >> lane) & 1ull) && (uint64_t)__popcll(empty & ((1ull << lane) - 1ull)) == k;
            it = Item{true, (int)(i % (uint64_t)P), (int)(i % per_seq / (uint64_t)P),
                      __ffsll((unsigned long long)__ballot(kth)) - 1, 0};
        }
    }
    it.chunk = __builtin_amdgcn_readfirstlane(it.chunk);
    it.hg = __builtin_amdgcn_readfirstlane(it.hg);
    it.b = __builtin_amdgcn_readfirstlane(it.b);
    it.n = __builtin_amdgcn_readfirstlane(it.n);
    return it;
}

template <typename T, int D, int GT, int NW, int TPL, int NBUF>
__global__ __launch_bounds__(NW * kWave) void partial_kernel(PartialParams p) {
    // Workgroups are handed to the eight XCDs in turn, so with the chunk index fastest
    // (and a multiple of 8 chunks per row) XCD k takes chunks k, k + 8, ... of every
    // row. Any permutation of the (chunk, row) pairs over the workgroups is correct.
    // Ragged grids of at most 64 sequences take the compacted order (compact_item):
    // the workgroups with work come first, one after the other, and the empty ones
    // after them. In the plain order about half the workgroups of a ragged batch are
    // empty, interleaved with the others; they leave CUs waiting for work for a fifth
    // of the time (per-workgroup timestamps, 32 sequences of 4k-64k tokens), and the
    // compacted order streamed 1.7-7% faster on such batches (chunks 1024-4096; 0.8%
    // slower at chunk 512). Larger ragged batches keep the older orders: rows of at
    // most 32 chunks walked chunk-major (workgroup L takes chunk L / rows of row
    // L % rows; with the chunk index fastest, rows of exactly 32 chunks streamed 7-10%
    // slower), others with the chunk index fastest, rotated by one XCD per row so that
    // each row's last, partly used group of 8 chunks does not always load the
    // low-numbered XCDs.
    int chunk_idx = blockIdx.x;
    int gy = blockIdx.y, gz = blockIdx.z;
    int n_read = -1;  // the row's clamped length, when the compacted order has read it
    if (p.seqlens && gridDim.z <= (unsigned)kCompactMaxBatch && (uint64_t)gridDim.x * gridDim.z < (1ull << 31)) {
        const uint64_t L = blockIdx.x + (uint64_t)gridDim.x * (blockIdx.y + (uint64_t)gridDim.y * blockIdx.z);
        const Item it = compact_item(p, L, (int)gridDim.x, (int)gridDim.y, (int)gridDim.z);
        if (!it.valid) return;
        chunk_idx = it.chunk;
        gy = it.hg;
        gz = it.b;
        n_read = it.n;
    } else if (p.seqlens && gridDim.x <= 32 && (gridDim.y & 7u) == 0) {
        const uint64_t rows = (uint64_t)gridDim.y * gridDim.z;
        const uint64_t L = blockIdx.x + (uint64_t)gridDim.x * (blockIdx.y + (uint64_t)gridDim.y * blockIdx.z);
        chunk_idx = (int)(L / rows);
        gy = (int)(L % rows % gridDim.y);
        gz = (int)(L % rows / gridDim.y);
    } else if (p.seqlens && (gridDim.x & 7u) == 0) {
        const unsigned row = blockIdx.y + gridDim.y * blockIdx.z;
        chunk_idx = (int)((blockIdx.x & ~7u) | ((blockIdx.x - row) & 7u));
    }
    const int h0 = gy * GT;
    const int b = gz;
    const int g = h0 / p.group;

    int n = n_read >= 0 ? n_read : (p.seqlens ? p.seqlens[b] : p.N);
    n = n < 0 ? 0 : (n > p.N ? p.N : n);

    // Chunks at or past nb hold no tokens. Their empty state (0, -inf) is written only
    // if the caller reads it, and then by the workgroups that have work (chunk j also
    // covers chunks j + nb, j + 2 nb, ...): an empty workgroup that stayed to store
    // 2 KB would hold its compute-unit slot for a whole write latency. A row with no
    // tokens at all has no such workgroup and writes its own.
    // in 32 bits: n <= N, and the launcher refuses N > INT32_MAX - chunk
    const int64_t nb = ((unsigned)n + (unsigned)p.chunk - 1u) / (unsigned)p.chunk;
    float* po_row = p.po + (int64_t)b * p.po_sb + (int64_t)h0 * p.po_sh;
    float* pl_row = p.plse + (int64_t)b * p.pl_sb + (int64_t)h0 * p.pl_sh;
    if (chunk_idx >= nb) {
        if (p.empty_states && nb == 0)
            write_empty<D, GT, NW>(po_row + (int64_t)chunk_idx * p.po_sp, pl_row + (int64_t)chunk_idx * p.pl_sp, p);
        return;
    }
    const int64_t c0 = (int64_t)chunk_idx * p.chunk;
    const int64_t c1 = (c0 + p.chunk < (int64_t)n) ? c0 + p.chunk : (int64_t)n;
    chunk_state<T, D, GT, NW, TPL, NBUF>(p, b, h0, g, c0, c1, po_row + (int64_t)chunk_idx * p.po_sp,
                                         pl_row + (int64_t)chunk_idx * p.pl_sp);
    if (p.empty_states)
        for (int64_t c = chunk_idx + nb; c < (int64_t)gridDim.x; c += nb)
            write_empty<D, GT, NW>(po_row + c * p.po_sp, pl_row + c * p.pl_sp, p);
}


// Rows of equal length whose chunks are all whole: workgroup x of a row streams the
// cpw chunks cpw * x, ..., cpw * x + cpw - 1 in one pass and writes one state per
// chunk (a row whose chunk count is no multiple of cpw would give its last
// workgroup fewer; the launcher does not ask for that).
template <typename T, int D, int GT, int NW, int TPL, int NBUF>
__global__ __launch_bounds__(NW * kWave) void partial_kernel_multi(PartialParams p, int n_chunks, int cpw) {
    const int first = blockIdx.x * cpw;
    const int nc = cpw < n_chunks - first ? cpw : n_chunks - first;
    const int h0 = blockIdx.y * GT;
    const int b = blockIdx.z;
    const int g = h0 / p.group;
    float* po = p.po + (int64_t)b * p.po_sb + (int64_t)h0 * p.po_sh + (int64_t)first * p.po_sp;
    float* pl = p.plse + (int64_t)b * p.pl_sb + (int64_t)h0 * p.pl_sh + (int64_t)first * p.pl_sp;
    const int64_t c0 = (int64_t)first * p.chunk;
    chunk_state<T, D, GT, NW, TPL, NBUF, true>(p, b, h0, g, c0, c0 + (int64_t)nc * p.chunk, po, pl, nc);
}

// Compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// A grid with fewer workgroups than compute units leaves compute units idle, and
// each busy one streams with only the bytes its waves keep in flight: such grids
// get more waves per workgroup (measured 16-20% faster at 64 and 128 workgroups,
// even at 256, slower from 512 on).
// Workgroups of the per-chunk kernel one CU holds at once (limited by its registers
// and LDS), from the runtime; 0 if it cannot say. One value serves every device: the
// library holds gfx950 code only, and the count depends on the kernel and the
// architecture.
template <typename T, int D, int GT, int NW, int TPL, int NBUF>
int per_chunk_capacity() {
    static std::atomic<int> cache{0};
    const int v = cache.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, partial_kernel<T, D, GT, NW, TPL, NBUF>, NW * kWave, 0) !=
            hipSuccess ||
        n <= 0)
        return 0;
    cache.store(n, std::memory_order_relaxed);
    return n;
}

template <typename T, int D, int GT>
hipError_t launch_typed(const PartialParams& p, int B, int Hq, int n_chunks, hipStream_t stream) {
    constexpr int TPL = GT >= 8 ? (TA_PARTIAL_TPL > 4 ? 4 : TA_PARTIAL_TPL) : TA_PARTIAL_TPL;
    constexpr int NBUF = TA_PARTIAL_NBUF;
    constexpr int NW = TA_PARTIAL_WAVES, NWS = TA_PARTIAL_WAVES_SMALL;
    dim3 grid(n_chunks, Hq / GT, B);
    const int64_t wgs = (int64_t)n_chunks * (Hq / GT) * B;
    const int cus = device_cus();
    // Nontemporal state stores pay off when the grid is more than about two rounds of
    // resident workgroups (8 per compute unit). With fewer, most states are written
    // near the tail of the stream, where write-back stores cost no more and leave the
    // states in L2 for the merge.
    PartialParams q = p;
    q.stream_states = wgs > 8 * (int64_t)cus ? 1 : 0;
    // A grid of a whole number k (2 to 16; GT of at most 4) of workgroups per CU streams
    // 0.4-2.2% faster as one workgroup per CU taking k consecutive chunks in one
    // stream, when that stream is at least 8192 tokens long (measured with k = 2 to
    // 16 on 256k to 4 x 512k tokens) -- unless the per-chunk grid itself fills whole
    // rounds of resident workgroups (k a multiple of the workgroups a CU holds: 3 for
    // the bf16 d = 128 kernel), which then stream at least as well (measured with
    // k = 3 and 6). Over shorter streams (4096 tokens per CU at 128k) the per-chunk
    // grid was 1-10% faster, the more so the more chunks. With a fraction of a
    // workgroup per CU the CUs that get two make it much slower. It needs rows of
    // equal length (no seqlens) cut into whole chunks, each a whole number of rounds
    // of NW blocks, so that every wave reaches each chunk's end at the same step.
    constexpr int BT = (kWave / (D / Storage<T>::kElems)) * TPL;
    const int64_t cpw = cus > 0 && wgs % cus == 0 ? wgs / cus : 0;
    const int cap = cpw >= 2 && max_chunks_per_wg<GT>() > 0 ? per_chunk_capacity<T, D, GT, NW, TPL, NBUF>() : 0;
    if constexpr (max_chunks_per_wg<GT>() > 0) {
        if (!p.seqlens && p.N > 0 && p.N % p.chunk == 0 && p.chunk % (BT * NW) == 0 && cpw >= 2 &&
            cpw <= max_chunks_per_wg<GT>() && n_chunks % cpw == 0 && cpw * p.chunk >= kMultiMinTokens && cap > 0 &&
            cpw % cap != 0) {
            dim3 gm((unsigned)((n_chunks + cpw - 1) / cpw), Hq / GT, B);
            hipLaunchKernelGGL((partial_kernel_multi<T, D, GT, NW, TPL, NBUF>), gm, dim3(NW * kWave), 0, stream, q,
                               n_chunks, (int)cpw);
            return hipGetLastError();
        }
    }
    constexpr bool kMeasuredTwoPerCu = std::is_same<T, uint16_t>::value && D == 128 && GT <= 4;
    const unsigned reserve = kMeasuredTwoPerCu && p.seqlens && wgs > 8 * (int64_t)cus ? kTwoPerCuLds : 0u;
    if (NWS != NW && wgs < cus)
        hipLaunchKernelGGL((partial_kernel<T, D, GT, NWS, TPL, NBUF>), grid, dim3(NWS * kWave), 0, stream, q);
    else
        hipLaunchKernelGGL((partial_kernel<T, D, GT, NW, TPL, NBUF>), grid, dim3(NW * kWave), reserve, stream, q);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_heads(const PartialParams& p, int gt, int B, int Hq, int n_chunks, hipStream_t stream) {
    switch (gt) {
        case 1: return launch_typed<T, D, 1>(p, B, Hq, n_chunks, stream);
        case 2: return launch_typed<T, D, 2>(p, B, Hq, n_chunks, stream);
        case 4: return launch_typed<T, D, 4>(p, B, Hq, n_chunks, stream);
        case 8: return launch_typed<T, D, 8>(p, B, Hq, n_chunks, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_partial(const PartialParams& p, Dtype dt, int d, int heads_per_wg, int B, int Hq,
                          int n_chunks, hipStream_t stream) {
    if (dt == Dtype::BF16) {
        if (d == 128) return launch_heads<uint16_t, 128>(p, heads_per_wg, B, Hq, n_chunks, stream);
        if (d == 64) return launch_heads<uint16_t, 64>(p, heads_per_wg, B, Hq, n_chunks, stream);
    } else {
        if (d == 128) return launch_heads<float, 128>(p, heads_per_wg, B, Hq, n_chunks, stream);
        if (d == 64) return launch_heads<float, 64>(p, heads_per_wg, B, Hq, n_chunks, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ta
