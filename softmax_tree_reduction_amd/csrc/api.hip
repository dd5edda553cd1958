// The C ABI declared in include/tree_attn.h: descriptor validation, dispatch to
// the partial-state and tree-merge kernels, and stream-ordered workspace.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>

#include "../../include/tree_attn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return TA_OK;
}

int64_t elem_size(int32_t dtype) { return dtype == TA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks ndim, dtype and non-negative sizes and strides. Tensors whose last
// dimension is the head dimension (rows_of_d) also need it contiguous and every
// row 16-byte aligned; the lse tensors take any strides.
int check_tensor(const ta_tensor* t, const char* name, int ndim, bool rows_of_d) {
    if (!t) return fail(TA_ERR_NULL, "%s: descriptor is NULL", name);
    if (t->ndim != ndim) return fail(TA_ERR_SHAPE, "%s: expected %d dimensions, got %d", name, ndim, t->ndim);
    if (t->dtype != TA_F32 && t->dtype != TA_BF16) return fail(TA_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
    bool empty = false;
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0) return fail(TA_ERR_SHAPE, "%s: negative size in dimension %d", name, i);
        if (t->stride[i] < 0) return fail(TA_ERR_STRIDE, "%s: negative stride in dimension %d", name, i);
        empty = empty || t->shape[i] == 0;
    }
    // a tensor with no elements is never read or written, so its pointer may be NULL
    if (!t->data && !empty) return fail(TA_ERR_NULL, "%s: data pointer is NULL", name);
    if (!rows_of_d) return TA_OK;
    if (t->shape[ndim - 1] > 1 && t->stride[ndim - 1] != 1)
        return fail(TA_ERR_STRIDE, "%s: the last dimension must be contiguous (stride 1), got %lld", name,
                    (long long)t->stride[ndim - 1]);
    if (!aligned16(t->data)) return fail(TA_ERR_STRIDE, "%s: data pointer is not 16-byte aligned", name);
    const int64_t es = elem_size(t->dtype);
    for (int i = 0; i < ndim - 1; ++i)
        if (t->shape[i] > 1 && (t->stride[i] * es) % 16 != 0)
            return fail(TA_ERR_STRIDE, "%s: stride of dimension %d (%lld elements) is not a multiple of 16 bytes",
                        name, i, (long long)t->stride[i]);
    return TA_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(TA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Device scratch of one call, ordered on the call's stream. Outside graph capture
// it is a buffer kept per (device, stream) and grown when a call needs more, so a
// steady decode loop allocates nothing. The buffer's lock is held from acquire()
// until the call returns, that is until its last kernel is enqueued: two host
// threads calling on one stream then enqueue their kernels back to back, never
// interleaved, so no call's merge reads another call's partial states, and a buffer
// released when it grows is released behind every kernel already enqueued on it.
// Under graph capture the scratch is allocated and released inside the captured
// work instead.
class CallWorkspace {
  public:
    explicit CallWorkspace(hipStream_t st) : st_(st) {}
    ~CallWorkspace() {
        if (owned_ && ptr_) (void)hipFreeAsync(ptr_, st_);
    }  // lock_ is released after this body, once every launch of the call is enqueued
    CallWorkspace(const CallWorkspace&) = delete;
    CallWorkspace& operator=(const CallWorkspace&) = delete;

    int acquire(size_t bytes) {
        if (bytes == 0) return TA_OK;
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(st_, &cap)) != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cap != hipStreamCaptureStatusNone) {
            if ((e = hipMallocAsync(&ptr_, bytes, st_)) != hipSuccess) return hip_fail(e, "hipMallocAsync (workspace)");
            owned_ = true;
            return TA_OK;
        }
        Entry* w = nullptr;
        {
            std::lock_guard<std::mutex> g(cache_mu());
            w = &cache()[{dev, reinterpret_cast<uintptr_t>(st_)}];  // map nodes never move or go away
        }
        lock_ = std::unique_lock<std::mutex>(w->mu);
        if (w->bytes < bytes) {
            const size_t nb = bytes > w->bytes + w->bytes / 2 ? bytes : w->bytes + w->bytes / 2;
            void* p = nullptr;
            if ((e = hipMallocAsync(&p, nb, st_)) != hipSuccess) return hip_fail(e, "hipMallocAsync (workspace)");
            if (w->ptr) (void)hipFreeAsync(w->ptr, st_);
            w->ptr = p;
            w->bytes = nb;
        }
        ptr_ = w->ptr;
        return TA_OK;
    }
    void* get() const { return ptr_; }

  private:
    struct Entry {
        std::mutex mu;  // held by the call using the buffer, from acquire() until it returns
        void* ptr = nullptr;
        size_t bytes = 0;
    };
    static std::mutex& cache_mu() {
        static std::mutex mu;
        return mu;
    }
    static std::map<std::pair<int, uintptr_t>, Entry>& cache() {
        static auto* m = new std::map<std::pair<int, uintptr_t>, Entry>();  // lives until exit
        return *m;
    }
    hipStream_t st_;
    void* ptr_ = nullptr;
    bool owned_ = false;
    std::unique_lock<std::mutex> lock_;
};

// Byte counts of scratch sub-buffers are rounded up to 256 bytes, so that every
// sub-buffer starts 256-byte aligned (the merge reads and writes float4 rows).
constexpr size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Leaves one merge workgroup takes: the binary kernel's tile (arity 0), or the
// largest power of `arity` the arity-K kernel holds.
int64_t merge_span(int64_t d, int arity) {
    return arity ? ta::combine_k_span((int)d, arity) : ta::combine_max_leaves((int)d);
}

// The merge's first pass puts one workgroup per group of leaves on the grid's third
// dimension, which holds at most 65535.
int check_merge_groups(int64_t n_parts, int64_t d, int arity) {
    const int64_t span = merge_span(d, arity);
    const int64_t groups = (n_parts + span - 1) / span;
    if (groups > 65535)
        return fail(TA_ERR_UNSUPPORTED, "%lld states per row exceed the merge's %lld (%lld groups of %lld)",
                    (long long)n_parts, (long long)(65535 * span), (long long)groups, (long long)span);
    return TA_OK;
}

// Bytes of one buffer of intermediate states: o [B, H, groups, d], then lse
// [B, H, groups] from the next 256-byte boundary.
size_t state_buffer_bytes(int64_t B, int64_t H, int64_t groups, int64_t d) {
    return align256((size_t)(B * H * groups * d) * sizeof(float)) + align256((size_t)(B * H * groups) * sizeof(float));
}

// Bytes of intermediate states the merge needs when a row has more leaves than one
// workgroup takes: two buffers of the first pass's output size.
size_t combine_scratch_bytes(int64_t n_parts, int64_t B, int64_t H, int64_t d, int arity = 0) {
    const int64_t span = merge_span(d, arity);
    if (n_parts <= span) return 0;
    const int64_t groups = (n_parts + span - 1) / span;
    return 2 * state_buffer_bytes(B, H, groups, d);
}

struct DecodeShape {
    int64_t B, Hq, Hkv, N, d;
    ta::Dtype dt;
};

int check_decode_inputs(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, int32_t chunk, DecodeShape* s) {
    int rc;
    if ((rc = check_tensor(q, "q", 3, true)) != TA_OK) return rc;
    if ((rc = check_tensor(k, "k", 4, true)) != TA_OK) return rc;
    if ((rc = check_tensor(v, "v", 4, true)) != TA_OK) return rc;
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(TA_ERR_DTYPE, "q, k and v must share a dtype (got %d, %d, %d)", q->dtype, k->dtype, v->dtype);
    for (int i = 0; i < 4; ++i)
        if (k->shape[i] != v->shape[i]) return fail(TA_ERR_SHAPE, "k and v shapes differ in dimension %d", i);
    s->B = q->shape[0];
    s->Hq = q->shape[1];
    s->d = q->shape[2];
    s->Hkv = k->shape[1];
    s->N = k->shape[2];
    s->dt = q->dtype == TA_BF16 ? ta::Dtype::BF16 : ta::Dtype::F32;
    if (k->shape[0] != s->B) return fail(TA_ERR_SHAPE, "k batch %lld != q batch %lld", (long long)k->shape[0], (long long)s->B);
    if (k->shape[3] != s->d) return fail(TA_ERR_SHAPE, "k head dim %lld != q head dim %lld", (long long)k->shape[3], (long long)s->d);
    if (s->Hkv <= 0 || s->Hq <= 0 || s->Hq % s->Hkv != 0)
        return fail(TA_ERR_SHAPE, "query heads (%lld) must be a positive multiple of KV heads (%lld)", (long long)s->Hq,
                    (long long)s->Hkv);
    if (s->d != 64 && s->d != 128) return fail(TA_ERR_UNSUPPORTED, "head dimension %lld: supported are 64 and 128", (long long)s->d);
    if (chunk < 1) return fail(TA_ERR_ARG, "chunk must be >= 1, got %d", chunk);
    if (s->B > 65535) return fail(TA_ERR_UNSUPPORTED, "batch %lld exceeds 65535", (long long)s->B);
    if (s->Hq > 65535) return fail(TA_ERR_UNSUPPORTED, "query heads %lld exceed 65535", (long long)s->Hq);
    if (s->N > INT32_MAX - chunk) return fail(TA_ERR_UNSUPPORTED, "cache length %lld too large", (long long)s->N);
    // the kernel addresses a row group's rows with 32-bit offsets from a shared base
    const int64_t es = elem_size(q->dtype);
    if (k->stride[2] * es >= (int64_t)1 << 28 || v->stride[2] * es >= (int64_t)1 << 28)
        return fail(TA_ERR_UNSUPPORTED, "token stride of k or v is 256 MiB or more");
    return TA_OK;
}

int check_partials(const ta_tensor* po, const ta_tensor* pl, int64_t B, int64_t H, int64_t d, int64_t min_parts,
                   const char* po_name, const char* pl_name) {
    int rc;
    if ((rc = check_tensor(po, po_name, 4, true)) != TA_OK) return rc;
    if ((rc = check_tensor(pl, pl_name, 3, false)) != TA_OK) return rc;
    if (po->dtype != TA_F32 || pl->dtype != TA_F32) return fail(TA_ERR_DTYPE, "%s and %s must be f32", po_name, pl_name);
    if (po->shape[0] != B || po->shape[1] != H || po->shape[3] != d)
        return fail(TA_ERR_SHAPE, "%s must be [%lld, %lld, P, %lld]", po_name, (long long)B, (long long)H, (long long)d);
    if (pl->shape[0] != B || pl->shape[1] != H || pl->shape[2] != po->shape[2])
        return fail(TA_ERR_SHAPE, "%s must be [%lld, %lld, %lld]", pl_name, (long long)B, (long long)H, (long long)po->shape[2]);
    if (po->shape[2] < min_parts)
        return fail(TA_ERR_SHAPE, "%s holds %lld partial states, needs %lld", po_name, (long long)po->shape[2], (long long)min_parts);
    return TA_OK;
}

int check_outputs(const ta_tensor* out, const ta_tensor* lse, int64_t B, int64_t H, int64_t d) {
    int rc;
    if ((rc = check_tensor(out, "out", 3, true)) != TA_OK) return rc;
    if (out->dtype != TA_F32) return fail(TA_ERR_DTYPE, "out must be f32");
    if (out->shape[0] != B || out->shape[1] != H || out->shape[2] != d)
        return fail(TA_ERR_SHAPE, "out must be [%lld, %lld, %lld]", (long long)B, (long long)H, (long long)d);
    if (lse) {
        if ((rc = check_tensor(lse, "lse", 2, false)) != TA_OK) return rc;
        if (lse->dtype != TA_F32) return fail(TA_ERR_DTYPE, "lse must be f32");
        if (lse->shape[0] != B || lse->shape[1] != H)
            return fail(TA_ERR_SHAPE, "lse must be [%lld, %lld]", (long long)B, (long long)H);
    }
    return TA_OK;
}

// Heads per workgroup: the largest of 8, 4, 2, 1 that divides the GQA group.
int heads_per_wg(int64_t group) {
    for (int g : {8, 4, 2, 1})
        if (group % g == 0) return g;
    return 1;
}

ta::PartialParams partial_params(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, const int32_t* seqlens,
                                 float* po, const int64_t po_st[3], float* pl, const int64_t pl_st[3],
                                 const DecodeShape& s, int32_t chunk, bool empty_states) {
    ta::PartialParams p{};
    p.q = q->data;
    p.k = k->data;
    p.v = v->data;
    p.seqlens = seqlens;
    p.po = po;
    p.plse = pl;
    p.q_sb = q->stride[0];
    p.q_sh = q->stride[1];
    p.k_sb = k->stride[0];
    p.k_sh = k->stride[1];
    p.k_st = k->stride[2];
    p.v_sb = v->stride[0];
    p.v_sh = v->stride[1];
    p.v_st = v->stride[2];
    p.po_sb = po_st[0];
    p.po_sh = po_st[1];
    p.po_sp = po_st[2];
    p.pl_sb = pl_st[0];
    p.pl_sh = pl_st[1];
    p.pl_sp = pl_st[2];
    p.N = (int32_t)s.N;
    p.chunk = chunk;
    p.group = (int32_t)(s.Hq / s.Hkv);
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s.d));
    p.empty_states = empty_states ? 1 : 0;
    return p;
}

// One pass of the merge: the binary kernel (arity 0) or the arity-K kernel.
hipError_t launch_pass(const ta::CombineParams& c, int64_t d, int arity, int64_t B, int64_t H, int64_t groups,
                       int64_t leaves_per_group, hipStream_t stream) {
    if (!arity) return ta::launch_combine_pass(c, (int)d, (int)B, (int)H, (int)groups, (int)leaves_per_group, stream);
    int64_t span = arity;  // the smallest power of K (at least K) holding the group's leaves
    while (span < leaves_per_group) span *= arity;
    return ta::launch_combine_k_pass(c, (int)d, arity, (int)B, (int)H, (int)groups, (int)span, stream);
}

// Runs the merge tree over n_parts leaves per row and writes (out, lse).
// Rows with more leaves than one workgroup takes go through intermediate levels
// held in `scratch` (combine_scratch_bytes of it). Arity 0 is the binary tree of
// the merge kernel; 2 <= arity <= 16 runs the arity-K kernel.
int run_combine(const float* po, const int64_t po_st[3], const float* pl, const int64_t pl_st[3], int64_t n_parts,
                const int32_t* seqlens, int32_t chunk, int64_t N, int64_t B, int64_t H, int64_t d, float* out,
                const int64_t out_st[2], float* lse, const int64_t lse_st[2], void* scratch, hipStream_t stream,
                int arity = 0) {
    const int64_t span = merge_span(d, arity);
    const float* cur_o = po;
    const float* cur_l = pl;
    int64_t cur_po[3] = {po_st[0], po_st[1], po_st[2]};
    int64_t cur_pl[3] = {pl_st[0], pl_st[1], pl_st[2]};
    int64_t leaves = n_parts;
    const int32_t* sl = seqlens;
    const int64_t first_groups = (n_parts + span - 1) / span;
    float* bufs[2] = {static_cast<float*>(scratch), nullptr};
    if (scratch) bufs[1] = reinterpret_cast<float*>(static_cast<char*>(scratch) + state_buffer_bytes(B, H, first_groups, d));
    int which = 0;
    hipError_t e = hipSuccess;

    while (leaves > span) {
        const int64_t groups = (leaves + span - 1) / span;
        float* nxt_o = bufs[which];
        float* nxt_l = reinterpret_cast<float*>(reinterpret_cast<char*>(nxt_o) + align256((size_t)(B * H * groups * d) * sizeof(float)));
        ta::CombineParams c{};
        c.po = cur_o;
        c.plse = cur_l;
        c.po_sb = cur_po[0]; c.po_sh = cur_po[1]; c.po_sp = cur_po[2];
        c.pl_sb = cur_pl[0]; c.pl_sh = cur_pl[1]; c.pl_sp = cur_pl[2];
        c.n_parts = (int32_t)leaves;
        c.seqlens = sl;
        c.chunk = chunk;
        c.N = (int32_t)N;
        c.out = nxt_o;
        c.lse = nxt_l;
        c.out_sb = H * groups * d; c.out_sh = groups * d; c.out_sg = d;
        c.lse_sb = H * groups; c.lse_sh = groups; c.lse_sg = 1;
        if ((e = launch_pass(c, d, arity, B, H, groups, span, stream)) != hipSuccess)
            return hip_fail(e, "merge kernel launch");
        cur_o = nxt_o;
        cur_l = nxt_l;
        cur_po[0] = c.out_sb; cur_po[1] = c.out_sh; cur_po[2] = c.out_sg;
        cur_pl[0] = c.lse_sb; cur_pl[1] = c.lse_sh; cur_pl[2] = c.lse_sg;
        leaves = groups;
        sl = nullptr;  // empty groups were written as empty states
        which ^= 1;
    }
    ta::CombineParams c{};
    c.po = cur_o;
    c.plse = cur_l;
    c.po_sb = cur_po[0]; c.po_sh = cur_po[1]; c.po_sp = cur_po[2];
    c.pl_sb = cur_pl[0]; c.pl_sh = cur_pl[1]; c.pl_sp = cur_pl[2];
    c.n_parts = (int32_t)leaves;
    c.seqlens = sl;
    c.chunk = chunk;
    c.N = (int32_t)N;
    c.out = out;
    c.lse = lse;
    c.out_sb = out_st[0]; c.out_sh = out_st[1]; c.out_sg = 0;
    c.lse_sb = lse ? lse_st[0] : 0; c.lse_sh = lse ? lse_st[1] : 0; c.lse_sg = 0;
    if ((e = launch_pass(c, d, arity, B, H, 1, leaves > 0 ? leaves : 1, stream)) != hipSuccess)
        return hip_fail(e, "merge kernel launch");
    return TA_OK;
}

// Workspace layout of one decode call: partial o [B, Hq, P, d], partial lse
// [B, Hq, P] from the next 256-byte boundary, then the merge's intermediate states.
struct DecodePlan {
    int64_t P;            // partial states per row (an N = 0 cache has one empty state)
    size_t lse_offset;    // bytes from the workspace start to partial lse
    size_t merge_offset;  // bytes to the merge scratch
    size_t merge_bytes;
    size_t total_bytes;
};

int check_decode(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, const ta_tensor* out, const ta_tensor* lse,
                 int32_t chunk, DecodeShape* s, DecodePlan* plan) {
    int rc;
    if ((rc = check_decode_inputs(q, k, v, chunk, s)) != TA_OK) return rc;
    if ((rc = check_outputs(out, lse, s->B, s->Hq, s->d)) != TA_OK) return rc;
    plan->P = s->N > 0 ? (s->N + chunk - 1) / chunk : 1;
    if ((rc = check_merge_groups(plan->P, s->d, 0)) != TA_OK) return rc;
    plan->lse_offset = align256((size_t)(s->B * s->Hq * plan->P * s->d) * sizeof(float));
    plan->merge_offset = state_buffer_bytes(s->B, s->Hq, plan->P, s->d);
    plan->merge_bytes = combine_scratch_bytes(plan->P, s->B, s->Hq, s->d);
    plan->total_bytes = s->B > 0 ? plan->merge_offset + plan->merge_bytes : 0;
    return TA_OK;
}

// Enqueues the partial kernel and the merge of one decode step on `st`, with the
// partial states and merge scratch in `ws` (plan.total_bytes of device memory).
int launch_decode(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, const int32_t* seqlens,
                  const ta_tensor* out, const ta_tensor* lse, int32_t chunk, const DecodeShape& s,
                  const DecodePlan& plan, void* ws, hipStream_t st) {
    const int64_t P = plan.P;
    float* po = static_cast<float*>(ws);
    float* pl = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.lse_offset);
    void* merge_scratch = plan.merge_bytes ? static_cast<char*>(ws) + plan.merge_offset : nullptr;
    const int64_t po_st[3] = {s.Hq * P * s.d, P * s.d, s.d};
    const int64_t pl_st[3] = {s.Hq * P, P, 1};
    const int gt = heads_per_wg(s.Hq / s.Hkv);
    // With seqlens the merge reads only the chunks below ceil(n / chunk) of each row, so
    // the chunks past a sequence's end need not be written; without, every chunk of the
    // grid holds tokens except the one of an N = 0 cache, which the merge does read.
    ta::PartialParams p = partial_params(q, k, v, seqlens, po, po_st, pl, pl_st, s, chunk,
                                         /*empty_states=*/seqlens == nullptr);
    hipError_t e = ta::launch_partial(p, s.dt, (int)s.d, gt, (int)s.B, (int)s.Hq, (int)P, st);
    if (e != hipSuccess) return hip_fail(e, "partial kernel launch");
    const int64_t out_st[2] = {out->stride[0], out->stride[1]};
    const int64_t lse_st[2] = {lse ? lse->stride[0] : 0, lse ? lse->stride[1] : 0};
    return run_combine(po, po_st, pl, pl_st, P, seqlens, chunk, s.N, s.B, s.Hq, s.d, static_cast<float*>(out->data),
                       out_st, lse ? static_cast<float*>(lse->data) : nullptr, lse_st, merge_scratch, st);
}

// ---- the allocation-free variant of ta_decode --------------------------------
// Its partial states and merge scratch live in this file-scope device array
// instead of library workspace, for callers that cannot allocate. Each device the
// library runs on holds its own copy, at its own address, until the process ends.
// In host code `scratch` is only a stand-in for the symbol: kernels get the device
// address that hipGetSymbolAddress returns for the current device, never the name.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device, looked up once per device
// with that device current. Returns TA_OK and sets *ptr, or a TA_ERR_HIP failure.
int noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(TA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (scratch)");
        if (!p) return fail(TA_ERR_HIP, "hipGetSymbolAddress (scratch) returned NULL");
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return TA_OK;
}

// Serialises the enqueueing of allocation-free calls per device, so that two host
// threads calling on one stream enqueue their kernels back to back.
std::mutex& noalloc_mutex(int dev) {
    static std::mutex mus[64];
    return mus[(unsigned)dev % 64];
}

}  // namespace

extern "C" {

int32_t ta_suggest_chunk(int64_t batch, int64_t q_heads, int64_t kv_heads, int64_t n, int32_t compute_units) {
    if (batch < 1 || q_heads < 1 || kv_heads < 1 || n < 1)
        return fail(TA_ERR_ARG, "batch, q_heads, kv_heads and n must be >= 1");
    if (q_heads % kv_heads != 0)
        return fail(TA_ERR_ARG, "q_heads (%lld) must be a multiple of kv_heads (%lld)", (long long)q_heads,
                    (long long)kv_heads);
    int cus = compute_units;
    if (cus <= 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "compute-unit count");
        if (cus <= 0) return fail(TA_ERR_HIP, "the device reports %d compute units", cus);
    }
    const int64_t rows = batch * (q_heads / heads_per_wg(q_heads / kv_heads));  // workgroups per chunk index
    int64_t chunk = 64;
    while (2 * chunk <= n && rows * ((n + 2 * chunk - 1) / (2 * chunk)) >= cus) chunk *= 2;
    ok();
    return (int32_t)chunk;
}

int ta_version(void) { return 1; }

const char* ta_last_error(void) { return g_last_error.c_str(); }

int ta_partial(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, const int32_t* seqlens,
               const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t chunk, void* stream) {
    DecodeShape s;
    int rc;
    if ((rc = check_decode_inputs(q, k, v, chunk, &s)) != TA_OK) return rc;
    const int64_t P = (s.N + chunk - 1) / chunk;
    if ((rc = check_partials(partial_o, partial_lse, s.B, s.Hq, s.d, P, "partial_o", "partial_lse")) != TA_OK) return rc;
    // An empty cache (N = 0) gives every row one empty state in slot 0, the state
    // ta_decode merges for it, when the caller's tensors have that slot.
    const int64_t P_launch = P > 0 ? P : (partial_o->shape[2] > 0 ? 1 : 0);
    if (s.B == 0 || P_launch == 0) return ok();
    const int gt = heads_per_wg(s.Hq / s.Hkv);
    ta::PartialParams p = partial_params(q, k, v, seqlens, static_cast<float*>(partial_o->data), partial_o->stride,
                                         static_cast<float*>(partial_lse->data), partial_lse->stride, s, chunk,
                                         /*empty_states=*/true);
    hipError_t e = ta::launch_partial(p, s.dt, (int)s.d, gt, (int)s.B, (int)s.Hq, (int)P_launch,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "partial kernel launch");
    return ok();
}

int ta_decode(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, const int32_t* seqlens,
              const ta_tensor* out, const ta_tensor* lse, int32_t chunk, void* stream) {
    DecodeShape s;
    DecodePlan plan;
    int rc;
    if ((rc = check_decode(q, k, v, out, lse, chunk, &s, &plan)) != TA_OK) return rc;
    if (s.B == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    CallWorkspace ws(st);
    if ((rc = ws.acquire(plan.total_bytes)) != TA_OK) return rc;
    if ((rc = launch_decode(q, k, v, seqlens, out, lse, chunk, s, plan, ws.get(), st)) != TA_OK) return rc;
    return ok();
}

int ta_decode_noalloc(const ta_tensor* q, const ta_tensor* k, const ta_tensor* v, const int32_t* seqlens,
                      const ta_tensor* out, const ta_tensor* lse, int32_t chunk, void* stream) {
    DecodeShape s;
    DecodePlan plan;
    int rc;
    if ((rc = check_decode(q, k, v, out, lse, chunk, &s, &plan)) != TA_OK) return rc;
    if (plan.total_bytes > kNoAllocScratchBytes)
        return fail(TA_ERR_UNSUPPORTED,
                    "ta_decode_noalloc: this call needs %zu bytes of partial states and merge scratch, above the "
                    "%zu bytes of its static scratch (use ta_decode)",
                    plan.total_bytes, kNoAllocScratchBytes);
    if (s.B == 0) return ok();
    void* ws = nullptr;
    if ((rc = noalloc_scratch(&ws)) != TA_OK) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(noalloc_mutex(dev));
    if ((rc = launch_decode(q, k, v, seqlens, out, lse, chunk, s, plan, ws, static_cast<hipStream_t>(stream))) != TA_OK)
        return rc;
    return ok();
}

}  // extern "C"

namespace {

constexpr int kChain = -1;  // combine_impl's arity for the sequential order

// Validates the merge arguments, then runs the merge: the binary tree (arity 0),
// the arity-K tree (2..16) or the sequential chain (kChain).
int combine_impl(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts, int arity,
                 const ta_tensor* out, const ta_tensor* lse, void* stream) {
    int rc;
    if (!partial_o) return fail(TA_ERR_NULL, "partial_o: descriptor is NULL");
    if (partial_o->ndim != 4) return fail(TA_ERR_SHAPE, "partial_o: expected 4 dimensions, got %d", partial_o->ndim);
    const int64_t B = partial_o->shape[0], H = partial_o->shape[1], d = partial_o->shape[3];
    if ((rc = check_partials(partial_o, partial_lse, B, H, d, 0, "partial_o", "partial_lse")) != TA_OK) return rc;
    if (d != 64 && d != 128) return fail(TA_ERR_UNSUPPORTED, "head dimension %lld: supported are 64 and 128", (long long)d);
    if (n_parts < 0 || n_parts > partial_o->shape[2])
        return fail(TA_ERR_ARG, "n_parts %d outside [0, %lld]", n_parts, (long long)partial_o->shape[2]);
    if ((rc = check_outputs(out, lse, B, H, d)) != TA_OK) return rc;
    if (B > 65535) return fail(TA_ERR_UNSUPPORTED, "batch %lld exceeds 65535", (long long)B);
    if (B == 0 || H == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t out_st[2] = {out->stride[0], out->stride[1]};
    const int64_t lse_st[2] = {lse ? lse->stride[0] : 0, lse ? lse->stride[1] : 0};
    if (arity == kChain) {
        ta::CombineParams c{};
        c.po = static_cast<const float*>(partial_o->data);
        c.plse = static_cast<const float*>(partial_lse->data);
        c.po_sb = partial_o->stride[0]; c.po_sh = partial_o->stride[1]; c.po_sp = partial_o->stride[2];
        c.pl_sb = partial_lse->stride[0]; c.pl_sh = partial_lse->stride[1]; c.pl_sp = partial_lse->stride[2];
        c.n_parts = n_parts;
        c.chunk = 1;
        c.out = static_cast<float*>(out->data);
        c.lse = lse ? static_cast<float*>(lse->data) : nullptr;
        c.out_sb = out_st[0]; c.out_sh = out_st[1];
        c.lse_sb = lse_st[0]; c.lse_sh = lse_st[1];
        hipError_t e = ta::launch_combine_chain(c, (int)d, (int)B, (int)H, st);
        if (e != hipSuccess) return hip_fail(e, "chain merge kernel launch");
        return ok();
    }
    if ((rc = check_merge_groups(n_parts, d, arity)) != TA_OK) return rc;
    CallWorkspace ws(st);
    if ((rc = ws.acquire(combine_scratch_bytes(n_parts, B, H, d, arity))) != TA_OK) return rc;
    rc = run_combine(static_cast<const float*>(partial_o->data), partial_o->stride,
                     static_cast<const float*>(partial_lse->data), partial_lse->stride, n_parts, nullptr, 1, 0, B, H, d,
                     static_cast<float*>(out->data), out_st, lse ? static_cast<float*>(lse->data) : nullptr, lse_st,
                     ws.get(), st, arity);
    if (rc != TA_OK) return rc;
    return ok();
}

}  // namespace

extern "C" {

int ta_combine(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts, const ta_tensor* out,
               const ta_tensor* lse, void* stream) {
    return combine_impl(partial_o, partial_lse, n_parts, 0, out, lse, stream);
}

int ta_combine_k(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts, int32_t arity,
                 const ta_tensor* out, const ta_tensor* lse, void* stream) {
    if (arity < 2 || arity > 16) return fail(TA_ERR_ARG, "arity %d outside [2, 16]", arity);
    return combine_impl(partial_o, partial_lse, n_parts, arity, out, lse, stream);
}

int ta_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(TA_ERR_NULL, "stream_read: buf or sink is NULL");
    if (bytes < 0 || bytes % 16 != 0) return fail(TA_ERR_ARG, "stream_read: %lld bytes is not a multiple of 16", (long long)bytes);
    if (!aligned16(buf)) return fail(TA_ERR_ARG, "stream_read: buf is not 16-byte aligned");
    if (bytes == 0) return ok();
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "stream_read: device query");
    const int64_t n16 = bytes / 16;
    if ((e = ta::launch_stream_read(buf, n16, sink, cus, static_cast<hipStream_t>(stream))) != hipSuccess)
        return hip_fail(e, "stream_read kernel launch");
    return ok();
}

int ta_combine_chain(const ta_tensor* partial_o, const ta_tensor* partial_lse, int32_t n_parts,
                     const ta_tensor* out, const ta_tensor* lse, void* stream) {
    return combine_impl(partial_o, partial_lse, n_parts, kChain, out, lse, stream);
}

}  // extern "C"
