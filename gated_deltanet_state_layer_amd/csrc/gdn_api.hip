// libgdn host API: descriptor checks, the slot pool, argument validation and
// dispatch to the kernels.  Every check runs before anything is enqueued, so
// a negative status leaves device memory untouched.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "gdn_common.h"

namespace gdn {
size_t decode_verify_lds_bytes(const gdn_pool* pool, int32_t n_tok);

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kMaxLds = 64 * 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

gdn_status check_desc(const gdn_pool_desc* d) {
    if (!d) return GDN_ERR_INVALID_ARG;
    if (d->n_slots < 1 || d->n_layers < 1 || d->h_k < 1 || d->h_v < 1 || d->d_k < 1 ||
        d->d_v < 1 || d->conv_k < 1)
        return GDN_ERR_INVALID_ARG;
    if (d->h_v % d->h_k != 0) return GDN_ERR_INVALID_ARG;
    if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
    if (!(d->q_scale >= 0.f) || !(d->norm_eps >= 0.f) || std::isinf(d->q_scale) ||
        std::isinf(d->norm_eps))
        return GDN_ERR_INVALID_ARG;
    if (d->flags & ~(GDN_VALIDATE | GDN_GROUP_KERNEL)) return GDN_ERR_INVALID_ARG;
    if (d->ring_len < 0) return GDN_ERR_INVALID_ARG;
    if (d->ring_len > kMaxRingSolve - kMaxVerifyTokens) return GDN_ERR_UNSUPPORTED;
    if (d->d_k != d->d_v) return GDN_ERR_UNSUPPORTED;
    if (d->d_k != 32 && d->d_k != 64 && d->d_k != 128) return GDN_ERR_UNSUPPORTED;
    if (d->conv_k < 2 || d->conv_k > kMaxConvK) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

// Byte offsets inside the aux buffer (the layout documented in gdn.h).
struct AuxLayout {
    size_t window_bytes, meta, ctr, ring_cnt, ring_arr, ring, total;
    int64_t ring_stride;   // floats per (slot, layer) ring block
};

AuxLayout aux_layout(const gdn_pool_desc* d) {
    AuxLayout x{};
    const size_t io = d->io_dtype == GDN_BF16 ? 2 : 4;
    const size_t c_conv = 2 * (size_t)d->h_k * d->d_k + (size_t)d->h_v * d->d_v;
    const size_t sl = (size_t)d->n_slots * d->n_layers;
    x.window_bytes = sl * (d->conv_k - 1) * c_conv * io;
    // windows | meta block (error word) | row-split decode counters | ring
    x.meta = align_up(x.window_bytes, kAlign);
    x.ctr = x.meta + kAlign;
    x.total = x.ctr + align_up(sl * d->h_k * sizeof(int32_t), kAlign);
    if (d->ring_len > 0) {
        const size_t per_tok = (size_t)d->h_k * d->d_k + (size_t)d->h_v * d->d_v + 2 * (size_t)d->h_v;
        x.ring_stride = (int64_t)align_up(d->ring_len * per_tok, 64);
        x.ring_cnt = x.total;
        x.ring_arr = x.ring_cnt + align_up(sl * sizeof(int32_t), kAlign);
        x.ring = x.ring_arr + align_up(sl * sizeof(int32_t), kAlign);
        x.total = x.ring + sl * x.ring_stride * sizeof(float);
    }
    return x;
}

void layout(const gdn_pool_desc* d, size_t* state_bytes, size_t* window_bytes, size_t* aux_bytes) {
    *state_bytes = (size_t)d->n_slots * d->n_layers * d->h_v * d->d_v * d->d_k * sizeof(float);
    const AuxLayout x = aux_layout(d);
    *window_bytes = x.window_bytes;
    *aux_bytes = x.total;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Host-side C++ failures (a host array that cannot be allocated in
// GDN_VALIDATE mode) never cross the C ABI: they become GDN_ERR_HOST, and
// nothing has been enqueued by then.
template <typename F>
gdn_status guarded(F&& f) noexcept {
    try {
        return f();
    } catch (...) {
        return GDN_ERR_HOST;
    }
}

// GDN_VALIDATE: copy a device index array to the host and check it.
gdn_status host_check_ids(const int32_t* ids, int32_t n, int32_t n_slots, hipStream_t s) {
    std::vector<int32_t> h(n);
    if (n == 0) return GDN_OK;
    if (hipMemcpyAsync(h.data(), ids, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return GDN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    std::vector<int32_t> seen;
    for (int32_t x : h) {
        if (x >= n_slots) return GDN_ERR_BAD_INDEX;
        if (x >= 0) seen.push_back(x);
    }
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return GDN_ERR_BAD_INDEX;
    return GDN_OK;
}

gdn_status host_check_seqlens(const int32_t* cu, int32_t n_seq, int64_t total, hipStream_t s) {
    std::vector<int32_t> h(n_seq + 1);
    if (hipMemcpyAsync(h.data(), cu, (n_seq + 1) * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return GDN_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    if (h[0] != 0 || h[n_seq] != total) return GDN_ERR_BAD_INDEX;
    for (int j = 0; j < n_seq; ++j)
        if (h[j + 1] < h[j]) return GDN_ERR_BAD_INDEX;
    return GDN_OK;
}

// Host check of the checkpoint lists (GDN_VALIDATE): offsets from 0,
// non-decreasing; every sequence and checkpoint slot in range and distinct.
// The row count is bounded before anything is sized from it: no sequence can
// use more than len_j / ckpt_every rows, so more than
// total_tokens / ckpt_every + n_seq rows in all is rejected.
gdn_status host_check_ckpt(const int32_t* slot_ids, int32_t n_seq, const int32_t* off,
                           const int32_t* slots, int32_t n_slots, int64_t total_tokens,
                           int32_t ckpt_every, hipStream_t s) {
    std::vector<int32_t> ho(n_seq + 1), hs(n_seq);
    if (hipMemcpyAsync(ho.data(), off, (n_seq + 1) * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(hs.data(), slot_ids, n_seq * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return GDN_ERR_HIP;
    if (ho[0] != 0) return GDN_ERR_BAD_INDEX;
    for (int j = 0; j < n_seq; ++j)
        if (ho[j + 1] < ho[j]) return GDN_ERR_BAD_INDEX;
    if ((int64_t)ho[n_seq] > total_tokens / ckpt_every + n_seq) return GDN_ERR_BAD_INDEX;
    std::vector<int32_t> hc(ho[n_seq]);
    if (!hc.empty() &&
        (hipMemcpyAsync(hc.data(), slots, hc.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
         hipStreamSynchronize(s) != hipSuccess))
        return GDN_ERR_HIP;
    std::vector<int32_t> seen;
    for (int32_t x : hs) if (x >= 0) seen.push_back(x);
    for (int32_t x : hc) if (x >= 0) seen.push_back(x);
    for (int32_t x : seen) if (x >= n_slots) return GDN_ERR_BAD_INDEX;
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return GDN_ERR_BAD_INDEX;
    return GDN_OK;
}

// GDN_VALIDATE for the one-call path on a ring pool: every listed slot's ring
// for `layer` must be empty (the call reads and writes the state tile).
gdn_status host_check_rings_empty(const gdn_pool* pool, int32_t layer, const int32_t* ids,
                                  int32_t n, hipStream_t s) {
    if (pool->desc.ring_len == 0 || n == 0) return GDN_OK;
    const size_t sl = (size_t)pool->desc.n_slots * pool->desc.n_layers;
    std::vector<int32_t> h(n), cnt(sl);
    if (hipMemcpyAsync(h.data(), ids, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(cnt.data(), pool->view.ring_cnt, sl * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return GDN_ERR_HIP;
    for (int32_t x : h)
        if (x >= 0 && x < pool->desc.n_slots && cnt[(size_t)x * pool->desc.n_layers + layer] != 0)
            return GDN_ERR_RING;
    return GDN_OK;
}

gdn_status prefill_common(gdn_pool* pool, int32_t layer, int32_t n_seq, const int32_t* cu_seqlens,
                          const int32_t* slot_ids, int64_t total_tokens, int32_t chunk,
                          const void* q, const void* k, const void* v, const float* a,
                          const float* b, const float* conv_w, void* out, int32_t ckpt_every,
                          const int32_t* ckpt_offsets, const int32_t* ckpt_slots, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!pool || layer < 0 || layer >= pool->desc.n_layers || n_seq < 0 || total_tokens < 0)
        return GDN_ERR_INVALID_ARG;
    if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_UNSUPPORTED;
    if (total_tokens > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if (ckpt_every < 0 || ckpt_every % chunk != 0) return GDN_ERR_INVALID_ARG;
    if (n_seq == 0) return GDN_OK;
    if (!cu_seqlens || !slot_ids || !conv_w) return GDN_ERR_INVALID_ARG;
    if (ckpt_every > 0 && (!ckpt_offsets || !ckpt_slots)) return GDN_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !a || !b || !out)) return GDN_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)))
        return GDN_ERR_INVALID_ARG;
    const size_t need = prefill_workspace_bytes(pool, n_seq, total_tokens, chunk);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDN_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, kAlign)) return GDN_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    if (pool->desc.flags & GDN_VALIDATE) {
        gdn_status st = ckpt_every > 0
                            ? host_check_ckpt(slot_ids, n_seq, ckpt_offsets, ckpt_slots,
                                              pool->desc.n_slots, total_tokens, ckpt_every, s)
                            : host_check_ids(slot_ids, n_seq, pool->desc.n_slots, s);
        if (st != GDN_OK) return st;
        st = host_check_seqlens(cu_seqlens, n_seq, total_tokens, s);
        if (st != GDN_OK) return st;
        st = host_check_rings_empty(pool, layer, slot_ids, n_seq, s);
        if (st == GDN_OK && ckpt_every > 0) {
            int32_t n_ck = 0;
            if (hipMemcpyAsync(&n_ck, ckpt_offsets + n_seq, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
                hipStreamSynchronize(s) != hipSuccess)
                return GDN_ERR_HIP;
            st = host_check_rings_empty(pool, layer, ckpt_slots, n_ck, s);
        }
        if (st != GDN_OK) return st;
    }
    const Ckpt ck{ckpt_every / chunk, ckpt_offsets, ckpt_slots};
    hipError_t e = launch_prefill(pool, layer, n_seq, cu_seqlens, slot_ids, total_tokens, chunk, q,
                                  k, v, a, b, conv_w, out, workspace, ck, s);
    if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

extern "C" {

gdn_status gdn_pool_bytes(const gdn_pool_desc* desc, size_t* state_bytes, size_t* aux_bytes) {
    gdn_status st = check_desc(desc);
    if (st != GDN_OK) return st;
    if (!state_bytes || !aux_bytes) return GDN_ERR_INVALID_ARG;
    size_t wb;
    layout(desc, state_bytes, &wb, aux_bytes);
    return GDN_OK;
}

gdn_status gdn_pool_create(const gdn_pool_desc* desc, void* state_buf, void* aux_buf, void* stream,
                           gdn_pool** out) {
    gdn_status st = check_desc(desc);
    if (st != GDN_OK) return st;
    if (!state_buf || !aux_buf || !out) return GDN_ERR_INVALID_ARG;
    if (!aligned(state_buf, kAlign) || !aligned(aux_buf, kAlign)) return GDN_ERR_INVALID_ARG;
    gdn_pool* p = new (std::nothrow) gdn_pool();
    if (!p) return GDN_ERR_INVALID_ARG;
    p->desc = *desc;
    if (p->desc.q_scale == 0.f) p->desc.q_scale = 1.0f / std::sqrt((float)desc->d_k);
    if (p->desc.norm_eps == 0.f) p->desc.norm_eps = 1e-6f;
    layout(desc, &p->state_bytes, &p->window_bytes, &p->aux_bytes);
    p->io_size = desc->io_dtype == GDN_BF16 ? 2 : 4;
    PoolView& v = p->view;
    v.state = static_cast<float*>(state_buf);
    v.window = aux_buf;
    const AuxLayout ax = aux_layout(desc);
    char* aux = static_cast<char*>(aux_buf);
    v.err = reinterpret_cast<int32_t*>(aux + ax.meta);
    v.ctr = reinterpret_cast<int32_t*>(aux + ax.ctr);
    v.ring_len = desc->ring_len;
    v.ring_cnt = desc->ring_len > 0 ? reinterpret_cast<int32_t*>(aux + ax.ring_cnt) : nullptr;
    v.ring_arr = desc->ring_len > 0 ? reinterpret_cast<int32_t*>(aux + ax.ring_arr) : nullptr;
    v.ring = desc->ring_len > 0 ? reinterpret_cast<float*>(aux + ax.ring) : nullptr;
    v.ring_stride = ax.ring_stride;
    v.n_slots = desc->n_slots;
    v.n_layers = desc->n_layers;
    v.h_k = desc->h_k;
    v.h_v = desc->h_v;
    v.d = desc->d_k;
    v.conv_k = desc->conv_k;
    v.c_conv = 2 * desc->h_k * desc->d_k + desc->h_v * desc->d_v;
    v.q_scale = p->desc.q_scale;
    v.eps = p->desc.norm_eps;
    hipStream_t s = as_stream(stream);
    if (launch_fill_zero(state_buf, p->state_bytes, s) != hipSuccess ||
        launch_fill_zero(aux_buf, p->aux_bytes, s) != hipSuccess) {
        delete p;
        return GDN_ERR_HIP;
    }
    *out = p;
    return GDN_OK;
}

gdn_status gdn_pool_destroy(gdn_pool* pool) {
    if (!pool) return GDN_ERR_INVALID_ARG;
    delete pool;
    return GDN_OK;
}

gdn_status gdn_slot_reset(gdn_pool* pool, int32_t n, const int32_t* slot_ids, void* stream) {
    return guarded([&]() -> gdn_status {
        if (!pool || n < 0 || (n > 0 && !slot_ids)) return GDN_ERR_INVALID_ARG;
        if (n == 0) return GDN_OK;
        if (n > 65535) return GDN_ERR_UNSUPPORTED;  // grid.y limit
        hipStream_t s = as_stream(stream);
        if (pool->desc.flags & GDN_VALIDATE) {
            gdn_status st = host_check_ids(slot_ids, n, pool->desc.n_slots, s);
            if (st != GDN_OK) return st;
        }
        return launch_slot_reset(pool, n, slot_ids, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    });
}

static gdn_status check_step_args(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                                  int32_t n_tok, const void* q, const void* k, const void* v,
                                  const float* a, const float* b, const float* conv_w,
                                  const void* out, bool out_optional = false) {
    if (!pool) return GDN_ERR_INVALID_ARG;
    if (layer < 0 || layer >= pool->desc.n_layers || n < 0) return GDN_ERR_INVALID_ARG;
    if (n_tok < 1 || n_tok > kMaxVerifyTokens) return GDN_ERR_INVALID_ARG;
    if (n > 0 && (!slot_ids || !q || !k || !v || !a || !b || !conv_w || (!out && !out_optional)))
        return GDN_ERR_INVALID_ARG;
    if (n > 65535) return GDN_ERR_UNSUPPORTED;  // grid.y limit
    if (n > 0 && out && !aligned(out, 16)) return GDN_ERR_INVALID_ARG;  // 16-byte output vectors
    if (decode_verify_lds_bytes(pool, n_tok) > kMaxLds) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

gdn_status gdn_decode_step(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           const void* q, const void* k, const void* v, const float* a,
                           const float* b, const float* conv_w, void* out, void* stream) {
    return guarded([&]() -> gdn_status {
        gdn_status st = check_step_args(pool, layer, n, slot_ids, 1, q, k, v, a, b, conv_w, out);
        if (st != GDN_OK || n == 0) return st;
        hipStream_t s = as_stream(stream);
        if (pool->desc.flags & GDN_VALIDATE) {
            st = host_check_ids(slot_ids, n, pool->desc.n_slots, s);
            if (st == GDN_OK) st = host_check_rings_empty(pool, layer, slot_ids, n, s);
            if (st != GDN_OK) return st;
        }
        // Few entries: split each head's rows over several workgroups so that
        // more CUs stream the state (same arithmetic, bitwise equal results).
        // Otherwise one value head per workgroup (d_k 64 or 128), else the
        // one-workgroup-per-group kernel.  All three are bitwise equal.
        const bool group = pool->desc.flags & GDN_GROUP_KERNEL;
        const int nrb = group ? 1 : decode_rows_split(pool, n);
        const hipError_t e =
            nrb > 1 ? launch_decode_rows(pool, nrb, layer, n, slot_ids, q, k, v, a, b, conv_w, out, s)
            : !group && decode_heads_ok(pool)
                ? launch_decode_heads(pool, layer, n, slot_ids, 1, q, k, v, a, b, conv_w, nullptr,
                                      out, s)
                : launch_decode_verify(pool, layer, n, slot_ids, 1, q, k, v, a, b, conv_w, nullptr,
                                       out, s);
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    });
}

gdn_status gdn_verify_step(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           int32_t n_tok, const void* q, const void* k, const void* v,
                           const float* a, const float* b, const float* conv_w,
                           const int32_t* accept_len, void* out, void* stream) {
    return guarded([&]() -> gdn_status {
        gdn_status st = check_step_args(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w, out, true);
        if (st != GDN_OK) return st;
        if (n > 0 && !accept_len) return GDN_ERR_INVALID_ARG;
        if (n == 0) return GDN_OK;
        hipStream_t s = as_stream(stream);
        if (pool->desc.flags & GDN_VALIDATE) {
            st = host_check_ids(slot_ids, n, pool->desc.n_slots, s);
            if (st == GDN_OK) st = host_check_rings_empty(pool, layer, slot_ids, n, s);
            if (st != GDN_OK) return st;
        }
        // One value head per workgroup where it applies (d_k 64 or 128),
        // else one workgroup per q/k group; bitwise equal.
        const hipError_t e =
            !(pool->desc.flags & GDN_GROUP_KERNEL) && decode_heads_ok(pool)
                ? launch_decode_heads(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                      accept_len, out, s)
                : launch_decode_verify(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                       accept_len, out, s);
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    });
}

gdn_status gdn_prefill_workspace_bytes(const gdn_pool* pool, int32_t n_seq, int64_t total_tokens,
                                       int32_t chunk, size_t* bytes) {
    if (!pool || !bytes || n_seq < 0 || total_tokens < 0) return GDN_ERR_INVALID_ARG;
    if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_UNSUPPORTED;
    *bytes = prefill_workspace_bytes(pool, n_seq, total_tokens, chunk);
    return GDN_OK;
}

gdn_status gdn_prefill_chunked(gdn_pool* pool, int32_t layer, int32_t n_seq,
                               const int32_t* cu_seqlens, const int32_t* slot_ids,
                               int64_t total_tokens, int32_t chunk, const void* q, const void* k,
                               const void* v, const float* a, const float* b, const float* conv_w,
                               void* out, void* workspace, size_t workspace_bytes, void* stream) {
    return guarded([&]() -> gdn_status {
        return prefill_common(pool, layer, n_seq, cu_seqlens, slot_ids, total_tokens, chunk, q, k, v,
                              a, b, conv_w, out, 0, nullptr, nullptr, workspace, workspace_bytes,
                              stream);
    });
}

gdn_status gdn_prefill_chunked_static(gdn_pool* pool, int32_t layer, int32_t n_seq,
                                      const int32_t* cu_seqlens, const int32_t* slot_ids,
                                      int64_t total_tokens, int32_t chunk, const void* q,
                                      const void* k, const void* v, const float* a,
                                      const float* b, const float* conv_w, void* out,
                                      void* stream) {
    return guarded([&]() -> gdn_status {
        if (!pool || n_seq < 0 || total_tokens < 0) return GDN_ERR_INVALID_ARG;
        if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_UNSUPPORTED;
        if (prefill_workspace_bytes(pool, n_seq, total_tokens, chunk) > kStaticScratchBytes)
            return GDN_ERR_WORKSPACE;
        void* ws = nullptr;
        if (prefill_static_scratch(&ws) != hipSuccess) return GDN_ERR_HIP;
        return prefill_common(pool, layer, n_seq, cu_seqlens, slot_ids, total_tokens, chunk, q, k,
                              v, a, b, conv_w, out, 0, nullptr, nullptr, ws, kStaticScratchBytes,
                              stream);
    });
}

gdn_status gdn_prefill_chunked_ckpt(gdn_pool* pool, int32_t layer, int32_t n_seq,
                                    const int32_t* cu_seqlens, const int32_t* slot_ids,
                                    int64_t total_tokens, int32_t chunk, const void* q,
                                    const void* k, const void* v, const float* a, const float* b,
                                    const float* conv_w, void* out, int32_t ckpt_every,
                                    const int32_t* ckpt_offsets, const int32_t* ckpt_slots,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    return guarded([&]() -> gdn_status {
        return prefill_common(pool, layer, n_seq, cu_seqlens, slot_ids, total_tokens, chunk, q, k, v,
                              a, b, conv_w, out, ckpt_every, ckpt_offsets, ckpt_slots, workspace,
                              workspace_bytes, stream);
    });
}

gdn_status gdn_slot_copy(gdn_pool* pool, int32_t n, const int32_t* src_ids,
                         const int32_t* dst_ids, void* stream) {
    return guarded([&]() -> gdn_status {
        if (!pool || n < 0 || (n > 0 && (!src_ids || !dst_ids))) return GDN_ERR_INVALID_ARG;
        if (n == 0) return GDN_OK;
        if (n > 65535) return GDN_ERR_UNSUPPORTED;  // grid.y limit
        hipStream_t s = as_stream(stream);
        if (pool->desc.flags & GDN_VALIDATE) {
            // sources in range; destinations in range, distinct and not sources
            std::vector<int32_t> hs(n), hd(n);
            if (hipMemcpyAsync(hs.data(), src_ids, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
                hipMemcpyAsync(hd.data(), dst_ids, n * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
                hipStreamSynchronize(s) != hipSuccess)
                return GDN_ERR_HIP;
            std::vector<int32_t> dst;
            for (int i = 0; i < n; ++i) {
                if (hs[i] >= pool->desc.n_slots || hd[i] >= pool->desc.n_slots) return GDN_ERR_BAD_INDEX;
                if (hs[i] >= 0 && hd[i] >= 0) dst.push_back(hd[i]);
            }
            std::sort(dst.begin(), dst.end());
            if (std::adjacent_find(dst.begin(), dst.end()) != dst.end()) return GDN_ERR_BAD_INDEX;
            for (int i = 0; i < n; ++i)
                if (hs[i] >= 0 && hd[i] >= 0 && std::binary_search(dst.begin(), dst.end(), hs[i]))
                    return GDN_ERR_BAD_INDEX;
        }
        return launch_slot_copy(pool, n, src_ids, dst_ids, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    });
}

static gdn_status ring_call(gdn_pool* pool, RingOp op, int32_t layer, int32_t n,
                            const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
                            const void* v, const float* a, const float* b, const float* conv_w,
                            const int32_t* accept_len, void* out, void* stream) {
    return guarded([&]() -> gdn_status {
        if (!pool || layer < 0 || layer >= pool->desc.n_layers || n < 0) return GDN_ERR_INVALID_ARG;
        if (pool->desc.ring_len == 0) return GDN_ERR_UNSUPPORTED;
        if (op != RingOp::kFlush) {
            if (n_tok < 1 || n_tok > kMaxVerifyTokens) return GDN_ERR_INVALID_ARG;
            if (pool->desc.ring_len + n_tok > kMaxRingSolve) return GDN_ERR_UNSUPPORTED;
            if (n > 0 && (!q || !k || !v || !a || !b || !conv_w)) return GDN_ERR_INVALID_ARG;
            if (n > 0 && op == RingOp::kVerify && !out) return GDN_ERR_INVALID_ARG;
            if (n > 0 && op == RingOp::kCommit && !accept_len) return GDN_ERR_INVALID_ARG;
        }
        if (n > 0 && !slot_ids) return GDN_ERR_INVALID_ARG;
        if (n == 0) return GDN_OK;
        hipStream_t s = as_stream(stream);
        if (pool->desc.flags & GDN_VALIDATE) {
            const gdn_status st = host_check_ids(slot_ids, n, pool->desc.n_slots, s);
            if (st != GDN_OK) return st;
        }
        const hipError_t e = launch_ring(pool, op, layer, n, slot_ids, op == RingOp::kFlush ? 0 : n_tok,
                                         q, k, v, a, b, conv_w, accept_len, out, s);
        if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    });
}

gdn_status gdn_ring_verify(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           int32_t n_tok, const void* q, const void* k, const void* v,
                           const float* a, const float* b, const float* conv_w, void* out,
                           void* stream) {
    return ring_call(pool, RingOp::kVerify, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                     nullptr, out, stream);
}

gdn_status gdn_ring_commit(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                           int32_t n_tok, const void* q, const void* k, const void* v,
                           const float* a, const float* b, const float* conv_w,
                           const int32_t* accept_len, void* stream) {
    return ring_call(pool, RingOp::kCommit, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                     accept_len, nullptr, stream);
}

gdn_status gdn_ring_flush(gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                          void* stream) {
    return ring_call(pool, RingOp::kFlush, layer, n, slot_ids, 0, nullptr, nullptr, nullptr,
                     nullptr, nullptr, nullptr, nullptr, nullptr, stream);
}

static gdn_status in_proj_args(const gdn_pool* pool, int64_t n_tok, int32_t hidden) {
    if (!pool || n_tok < 0 || hidden < 1) return GDN_ERR_INVALID_ARG;
    if (hidden % 32 != 0) return GDN_ERR_UNSUPPORTED;
    const int64_t n_out = pool->view.c_conv + 2 * pool->view.h_v;
    // 32-bit byte offsets inside x and W (128 rows of slack for ragged tiles)
    if ((n_tok + 128) * hidden * 2 >= INT32_MAX || (n_out + 128) * hidden * 2 >= INT32_MAX)
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

gdn_status gdn_in_proj_workspace_bytes(const gdn_pool* pool, int64_t n_tok, int32_t hidden,
                                       size_t* bytes) {
    const gdn_status st = in_proj_args(pool, n_tok, hidden);
    if (st != GDN_OK) return st;
    if (!bytes) return GDN_ERR_INVALID_ARG;
    *bytes = in_proj_workspace_bytes(pool, n_tok, hidden);
    return GDN_OK;
}

gdn_status gdn_in_proj(gdn_pool* pool, int64_t n_tok, int32_t hidden, const void* x, const void* w,
                       void* q, void* k, void* v, float* a, float* b, void* workspace,
                       size_t workspace_bytes, void* stream) {
    const gdn_status st = in_proj_args(pool, n_tok, hidden);
    if (st != GDN_OK) return st;
    if (n_tok == 0) return GDN_OK;
    if (!x || !w || !q || !k || !v || !a || !b) return GDN_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w, 16)) return GDN_ERR_INVALID_ARG;
    const size_t need = in_proj_workspace_bytes(pool, n_tok, hidden);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDN_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, kAlign)) return GDN_ERR_INVALID_ARG;
    return launch_in_proj(pool, n_tok, hidden, x, w, q, k, v, a, b, workspace,
                          as_stream(stream)) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

gdn_status gdn_pool_error(gdn_pool* pool, void* stream, int32_t* device_error) {
    if (!pool || !device_error) return GDN_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    int32_t h = 0;
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    if (hipMemcpy(&h, pool->view.err, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return GDN_ERR_HIP;
    if (h != 0) {
        if (launch_fill_zero(pool->view.err, kAlign, s) != hipSuccess) return GDN_ERR_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_HIP;
    }
    *device_error = h;
    return GDN_OK;
}

const char* gdn_status_string(gdn_status status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported shape or option";
        case GDN_ERR_BAD_INDEX: return "slot id out of range or repeated, or malformed cu_seqlens";
        case GDN_ERR_WORKSPACE: return "prefill workspace too small";
        case GDN_ERR_HIP: return "HIP runtime error";
        case GDN_ERR_RING: return "a listed slot's verify ring is not empty (flush it first)";
        case GDN_ERR_HOST: return "host-side failure (host memory)";
        default: return "unknown status";
    }
}

}  // extern "C"
