// C ABI of libh2o: argument validation, kernel dispatch, optional timers.
// Entry points are declared and documented in include/h2o.h.
#include "h2o_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

namespace h2o {
namespace {

thread_local std::string g_error;

h2o_status_t fail(h2o_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

h2o_status_t ok() {
    g_error.clear();
    return H2O_OK;
}

h2o_status_t check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(H2O_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return H2O_OK;
}

h2o_status_t validate_dims(const h2o_dims_t* d) {
    if (!d) return fail(H2O_ERR_INVALID_ARG, "dims is NULL");
    if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
        return fail(H2O_ERR_INVALID_ARG, "batch, n_q_heads and n_kv_heads must be >= 1");
    if (d->n_q_heads % d->n_kv_heads != 0)
        return fail(H2O_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                    d->n_q_heads, d->n_kv_heads);
    if (d->dtype != H2O_F32 && d->dtype != H2O_BF16)
        return fail(H2O_ERR_UNSUPPORTED, "dtype %d is not supported", d->dtype);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(H2O_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
    if (d->capacity < 1 || d->capacity > kMaxCapacity)
        return fail(H2O_ERR_UNSUPPORTED, "capacity %d outside 1..%d", d->capacity, kMaxCapacity);
    if (d->recent_window < 0) return fail(H2O_ERR_INVALID_ARG, "recent_window must be >= 0");
    const long long groups = (long long)d->batch * d->n_kv_heads;
    if (groups > 65535 || (long long)d->batch * d->n_q_heads > (1LL << 24))
        return fail(H2O_ERR_UNSUPPORTED, "batch x heads too large");
    return H2O_OK;
}

h2o_status_t validate_cache(const h2o_dims_t* d, const h2o_cache_t* c) {
    if (!c) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
    if (!c->k || !c->v || !c->pos || !c->score)
        return fail(H2O_ERR_INVALID_ARG, "cache k, v, pos and score must be non-NULL");
    if (c->n_valid < 0 || c->n_valid > d->capacity)
        return fail(H2O_ERR_INVALID_ARG, "n_valid %d outside 0..capacity (%d)", c->n_valid,
                    d->capacity);
    return H2O_OK;
}

h2o_status_t validate_chunk(int64_t chunk_start, int32_t chunk_len) {
    if (chunk_len < 1) return fail(H2O_ERR_INVALID_ARG, "chunk_len must be >= 1");
    if (chunk_len > (1 << 20)) return fail(H2O_ERR_UNSUPPORTED, "chunk_len too large");
    if (chunk_start < 0) return fail(H2O_ERR_INVALID_ARG, "chunk_start must be >= 0");
    if (chunk_start + (int64_t)chunk_len > 2147483647LL)
        return fail(H2O_ERR_UNSUPPORTED, "chunk_start + chunk_len exceeds INT32_MAX");
    return H2O_OK;
}

// Kernel timers --------------------------------------------------------------
struct Timer {
    bool on = false;
    int max = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;
};
Timer g_timer[H2O_KERNEL_COUNT];

void destroy_events(Timer& t) {
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
    t.ev.clear();
    t.on = false;
    t.used = 0;
    t.max = 0;
}

}  // namespace

void timer_begin(int kernel, hipStream_t s) {
    Timer& t = g_timer[kernel];
    if (t.on && t.used < t.max) (void)hipEventRecord(t.ev[2 * t.used], s);
}

void timer_end(int kernel, hipStream_t s) {
    Timer& t = g_timer[kernel];
    if (t.on && t.used < t.max) {
        (void)hipEventRecord(t.ev[2 * t.used + 1], s);
        ++t.used;
    }
}

// The S = 1 split-KV specialisation (bf16, d = 128, at most 32 query heads per KV head).
bool uses_decode(const h2o_dims_t* dims, int32_t chunk_len) {
    return chunk_len == 1 && dims->dtype == H2O_BF16 && dims->head_dim == 128 &&
           dims->n_q_heads / dims->n_kv_heads <= 32;
}

// Compute units of the current device, read once per device.
hipError_t cu_count(int* cus) {
    static int cached[64] = {0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (cached[dev] == 0) {
        int v = 0;
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cached[dev] = v > 0 ? v : 1;
    }
    *cus = cached[dev];
    return hipSuccess;
}

// One SideStream per device, made at its first use; the lock is held from the
// fork to the join of a call, so calls from several host threads do not mix
// their forks on one device.
std::mutex& side_stream_lock() {
    static std::mutex mu;
    return mu;
}
// Caller holds side_stream_lock().  nullptr if the stream or events cannot be
// made (the call then runs its launches on the caller's stream alone).
const SideStream* side_stream() {
    static SideStream side[64];
    static bool tried[64] = {false};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    if (!tried[dev]) {
        tried[dev] = true;
        SideStream t;
        if (hipStreamCreateWithFlags(&t.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&t.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&t.join, hipEventDisableTiming) == hipSuccess) {
            side[dev] = t;
        } else {
            // release whatever was made; the error is not left for the next call
            if (t.fork) (void)hipEventDestroy(t.fork);
            if (t.s) (void)hipStreamDestroy(t.s);
            (void)hipGetLastError();
        }
    }
    return side[dev].join != nullptr ? &side[dev] : nullptr;
}

// Workspace layout of a non-decode chunk: the split summed-weights partials
// (bf16) and then, 256-byte aligned, the exclusion bits of the buffer form.
size_t excl_offset(const h2o_dims_t* dims, int32_t chunk_len) {
    if (dims->dtype != H2O_BF16) return 0;
    const size_t b = colsum_workspace_bytes(dims->batch, dims->n_kv_heads, dims->capacity,
                                            chunk_len);
    return (b + 255) / 256 * 256;
}
size_t excl_bytes(const h2o_dims_t* dims) {
    return (size_t)dims->batch * dims->n_kv_heads * excl_tiles(dims->capacity) * sizeof(uint64_t);
}

// H2O_ERR_CAPACITY when k = n + S - N_C > 0 slots must go and the chunk plus the
// protected slots (recent window, or lastrec's sink) exceed the capacity.
h2o_status_t check_capacity(const h2o_dims_t* dims, const h2o_cache_t* cache, int32_t S,
                            int mode, int sink) {
    const int n = cache->n_valid, NC = dims->capacity;
    const int k = n + S - NC;
    const bool lastrec = mode == kModeLastrec;
    const long long guard = lastrec ? sink : dims->recent_window;
    if (k > 0 && (long long)S + guard > NC)
        return fail(H2O_ERR_CAPACITY, "cannot evict %d slots: capacity %d < chunk_len %d + %s %lld",
                    k, NC, S, lastrec ? "sink_tokens" : "recent_window", guard);
    return H2O_OK;
}

// Shared body of the eviction entry points.  mode: h2o_score_mode_t, or
// kModeLastrec with `sink` protected leading positions; colsum_new NULL gives
// inserted slots score 0.  do_select / do_insert: run the selection (targets
// into freed_slots) and / or the insertion (from freed_slots).
h2o_status_t evict_and_insert(const h2o_dims_t* dims, h2o_cache_t* cache, int64_t chunk_start,
                              int32_t chunk_len, int mode, int sink, const void* k_new,
                              const void* v_new, const float* colsum_new, int32_t* freed_slots,
                              void* stream, bool do_select = true, bool do_insert = true,
                              const float* cs_upd = nullptr) {
    h2o_status_t st;
    if ((st = validate_dims(dims)) != H2O_OK) return st;
    if ((st = validate_cache(dims, cache)) != H2O_OK) return st;
    if ((st = validate_chunk(chunk_start, chunk_len)) != H2O_OK) return st;
    if ((do_insert && (!k_new || !v_new)) || !freed_slots)
        return fail(H2O_ERR_INVALID_ARG, "k_new, v_new and freed_slots must be non-NULL");
    if ((st = check_capacity(dims, cache, chunk_len, mode, sink)) != H2O_OK) return st;
    const int n = cache->n_valid, S = chunk_len, NC = dims->capacity;
    const int k = n + S - NC;
    EvictArgs a;
    a.kc = cache->k;
    a.vc = cache->v;
    a.pos = cache->pos;
    a.score = cache->score;
    a.kn = k_new;
    a.vn = v_new;
    a.cs_new = colsum_new;
    a.freed = freed_slots;
    a.B = dims->batch;
    a.Hkv = dims->n_kv_heads;
    a.D = dims->head_dim;
    a.S = S;
    a.NC = NC;
    a.n = n;
    a.W = dims->recent_window;
    a.P = (int)chunk_start;
    a.elem_bytes = dims->dtype == H2O_BF16 ? 2 : 4;
    a.score_mode = mode;
    a.sink = sink;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (cs_upd != nullptr) {
        // The score update of h2o_update_scores: inside the selection when there is
        // one (it reads every score anyway), else on its own.
        if (k > 0 && do_select) {
            a.cs_upd = cs_upd;
        } else {
            timer_begin(H2O_KERNEL_UPDATE, s);
            hipError_t e = launch_update_scores(cache->score, cs_upd, a.B * a.Hkv, NC, n, s);
            timer_end(H2O_KERNEL_UPDATE, s);
            if ((st = check_hip(e, "update launch")) != H2O_OK) return st;
        }
    }
    if (do_select && do_insert && k == 1 && S == 1) {
        // one victim and one token: one launch, timed as the selection
        timer_begin(H2O_KERNEL_SELECT, s);
        hipError_t e = launch_select1_insert(a, s);
        timer_end(H2O_KERNEL_SELECT, s);
        if ((st = check_hip(e, "select/insert launch")) != H2O_OK) return st;
        cache->n_valid = NC;
        return ok();
    }
    if (do_select) {
        timer_begin(H2O_KERNEL_SELECT, s);
        hipError_t e = launch_select(a, s);
        timer_end(H2O_KERNEL_SELECT, s);
        if ((st = check_hip(e, "select launch")) != H2O_OK) return st;
    }
    if (do_insert) {
        timer_begin(H2O_KERNEL_INSERT, s);
        hipError_t e = launch_insert(a, s);
        timer_end(H2O_KERNEL_INSERT, s);
        if ((st = check_hip(e, "insert launch")) != H2O_OK) return st;
        cache->n_valid = n + S < NC ? n + S : NC;
    }
    return ok();
}

}  // namespace h2o

using namespace h2o;

extern "C" {

int32_t h2o_abi_version(void) { return H2O_ABI_VERSION; }

const char* h2o_last_error(void) { return g_error.c_str(); }

size_t h2o_workspace_bytes(const h2o_dims_t* dims, int32_t chunk_len) {
    if (validate_dims(dims) != H2O_OK || chunk_len < 1) return 0;
    if (uses_decode(dims, chunk_len))
        return decode_workspace_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads,
                                      dims->capacity);
    return excl_offset(dims, chunk_len) + excl_bytes(dims);
}

}  // extern "C"

namespace h2o {

h2o_status_t set_error(h2o_status_t st, const char* msg) { return fail(st, "%s", msg); }

// Workspace: the decode partials; else the split summed-weights partials (bf16,
// when summed weights are asked for) and the exclusion bits (buffer form).
size_t chunk_attn_workspace_need(const h2o_dims_t* dims, int32_t chunk_len, bool summed_weights,
                                 bool buffer_form) {
    if (validate_dims(dims) != H2O_OK || chunk_len < 1) return 0;
    if (uses_decode(dims, chunk_len)) return h2o_workspace_bytes(dims, chunk_len);
    if (buffer_form) return excl_offset(dims, chunk_len) + excl_bytes(dims);
    if (summed_weights && dims->dtype == H2O_BF16) return excl_offset(dims, chunk_len);
    return 0;
}

// Shared body of h2o_chunk_attn and h2o_buffer_attn (freed != NULL: the
// victims among the targets are not keys).
h2o_status_t chunk_attn(const h2o_dims_t* dims, const h2o_cache_t* cache, int64_t chunk_start,
                        int32_t chunk_len, float sm_scale, const void* q, const void* k_new,
                        const void* v_new, const int32_t* freed, void* out, float* lse,
                        float* colsum_cache, float* colsum_new, void* workspace,
                        size_t workspace_bytes, void* stream, const EvictArgs* ev) {
    h2o_status_t st;

    if ((st = validate_dims(dims)) != H2O_OK) return st;
    if ((st = validate_cache(dims, cache)) != H2O_OK) return st;
    if ((st = validate_chunk(chunk_start, chunk_len)) != H2O_OK) return st;
    if (!q || !k_new || !v_new || !out || !lse)
        return fail(H2O_ERR_INVALID_ARG, "q, k_new, v_new, out and lse must be non-NULL");
    if ((colsum_cache == nullptr) != (colsum_new == nullptr))
        return fail(H2O_ERR_INVALID_ARG, "colsum_cache and colsum_new must both be set or both be NULL");
    const bool want_cs = colsum_cache != nullptr;
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
        return fail(H2O_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
    {
        const long long G = dims->n_q_heads / dims->n_kv_heads;
        if (G * G * (long long)chunk_len >= (1LL << 31) ||
            G * (long long)chunk_len * dims->head_dim * 4 >= (1LL << 31))
            return fail(H2O_ERR_UNSUPPORTED, "query heads per KV head (%lld) too large for chunk_len %d",
                        G, chunk_len);
    }
    const bool decode = uses_decode(dims, chunk_len);
    const size_t ws_need = chunk_attn_workspace_need(dims, chunk_len, want_cs, freed != nullptr);
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need))
        return fail(H2O_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", ws_need,
                    workspace ? workspace_bytes : (size_t)0);

    ChunkArgs a;
    a.q = q;
    a.kc = cache->k;
    a.vc = cache->v;
    a.kn = k_new;
    a.vn = v_new;
    a.pos = cache->pos;
    a.out = out;
    a.lse = lse;
    a.cs_cache = colsum_cache;
    a.cs_new = colsum_new;
    a.B = dims->batch;
    a.Hq = dims->n_q_heads;
    a.Hkv = dims->n_kv_heads;
    a.G = dims->n_q_heads / dims->n_kv_heads;
    a.D = dims->head_dim;
    a.S = chunk_len;
    a.NC = dims->capacity;
    a.n = cache->n_valid;
    a.P = (int)chunk_start;
    a.sm_scale = sm_scale;
    a.freed = freed;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int rows = a.B * a.Hkv;
    if (freed && !decode) {
        uint64_t* excl = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) +
                                                     excl_offset(dims, chunk_len));
        if ((st = check_hip(launch_build_excl(a, excl, s), "exclusion masks")) != H2O_OK)
            return st;
        a.excl = excl;
    }

    const bool bf16 = dims->dtype == H2O_BF16;
    int parts = 1;
    if (want_cs && bf16 && !decode) {
        int cus = 0;
        if ((st = check_hip(cu_count(&cus), "device attributes")) != H2O_OK) return st;
        parts = colsum_parts(a, cus);
    }
    // The reduction of a split colsum writes the empty slots itself.
    if (want_cs && parts == 1 && a.n < a.NC) {
        if ((st = check_hip(launch_zero_f32(colsum_cache, a.NC - a.n, a.NC, rows, a.n, s),
                            "zero colsum tail")) != H2O_OK)
            return st;
    }
    if (decode) {
        hipError_t e = launch_decode(a, workspace, s, ev);  // times its two kernels
        if ((st = check_hip(e, "decode attention launch")) != H2O_OK) return st;
        return ok();
    }
    timer_begin(H2O_KERNEL_ATTN, s);
    hipError_t e = bf16 ? launch_attn_bf16(a, s) : launch_attn_f32(a, s);
    timer_end(H2O_KERNEL_ATTN, s);
    if ((st = check_hip(e, "attention launch")) != H2O_OK) return st;
    if (!want_cs) return ok();
    timer_begin(H2O_KERNEL_COLSUM, s);
    e = bf16 ? launch_colsum_bf16(a, parts, static_cast<float*>(workspace), s)
             : launch_colsum_f32(a, s);
    timer_end(H2O_KERNEL_COLSUM, s);
    if ((st = check_hip(e, "colsum launch")) != H2O_OK) return st;
    return ok();
}


}  // namespace h2o

extern "C" {

h2o_status_t h2o_chunk_attn(const h2o_dims_t* dims, const h2o_cache_t* cache,
                            int64_t chunk_start, int32_t chunk_len, float sm_scale,
                            const void* q, const void* k_new, const void* v_new, void* out,
                            float* lse, float* colsum_cache, float* colsum_new,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_attn(dims, cache, chunk_start, chunk_len, sm_scale, q, k_new, v_new, nullptr,
                      out, lse, colsum_cache, colsum_new, workspace, workspace_bytes, stream);
}

h2o_status_t h2o_buffer_attn(const h2o_dims_t* dims, const h2o_cache_t* cache,
                             int64_t chunk_start, int32_t chunk_len, float sm_scale,
                             const void* q, const void* k_new, const void* v_new,
                             const int32_t* freed_slots, void* out, float* lse,
                             float* colsum_cache, float* colsum_new, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (!freed_slots) return fail(H2O_ERR_INVALID_ARG, "freed_slots is NULL");
    return chunk_attn(dims, cache, chunk_start, chunk_len, sm_scale, q, k_new, v_new,
                      freed_slots, out, lse, colsum_cache, colsum_new, workspace,
                      workspace_bytes, stream);
}

size_t h2o_backward_workspace_bytes(const h2o_dims_t* dims, int32_t chunk_len) {
    if (validate_dims(dims) != H2O_OK || chunk_len < 1) return 0;
    return backward_workspace_bytes(dims->batch, dims->n_q_heads, chunk_len) + excl_bytes(dims);
}

h2o_status_t h2o_chunk_attn_backward(const h2o_dims_t* dims, const h2o_cache_t* cache,
                                     int64_t chunk_start, int32_t chunk_len, float sm_scale,
                                     const void* q, const void* k_new, const void* v_new,
                                     const void* out, const float* lse, const void* dout,
                                     const int32_t* freed_slots, float* dq, float* dk_new,
                                     float* dv_new, float* dk_cache, float* dv_cache,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    h2o_status_t st;
    if ((st = validate_dims(dims)) != H2O_OK) return st;
    if ((st = validate_cache(dims, cache)) != H2O_OK) return st;
    if ((st = validate_chunk(chunk_start, chunk_len)) != H2O_OK) return st;
    if (!q || !k_new || !v_new || !out || !lse || !dout)
        return fail(H2O_ERR_INVALID_ARG, "q, k_new, v_new, out, lse and dout must be non-NULL");
    if (!dq || !dk_new || !dv_new || !dk_cache || !dv_cache)
        return fail(H2O_ERR_INVALID_ARG, "gradient buffers must be non-NULL");
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
        return fail(H2O_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
    {
        const long long G = dims->n_q_heads / dims->n_kv_heads;
        if (G * G * (long long)chunk_len >= (1LL << 31) ||
            G * (long long)chunk_len * dims->head_dim * 4 >= (1LL << 31))
            return fail(H2O_ERR_UNSUPPORTED, "query heads per KV head (%lld) too large for chunk_len %d",
                        G, chunk_len);
    }
    const size_t ws_drow = backward_workspace_bytes(dims->batch, dims->n_q_heads, chunk_len);
    const size_t ws_need = ws_drow + (freed_slots ? excl_bytes(dims) : 0);
    if (!workspace || workspace_bytes < ws_need)
        return fail(H2O_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", ws_need,
                    workspace ? workspace_bytes : (size_t)0);
    ChunkArgs a;
    a.q = q;
    a.kc = cache->k;
    a.vc = cache->v;
    a.kn = k_new;
    a.vn = v_new;
    a.pos = cache->pos;
    a.out = const_cast<void*>(out);
    a.lse = const_cast<float*>(lse);
    a.cs_cache = nullptr;
    a.cs_new = nullptr;
    a.B = dims->batch;
    a.Hq = dims->n_q_heads;
    a.Hkv = dims->n_kv_heads;
    a.G = dims->n_q_heads / dims->n_kv_heads;
    a.D = dims->head_dim;
    a.S = chunk_len;
    a.NC = dims->capacity;
    a.n = cache->n_valid;
    a.P = (int)chunk_start;
    a.sm_scale = sm_scale;
    a.freed = freed_slots;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* drow = static_cast<float*>(workspace);
    if (freed_slots) {
        uint64_t* excl = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + ws_drow);
        if ((st = check_hip(launch_build_excl(a, excl, s), "exclusion masks")) != H2O_OK) return st;
        a.excl = excl;
    }
    const int rows = a.B * a.Hkv;
    // bf16: key blocks may be split into two row halves that add into zeroed
    // dK/dV buffers; otherwise only the empty slots' rows are zeroed here.
    int parts = 1;
    if (dims->dtype == H2O_BF16) {
        int cus = 0;
        if ((st = check_hip(cu_count(&cus), "device attributes")) != H2O_OK) return st;
        parts = backward_dkdv_parts(a, cus);
    }
    timer_begin(H2O_KERNEL_BACKWARD, s);
    const size_t cstride = (size_t)a.NC * a.D, nstride = (size_t)a.S * a.D;
    if (parts == 2) {
        float* const bufs[4] = {dk_cache, dv_cache, dk_new, dv_new};
        const size_t counts[4] = {cstride * rows, cstride * rows, nstride * rows, nstride * rows};
        if ((st = check_hip(launch_zero_f32_list(bufs, counts, 4, s), "zero dk, dv")) != H2O_OK)
            return st;
    } else if (a.n < a.NC) {
        const size_t per = (size_t)(a.NC - a.n) * a.D;
        if ((st = check_hip(launch_zero_f32(dk_cache, per, cstride, rows, (size_t)a.n * a.D, s),
                            "zero dk tail")) != H2O_OK ||
            (st = check_hip(launch_zero_f32(dv_cache, per, cstride, rows, (size_t)a.n * a.D, s),
                            "zero dv tail")) != H2O_OK)
            return st;
    }
    hipError_t e;
    if (dims->dtype == H2O_BF16) {
        std::lock_guard<std::mutex> lock(side_stream_lock());
        e = launch_backward_bf16(a, out, dout, drow, dq, dk_new, dv_new, dk_cache, dv_cache, parts,
                                 s, side_stream());
    } else {
        e = launch_backward_f32(a, out, dout, drow, dq, dk_new, dv_new, dk_cache, dv_cache, s);
    }
    timer_end(H2O_KERNEL_BACKWARD, s);
    if ((st = check_hip(e, "backward launch")) != H2O_OK) return st;
    return ok();
}

h2o_status_t h2o_update_scores(const h2o_dims_t* dims, const h2o_cache_t* cache,
                               const float* colsum_cache, void* stream) {
    h2o_status_t st;
    if ((st = validate_dims(dims)) != H2O_OK) return st;
    if ((st = validate_cache(dims, cache)) != H2O_OK) return st;
    if (!colsum_cache) return fail(H2O_ERR_INVALID_ARG, "colsum_cache is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    timer_begin(H2O_KERNEL_UPDATE, s);
    hipError_t e = launch_update_scores(cache->score, colsum_cache,
                                        dims->batch * dims->n_kv_heads, dims->capacity,
                                        cache->n_valid, s);
    timer_end(H2O_KERNEL_UPDATE, s);
    if ((st = check_hip(e, "update launch")) != H2O_OK) return st;
    return ok();
}

h2o_status_t h2o_update_evict_and_insert(const h2o_dims_t* dims, h2o_cache_t* cache,
                                         const float* colsum_cache, int64_t chunk_start,
                                         int32_t chunk_len, int32_t score_mode,
                                         const void* k_new, const void* v_new,
                                         const float* colsum_new, int32_t* freed_slots,
                                         void* stream) {
    if (!colsum_cache) return fail(H2O_ERR_INVALID_ARG, "colsum_cache is NULL");
    if (!colsum_new) return fail(H2O_ERR_INVALID_ARG, "colsum_new is NULL");
    if (score_mode != H2O_SCORE_H2O && score_mode != H2O_SCORE_H2O_NORM)
        return fail(H2O_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
    return evict_and_insert(dims, cache, chunk_start, chunk_len, score_mode, 0, k_new, v_new,
                            colsum_new, freed_slots, stream, true, true, colsum_cache);
}

h2o_status_t h2o_chunk_step(const h2o_dims_t* dims, h2o_cache_t* cache, int64_t chunk_start,
                            int32_t chunk_len, float sm_scale, int32_t score_mode,
                            const void* q, const void* k_new, const void* v_new, void* out,
                            float* lse, float* colsum_cache, float* colsum_new,
                            int32_t* freed_slots, void* workspace, size_t workspace_bytes,
                            void* stream) {
    h2o_status_t st;
    if (score_mode != H2O_SCORE_H2O && score_mode != H2O_SCORE_H2O_NORM)
        return fail(H2O_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
    if (!colsum_cache || !colsum_new)
        return fail(H2O_ERR_INVALID_ARG, "colsum_cache and colsum_new must be non-NULL");
    if (!freed_slots) return fail(H2O_ERR_INVALID_ARG, "freed_slots is NULL");
    if ((st = validate_dims(dims)) != H2O_OK) return st;
    if ((st = validate_cache(dims, cache)) != H2O_OK) return st;
    if ((st = validate_chunk(chunk_start, chunk_len)) != H2O_OK) return st;
    // Everything the eviction would refuse is refused before the attention launches.
    if ((st = check_capacity(dims, cache, chunk_len, score_mode, 0)) != H2O_OK) return st;
    const int n = cache->n_valid, NC = dims->capacity;
    if (uses_decode(dims, chunk_len)) {
        // S = 1: the update, selection and insertion run in the finishing kernel.
        EvictArgs ev;
        ev.kc = cache->k;
        ev.vc = cache->v;
        ev.pos = cache->pos;
        ev.score = cache->score;
        ev.kn = k_new;
        ev.vn = v_new;
        ev.cs_new = colsum_new;
        ev.freed = freed_slots;
        ev.B = dims->batch;
        ev.Hkv = dims->n_kv_heads;
        ev.D = dims->head_dim;
        ev.S = 1;
        ev.NC = NC;
        ev.n = n;
        ev.W = dims->recent_window;
        ev.P = (int)chunk_start;
        ev.elem_bytes = 2;
        ev.score_mode = score_mode;
        ev.sink = 0;
        if ((st = chunk_attn(dims, cache, chunk_start, chunk_len, sm_scale, q, k_new, v_new,
                             nullptr, out, lse, colsum_cache, colsum_new, workspace,
                             workspace_bytes, stream, &ev)) != H2O_OK)
            return st;
        cache->n_valid = n + 1 < NC ? n + 1 : NC;
        return ok();
    }
    if (!k_new || !v_new)
        return fail(H2O_ERR_INVALID_ARG, "k_new, v_new and freed_slots must be non-NULL");
    if ((st = chunk_attn(dims, cache, chunk_start, chunk_len, sm_scale, q, k_new, v_new, nullptr,
                         out, lse, colsum_cache, colsum_new, workspace, workspace_bytes,
                         stream)) != H2O_OK)
        return st;
    return evict_and_insert(dims, cache, chunk_start, chunk_len, score_mode, 0, k_new, v_new,
                            colsum_new, freed_slots, stream, true, true, colsum_cache);
}

h2o_status_t h2o_evict_and_insert(const h2o_dims_t* dims, h2o_cache_t* cache,
                                  int64_t chunk_start, int32_t chunk_len, int32_t score_mode,
                                  const void* k_new, const void* v_new,
                                  const float* colsum_new, int32_t* freed_slots, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (!colsum_new) return fail(H2O_ERR_INVALID_ARG, "colsum_new is NULL");
    if (score_mode != H2O_SCORE_H2O && score_mode != H2O_SCORE_H2O_NORM)
        return fail(H2O_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
    return evict_and_insert(dims, cache, chunk_start, chunk_len, score_mode, 0, k_new, v_new,
                            colsum_new, freed_slots, stream);
}

h2o_status_t h2o_evict_and_insert_lastrec(const h2o_dims_t* dims, h2o_cache_t* cache,
                                          int64_t chunk_start, int32_t chunk_len,
                                          int32_t sink_tokens, const void* k_new,
                                          const void* v_new, int32_t* freed_slots,
                                          void* stream) {
    if (sink_tokens < 0) return fail(H2O_ERR_INVALID_ARG, "sink_tokens %d < 0", sink_tokens);
    return evict_and_insert(dims, cache, chunk_start, chunk_len, kModeLastrec, sink_tokens,
                            k_new, v_new, nullptr, freed_slots, stream);
}

h2o_status_t h2o_select_slots(const h2o_dims_t* dims, const h2o_cache_t* cache,
                              int64_t chunk_start, int32_t chunk_len, int32_t score_mode,
                              int32_t* freed_slots, void* stream) {
    if (score_mode != H2O_SCORE_H2O && score_mode != H2O_SCORE_H2O_NORM)
        return fail(H2O_ERR_INVALID_ARG, "unknown score_mode %d", score_mode);
    if (!cache) return fail(H2O_ERR_INVALID_ARG, "cache is NULL");
    h2o_cache_t c = *cache;                      // n_valid is not advanced
    return evict_and_insert(dims, &c, chunk_start, chunk_len, score_mode, 0, nullptr, nullptr,
                            nullptr, freed_slots, stream, true, false);
}

h2o_status_t h2o_insert(const h2o_dims_t* dims, h2o_cache_t* cache, int64_t chunk_start,
                        int32_t chunk_len, const void* k_new, const void* v_new,
                        const float* colsum_new, const int32_t* freed_slots, void* stream) {
    return evict_and_insert(dims, cache, chunk_start, chunk_len, H2O_SCORE_H2O, 0, k_new, v_new,
                            colsum_new, const_cast<int32_t*>(freed_slots), stream, false, true);
}

h2o_status_t h2o_kernel_timer_start(int32_t kernel, int32_t max_launches) {
    if (kernel < 0 || kernel >= H2O_KERNEL_COUNT)
        return fail(H2O_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
    if (max_launches < 1 || max_launches > (1 << 20))
        return fail(H2O_ERR_INVALID_ARG, "max_launches outside 1..2^20");
    Timer& t = g_timer[kernel];
    destroy_events(t);
    t.ev.resize(2 * (size_t)max_launches);
    for (size_t i = 0; i < t.ev.size(); ++i) {
        hipError_t e = hipEventCreateWithFlags(&t.ev[i], hipEventDisableSystemFence);
        if (e != hipSuccess) {
            t.ev.resize(i);
            destroy_events(t);
            return check_hip(e, "hipEventCreateWithFlags");
        }
    }
    t.max = max_launches;
    t.used = 0;
    t.on = true;
    return ok();
}

h2o_status_t h2o_kernel_timer_stop(int32_t kernel, double* total_ms, int64_t* launches) {
    if (kernel < 0 || kernel >= H2O_KERNEL_COUNT)
        return fail(H2O_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
    if (!total_ms || !launches) return fail(H2O_ERR_INVALID_ARG, "NULL output pointer");
    Timer& t = g_timer[kernel];
    double sum = 0.0;
    h2o_status_t st = H2O_OK;
    for (int i = 0; i < t.used && st == H2O_OK; ++i) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(t.ev[2 * i + 1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
        st = check_hip(e, "kernel timer");
        sum += ms;
    }
    *total_ms = sum;
    *launches = t.used;
    destroy_events(t);
    return st == H2O_OK ? ok() : st;
}

}  // extern "C"
