// h2o_chunk_attn_noalloc: h2o_chunk_attn with its workspace taken from a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in this file's code object; every GPU the library runs on
// holds its own copy until the process ends.  Its address on a device comes
// from hipGetSymbolAddress, looked up once per device with that device current
// and kept; the array's name itself is only a host-side stand-in and is never
// handed to a kernel or a copy.
#include "h2o_internal.h"

#include <cstdio>
#include <mutex>

namespace h2o {
namespace {

// Largest workspace the variant serves: the decode workload (16 sequences, 8 KV
// heads, 4 query heads each, 16384 slots) needs 34.6 MB of logits and split
// partials; a bf16 chunk's split summed weights need 4 * B * Hkv * (N_C + S)
// floats (1.2 MB at chunk 1k / 8192 slots).
constexpr size_t kScratchBytes = size_t(40) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device.
h2o_status_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        char msg[160];
        snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
        return set_error(H2O_ERR_HIP, msg);
    }
    if (dev < 0 || dev >= kMaxDevices) return set_error(H2O_ERR_UNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            char msg[160];
            snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return set_error(H2O_ERR_HIP, msg);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return H2O_OK;
}

}  // namespace
}  // namespace h2o

using namespace h2o;

extern "C" {

size_t h2o_noalloc_scratch_bytes(void) { return kScratchBytes; }

h2o_status_t h2o_chunk_attn_noalloc(const h2o_dims_t* dims, const h2o_cache_t* cache,
                                    int64_t chunk_start, int32_t chunk_len, float sm_scale,
                                    const void* q, const void* k_new, const void* v_new,
                                    void* out, float* lse, float* colsum_cache,
                                    float* colsum_new, void* stream) {
    const size_t need = chunk_attn_workspace_need(dims, chunk_len, colsum_cache != nullptr,
                                                  false);
    if (need > kScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof(msg),
                 "this call needs %zu bytes of workspace; the static scratch of "
                 "h2o_chunk_attn_noalloc holds %zu (use h2o_chunk_attn with a workspace)",
                 need, kScratchBytes);
        return set_error(H2O_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if (need > 0) {
        const h2o_status_t st = scratch_on_current_device(&ws);
        if (st != H2O_OK) return st;
    }
    return chunk_attn(dims, cache, chunk_start, chunk_len, sm_scale, q, k_new, v_new, nullptr,
                      out, lse, colsum_cache, colsum_new, ws, need > 0 ? kScratchBytes : 0,
                      stream);
}

}  // extern "C"
