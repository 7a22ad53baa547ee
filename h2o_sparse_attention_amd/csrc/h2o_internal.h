// Internal declarations shared by the HIP translation units of libh2o.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/h2o.h"

namespace h2o {

// Problem description handed to every kernel (plain values, device pointers).
struct ChunkArgs {
    const void* q;          // [B][Hq][S][D]
    const void* kc;         // [B][Hkv][NC][D]  cache keys
    const void* vc;         // [B][Hkv][NC][D]  cache values
    const void* kn;         // [B][Hkv][S][D]   chunk keys
    const void* vn;         // [B][Hkv][S][D]   chunk values
    const int32_t* pos;     // [B][Hkv][NC]     t(b,g,j)
    void* out;              // [B][Hq][S][D]
    float* lse;             // [B][Hq][S]
    float* cs_cache;        // [B][Hkv][NC]
    float* cs_new;          // [B][Hkv][S]
    int B, Hq, Hkv, G, D, S, NC, n;
    int P;                  // absolute position of the chunk's first query row
    float sm_scale;
    // Buffer form: cache slots the chunk is about to overwrite are not keys.
    const int32_t* freed = nullptr;   // [B][Hkv][S] targets, ascending (victims are < n)
    const uint64_t* excl = nullptr;   // [B][Hkv][ceil(NC/64)] excluded-slot bits per 64 slots
};

// Tiles of 64 slots per (b, kv head) row of the exclusion masks.
__host__ __device__ inline int excl_tiles(int NC) { return (NC + 63) / 64; }

struct EvictArgs {
    void* kc;
    void* vc;
    int32_t* pos;
    float* score;
    const void* kn;
    const void* vn;
    const float* cs_new;
    int32_t* freed;
    int B, Hkv, D, S, NC, n, W, P, elem_bytes, score_mode;
    int sink;               // lastrec: slots at positions < sink are never evicted
    // If set, the selection first adds these summed weights to the scores of the
    // filled slots (and writes the sums back), as h2o_update_scores would.
    const float* cs_upd = nullptr;
};

// Internal ranking mode of the select kernel, beside h2o_score_mode_t.
constexpr int kModeLastrec = 2;     // rank by position t(j), eligible iff t(j) >= sink

// Launchers (return the hipError_t of the launch).
hipError_t launch_attn_bf16(const ChunkArgs& a, hipStream_t s);
// bf16 summed weights: `parts` row ranges per key block (1: written straight to
// the outputs; else partial sums in part_ws, then a reduction launch).
size_t colsum_workspace_bytes(int B, int Hkv, int NC, int S);
int colsum_parts(const ChunkArgs& a, int cus);
hipError_t launch_colsum_bf16(const ChunkArgs& a, int parts, float* part_ws, hipStream_t s);
hipError_t launch_attn_f32(const ChunkArgs& a, hipStream_t s);
hipError_t launch_colsum_f32(const ChunkArgs& a, hipStream_t s);
hipError_t launch_zero_f32(float* p, size_t count_per_row, size_t row_stride, int rows,
                           size_t offset, hipStream_t s);
// Zero count (1..4) whole buffers of n[i] floats in one launch.
hipError_t launch_zero_f32_list(float* const* p, const size_t* n, int count, hipStream_t s);
hipError_t launch_update_scores(float* score, const float* cs, int rows, int NC, int n,
                                hipStream_t s);
hipError_t launch_select(const EvictArgs& a, hipStream_t s);
// excl[bg][t] = bits of the victims (freed slots below n) among slots 64t .. 64t+63.
hipError_t launch_build_excl(const ChunkArgs& a, uint64_t* excl, hipStream_t s);
hipError_t launch_insert(const EvictArgs& a, hipStream_t s);
// k = 1 and S = 1 (decode on a full cache): selection and insertion in one launch.
hipError_t launch_select1_insert(const EvictArgs& a, hipStream_t s);

// Backward of the chunk attention (fp32 gradients).  Workspace: D per row
// (drow, B*Hq*S floats), then at backward_lse2_offset the rows' lse * log2(e).
size_t backward_workspace_bytes(int B, int Hq, int S);
size_t backward_lse2_offset(int B, int Hq, int S);
hipError_t launch_backward_f32(const ChunkArgs& a, const void* out, const void* dout,
                               float* drow, float* dq, float* dk_new, float* dv_new,
                               float* dk_cache, float* dv_cache, hipStream_t s);
// Row parts (1 or 2) of the bf16 dK/dV kernel for `cus` compute units; with 2
// the dK/dV outputs must be zero before the launch.
int backward_dkdv_parts(const ChunkArgs& a, int cus);
// A second stream of a device (default priority) and two events, to run
// independent launches of one call side by side: `fork` is recorded on the
// caller's stream and waited for by `s`; `join` the other way round.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
// side != nullptr: the dQ kernel runs on side->s beside the dK/dV kernel (the
// caller serialises the use of one SideStream).
hipError_t launch_backward_bf16(const ChunkArgs& a, const void* out, const void* dout,
                                float* drow, float* dq, float* dk_new, float* dv_new,
                                float* dk_cache, float* dv_cache, int parts, hipStream_t s,
                                const SideStream* side = nullptr);

// Compute units of the current device (api.hip), read once per device.
hipError_t cu_count(int* cus);

// Decode (S = 1) specialisation.
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int NC);
// ev != NULL (summed weights required): the finishing kernel also updates the
// scores with the summed weights, selects the victim (full cache) and inserts
// the new token -- h2o_update_evict_and_insert for S = 1 inside the same launch.
hipError_t launch_decode(const ChunkArgs& a, void* ws, hipStream_t s,
                         const EvictArgs* ev = nullptr);

// Kernel timers (api.hip): bracket a launch with events when enabled.
void timer_begin(int kernel, hipStream_t s);
void timer_end(int kernel, hipStream_t s);

constexpr int kMaxCapacity = 32768;

// Shared body of h2o_chunk_attn and h2o_buffer_attn (api.hip); freed != NULL is
// the buffer form.
h2o_status_t chunk_attn(const h2o_dims_t* dims, const h2o_cache_t* cache, int64_t chunk_start,
                        int32_t chunk_len, float sm_scale, const void* q, const void* k_new,
                        const void* v_new, const int32_t* freed, void* out, float* lse,
                        float* colsum_cache, float* colsum_new, void* workspace,
                        size_t workspace_bytes, void* stream, const EvictArgs* ev = nullptr);
// Workspace bytes chunk_attn needs for this call (0: none, or invalid dims).
size_t chunk_attn_workspace_need(const h2o_dims_t* dims, int32_t chunk_len, bool summed_weights,
                                 bool buffer_form);
// Records a non-OK status and its message for h2o_last_error (api.hip).
h2o_status_t set_error(h2o_status_t st, const char* msg);

}  // namespace h2o
