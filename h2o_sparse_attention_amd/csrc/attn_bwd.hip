// Backward of the chunk attention with the cache decisions fixed.
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention",
// montaan paper page, "Gradient Computation Strategy", item 1: the policy's
// choices are replayed, not differentiated, so the keys and the mask of a chunk
// are constants and the gradient is that of masked softmax attention.  With
// m = softmax(sm_scale * q.k) over the visible keys, per query row i:
//   D_i = sum_d dO[i,d] O[i,d],   ds_ij = m_ij (dO_i . v_j - D_i),
//   dQ_i = sm_scale sum_j ds_ij k_j,   dK_j = sm_scale sum_i ds_ij q_i,
//   dV_j = sum_i m_ij dO_i   (dK, dV summed over the G query heads of a KV head).
// Visibility is that of the forward pass: every filled slot (minus the slots the
// buffer form overwrites) for every row, chunk key i' for rows i >= i'.
// All gradients are fp32.
#include "h2o_internal.h"
#include "device_common.h"

#include <hip/hip_bf16.h>

#include <climits>
#include <cmath>
#include <type_traits>

namespace h2o {
namespace {

using namespace dev;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(u16 x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ bool excluded(const ChunkArgs& a, int bg, int slot) {
    return a.excl != nullptr &&
           ((a.excl[(size_t)bg * excl_tiles(a.NC) + slot / 64] >> (slot % 64)) & 1);
}

// D_i = dO_i . O_i: 16 lanes per row, 8 elements per lane per step.  With
// lse2 != nullptr also lse2_i = lse_i * log2(e), the row's log-sum-exp in the
// units of the exponentials (read once per row instead of scaled per pair).
template <typename T>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ o,
                                                     const T* __restrict__ dout,
                                                     float* __restrict__ drow,
                                                     const float* __restrict__ lse,
                                                     float* __restrict__ lse2, int rows, int D) {
    const int row = blockIdx.x * 16 + threadIdx.x / 16;
    const int l = threadIdx.x % 16;
    float acc = 0.f;
    if (row < rows) {
        const T* orow = o + (size_t)row * D;
        const T* drw = dout + (size_t)row * D;
        for (int d = l; d < D; d += 16) acc = fmaf(to_f32(orow[d]), to_f32(drw[d]), acc);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (row < rows && l == 0) {
        drow[row] = acc;
        if (lse2 != nullptr) lse2[row] = lse[row] * kLog2e;
    }
}

// ------------------------------------------------------------------ f32 path
// Four lanes per query row (dQ) or per key (dK, dV), a quarter of head_dim each.
constexpr int kThreads = 256;
constexpr int kLanes = 4;
constexpr int kItems = kThreads / kLanes;

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(ChunkArgs a, const float* drow,
                                                              const float* dout, float* dq) {
    constexpr int DL = D / kLanes;
    const int R = a.G * a.S;
    const int nrb = (R + kItems - 1) / kItems;
    const int bg = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    if (bg >= a.B * a.Hkv) return;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int part = threadIdx.x % kLanes;
    const int row = rb * kItems + threadIdx.x / kLanes;
    const bool row_ok = row < R;
    const int i = row_ok ? row / a.G : a.S - 1;
    const int h = g * a.G + (row_ok ? row % a.G : 0);
    const int qpos = a.P + i;
    const size_t qi = (size_t)(b * a.Hq + h) * a.S + i;
    const float* Q = static_cast<const float*>(a.q) + qi * D;
    const float* dO = dout + qi * D;
    const float* Kc = static_cast<const float*>(a.kc) + (size_t)bg * a.NC * D;
    const float* Vc = static_cast<const float*>(a.vc) + (size_t)bg * a.NC * D;
    const float* Kn = static_cast<const float*>(a.kn) + (size_t)bg * a.S * D;
    const float* Vn = static_cast<const float*>(a.vn) + (size_t)bg * a.S * D;
    const int32_t* posg = a.pos + (size_t)bg * a.NC;
    const float lse = a.lse[qi], Di = drow[qi];
    float qv[DL], dov[DL], acc[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) {
        qv[e] = Q[part * DL + e];
        dov[e] = dO[part * DL + e];
        acc[e] = 0.f;
    }
    for (int kk = 0; kk < a.n + a.S; ++kk) {
        const bool cached = kk < a.n;
        const int kp = cached ? posg[kk] : a.P + (kk - a.n);
        const float* kr = cached ? Kc + (size_t)kk * D : Kn + (size_t)(kk - a.n) * D;
        const float* vr = cached ? Vc + (size_t)kk * D : Vn + (size_t)(kk - a.n) * D;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
            s = fmaf(qv[e], kr[part * DL + e], s);
            dp = fmaf(dov[e], vr[part * DL + e], dp);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dp += __shfl_xor(dp, 1);
        dp += __shfl_xor(dp, 2);
        if (!(kp >= 0 && kp <= qpos) || (cached && excluded(a, bg, kk))) continue;
        const float ds = expf(s * a.sm_scale - lse) * (dp - Di);
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[e] = fmaf(ds, kr[part * DL + e], acc[e]);
    }
    if (!row_ok) return;
#pragma unroll
    for (int e = 0; e < DL; ++e) dq[qi * D + part * DL + e] = a.sm_scale * acc[e];
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32_kernel(ChunkArgs a, const float* drow,
                                                                const float* dout, float* dk_new,
                                                                float* dv_new, float* dk_cache,
                                                                float* dv_cache) {
    constexpr int DL = D / kLanes;
    const int nkeys = a.n + a.S;
    const int nkb = (nkeys + kItems - 1) / kItems;
    const int bg = blockIdx.x / nkb, kb = blockIdx.x % nkb;
    if (bg >= a.B * a.Hkv) return;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int part = threadIdx.x % kLanes;
    const int kk = kb * kItems + threadIdx.x / kLanes;
    const bool key_ok = kk < nkeys;
    const int kc = key_ok ? kk : 0;
    const bool cached = kc < a.n;
    const int kp = !key_ok ? INT_MAX : (cached ? a.pos[(size_t)bg * a.NC + kc] : a.P + (kc - a.n));
    const bool ex = key_ok && cached && excluded(a, bg, kc);
    const float* kr = cached ? static_cast<const float*>(a.kc) + ((size_t)bg * a.NC + kc) * D
                             : static_cast<const float*>(a.kn) + ((size_t)bg * a.S + (kc - a.n)) * D;
    const float* vr = cached ? static_cast<const float*>(a.vc) + ((size_t)bg * a.NC + kc) * D
                             : static_cast<const float*>(a.vn) + ((size_t)bg * a.S + (kc - a.n)) * D;
    float kv[DL], vv[DL], dk[DL], dv[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) {
        kv[e] = kr[part * DL + e];
        vv[e] = vr[part * DL + e];
        dk[e] = 0.f;
        dv[e] = 0.f;
    }
    const float* Q = static_cast<const float*>(a.q);
    const int R = a.G * a.S;
    for (int r = 0; r < R; ++r) {
        const int h = g * a.G + r % a.G, i = r / a.G;
        const size_t qi = (size_t)(b * a.Hq + h) * a.S + i;
        const float* qr = Q + qi * D;
        const float* dr = dout + qi * D;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
            s = fmaf(qr[part * DL + e], kv[e], s);
            dp = fmaf(dr[part * DL + e], vv[e], dp);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        dp += __shfl_xor(dp, 1);
        dp += __shfl_xor(dp, 2);
        if (!(kp >= 0 && kp <= a.P + i) || ex) continue;
        const float p = expf(s * a.sm_scale - a.lse[qi]);
        const float ds = p * (dp - drow[qi]);
#pragma unroll
        for (int e = 0; e < DL; ++e) {
            dv[e] = fmaf(p, dr[part * DL + e], dv[e]);
            dk[e] = fmaf(ds, qr[part * DL + e], dk[e]);
        }
    }
    if (!key_ok) return;
    float* dkr = cached ? dk_cache + ((size_t)bg * a.NC + kc) * D : dk_new + ((size_t)bg * a.S + (kc - a.n)) * D;
    float* dvr = cached ? dv_cache + ((size_t)bg * a.NC + kc) * D : dv_new + ((size_t)bg * a.S + (kc - a.n)) * D;
#pragma unroll
    for (int e = 0; e < DL; ++e) {
        dkr[part * DL + e] = a.sm_scale * dk[e];
        dvr[part * DL + e] = dv[e];
    }
}

// ------------------------------------------------------------------ bf16 path
// MFMA layout as in the forward kernels (v_mfma_f32_32x32x16_bf16, lane
// l = 32*hh + lq): A lane holds A[m = lq][k = 8hh..8hh+7], B lane holds
// B[k = 8hh..8hh+7][n = lq], C lane holds C[8(r/4) + 4hh + r%4][lq].  An A
// operand whose rows are read through perm_key puts physical row
// 16(r/8) + 8hh + r%8 in C register r, i.e. eight consecutive rows per lane
// and 16-row step -- the k order of a following product's A or B operand.
// Operands read transposed (column lq, eight consecutive rows) use
// ds_read_b64_tr_b16: a 16-lane group addresses a 4 x 16 block (row 4-group
// + j16/4, columns 4*(j16%4)..+3 of its 16) and each lane receives one column
// of the four rows; two reads, four rows apart, give eight rows.
constexpr int kBwWaves = 4;
constexpr int kBwThreads = 64 * kBwWaves;
constexpr int kBwRowsPerTile = 64;            // dK/dV kernel: query rows per LDS tile
constexpr int kBwKeysPerBlock = 32 * kBwWaves;
constexpr int kBwKeysPerTile = 64;            // dQ kernel: keys per LDS tile
constexpr int kBwRowsPerBlock = 32 * kBwWaves;
constexpr int kWaitVmcnt0 = 0x0F70;           // s_waitcnt vmcnt(0), others at maximum

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Loads that write LDS are this wave's own as far as the compiler knows: each
// wave waits for its own before the barrier that publishes them.
__device__ __forceinline__ void publish() {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
}
__device__ __forceinline__ void lds16(Rsrc r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds4(Rsrc r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld_tr(const unsigned char* p0, const unsigned char* p1) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
}
// Byte offset, in a row-major tile of RB-byte rows whose 16-byte chunks are
// XOR-swizzled by swz_kt, of row r, 16-byte chunk c, 8-byte half h.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c, int h) {
    return r * (2 * D) + 16 * (c ^ swz_kt<D>(r)) + 8 * h;
}
// This lane's two transposed-read offsets for rows 8hh..8hh+7 (plus a multiple
// of 16) and columns 32*dt + lq: XOR 64*dt selects dt, adding 16*RB moves 16 rows.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int& o0, int& o1) {
    const int hh = lane >> 5, g16 = lane >> 4, j16 = lane & 15;
    const int r = 8 * hh + (j16 >> 2);
    const int c = 2 * (g16 & 1) + ((j16 & 3) >> 1);
    o0 = tile_off<D>(r, c, j16 & 1);
    o1 = tile_off<D>(r + 4, c, j16 & 1);
}

// dQ: one workgroup per 128 packed query rows (row r = i*G + head) of a KV
// head; each wave keeps its 32 rows' Q and dO (the B operands) in registers
// and walks the key tiles (K, V staged in LDS): S^T = K Q^T, dP^T = V dO^T,
// dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
template <int D>
__global__ __launch_bounds__(kBwThreads) void bwd_dq_bf16_kernel(ChunkArgs a, const float* drow,
                                                                 const u16* dout, float* dq) {
    constexpr int KS = D / 16, DT = D / 32, RB = 2 * D;
    constexpr int TB = kBwKeysPerTile * RB;            // bytes per K or V tile
    constexpr int LOADS = TB / 1024 / kBwWaves;        // 1 KB loads per wave per tile
    // One array per stage: the compiler tells the loads in flight into one
    // stage from the reads of the other only if they are distinct objects
    // (reading a slice of an array that loads are filling costs a wait for
    // every load in flight).
    __shared__ __attribute__((aligned(1024))) unsigned char sK0[TB], sK1[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sV0[TB], sV1[TB];
    __shared__ __attribute__((aligned(256))) int sPos0[kBwKeysPerTile], sPos1[kBwKeysPerTile];

    const int R = a.G * a.S;
    const int nrb = (R + kBwRowsPerBlock - 1) / kBwRowsPerBlock;
    const int total = nrb * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nrb, rb = t % nrb;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int row = rb * kBwRowsPerBlock + wave * 32 + lq;
    const bool row_ok = row < R;
    const int i = row_ok ? row / a.G : a.S - 1;
    const int h = g * a.G + (row_ok ? row % a.G : 0);
    const size_t qi = (size_t)(b * a.Hq + h) * a.S + i;

    bf16x8 qf[KS], df[KS];
    {
        const u16* Q = static_cast<const u16*>(a.q) + qi * D;
        const u16* dO = dout + qi * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u}, w = {0u, 0u, 0u, 0u};
            if (row_ok) {
                v = ld16(Q + 16 * ks + 8 * hh);
                w = ld16(dO + 16 * ks + 8 * hh);
            }
            qf[ks] = as_bf16x8(v);
            df[ks] = as_bf16x8(w);
        }
    }
    const float c = a.sm_scale * kLog2e;
    // log2-scaled LSE; +inf for rows past the end makes their weights zero
    const float lse2 = row_ok ? a.lse[qi] * kLog2e : INFINITY;
    const float Di = row_ok ? drow[qi] : 0.f;

    const int n = a.n, S = a.S;
    const int cache_tiles = (n + kBwKeysPerTile - 1) / kBwKeysPerTile;
    const int last_row = min(R - 1, rb * kBwRowsPerBlock + kBwRowsPerBlock - 1);
    const int ntiles = cache_tiles + (last_row / a.G) / kBwKeysPerTile + 1;
    const int wave_row0 = min(R - 1, rb * kBwRowsPerBlock + wave * 32);
    const int i_wave_min = wave_row0 / a.G;
    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D;
    const u16* Vc = static_cast<const u16*>(a.vc) + (size_t)bg * a.NC * D;
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
    const u16* Vn = static_cast<const u16*>(a.vn) + (size_t)bg * S * D;
    const uint64_t* exrow = a.excl ? a.excl + (size_t)bg * excl_tiles(a.NC) : nullptr;

    // Tile jt: cache slots 64jt.. (jt < cache_tiles) or chunk keys 64(jt - cache_tiles)..
    auto tile_first = [&](int jt) { return (jt < cache_tiles ? jt : jt - cache_tiles) * kBwKeysPerTile; };
    auto tile_valid = [&](int jt) {
        return min(kBwKeysPerTile, (jt < cache_tiles ? n : S) - tile_first(jt));
    };
    auto issue = [&](auto stage_c, int jt) {
        constexpr int stage = decltype(stage_c)::value;
        unsigned char* dk_ = stage ? sK1 : sK0;
        unsigned char* dv_ = stage ? sV1 : sV0;
        const bool cache = jt < cache_tiles;
        const int first = tile_first(jt), valid = tile_valid(jt);
        const Rsrc rk = make_rsrc((cache ? Kc : Kn) + (size_t)first * D, valid * RB);
        const Rsrc rv = make_rsrc((cache ? Vc : Vn) + (size_t)first * D, valid * RB);
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int off = (it * kBwWaves + wave) * 1024 + 16 * lane;
            const int r = off / RB, cp = (off % RB) / 16;
            const int go = r * RB + 16 * (cp ^ swz_kt<D>(r));
            lds16(rk, dk_ + (it * kBwWaves + wave) * 1024, go);
            lds16(rv, dv_ + (it * kBwWaves + wave) * 1024, go);
        }
        if (cache && wave == 0)
            lds4(make_rsrc(a.pos + (size_t)bg * a.NC + first, valid * 4), stage ? sPos1 : sPos0,
                 4 * lane);
    };
    // A operand rows: physical key perm_key(lq) (+32 per sub-tile), k-step ks.
    const int prow = perm_key(lq);
    const int kb = prow * RB + 16 * (hh ^ swz_kt<D>(prow));
    int t0, t1;
    tr_offsets<D>(lane, t0, t1);

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // Exclusion bits (buffer form) are loaded one tile ahead, so the wait that
    // ends each iteration covers them: a wait for them in the iteration that
    // uses them would also wait for the tile loads issued before (vmcnt counts
    // in order).
    auto tile_ex = [&](int jt) {
        return (jt < cache_tiles && exrow != nullptr) ? exrow[jt] : 0ull;
    };
    uint64_t ex_next = tile_ex(0);
    issue(S0{}, 0);
    publish();
    // Tile jt sits in stage jt & 1; the loop runs two tiles per trip so that
    // each body names its stages at compile time.
    auto body = [&](auto stage_c, int jt) {
        constexpr int stage = decltype(stage_c)::value;
        // The dQ accumulators only meet MFMAs inside the loop: keep them in AGPRs
        // across the two bodies (left to itself the compiler moved all 64 values
        // between VGPRs and AGPRs once per trip).
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+a"(o[dt]));
        if (jt + 1 < ntiles) issue(std::integral_constant<int, stage ^ 1>{}, jt + 1);
        const uint64_t ex = ex_next;
        ex_next = tile_ex(jt + 1);
        const unsigned char* tk = stage ? sK1 : sK0;
        const unsigned char* tv = stage ? sV1 : sV0;
        const int* tpos = stage ? sPos1 : sPos0;
        const bool cache = jt < cache_tiles;
        const int first = tile_first(jt), valid = tile_valid(jt);
        // keys k of the tile with k > lim are not visible to this lane's row
        const int lim = cache ? valid - 1 : min(valid - 1, i - first);
        // Cache keys whose position lies outside [0, P) are visible iff
        // 0 <= t(j) <= P + i (none in a cache built by this library's insertions).
        const bool irr = cache && __ballot(lane < valid && (tpos[lane] < 0 ||
                                                           tpos[lane] >= a.P)) != 0;
        const bool all_vis = ex == 0 && !irr && valid == kBwKeysPerTile &&
                             (cache || first + kBwKeysPerTile - 1 <= i_wave_min);
        const uint32_t lb = __builtin_amdgcn_perm((uint32_t)(ex >> 32), (uint32_t)ex,
                                                  hh ? 0x07050301u : 0x06040200u);
        // The two 32-key sub-tiles are pipelined inside the wave (one wave per SIMD):
        // sub-tile 0's dS runs under sub-tile 1's S and dP MFMAs, sub-tile 1's under
        // sub-tile 0's dQ MFMAs.  Invisible keys get score -inf (weight 0) first.
        // K and V rows of k-step ks of a sub-tile (the A operands of S^T and
        // dP^T).  They are read two k-steps ahead of their MFMAs through a ring
        // of three: all KS at once held 64 more registers per sub-tile, and the
        // pressure moved the S and dP tiles through AGPRs (copies per value).
        auto kv_at = [&](int sub, int ks, bf16x8& ka, bf16x8& va) {
            const int ob = (kb ^ (32 * ks)) + sub * 32 * RB;
            ka = as_bf16x8(ld16(tk + ob));
            va = as_bf16x8(ld16(tv + ob));
        };
        auto ktr_of = [&](int sub, int dt, int s2) {
            const int rows = (sub * 32 + 16 * s2) * RB;
            return ld_tr(tk + ((t0 + rows) ^ (64 * dt)), tk + ((t1 + rows) ^ (64 * dt)));
        };
        // this lane's keys 32*sub + 16*(r/8) + 8*hh + r%8 and its row
        auto mask_sub = [&](int sub, f32x16& stv) {
            if (all_vis) return;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = 32 * sub + 16 * (r >> 3) + 8 * hh + (r & 7);
                if (kk > lim || ((lb >> (16 * sub + r)) & 1u)) stv[r] = -INFINITY;
            }
            if (irr) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tp = tpos[32 * sub + 16 * (r >> 3) + 8 * hh + (r & 7)];
                    if (tp < 0 || tp > a.P + i) stv[r] = -INFINITY;
                }
            }
        };
        auto pack = [&](const float (&v)[16], bf16x8 (&b)[2]) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                b[s2] = as_bf16x8(u32x4{pack2(v[8 * s2 + 0], v[8 * s2 + 1]), pack2(v[8 * s2 + 2], v[8 * s2 + 3]),
                                        pack2(v[8 * s2 + 4], v[8 * s2 + 5]), pack2(v[8 * s2 + 6], v[8 * s2 + 7])});
        };
        // A: sub-tile 0's S and dP.
        bf16x8 kw[3], vw[3];
        kv_at(0, 0, kw[0], vw[0]);
        kv_at(0, 1, kw[1], vw[1]);
        f32x16 st0 = f32x16{}, dp0 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) kv_at(0, ks + 2, kw[(ks + 2) % 3], vw[(ks + 2) % 3]);
            st0 = mfma32(kw[ks % 3], qf[ks], st0);
            dp0 = mfma32(vw[ks % 3], df[ks], dp0);
            __builtin_amdgcn_sched_barrier(0);
        }
        kv_at(1, 0, kw[0], vw[0]);
        kv_at(1, 1, kw[1], vw[1]);
        __builtin_amdgcn_sched_barrier(0);
        mask_sub(0, st0);
        // B: sub-tile 1's S and dP with sub-tile 0's dS.
        float dsv[16];
        f32x16 st1 = f32x16{}, dp1 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) kv_at(1, ks + 2, kw[(ks + 2) % 3], vw[(ks + 2) % 3]);
            st1 = mfma32(kw[ks % 3], qf[ks], st1);
            dp1 = mfma32(vw[ks % 3], df[ks], dp1);
#pragma unroll
            for (int r = 16 * ks / KS; r < 16 * (ks + 1) / KS; ++r)
                dsv[r] = fast_exp2(fmaf(st0[r], c, -lse2)) * (dp0[r] - Di);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 dsb0[2];
        pack(dsv, dsb0);
        __builtin_amdgcn_sched_barrier(0);
        mask_sub(1, st1);
        // The K^T operands of the dQ product (K^T columns d = 32*dt + lq, keys
        // 16*s2 + 8*hh.. of a sub-tile), step x = 8*sub + 2*dt + s2 of the
        // sixteen, go through a ring of three, two steps ahead.
        bf16x8 ktw[3];
        auto ktr_at = [&](int x) {
            return ktr_of(x / (2 * DT), (x % (2 * DT)) >> 1, x & 1);
        };
        ktw[0] = ktr_at(0);
        ktw[1] = ktr_at(1);
        __builtin_amdgcn_sched_barrier(0);
        // C: sub-tile 0's dQ^T += K^T dS^T with sub-tile 1's dS.
#pragma unroll
        for (int x = 0; x < 2 * DT; ++x) {
            const int dt = x >> 1, s2 = x & 1;
            ktw[(x + 2) % 3] = ktr_at(x + 2);
            o[dt] = mfma32(ktw[x % 3], dsb0[s2], o[dt]);
#pragma unroll
            for (int r = 16 * x / (2 * DT); r < 16 * (x + 1) / (2 * DT); ++r)
                dsv[r] = fast_exp2(fmaf(st1[r], c, -lse2)) * (dp1[r] - Di);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 dsb1[2];
        pack(dsv, dsb1);
        // E: sub-tile 1's dQ.
#pragma unroll
        for (int x = 2 * DT; x < 4 * DT; ++x) {
            if (x + 2 < 4 * DT) ktw[(x + 2) % 3] = ktr_at(x + 2);
            o[(x - 2 * DT) >> 1] = mfma32(ktw[x % 3], dsb1[x & 1], o[(x - 2 * DT) >> 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        publish();
    };
    for (int jt = 0; jt < ntiles; jt += 2) {
        body(S0{}, jt);
        if (jt + 1 < ntiles) body(S1{}, jt + 1);
    }
    if (!row_ok) return;
    // o[dt][r] = dQ^T[d = 32dt + 8(r/4) + 4hh + r%4][row lq]
    float* out = dq + qi * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float4 w;
            w.x = a.sm_scale * o[dt][4 * r4 + 0];
            w.y = a.sm_scale * o[dt][4 * r4 + 1];
            w.z = a.sm_scale * o[dt][4 * r4 + 2];
            w.w = a.sm_scale * o[dt][4 * r4 + 3];
            *reinterpret_cast<float4*>(out + 32 * dt + 8 * r4 + 4 * hh) = w;
        }
}

// dK, dV: one workgroup per 128 keys of a KV head (cache slots or chunk keys)
// and per part of the query rows; each wave keeps its 32 keys' K and V (the B
// operands) in registers and walks its part's packed query rows in 64-row
// tiles (Q, dO, LSE, D staged in LDS):
// S = Q K^T, dP = dO V^T (rows through perm_key), P, dS = P (dP - D),
// dV += P^T dO, dK += dS^T Q.
// With parts == 2 the two row halves of a key block add their sums into
// gradient buffers zeroed beforehand: two additions to zero give the same bits
// in either order, so the result stays deterministic.  (At one wave per SIMD,
// 576 whole blocks at chunk 1k / 8192 slots take three rounds of 256 CUs for
// 2.25 rounds of work; halves take 2.5.)
template <int D>
__global__ __launch_bounds__(kBwThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_bf16_kernel(ChunkArgs a, const float* drow, const float* lse2, const u16* dout,
                          uint32_t g_magic, int parts, float* dk_new, float* dv_new,
                          float* dk_cache, float* dv_cache) {
    constexpr int KS = D / 16, DT = D / 32, RB = 2 * D;
    constexpr int TB = kBwRowsPerTile * RB;
    constexpr int LOADS = TB / 1024 / kBwWaves;
    constexpr int ROWS_PER_LOAD = 4096 / RB;
    // One array per stage (as in the dQ kernel).
    __shared__ __attribute__((aligned(1024))) unsigned char sQ0[TB], sQ1[TB];
    __shared__ __attribute__((aligned(1024))) unsigned char sD0[TB], sD1[TB];
    __shared__ __attribute__((aligned(16))) float sL0[kBwRowsPerTile], sL1[kBwRowsPerTile];
    __shared__ __attribute__((aligned(16))) float sR0[kBwRowsPerTile], sR1[kBwRowsPerTile];

    const int n = a.n, S = a.S, G = a.G;
    const int cache_blocks = (n + kBwKeysPerBlock - 1) / kBwKeysPerBlock;
    const int nkb = cache_blocks + (S + kBwKeysPerBlock - 1) / kBwKeysPerBlock;
    const int total = nkb * a.B * a.Hkv * parts;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int kbk = t % nkb, part = (t / nkb) % parts, bg = t / nkb / parts;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const bool is_cache = kbk < cache_blocks;
    const int block_first = (is_cache ? kbk : kbk - cache_blocks) * kBwKeysPerBlock;
    const int limit = is_cache ? n : S;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int first = block_first + wave * 32;
    const int key = first + lq;                          // this lane's key (B operand column)

    bf16x8 kf[KS], vf[KS];
    {
        const u16* Ks = is_cache ? static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D
                                 : static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
        const u16* Vs = is_cache ? static_cast<const u16*>(a.vc) + (size_t)bg * a.NC * D
                                 : static_cast<const u16*>(a.vn) + (size_t)bg * S * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u}, w = {0u, 0u, 0u, 0u};
            if (key < limit) {
                v = ld16(Ks + (size_t)key * D + 16 * ks + 8 * hh);
                w = ld16(Vs + (size_t)key * D + 16 * ks + 8 * hh);
            }
            kf[ks] = as_bf16x8(v);
            vf[ks] = as_bf16x8(w);
        }
    }

    // This lane's cache key position; irr: some key of the wave lies outside
    // [0, P) and is visible iff 0 <= t(j) <= P + i (none in a cache built by this
    // library's insertions).
    const int tpos = (is_cache && key < limit) ? a.pos[(size_t)bg * a.NC + key] : 0;
    const bool irr = __ballot(tpos < 0 || tpos >= a.P) != 0 && is_cache;

    const int R = G * S;
    const int ntile = (R + kBwRowsPerTile - 1) / kBwRowsPerTile;
    const int tile0 = is_cache ? 0 : (block_first * G) / kBwRowsPerTile;
    // This workgroup's row tiles [t_lo, t_hi).
    const int per_part = (ntile - tile0 + parts - 1) / parts;
    const int t_lo = tile0 + part * per_part, t_hi = min(ntile, t_lo + per_part);
    if (t_lo >= t_hi) return;                 // nothing to add (parts > 1 only)
    const u16* Qg = static_cast<const u16*>(a.q) + (size_t)(b * a.Hq + g * G) * S * D;
    const u16* Dg = dout + (size_t)(b * a.Hq + g * G) * S * D;
    const float* Lg = lse2 + (size_t)(b * a.Hq + g * G) * S;
    const float* Rg = drow + (size_t)(b * a.Hq + g * G) * S;
    const int q_bytes = G * S * D * 2;
    auto row_split = [&](int r, int& hl, int& ipos) {
        ipos = G == 1 ? r : (int)__umulhi((uint32_t)r, g_magic);
        hl = r - ipos * G;
    };
    const int rl_base = (wave * 1024 + 16 * lane) / RB;
    const int cp = (16 * lane % RB) / 16;
    // When a tile holds whole positions (G divides 64) and the chunk whole tiles,
    // row rl of tile rt is head rl % G at position rt*64/G + rl/G: each load's
    // offset is a fixed per-lane value past a base that moves by 64/G positions a
    // tile, and no row lies past the end.  Otherwise each row is split per load.
    const int ppt = kBwRowsPerTile / G;
    const bool even = kBwRowsPerTile % G == 0 && S % ppt == 0;
    int qoff[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
        const int rl = rl_base + it * ROWS_PER_LOAD;
        qoff[it] = (((rl % G) * S + rl / G) * D) * 2 + 16 * (cp ^ swz_kt<D>(rl));
    }
    const int loff = ((lane % G) * S + lane / G) * 4;
    auto issue = [&](auto stage_c, int rt) {
        constexpr int stage = decltype(stage_c)::value;
        unsigned char* dq_ = stage ? sQ1 : sQ0;
        unsigned char* dd_ = stage ? sD1 : sD0;
        if (even) {
            const size_t p0 = (size_t)rt * ppt;
            const int rem = q_bytes - (int)p0 * D * 2;
            const Rsrc rq = make_rsrc(Qg + p0 * D, rem), rd = make_rsrc(Dg + p0 * D, rem);
#pragma unroll
            for (int it = 0; it < LOADS; ++it) {
                lds16(rq, dq_ + (it * kBwWaves + wave) * 1024, qoff[it]);
                lds16(rd, dd_ + (it * kBwWaves + wave) * 1024, qoff[it]);
            }
            if (wave == 0) {
                const int lrem = (G * S - (int)p0) * 4;
                lds4(make_rsrc(Lg + p0, lrem), stage ? sL1 : sL0, loff);
                lds4(make_rsrc(Rg + p0, lrem), stage ? sR1 : sR0, loff);
            }
            return;
        }
        const Rsrc rq = make_rsrc(Qg, q_bytes), rd = make_rsrc(Dg, q_bytes);
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
            const int rl = rl_base + it * ROWS_PER_LOAD;
            const int r = rt * kBwRowsPerTile + rl;
            int hl = 0, ipos = 0;
            row_split(min(r, R - 1), hl, ipos);
            const int off = r < R ? ((hl * S + ipos) * D) * 2 + 16 * (cp ^ swz_kt<D>(rl)) : q_bytes;
            lds16(rq, dq_ + (it * kBwWaves + wave) * 1024, off);
            lds16(rd, dd_ + (it * kBwWaves + wave) * 1024, off);
        }
        if (wave == 0) {
            const int r = rt * kBwRowsPerTile + lane;
            int hl = 0, ipos = 0;
            row_split(min(r, R - 1), hl, ipos);
            const int off = r < R ? (hl * S + ipos) * 4 : G * S * 4;
            lds4(make_rsrc(Lg, G * S * 4), stage ? sL1 : sL0, off);
            lds4(make_rsrc(Rg, G * S * 4), stage ? sR1 : sR0, off);
        }
    };
    const float c = a.sm_scale * kLog2e;
    const int prow = perm_key(lq);
    const int qb = prow * RB + 16 * (hh ^ swz_kt<D>(prow));
    int t0, t1;
    tr_offsets<D>(lane, t0, t1);

    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dk[dt] = f32x16{};
        dv[dt] = f32x16{};
    }
    const int kmax = min(first + 31, limit - 1);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    issue(S0{}, t_lo);
    publish();
    // Tile rt sits in stage (rt - t_lo) & 1; the loop runs two tiles per trip
    // so that each body names its stages at compile time.
    auto body = [&](auto stage_c, int rt) {
        constexpr int stage = decltype(stage_c)::value;
        if (rt + 1 < t_hi) issue(std::integral_constant<int, stage ^ 1>{}, rt + 1);
        const unsigned char* tq = stage ? sQ1 : sQ0;
        const unsigned char* td = stage ? sD1 : sD0;
        const float* tl = stage ? sL1 : sL0;
        const float* tr = stage ? sR1 : sR0;
        // The two 32-row sub-tiles are pipelined inside the wave (one wave per
        // SIMD): sub-tile 0's exponentials and dS run under sub-tile 1's S and dP
        // MFMAs, sub-tile 1's under sub-tile 0's dV and dK MFMAs.
        // Q and dO rows of k-step ks of a sub-tile (the A operands of S and dP),
        // read two k-steps ahead of their MFMAs through a ring of three (as in
        // the dQ kernel).
        auto qd_at = [&](int sub, int ks, bf16x8& qa, bf16x8& da) {
            const int ob = (qb ^ (32 * ks)) + sub * 32 * RB;
            qa = as_bf16x8(ld16(tq + ob));
            da = as_bf16x8(ld16(td + ob));
        };
        // log2-scaled LSE and D of the lane's rows 32*sub + 16*(r/8) + 8*hh + r%8.
        // Rows past the last read zeros (out-of-range loads), and so do their Q
        // and dO: the weight exp2(0) = 1 multiplies dO = 0 and dS = 1 * (0 - 0)
        // multiplies Q = 0, so those rows add nothing.
        float l2v[16], drv[16];
        auto read_ld = [&](int sub) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = 32 * sub + 16 * (r >> 3) + 8 * hh + (r & 7);
                l2v[r] = tl[rl];
                drv[r] = tr[rl];
            }
        };
        // Chunk keys near the diagonal: -inf for this lane's key at rows before it;
        // cache keys outside [0, P): -inf where t(j) < 0 or t(j) > P + i.
        auto mask_sub = [&](int sub, f32x16& stv) {
            const int r0 = rt * kBwRowsPerTile + 32 * sub;
            const int i0 = G == 1 ? min(r0, R - 1) : (int)__umulhi((uint32_t)min(r0, R - 1), g_magic);
            if (is_cache ? !irr : kmax <= i0) return;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = min(r0 + 16 * (r >> 3) + 8 * hh + (r & 7), R - 1);
                const int ipos = G == 1 ? rr : (int)__umulhi((uint32_t)rr, g_magic);
                if (is_cache ? (tpos < 0 || tpos > a.P + ipos) : key > ipos) stv[r] = -INFINITY;
            }
        };
        // P and dS = P (dP - D) of value r of a sub-tile.
        auto pds = [&](const f32x16& stv, const f32x16& dpv, int r, float& pr, float& dsr) {
            pr = fast_exp2(fmaf(stv[r], c, -l2v[r]));
            dsr = pr * (dpv[r] - drv[r]);
        };
        auto pack = [&](const float (&v)[16], bf16x8 (&b)[2]) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                b[s2] = as_bf16x8(u32x4{pack2(v[8 * s2 + 0], v[8 * s2 + 1]), pack2(v[8 * s2 + 2], v[8 * s2 + 3]),
                                        pack2(v[8 * s2 + 4], v[8 * s2 + 5]), pack2(v[8 * s2 + 6], v[8 * s2 + 7])});
        };

        // A: sub-tile 0's S and dP.
        bf16x8 qw[3], dw[3];
        qd_at(0, 0, qw[0], dw[0]);
        qd_at(0, 1, qw[1], dw[1]);
        f32x16 st0 = f32x16{}, dp0 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) qd_at(0, ks + 2, qw[(ks + 2) % 3], dw[(ks + 2) % 3]);
            st0 = mfma32(qw[ks % 3], kf[ks], st0);
            dp0 = mfma32(dw[ks % 3], vf[ks], dp0);
            __builtin_amdgcn_sched_barrier(0);
        }
        qd_at(1, 0, qw[0], dw[0]);
        qd_at(1, 1, qw[1], dw[1]);
        read_ld(0);
        __builtin_amdgcn_sched_barrier(0);
        mask_sub(0, st0);
        // B: sub-tile 1's S and dP with sub-tile 0's P and dS.
        float pv[16], dsv[16];
        f32x16 st1 = f32x16{}, dp1 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) qd_at(1, ks + 2, qw[(ks + 2) % 3], dw[(ks + 2) % 3]);
            st1 = mfma32(qw[ks % 3], kf[ks], st1);
            dp1 = mfma32(dw[ks % 3], vf[ks], dp1);
#pragma unroll
            for (int r = 16 * ks / KS; r < 16 * (ks + 1) / KS; ++r) pds(st0, dp0, r, pv[r], dsv[r]);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pb0[2], db0[2];
        pack(pv, pb0);
        pack(dsv, db0);
        read_ld(1);
        // The transposed operands of the dV and dK products (dO / Q columns
        // 32*dt + lq, rows 16*s2 + 8*hh.. of a sub-tile), step x = 8*sub + 2*dt +
        // s2 of the sixteen, go through a ring of three, two steps ahead.
        bf16x8 dtw[3], qtw[3];
        auto tr_at = [&](int x, bf16x8& dtv, bf16x8& qtv) {
            const int sub = x / (2 * DT), dt = (x % (2 * DT)) >> 1, s2 = x & 1;
            const int rows = (sub * 32 + 16 * s2) * RB;
            const int o0 = (t0 + rows) ^ (64 * dt), o1 = (t1 + rows) ^ (64 * dt);
            dtv = ld_tr(td + o0, td + o1);
            qtv = ld_tr(tq + o0, tq + o1);
        };
        tr_at(0, dtw[0], qtw[0]);
        tr_at(1, dtw[1], qtw[1]);
        __builtin_amdgcn_sched_barrier(0);
        mask_sub(1, st1);
        // C: sub-tile 0's dV and dK with sub-tile 1's P and dS.
#pragma unroll
        for (int x = 0; x < 2 * DT; ++x) {
            const int dt = x >> 1, s2 = x & 1;
            tr_at(x + 2, dtw[(x + 2) % 3], qtw[(x + 2) % 3]);
            dv[dt] = mfma32(pb0[s2], dtw[x % 3], dv[dt]);
            dk[dt] = mfma32(db0[s2], qtw[x % 3], dk[dt]);
#pragma unroll
            for (int r = 16 * x / (2 * DT); r < 16 * (x + 1) / (2 * DT); ++r)
                pds(st1, dp1, r, pv[r], dsv[r]);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pb1[2], db1[2];
        pack(pv, pb1);
        pack(dsv, db1);
        // E: sub-tile 1's dV and dK.
#pragma unroll
        for (int x = 2 * DT; x < 4 * DT; ++x) {
            const int dt = (x - 2 * DT) >> 1, s2 = x & 1;
            if (x + 2 < 4 * DT) tr_at(x + 2, dtw[(x + 2) % 3], qtw[(x + 2) % 3]);
            dv[dt] = mfma32(pb1[s2], dtw[x % 3], dv[dt]);
            dk[dt] = mfma32(db1[s2], qtw[x % 3], dk[dt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        publish();
    };
    for (int rt = t_lo; rt < t_hi; rt += 2) {
        body(S0{}, rt);
        if (rt + 1 < t_hi) body(S1{}, rt + 1);
    }
    // dk[dt][r] = dK[key first + 8(r/4) + 4hh + r%4][d = 32dt + lq]
    float* dkb = is_cache ? dk_cache + (size_t)bg * a.NC * D : dk_new + (size_t)bg * S * D;
    float* dvb = is_cache ? dv_cache + (size_t)bg * a.NC * D : dv_new + (size_t)bg * S * D;
    // The wave's 32 keys lie in one 64-slot word of the exclusion bits.
    const uint64_t exw = (is_cache && a.excl != nullptr)
                             ? a.excl[(size_t)bg * excl_tiles(a.NC) + first / 64] : 0ull;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kk = first + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (kk >= limit) continue;
        const bool ex = (exw >> (kk % 64)) & 1;
        if (parts == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                dkb[(size_t)kk * D + 32 * dt + lq] = ex ? 0.f : a.sm_scale * dk[dt][r];
                dvb[(size_t)kk * D + 32 * dt + lq] = ex ? 0.f : dv[dt][r];
            }
        } else if (!ex) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                atomicAdd(&dkb[(size_t)kk * D + 32 * dt + lq], a.sm_scale * dk[dt][r]);
                atomicAdd(&dvb[(size_t)kk * D + 32 * dt + lq], dv[dt][r]);
            }
        }
    }
}

}  // namespace

size_t backward_workspace_bytes(int B, int Hq, int S) {
    return 2 * backward_lse2_offset(B, Hq, S);
}

size_t backward_lse2_offset(int B, int Hq, int S) {
    return ((size_t)B * Hq * S * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_backward_f32(const ChunkArgs& a, const void* out, const void* dout,
                               float* drow, float* dq, float* dk_new, float* dv_new,
                               float* dk_cache, float* dv_cache, hipStream_t s) {
    const int rows = a.B * a.Hq * a.S;
    hipLaunchKernelGGL(rowdot_kernel<float>, dim3((rows + 15) / 16), dim3(256), 0, s,
                       static_cast<const float*>(out), static_cast<const float*>(dout), drow,
                       static_cast<const float*>(nullptr), static_cast<float*>(nullptr), rows,
                       a.D);
    const float* dO = static_cast<const float*>(dout);
    const int nrb = (a.G * a.S + kItems - 1) / kItems;
    const int nkb = (a.n + a.S + kItems - 1) / kItems;
    if (a.D == 128) {
        hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, dim3(nrb * a.B * a.Hkv), dim3(kThreads), 0, s, a,
                           drow, dO, dq);
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, dim3(nkb * a.B * a.Hkv), dim3(kThreads), 0, s,
                           a, drow, dO, dk_new, dv_new, dk_cache, dv_cache);
    } else {
        hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, dim3(nrb * a.B * a.Hkv), dim3(kThreads), 0, s, a,
                           drow, dO, dq);
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, dim3(nkb * a.B * a.Hkv), dim3(kThreads), 0, s,
                           a, drow, dO, dk_new, dv_new, dk_cache, dv_cache);
    }
    return hipGetLastError();
}

int backward_dkdv_parts(const ChunkArgs& a, int cus) {
    // Whole key blocks or row halves, whichever needs fewer rounds of one
    // workgroup per CU, counted in whole-block units (ties: whole blocks).
    const long long blocks = (long long)((a.n + kBwKeysPerBlock - 1) / kBwKeysPerBlock +
                                         (a.S + kBwKeysPerBlock - 1) / kBwKeysPerBlock) *
                             a.B * a.Hkv;
    const double r1 = (double)((blocks + cus - 1) / cus);
    const double r2 = (double)((2 * blocks + cus - 1) / cus) / 2.0;
    return r2 < r1 - 1e-9 ? 2 : 1;
}

hipError_t launch_backward_bf16(const ChunkArgs& a, const void* out, const void* dout,
                                float* drow, float* dq, float* dk_new, float* dv_new,
                                float* dk_cache, float* dv_cache, int parts, hipStream_t s,
                                const SideStream* side) {
    const int rows = a.B * a.Hq * a.S;
    // lse * log2(e) per row, for the dK/dV kernel, after D in the workspace
    float* lse2 = drow + backward_lse2_offset(a.B, a.Hq, a.S) / sizeof(float);
    hipLaunchKernelGGL(rowdot_kernel<u16>, dim3((rows + 15) / 16), dim3(256), 0, s,
                       static_cast<const u16*>(out), static_cast<const u16*>(dout), drow,
                       static_cast<const float*>(a.lse), lse2, rows, a.D);
    const u16* dO = static_cast<const u16*>(dout);
    const int nrb = (a.G * a.S + kBwRowsPerBlock - 1) / kBwRowsPerBlock;
    const int nkb = (a.n + kBwKeysPerBlock - 1) / kBwKeysPerBlock +
                    (a.S + kBwKeysPerBlock - 1) / kBwKeysPerBlock;
    const uint32_t magic = a.G > 1 ? (uint32_t)((0x100000000ull + a.G - 1) / a.G) : 0u;
    const dim3 gq(xcd_grid(nrb * a.B * a.Hkv)), gk(xcd_grid(nkb * a.B * a.Hkv * parts));
    // The two kernels write disjoint outputs and each holds one workgroup per
    // CU.  Side by side, the dQ kernel's long workgroups (one round) fill the
    // CUs that the dK/dV kernel's last, partial round leaves idle.  dK/dV is
    // enqueued first, on the caller's stream.
    hipStream_t sq = s;
    if (side != nullptr) {
        hipError_t e = hipEventRecord(side->fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
        if (e != hipSuccess) return e;
        sq = side->s;
    }
    if (a.D == 128)
        hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<128>, gk, dim3(kBwThreads), 0, s, a, drow, lse2,
                           dO, magic, parts, dk_new, dv_new, dk_cache, dv_cache);
    else
        hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<64>, gk, dim3(kBwThreads), 0, s, a, drow, lse2,
                           dO, magic, parts, dk_new, dv_new, dk_cache, dv_cache);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.D == 128)
        hipLaunchKernelGGL(bwd_dq_bf16_kernel<128>, gq, dim3(kBwThreads), 0, sq, a, drow, dO, dq);
    else
        hipLaunchKernelGGL(bwd_dq_bf16_kernel<64>, gq, dim3(kBwThreads), 0, sq, a, drow, dO, dq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (side != nullptr) {
        e = hipEventRecord(side->join, side->s);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
    }
    return e;
}

}  // namespace h2o
