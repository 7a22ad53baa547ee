// Score accumulation, heavy-hitter selection and chunk insertion.
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention",
// montaan paper page, "Improvements to Heavy-Hitter Oracle (H2O)", item 2: the
// H2O score is the running sum of the summed attention weights, optionally
// normalised by age, and new content overwrites the slots of smallest score.
#include "h2o_internal.h"
#include "device_common.h"

#include <climits>

namespace h2o {
namespace {

// ------------------------------------------------------------------ update
// One (b, kv head) row per blockIdx.y; float4 where the row allows it.
__global__ __launch_bounds__(256) void update_scores_kernel(float* __restrict__ score,
                                                            const float* __restrict__ cs,
                                                            int NC, int n, bool vec) {
    const size_t base = (size_t)blockIdx.y * NC;
    if (vec) {
        const int n4 = n / 4;
        float4* s4 = reinterpret_cast<float4*>(score + base);
        const float4* c4 = reinterpret_cast<const float4*>(cs + base);
        for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) {
            float4 v = s4[i];
            const float4 w = c4[i];
            v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
            s4[i] = v;
        }
        for (int j = n4 * 4 + blockIdx.x * blockDim.x + threadIdx.x; j < n;
             j += gridDim.x * blockDim.x)
            score[base + j] += cs[base + j];
    } else {
        for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x)
            score[base + j] += cs[base + j];
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int per_row,
                                                   size_t stride, size_t offset) {
    float* row = p + (size_t)blockIdx.y * stride + offset;
    const int step = gridDim.x * blockDim.x;
    if (((reinterpret_cast<uintptr_t>(row) & 15u) | (uintptr_t)(per_row & 3)) == 0) {
        // 16-byte stores when the row start is 16-byte aligned and the length a
        // multiple of 4 floats
        float4* row4 = reinterpret_cast<float4*>(row);
        const float4 z = {0.f, 0.f, 0.f, 0.f};
        for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < per_row / 4; j += step)
            row4[j] = z;
        return;
    }
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < per_row; j += step) row[j] = 0.f;
}

// Up to four whole buffers in one launch (blockIdx.y picks the buffer).
struct ZeroList {
    float* p[4];
    size_t n[4];
};
__global__ __launch_bounds__(256) void zero_list_kernel(ZeroList z) {
    float* p = z.p[blockIdx.y];
    const size_t n = z.n[blockIdx.y];
    const size_t step = (size_t)gridDim.x * blockDim.x;
    const size_t first = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (((reinterpret_cast<uintptr_t>(p) & 15u) | (uintptr_t)(n & 3)) == 0) {
        float4* p4 = reinterpret_cast<float4*>(p);
        const float4 zero = {0.f, 0.f, 0.f, 0.f};
        for (size_t j = first; j < n / 4; j += step) p4[j] = zero;
        return;
    }
    for (size_t j = first; j < n; j += step) p[j] = 0.f;
}

// ------------------------------------------------------------------ select
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistCopies = 4;
using dev::kIneligible;
using dev::kAbsent;
using dev::order_key;

__device__ __forceinline__ int wave_count(bool pred) {
    return __popcll(__ballot(pred));
}

// Exclusive prefix sum over the block in thread order; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sWave, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) sWave[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int x = sWave[w];
        before += w < wave ? x : 0;
        total += x;
    }
    __syncthreads();
    return before + incl - v;
}

// One workgroup per (b, kv head); KPT consecutive slots per thread, held in
// registers.  The k-th smallest key T is found by a most-significant-digit-
// first radix select over four 8-bit digits: each pass builds an LDS
// histogram of the digit among the keys that match the digits fixed so far,
// and one wave scans it for the bin that holds the k-th key.  Victims are
// every key below T plus the lowest-index slots equal to T, which gives the
// (score, slot index) order exactly.
template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(EvictArgs a) {
    // kHistCopies copies of every bin, lane l adding to copy l % kHistCopies:
    // scores cluster in a few exponent bins, and lanes of one instruction that
    // hit the same LDS word serialize.
    __shared__ int sHist[2][256 * kHistCopies];
    __shared__ int sSel[2];
    __shared__ int sWave[kSelWaves];
    const int bg = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n, S = a.S, NC = a.NC;
    const int n_new = min(NC, n + S);
    const int k = max(0, n + S - NC);
    int32_t* freed = a.freed + (size_t)bg * S;

    if (k > 0) {
        const float* sc = a.score + (size_t)bg * NC;
        const int32_t* ps = a.pos + (size_t)bg * NC;
        const int thr = a.P - a.W;            // eligible iff t(j) < P - W
        const int t_now = a.P + S;
        const int j0 = tid * KPT;
        uint32_t key[KPT];
        // Coalesced pass: slot j = e*1024 + tid forms its order key into LDS; then
        // each thread takes KPT consecutive slots, so thread order is slot order.
        extern __shared__ uint32_t sKeys[];
        // All loads first (buffer loads past slot n return zero), then the keys.
        const dev::Rsrc rs = dev::make_rsrc(sc, n * 4), rp = dev::make_rsrc(ps, n * 4);
        uint32_t sraw[KPT], praw[KPT];
        const bool need_score = a.score_mode != kModeLastrec;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            sraw[e] = need_score ? dev::bload4(rs, (e * kSelThreads + tid) * 4) : 0u;
            praw[e] = dev::bload4(rp, (e * kSelThreads + tid) * 4);
        }
        if (a.cs_upd != nullptr) {
            // The score update first: phi += colsum for the filled slots, written back.
            const dev::Rsrc rc = dev::make_rsrc(a.cs_upd + (size_t)bg * NC, n * 4);
            uint32_t craw[KPT];
#pragma unroll
            for (int e = 0; e < KPT; ++e) craw[e] = dev::bload4(rc, (e * kSelThreads + tid) * 4);
            float* scw = a.score + (size_t)bg * NC;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int j = e * kSelThreads + tid;
                const float v = __uint_as_float(sraw[e]) + __uint_as_float(craw[e]);
                if (j < n) scw[j] = v;
                sraw[e] = __float_as_uint(v);
            }
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int j = e * kSelThreads + tid;
            const int pj = (int)praw[e];
            uint32_t kv;
            if (a.score_mode == kModeLastrec) {
                // Positions are non-negative int32: their uint order is their order.
                kv = j >= n ? kAbsent : (pj >= a.sink ? (uint32_t)pj : kIneligible);
            } else {
                float v = __uint_as_float(sraw[e]);
                if (a.score_mode == H2O_SCORE_H2O_NORM) v = v / (float)(t_now - pj);
                kv = j >= n ? kAbsent : (pj < thr ? order_key(v) : kIneligible);
            }
            sKeys[j + j / 16] = kv;               // one pad word per 16: no bank conflicts
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e) key[e] = sKeys[j0 + e + (j0 + e) / 16];

        if (k == 1) {
            // Single victim: argmin of (key, slot), one reduction.  The empty-slot
            // targets (S > 1) follow below like those of the radix path.
            uint64_t best = ~0ull;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const uint64_t v = ((uint64_t)key[e] << 32) | (uint32_t)(j0 + e);
                best = v < best ? v : best;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const uint64_t o = __shfl_xor(best, off);
                best = o < best ? o : best;
            }
            __shared__ uint64_t sBest[kSelWaves];
            if (lane == 0) sBest[wave] = best;
            __syncthreads();
            if (tid == 0) {
                uint64_t m = sBest[0];
                for (int w = 1; w < kSelWaves; ++w) m = sBest[w] < m ? sBest[w] : m;
                freed[0] = (int)(uint32_t)m;
            }
        } else {
            // Skip the leading digits that every candidate for T shares: T lies in
            // [lo, hi] with lo the smallest key and hi the largest eligible key when
            // at least k are eligible (else the largest possible key), so digits
            // where lo and hi agree are T's digits too, and no key lies below them.
            // Positions (lastrec) share their high bytes: their passes would pile
            // every key into one histogram bin.
            uint32_t lo = ~0u, hi = 0u;
            int elig = 0;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                lo = min(lo, key[e]);
                const bool is_e = key[e] < kIneligible;
                hi = is_e ? max(hi, key[e]) : hi;
                elig += is_e;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
                hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
                elig += __shfl_xor(elig, off);
            }
            __shared__ uint32_t sLo[kSelWaves], sHi[kSelWaves];
            __shared__ int sElig[kSelWaves];
            if (lane == 0) {
                sLo[wave] = lo;
                sHi[wave] = hi;
                sElig[wave] = elig;
            }
            __syncthreads();
            lo = ~0u;
            hi = 0u;
            elig = 0;
#pragma unroll
            for (int w = 0; w < kSelWaves; ++w) {
                lo = min(lo, sLo[w]);
                hi = max(hi, sHi[w]);
                elig += sElig[w];
            }
            if (elig < k) hi = ~0u;
            const uint32_t diff = lo ^ hi;
            // Highest digit where lo and hi differ (-8: none, T == lo).
            const int top = diff ? ((31 - __clz((int)diff)) & ~7) : -8;
            uint32_t mask = top >= 24 ? 0u : ~0u << (top + 8);
            uint32_t prefix = lo & mask;
            int k_rem = k;                        // rank of T among the keys matching prefix
            // Two histograms: while wave 0 scans one, the other waves clear the other
            // for the next pass (its last reader, the scan before, ended at a barrier).
            for (int x = tid; x < 256 * kHistCopies; x += kSelThreads) {
                sHist[0][x] = 0;
                sHist[1][x] = 0;
            }
            __syncthreads();
            int hb = 0;
            for (int shift = top; shift >= 0; shift -= 8, hb ^= 1) {
                int* hist = sHist[hb];
#pragma unroll
                for (int e = 0; e < KPT; ++e)
                    if ((key[e] & mask) == prefix)
                        atomicAdd(&hist[((key[e] >> shift) & 255u) * kHistCopies +
                                        (lane & (kHistCopies - 1))], 1);
                __syncthreads();
                if (wave != 0) {
                    for (int x = tid - 64; x < 256 * kHistCopies; x += kSelThreads - 64)
                        sHist[hb ^ 1][x] = 0;
                } else {
                    int c4[4], sum = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        c4[q] = 0;
#pragma unroll
                        for (int cp = 0; cp < kHistCopies; ++cp)
                            c4[q] += hist[(4 * lane + q) * kHistCopies + cp];
                        sum += c4[q];
                    }
                    int incl = sum;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const int y = __shfl_up(incl, off);
                        if (lane >= off) incl += y;
                    }
                    int before = incl - sum;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (before < k_rem && before + c4[q] >= k_rem) {
                            sSel[0] = 4 * lane + q;
                            sSel[1] = before;
                        }
                        before += c4[q];
                    }
                }
                __syncthreads();
                prefix |= (uint32_t)sSel[0] << shift;
                mask |= 255u << shift;
                k_rem -= sSel[1];
            }
            const uint32_t T = prefix;
            // T is the k-th smallest key: count(< T) < k <= count(<= T).  One scan of
            // the packed counts (less in the low 16 bits, equal in the high: at most
            // N_C <= 32768 each) gives, in slot order, the keys below T and the keys
            // equal to T before each thread; a victim's output index is the number of
            // victims before it: the keys below T plus the first need_eq equal keys.
            int my_less = 0, my_eq = 0;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                my_less += key[e] < T;
                my_eq += (key[e] == T) && (j0 + e < n);
            }
            int total;
            const int before = block_exclusive_scan(my_less | (my_eq << 16), sWave, total);
            const int need_eq = k - (total & 0xFFFF);
            int less_run = before & 0xFFFF, eq_run = before >> 16;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const bool lt = key[e] < T;
                const bool eq = (key[e] == T) && (j0 + e < n);
                if (lt || (eq && eq_run < need_eq)) freed[less_run + min(eq_run, need_eq)] = j0 + e;
                less_run += lt;
                eq_run += eq;
            }
        }
    }
    for (int e = tid; e < n_new - n; e += kSelThreads) freed[k + e] = n + e;
}

// ------------------------------------------------------------- exclusion masks
// One workgroup per (b, kv head): the row's words are cleared in LDS, every
// thread ORs in the bits of its targets below n (the slots >= n it gets are
// empty, not keys), and the row is written out.  One load per target and no
// dependent chain (OR does not depend on the order).
constexpr int kExclThreads = 1024;
constexpr int kExclMaxWords = (kMaxCapacity + 63) / 64;
__global__ __launch_bounds__(kExclThreads) void build_excl_kernel(const int32_t* __restrict__ freed,
                                                                  uint64_t* __restrict__ excl,
                                                                  int S, int n, int ntc) {
    __shared__ unsigned long long sW[kExclMaxWords];
    const int bg = blockIdx.x;
    for (int t = threadIdx.x; t < ntc; t += kExclThreads) sW[t] = 0ull;
    __syncthreads();
    const int32_t* f = freed + (size_t)bg * S;
    for (int i = threadIdx.x; i < S; i += kExclThreads) {
        const int slot = f[i];
        if (slot >= 0 && slot < n) atomicOr(&sW[slot >> 6], 1ull << (slot & 63));
    }
    __syncthreads();
    uint64_t* out = excl + (size_t)bg * ntc;
    for (int t = threadIdx.x; t < ntc; t += kExclThreads) out[t] = sW[t];
}

// ------------------------------------------------------------------ insert
constexpr int kInsTokens = 16;

__global__ __launch_bounds__(256) void insert_kernel(EvictArgs a) {
    const int bg = blockIdx.y;
    const int tok0 = blockIdx.x * kInsTokens;
    const int units = a.D * a.elem_bytes / 16;    // 16-byte units per row
    const int32_t* freed = a.freed + (size_t)bg * a.S;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const size_t row_units_cache = (size_t)bg * a.NC * units;
    const size_t row_units_chunk = (size_t)bg * a.S * units;
    u32x4* kc = static_cast<u32x4*>(a.kc);
    u32x4* vc = static_cast<u32x4*>(a.vc);
    const u32x4* kn = static_cast<const u32x4*>(a.kn);
    const u32x4* vn = static_cast<const u32x4*>(a.vn);
    for (int u = threadIdx.x; u < kInsTokens * units; u += blockDim.x) {
        const int tok = tok0 + u / units, part = u % units;
        if (tok >= a.S) break;
        const int slot = freed[tok];
        kc[row_units_cache + (size_t)slot * units + part] = kn[row_units_chunk + (size_t)tok * units + part];
        vc[row_units_cache + (size_t)slot * units + part] = vn[row_units_chunk + (size_t)tok * units + part];
    }
    if (threadIdx.x < kInsTokens) {
        const int tok = tok0 + threadIdx.x;
        if (tok < a.S) {
            const int slot = freed[tok];
            a.pos[(size_t)bg * a.NC + slot] = a.P + tok;
            a.score[(size_t)bg * a.NC + slot] = a.cs_new ? a.cs_new[(size_t)bg * a.S + tok] : 0.f;
        }
    }
}

// --------------------------------------------------- one victim, one token
// k = 1 and S = 1 (a decode step on a full cache): the victim is the smallest
// (key, slot) pair under the same order keys as select_kernel, found in one
// pass of 16-byte loads and a reduction, and the same workgroup writes the new
// token into it.  Same victims and cache contents as select_kernel followed by
// insert_kernel, in one launch instead of two.
constexpr int kOneThreads = 1024;
constexpr int kOneLoads = 4;                     // 16-byte loads in flight per array

__global__ __launch_bounds__(kOneThreads) void select1_insert_kernel(EvictArgs a) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ uint64_t sBest[kOneThreads / 64];
    const int bg = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = a.n, NC = a.NC;
    const float* sc = a.score + (size_t)bg * NC;
    const int32_t* ps = a.pos + (size_t)bg * NC;
    const int thr = a.P - a.W;                   // eligible iff t(j) < P - W
    const int t_now = a.P + 1;
    const bool need_score = a.score_mode != kModeLastrec;
    // The new token's K / V row and summed weight do not depend on the victim:
    // load them with the scores so the insertion at the end only stores.
    const int units = a.D * a.elem_bytes / 16;    // 16-byte units per row (<= 32)
    const u32x4* kn = static_cast<const u32x4*>(a.kn) + (size_t)bg * units;
    const u32x4* vn = static_cast<const u32x4*>(a.vn) + (size_t)bg * units;
    u32x4 knv = {0u, 0u, 0u, 0u}, vnv = {0u, 0u, 0u, 0u};
    if (tid < units) {
        knv = kn[tid];
        vnv = vn[tid];
    }
    const float cs_tok = (tid == 0 && a.cs_new) ? a.cs_new[bg] : 0.f;
    const dev::Rsrc rs = dev::make_rsrc(sc, n * 4), rp = dev::make_rsrc(ps, n * 4);
    uint64_t best = ~0ull;
    for (int base = 0; base < n; base += 4 * kOneThreads * kOneLoads) {
        u32x4 s4[kOneLoads], p4[kOneLoads];
#pragma unroll
        for (int u = 0; u < kOneLoads; ++u) {
            const int j = base + 4 * (u * kOneThreads + tid);
            s4[u] = need_score ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              rs, j * 4, 0, 0))
                               : u32x4{0u, 0u, 0u, 0u};
            p4[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, j * 4, 0, 0));
        }
        if (a.cs_upd != nullptr) {
            // The score update first: phi += colsum for the filled slots, written back.
            const dev::Rsrc rc = dev::make_rsrc(a.cs_upd + (size_t)bg * NC, n * 4);
            u32x4 c4[kOneLoads];
#pragma unroll
            for (int u = 0; u < kOneLoads; ++u)
                c4[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rc, (base + 4 * (u * kOneThreads + tid)) * 4,
                                                      0, 0));
            float* scw = a.score + (size_t)bg * NC;
#pragma unroll
            for (int u = 0; u < kOneLoads; ++u) {
                const int j = base + 4 * (u * kOneThreads + tid);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = __uint_as_float(s4[u][e]) + __uint_as_float(c4[u][e]);
                    s4[u][e] = __float_as_uint(v[e]);
                }
                if (j + 3 < n && (((reinterpret_cast<uintptr_t>(scw) & 15u) | (NC & 3)) == 0)) {
                    *reinterpret_cast<float4*>(scw + j) = float4{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (j + e < n) scw[j + e] = v[e];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kOneLoads; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = base + 4 * (u * kOneThreads + tid) + e;
                const int pj = (int)p4[u][e];
                uint32_t kv;
                if (a.score_mode == kModeLastrec) {
                    kv = j >= n ? kAbsent : (pj >= a.sink ? (uint32_t)pj : kIneligible);
                } else {
                    float v = __uint_as_float(s4[u][e]);
                    if (a.score_mode == H2O_SCORE_H2O_NORM) v = v / (float)(t_now - pj);
                    kv = j >= n ? kAbsent : (pj < thr ? order_key(v) : kIneligible);
                }
                const uint64_t key = ((uint64_t)kv << 32) | (uint32_t)j;
                best = key < best ? key : best;
            }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(best, off);
        best = o < best ? o : best;
    }
    if (lane == 0) sBest[wave] = best;
    __syncthreads();
    uint64_t m = sBest[0];
#pragma unroll
    for (int w = 1; w < kOneThreads / 64; ++w) m = sBest[w] < m ? sBest[w] : m;
    const int victim = (int)(uint32_t)m;
    // The new token into the victim's slot.
    u32x4* kc = static_cast<u32x4*>(a.kc) + ((size_t)bg * NC + victim) * units;
    u32x4* vc = static_cast<u32x4*>(a.vc) + ((size_t)bg * NC + victim) * units;
    if (tid < units) {
        kc[tid] = knv;
        vc[tid] = vnv;
    }
    if (tid == 0) {
        a.freed[bg] = victim;
        a.pos[(size_t)bg * NC + victim] = a.P;
        a.score[(size_t)bg * NC + victim] = cs_tok;
    }
}

}  // namespace

hipError_t launch_update_scores(float* score, const float* cs, int rows, int NC, int n,
                                hipStream_t s) {
    if (rows == 0 || n == 0) return hipSuccess;
    const int per_block = 256 * 4;
    int bx = (n + per_block - 1) / per_block;
    if (bx > 64) bx = 64;
    // float4 rows need 16-byte aligned row starts in both arrays.
    const bool vec = NC % 4 == 0 && ((reinterpret_cast<uintptr_t>(score) |
                                      reinterpret_cast<uintptr_t>(cs)) & 15) == 0;
    hipLaunchKernelGGL(update_scores_kernel, dim3(bx, rows), dim3(256), 0, s, score, cs, NC, n,
                       vec);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, size_t per_row, size_t stride, int rows, size_t offset,
                           hipStream_t s) {
    if (rows == 0 || per_row == 0) return hipSuccess;
    int bx = (int)((per_row + 1023) / 1024);
    if (bx > 256) bx = 256;
    hipLaunchKernelGGL(zero_kernel, dim3(bx, rows), dim3(256), 0, s, p, (int)per_row, stride,
                       offset);
    return hipGetLastError();
}

hipError_t launch_zero_f32_list(float* const* p, const size_t* n, int count, hipStream_t s) {
    if (count < 1 || count > 4) return hipErrorInvalidValue;
    ZeroList z;
    size_t most = 0;
    for (int i = 0; i < 4; ++i) {
        z.p[i] = i < count ? p[i] : p[0];
        z.n[i] = i < count ? n[i] : 0;
        most = z.n[i] > most ? z.n[i] : most;
    }
    if (most == 0) return hipSuccess;
    int bx = (int)((most + 1023) / 1024);
    if (bx > 512) bx = 512;
    hipLaunchKernelGGL(zero_list_kernel, dim3(bx, count), dim3(256), 0, s, z);
    return hipGetLastError();
}

hipError_t launch_select(const EvictArgs& a, hipStream_t s) {
    const dim3 grid(a.B * a.Hkv), block(kSelThreads);
    const int kpt = (a.NC + kSelThreads - 1) / kSelThreads;
    int p2 = 1;
    while (p2 < kpt) p2 <<= 1;
    const size_t lds = (size_t)p2 * kSelThreads * 4 * 17 / 16;   // order keys, padded
    auto go = [&](auto kernel) -> hipError_t {
        // Above 64 KB of LDS the attribute must be raised first (once per device).
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(kernel, grid, block, lds, s, a);
        return hipGetLastError();
    };
    if (p2 <= 1) return go(select_kernel<1>);
    if (p2 <= 2) return go(select_kernel<2>);
    if (p2 <= 4) return go(select_kernel<4>);
    if (p2 <= 8) return go(select_kernel<8>);
    if (p2 <= 16) return go(select_kernel<16>);
    return go(select_kernel<32>);
}

hipError_t launch_build_excl(const ChunkArgs& a, uint64_t* excl, hipStream_t s) {
    const int rows = a.B * a.Hkv, ntc = excl_tiles(a.NC);
    if (ntc > kExclMaxWords) return hipErrorInvalidValue;
    hipLaunchKernelGGL(build_excl_kernel, dim3(rows), dim3(kExclThreads), 0, s, a.freed, excl,
                       a.S, a.n, ntc);
    return hipGetLastError();
}

hipError_t launch_insert(const EvictArgs& a, hipStream_t s) {
    const dim3 grid((a.S + kInsTokens - 1) / kInsTokens, a.B * a.Hkv), block(256);
    hipLaunchKernelGGL(insert_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_select1_insert(const EvictArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(select1_insert_kernel, dim3(a.B * a.Hkv), dim3(kOneThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace h2o
