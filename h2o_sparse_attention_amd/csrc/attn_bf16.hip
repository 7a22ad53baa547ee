// bf16 chunk attention for gfx950: the attention pass (output + log-sum-exp)
// and the recompute pass that forms the summed attention weights.
//
// Method: "Learning how to Forget: Fine-tuning for Long-Context Sparse
// Attention", montaan paper page, "Kernel Support Needs": the SDPA kernel
// must also return sum_i m_{b,h,i,j}, and the causal mask is implicit,
// -inf * 1[P+i < t(b,h,j)].  Keys are the filled cache slots followed by the
// chunk's own keys ("virtual key" kk: kk < n is slot kk, else chunk key kk-n).
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64).  Lane l = 32*hh + lq.
//   A operand: lane holds A[m = lq][k = 8*hh + 0..7]
//   B operand: lane holds B[k = 8*hh + 0..7][n = lq]
//   C/D:       lane holds C[8*(r/4) + 4*hh + r%4][lq], r = 0..15
// The attention pass computes S^T = K Q^T (A = K from LDS, B = Q^T from
// registers), so each lane owns one query row (lq) and 16 of the 32 keys of a
// sub-tile; the two lanes lq and lq+32 together see all 32.  The K rows fed
// to A are permuted (perm_key) so that C register r of half hh lands on
// physical key 16*(r/8) + 8*hh + r%8: eight consecutive keys per lane and
// per 16-key step, which is exactly the k-slot order of the B operand of the
// P V product.  O^T = V^T P^T then takes P^T straight from registers (no
// shuffle) and V^T from LDS (V is transposed while it is staged), and the
// O^T accumulator keeps the lane's own query row, so the softmax rescale
// needs no cross-lane traffic.
#include "h2o_internal.h"

#include <climits>
#include <cmath>

namespace h2o {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;   // attention pass: 32 query rows per wave
constexpr int kKeysPerTile = 64;             // attention pass: keys staged per step
constexpr int kKeysPerBlock = 32 * kWaves;   // colsum pass: 32 keys per wave
constexpr int kRowsPerTile = 64;             // colsum pass: query rows staged per step
constexpr float kLog2e = 1.4426950408889634f;
// The running max is only raised when it grows by more than 2^8 (log2 units),
// so most tiles skip the O rescale; p = exp2(s - m) then stays below 2^8,
// which bf16 and fp32 hold without loss of relative precision.
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup ids are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles that share K/V (or Q) share an L2.
__device__ __forceinline__ int xcd_tile(int lin, int total) {
    const int per = (total + 7) >> 3;
    return (lin & 7) * per + (lin >> 3);
}

__host__ __device__ inline int xcd_grid(int total) { return ((total + 7) >> 3) << 3; }

// A-operand row m of the QK^T product reads physical key perm_key(m).
__device__ __forceinline__ int perm_key(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// ---------------------------------------------------------------------------
// Attention pass: O and LSE for 128 query rows of one (b, kv head).
// Rows of a KV head are ordered position-major: row r = i*G + hh is query
// head g*G + hh at chunk position i.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(ChunkArgs a) {
    constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
    constexpr int DT = D / 32;                    // 32-row tiles of O^T
    constexpr int KROW = D + 8;                   // LDS K row, +16 B pad
    constexpr int VROW = kKeysPerTile + 8;        // LDS V^T row, +16 B pad
    constexpr int KCH = D / 8;                    // 16-byte chunks per key row
    constexpr int K_LD = kKeysPerTile * KCH / kThreads;
    constexpr int VP = D / 2;                     // d pairs
    constexpr int VKG = kThreads / VP;            // key groups for V staging
    constexpr int VKPG = kKeysPerTile / VKG;      // keys per group (8 or 16)
    static_assert(K_LD >= 1 && VKPG % 8 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sK[kKeysPerTile * KROW];
    __shared__ __attribute__((aligned(16))) u16 sVt[D * VROW];
    __shared__ __attribute__((aligned(16))) int sPos[kKeysPerTile];

    const int R = a.G * a.S;
    const int nrb = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    const int total = nrb * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nrb, rb = t % nrb;
    const int b = bg / a.Hkv, g = bg % a.Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hh = lane >> 5;
    const int row = rb * kRowsPerBlock + wave * 32 + lq;
    const bool row_ok = row < R;
    const int i = row_ok ? row / a.G : a.S - 1;
    const int h = g * a.G + (row_ok ? row % a.G : 0);
    const int qpos = a.P + i;

    const u16* Q = static_cast<const u16*>(a.q);
    const size_t qoff = ((size_t)(b * a.Hq + h) * a.S + i) * D;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok) v = ld16(Q + qoff + 16 * ks + 8 * hh);
        qf[ks] = as_bf16x8(v);
    }

    const int last_row = min(R - 1, rb * kRowsPerBlock + kRowsPerBlock - 1);
    const int nkeys = a.n + last_row / a.G + 1;
    const int ntiles = (nkeys + kKeysPerTile - 1) / kKeysPerTile;
    const int wave_row0 = min(R - 1, rb * kRowsPerBlock + wave * 32);
    const int qpos_wave_min = a.P + wave_row0 / a.G;

    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D;
    const u16* Vc = static_cast<const u16*>(a.vc) + (size_t)bg * a.NC * D;
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * a.S * D;
    const u16* Vn = static_cast<const u16*>(a.vn) + (size_t)bg * a.S * D;
    const int32_t* posg = a.pos + (size_t)bg * a.NC;
    const int n = a.n, S = a.S;

    u32x4 kreg[K_LD];
    uint32_t vreg[VKPG];
    int preg = INT_MAX;

    auto gload = [&](int tile) {
        const int base = tile * kKeysPerTile;
#pragma unroll
        for (int it = 0; it < K_LD; ++it) {
            const int c = tid + it * kThreads;
            const int kk = base + c / KCH, col = (c % KCH) * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (kk < n) v = ld16(Kc + (size_t)kk * D + col);
            else if (kk < n + S) v = ld16(Kn + (size_t)(kk - n) * D + col);
            kreg[it] = v;
        }
        const int dp = tid % VP, kg = tid / VP;
#pragma unroll
        for (int e = 0; e < VKPG; ++e) {
            const int kk = base + kg * VKPG + e;
            uint32_t v = 0u;
            if (kk < n) v = *reinterpret_cast<const uint32_t*>(Vc + (size_t)kk * D + 2 * dp);
            else if (kk < n + S)
                v = *reinterpret_cast<const uint32_t*>(Vn + (size_t)(kk - n) * D + 2 * dp);
            vreg[e] = v;
        }
        if (tid < kKeysPerTile) {
            const int kk = base + tid;
            preg = kk < n ? posg[kk] : (kk < n + S ? a.P + (kk - n) : INT_MAX);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < K_LD; ++it) {
            const int c = tid + it * kThreads;
            *reinterpret_cast<u32x4*>(&sK[(c / KCH) * KROW + (c % KCH) * 8]) = kreg[it];
        }
        const int dp = tid % VP, kg = tid / VP;
#pragma unroll
        for (int e0 = 0; e0 < VKPG; e0 += 8) {
            u32x4 lo, hi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w0 = vreg[e0 + 2 * j], w1 = vreg[e0 + 2 * j + 1];
                lo[j] = (w0 & 0xffffu) | (w1 << 16);
                hi[j] = (w0 >> 16) | (w1 & 0xffff0000u);
            }
            *reinterpret_cast<u32x4*>(&sVt[(2 * dp) * VROW + kg * VKPG + e0]) = lo;
            *reinterpret_cast<u32x4*>(&sVt[(2 * dp + 1) * VROW + kg * VKPG + e0]) = hi;
        }
        if (tid < kKeysPerTile) sPos[tid] = preg;
    };

    const float c = a.sm_scale * kLog2e;          // logits -> log2 units
    const float tau_raw = kRescaleLog2 / c;
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int prow = perm_key(lq);

    if (ntiles > 0) gload(0);
    for (int tile = 0; tile < ntiles; ++tile) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (tile + 1 < ntiles) gload(tile + 1);

        f32x16 s[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            s[sub] = f32x16{};
            const u16* kp = &sK[(sub * 32 + prow) * KROW + 8 * hh];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[sub] = mfma32(as_bf16x8(ld16(kp + 16 * ks)), qf[ks], s[sub]);
        }

        // Implicit positional mask; skipped when every key of the tile is
        // visible to every row of this wave.
        const int kp_lane = sPos[lane];
        const bool vis_all = kp_lane >= 0 && kp_lane <= qpos_wave_min;
        if (!__all(vis_all)) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int k0 = sub * 32 + 16 * s2 + 8 * hh;
                    const i32x4 p0 = *reinterpret_cast<const i32x4*>(&sPos[k0]);
                    const i32x4 p1 = *reinterpret_cast<const i32x4*>(&sPos[k0 + 4]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int kpv = e < 4 ? p0[e] : p1[e - 4];
                        if (!(kpv >= 0 && kpv <= qpos)) s[sub][8 * s2 + e] = -INFINITY;
                    }
                }
        }

        float mt = s[0][0];
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(s[0][r], s[1][r]));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const bool need = m_new > m_run + tau_raw;
        if (__any(need)) {
            const float m_next = need ? m_new : m_run;
            const float alpha = (m_next == m_run) ? 1.f : fast_exp2((m_run - m_next) * c);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            m_run = m_next;
        }
        const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;

        bf16x8 pb[2][2];
        float lsum = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = fast_exp2(fmaf(s[sub][8 * s2 + e], c, -mc));
                    lsum += p[e];
                }
                u32x4 w = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]),
                           pack2(p[6], p[7])};
                pb[sub][s2] = as_bf16x8(w);
            }
        l_run += lsum;

#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u16* vp = &sVt[(dt * 32 + lq) * VROW + 8 * hh];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    o[dt] = mfma32(as_bf16x8(ld16(vp + sub * 32 + 16 * s2)), pb[sub][s2], o[dt]);
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_ok) {
        const float inv = 1.f / l_tot;
        u16* O = static_cast<u16*>(a.out) + qoff;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = dt * 32 + 8 * r4 + 4 * hh;
                u32x2 w = {pack2(o[dt][4 * r4 + 0] * inv, o[dt][4 * r4 + 1] * inv),
                           pack2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(O + d0) = w;
            }
        if (hh == 0)
            a.lse[(size_t)(b * a.Hq + h) * a.S + i] = fmaf(m_run, a.sm_scale, logf(l_tot));
    }
}

// ---------------------------------------------------------------------------
// Colsum pass: for 128 keys of one (b, kv head), sum exp(s - lse) over every
// query row of the group (G heads x S positions).  K stays in registers; Q
// and LSE tiles stream through LDS.  Each lane accumulates its 16 keys over
// its query column, and the 32 columns are added in a fixed order at the end,
// so the result is deterministic (no atomics).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void colsum_bf16_kernel(ChunkArgs a) {
    constexpr int KS = D / 16;
    constexpr int QROW = D + 8;
    constexpr int QCH = D / 8;
    constexpr int Q_LD = kRowsPerTile * QCH / kThreads;
    static_assert(Q_LD >= 1, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sQ[kRowsPerTile * QROW];
    __shared__ float sL[kRowsPerTile];
    __shared__ float sRed[kWaves][32][33];

    const int n = a.n, S = a.S, G = a.G;
    const int nkeys = n + S;
    const int nkb = (nkeys + kKeysPerBlock - 1) / kKeysPerBlock;
    const int total = nkb * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nkb, kb = t % nkb;
    const int b = bg / a.Hkv, g = bg % a.Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hh = lane >> 5;
    const int key0 = kb * kKeysPerBlock + wave * 32;

    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D;
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
    const int32_t* posg = a.pos + (size_t)bg * a.NC;
    auto key_pos = [&](int kk) -> int {
        return kk < n ? posg[kk] : (kk < n + S ? a.P + (kk - n) : INT_MAX);
    };

    // A operand: this lane's key row.
    bf16x8 kf[KS];
    {
        const int kk = key0 + lq;
        const u16* src = kk < n ? Kc + (size_t)kk * D
                                : (kk < n + S ? Kn + (size_t)(kk - n) * D : nullptr);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (src) v = ld16(src + 16 * ks + 8 * hh);
            kf[ks] = as_bf16x8(v);
        }
    }
    // Positions of the 16 keys of this lane's C registers.
    int kpos[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) kpos[r] = key_pos(key0 + 8 * (r >> 2) + 4 * hh + (r & 3));
    int kmin = key_pos(key0 + lq), kmax = kmin;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kmin = min(kmin, __shfl_xor(kmin, off));
        kmax = max(kmax, __shfl_xor(kmax, off));
    }

    const int R = G * S;
    const int ntile = (R + kRowsPerTile - 1) / kRowsPerTile;
    // Blocks made only of chunk keys are invisible to rows before their first key.
    const int first_key = kb * kKeysPerBlock;
    const int tile0 = first_key >= n ? ((first_key - n) * G) / kRowsPerTile : 0;

    const u16* Q = static_cast<const u16*>(a.q);
    u32x4 qreg[Q_LD];
    float lreg = INFINITY;
    auto gload = [&](int rt) {
#pragma unroll
        for (int it = 0; it < Q_LD; ++it) {
            const int cidx = tid + it * kThreads;
            const int r = rt * kRowsPerTile + cidx / QCH, col = (cidx % QCH) * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < R) {
                const int hq = g * G + r % G, ipos = r / G;
                v = ld16(Q + ((size_t)(b * a.Hq + hq) * S + ipos) * D + col);
            }
            qreg[it] = v;
        }
        if (tid < kRowsPerTile) {
            const int r = rt * kRowsPerTile + tid;
            lreg = r < R ? a.lse[(size_t)(b * a.Hq + g * G + r % G) * S + r / G] * kLog2e
                         : INFINITY;
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < Q_LD; ++it) {
            const int cidx = tid + it * kThreads;
            *reinterpret_cast<u32x4*>(&sQ[(cidx / QCH) * QROW + (cidx % QCH) * 8]) = qreg[it];
        }
        if (tid < kRowsPerTile) sL[tid] = lreg;
    };

    const float c = a.sm_scale * kLog2e;
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    if (tile0 < ntile) gload(tile0);
    for (int rt = tile0; rt < ntile; ++rt) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (rt + 1 < ntile) gload(rt + 1);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int rloc = sub * 32 + lq;
            const float lse2 = sL[rloc];
            f32x16 sacc = f32x16{};
            const u16* qp = &sQ[rloc * QROW + 8 * hh];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc = mfma32(kf[ks], as_bf16x8(ld16(qp + 16 * ks)), sacc);
            const int row_first = rt * kRowsPerTile + sub * 32;
            const int qpos_min = a.P + min(row_first, R - 1) / G;
            if (kmin >= 0 && kmax <= qpos_min) {
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] += fast_exp2(fmaf(sacc[r], c, -lse2));
            } else {
                const int qpos = a.P + min(row_first + lq, R - 1) / G;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sacc[r], c, -lse2));
                    acc[r] += (kpos[r] >= 0 && kpos[r] <= qpos) ? p : 0.f;
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < 16; ++r) sRed[wave][8 * (r >> 2) + 4 * hh + (r & 3)][lq] = acc[r];
    __syncthreads();
    if (lane < 32) {
        float sum = 0.f;
#pragma unroll 8
        for (int j = 0; j < 32; ++j) sum += sRed[wave][lane][j];
        const int kk = key0 + lane;
        if (kk < n) a.cs_cache[(size_t)bg * a.NC + kk] = sum;
        else if (kk < n + S) a.cs_new[(size_t)bg * S + (kk - n)] = sum;
    }
}

}  // namespace

hipError_t launch_attn_bf16(const ChunkArgs& a, hipStream_t s) {
    const int R = a.G * a.S;
    const int total = ((R + kRowsPerBlock - 1) / kRowsPerBlock) * a.B * a.Hkv;
    const dim3 grid(xcd_grid(total)), block(kThreads);
    if (a.D == 128) hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_colsum_bf16(const ChunkArgs& a, hipStream_t s) {
    const int total = ((a.n + a.S + kKeysPerBlock - 1) / kKeysPerBlock) * a.B * a.Hkv;
    const dim3 grid(xcd_grid(total)), block(kThreads);
    if (a.D == 128) hipLaunchKernelGGL(colsum_bf16_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(colsum_bf16_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace h2o
