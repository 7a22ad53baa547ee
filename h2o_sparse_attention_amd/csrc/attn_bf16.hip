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
#include "device_common.h"

#include <climits>
#include <cmath>

namespace h2o {
namespace {

using namespace dev;


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;   // attention pass: 32 query rows per wave
constexpr int kKeysPerTile = 64;             // attention pass: keys staged per step
constexpr int kKeysPerBlock = 32 * kWaves;   // colsum pass: 32 keys per wave
constexpr int kRowsPerTile = 64;             // colsum pass: query rows staged per step

// ---------------------------------------------------------------------------
// Key tiles.  The filled cache slots form ceil(n/64) tiles (the last one may be
// partial) and the chunk's own keys follow in tiles of their own, so a tile
// never mixes cache rows and chunk rows: one base pointer and one count of
// valid keys describe it, and full tiles load with no per-key tests.
// ---------------------------------------------------------------------------
struct TileRef {
    const u16* k;
    const u16* v;
    int first;      // index of the tile's first key in its source (cache or chunk)
    int valid;      // keys of the tile that exist (1..64)
    bool cache;
};

__device__ __forceinline__ TileRef tile_ref(int tile, int cache_tiles, int n, int S, int D,
                                            const u16* Kc, const u16* Vc, const u16* Kn,
                                            const u16* Vn) {
    TileRef t;
    t.cache = tile < cache_tiles;
    t.first = (t.cache ? tile : tile - cache_tiles) * kKeysPerTile;
    t.valid = min(kKeysPerTile, (t.cache ? n : S) - t.first);
    t.k = (t.cache ? Kc : Kn) + (size_t)t.first * D;
    t.v = (t.cache ? Vc : Vn) + (size_t)t.first * D;
    return t;
}

template <int D>
struct AttnSmem {
    static constexpr int KROW = D + 8;                  // LDS K row, +16 B pad
    static constexpr int VROW = kKeysPerTile + 8;       // LDS V^T row, +16 B pad
    static constexpr int K_BYTES = kKeysPerTile * KROW * 2;
    static constexpr int V_BYTES = D * VROW * 2;
    static constexpr int BUF_BYTES = K_BYTES + V_BYTES + kKeysPerTile * 4;
    static constexpr int MERGE_FLOATS = 2 + (D / 32) * 16;   // m, l, O^T accumulators
    static constexpr int MERGE_BYTES = 4 * MERGE_FLOATS * 64 * 4;
    static constexpr int BYTES = 4 * BUF_BYTES > MERGE_BYTES ? 4 * BUF_BYTES : MERGE_BYTES;
};

// ---------------------------------------------------------------------------
// Attention pass: O and LSE for 128 query rows of one (b, kv head).
// Rows of a KV head are ordered position-major: row r = i*G + hh is query
// head g*G + hh at chunk position i.  Eight waves: waves 0-3 and 4-7 own the
// same four 32-row groups and split the key tiles between them (even / odd
// tiles), each half with its own double-buffered LDS tiles; the two partial
// softmax states are merged through LDS at the end.
// ---------------------------------------------------------------------------
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kHalfThreads = kAttnThreads / 2;

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_bf16_kernel(ChunkArgs a) {
    using L = AttnSmem<D>;
    constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
    constexpr int DT = D / 32;                    // 32-row tiles of O^T
    constexpr int KROW = L::KROW, VROW = L::VROW;
    constexpr int KCH = D / 8;                    // 16-byte chunks per key row
    constexpr int K_LD = kKeysPerTile * KCH / kHalfThreads;
    constexpr int VP = D / 2;                     // d pairs
    constexpr int VKG = kHalfThreads / VP;        // key groups for V staging
    constexpr int VKPG = kKeysPerTile / VKG;      // keys per group (8 or 16)
    static_assert(K_LD >= 1 && VKPG % 8 == 0, "tile shape");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int R = a.G * a.S;
    const int nrb = (R + kRowsPerBlock - 1) / kRowsPerBlock;
    const int total = nrb * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nrb, rb = t % nrb;
    const int b = bg / a.Hkv, g = bg % a.Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep it scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wave >> 2, rw = wave & 3, htid = tid & (kHalfThreads - 1);
    const int lq = lane & 31, hh = lane >> 5;
    const int row = rb * kRowsPerBlock + rw * 32 + lq;
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

    const int n = a.n, S = a.S;
    const int cache_tiles = (n + kKeysPerTile - 1) / kKeysPerTile;
    const int last_row = min(R - 1, rb * kRowsPerBlock + kRowsPerBlock - 1);
    const int ntiles = cache_tiles + (last_row / a.G) / kKeysPerTile + 1;
    const int steps = (ntiles + 1) / 2;
    const int wave_row0 = min(R - 1, rb * kRowsPerBlock + rw * 32);
    const int qpos_wave_min = a.P + wave_row0 / a.G;

    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D;
    const u16* Vc = static_cast<const u16*>(a.vc) + (size_t)bg * a.NC * D;
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
    const u16* Vn = static_cast<const u16*>(a.vn) + (size_t)bg * S * D;
    const int32_t* posg = a.pos + (size_t)bg * a.NC;

    u32x4 kreg[K_LD];
    uint32_t vreg[VKPG];
    int preg = INT_MAX;
    bool pvalid = false;
    const int dp = htid % VP, kg = htid / VP;

    // Loop-invariant lane offsets (bytes) into a tile.
    int koff[K_LD];
#pragma unroll
    for (int it = 0; it < K_LD; ++it) {
        const int c = htid + it * kHalfThreads;
        koff[it] = ((c / KCH) * D + (c % KCH) * 8) * 2;
    }
    const int voff = (kg * VKPG * D + 2 * dp) * 2;
    auto gload = [&](int tile) {
        const TileRef tr = tile_ref(tile, cache_tiles, n, S, D, Kc, Vc, Kn, Vn);
        const Rsrc rk = make_rsrc(tr.k, tr.valid * D * 2);
        const Rsrc rv = make_rsrc(tr.v, tr.valid * D * 2);
#pragma unroll
        for (int it = 0; it < K_LD; ++it) kreg[it] = bload16(rk, koff[it]);
#pragma unroll
        for (int e = 0; e < VKPG; ++e) vreg[e] = bload4(rv, voff + e * D * 2);
        // The loaded position is only consumed in lstore (after compute), so the
        // prefetch stays in flight; invalid keys are marked there.
        if (htid < kKeysPerTile) {
            pvalid = htid < tr.valid;
            if (tr.cache) {
                const Rsrc rp = make_rsrc(posg + tr.first, tr.valid * 4);
                preg = (int)bload4(rp, htid * 4);
            } else {
                preg = a.P + tr.first + htid;
            }
        }
    };
    auto bufs = [&](int which, u16*& sK, u16*& sVt, int*& sPos) {
        unsigned char* base = smem + (kh * 2 + which) * L::BUF_BYTES;
        sK = reinterpret_cast<u16*>(base);
        sVt = reinterpret_cast<u16*>(base + L::K_BYTES);
        sPos = reinterpret_cast<int*>(base + L::K_BYTES + L::V_BYTES);
    };
    auto lstore = [&](int which) {
        u16 *sK, *sVt;
        int* sPos;
        bufs(which, sK, sVt, sPos);
#pragma unroll
        for (int it = 0; it < K_LD; ++it) {
            const int c = htid + it * kHalfThreads;
            *reinterpret_cast<u32x4*>(&sK[(c / KCH) * KROW + (c % KCH) * 8]) = kreg[it];
        }
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
        if (htid < kKeysPerTile) sPos[htid] = pvalid ? preg : INT_MAX;
    };

    const float c = a.sm_scale * kLog2e;          // logits -> log2 units
    const float tau_raw = kRescaleLog2 / c;
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int prow = perm_key(lq);

    auto compute = [&](int which) {
        u16 *sK, *sVt;
        int* sPos;
        bufs(which, sK, sVt, sPos);
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
    };

    // Half kh owns tiles kh, kh+2, kh+4, ...; both halves step together.
    // Unconditional prologue (a half with no tile stages tile 0 and never reads
    // it), so every path has waited for the Q loads before the loop.
    gload(min(kh, ntiles - 1));
    lstore(0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const int cur = st & 1;
        const int my_tile = 2 * st + kh, next_tile = my_tile + 2;
        if (next_tile < ntiles) gload(next_tile);
        if (my_tile < ntiles) compute(cur);
        if (next_tile < ntiles) lstore(cur ^ 1);
        __syncthreads();
    }

    // Merge the two halves' (m, l, O) for each row (all LDS tile reads are done).
    constexpr int MF = L::MERGE_FLOATS;
    float* mb = reinterpret_cast<float*>(smem) + rw * MF * 64;
    if (kh == 1) {
        mb[lane] = m_run;
        mb[64 + lane] = l_run;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mb[(2 + dt * 16 + r) * 64 + lane] = o[dt][r];
    }
    __syncthreads();
    if (kh == 1) return;
    {
        const float m1 = mb[lane], l1 = mb[64 + lane];
        const float m = fmaxf(m_run, m1);
        const float a0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m) * c);
        const float a1 = m1 == -INFINITY ? 0.f : fast_exp2((m1 - m) * c);
        l_run = l_run * a0 + l1 * a1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[dt][r] = o[dt][r] * a0 + mb[(2 + dt * 16 + r) * 64 + lane] * a1;
        m_run = m;
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
// and LSE tiles stream through double-buffered LDS.  Each lane accumulates its
// 16 keys over its query column, and the 32 columns are added in a fixed
// order at the end, so the result is deterministic (no atomics).  Key blocks
// follow the same cache / chunk split as the attention tiles.
// ---------------------------------------------------------------------------
template <int D, bool EVEN_ROWS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void colsum_bf16_kernel(ChunkArgs a, uint32_t g_magic) {
    constexpr int KS = D / 16;
    constexpr int QROW = D + 8;
    constexpr int QCH = D / 8;
    constexpr int Q_LD = kRowsPerTile * QCH / kThreads;
    constexpr int QBUF = kRowsPerTile * QROW;      // u16 per Q buffer
    static_assert(Q_LD >= 1, "tile shape");

    __shared__ __attribute__((aligned(16))) u16 sQ[2][QBUF];
    __shared__ float sL[2][kRowsPerTile];
    __shared__ float sRed[kWaves][32][33];

    const int n = a.n, S = a.S, G = a.G;
    const int cache_blocks = (n + kKeysPerBlock - 1) / kKeysPerBlock;
    const int nkb = cache_blocks + (S + kKeysPerBlock - 1) / kKeysPerBlock;
    const int total = nkb * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nkb, kb = t % nkb;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const bool is_cache = kb < cache_blocks;
    const int block_first = (is_cache ? kb : kb - cache_blocks) * kKeysPerBlock;
    const int limit = is_cache ? n : S;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hh = lane >> 5;
    const int first = block_first + wave * 32;    // this wave's first key in its source

    const u16* Ksrc = is_cache ? static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D
                               : static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
    const int32_t* posg = a.pos + (size_t)bg * a.NC;
    auto key_pos = [&](int idx) -> int {
        return idx < limit ? (is_cache ? posg[idx] : a.P + idx) : INT_MAX;
    };

    bf16x8 kf[KS];
    {
        const int idx = first + lq;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (idx < limit) v = ld16(Ksrc + (size_t)idx * D + 16 * ks + 8 * hh);
            kf[ks] = as_bf16x8(v);
        }
    }
    int kmin = key_pos(first + lq), kmax = kmin;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kmin = min(kmin, __shfl_xor(kmin, off));
        kmax = max(kmax, __shfl_xor(kmax, off));
    }

    const int R = G * S;
    const int ntile = (R + kRowsPerTile - 1) / kRowsPerTile;
    // Chunk keys are invisible to the rows before their own position.
    const int tile0 = is_cache ? 0 : (block_first * G) / kRowsPerTile;

    // The G query heads of KV head g are contiguous in Q and in LSE.
    const u16* Qg = static_cast<const u16*>(a.q) + (size_t)(b * a.Hq + g * G) * S * D;
    const float* Lg = a.lse + (size_t)(b * a.Hq + g * G) * S;
    const int q_bytes = G * S * D * 2;
    u32x4 qreg[Q_LD];
    uint32_t lraw = 0u;          // LSE bits as loaded; scaled and masked in lstore
    bool lvalid = false;
    // When G divides the tile height every tile holds 64/G positions of all G
    // heads, so a lane's offset inside the tile is loop-invariant.
    // EVEN_ROWS: G divides the tile height (checked by the launcher).
    constexpr bool even_rows = EVEN_ROWS;
    const int pos_per_tile = even_rows ? kRowsPerTile / G : 0;
    int qoff[Q_LD];
    int l_il = 0, l_off = 0;
#pragma unroll
    for (int it = 0; it < Q_LD; ++it) {
        const int cidx = tid + it * kThreads;
        const int rloc = cidx / QCH, col = (cidx % QCH) * 8;
        qoff[it] = even_rows ? (((rloc % G) * S + rloc / G) * D + col) * 2 : col * 2;
    }
    if (even_rows && tid < kRowsPerTile) {
        l_il = tid / G;
        l_off = ((tid % G) * S + l_il) * 4;
    }
    auto row_split = [&](int r, int& hh_, int& ipos) {
        ipos = G == 1 ? r : (int)__umulhi((uint32_t)r, g_magic);
        hh_ = r - ipos * G;
    };
    auto gload = [&](int rt) {
        if constexpr (even_rows) {
            const int p0 = rt * pos_per_tile;                 // first position of the tile
            const Rsrc rq = make_rsrc(Qg + (size_t)p0 * D, q_bytes - p0 * D * 2);
#pragma unroll
            for (int it = 0; it < Q_LD; ++it) qreg[it] = bload16(rq, qoff[it]);
            if (tid < kRowsPerTile) {
                const Rsrc rl = make_rsrc(Lg + p0, (G * S - p0) * 4);
                lraw = bload4(rl, l_off);
                lvalid = p0 + l_il < S;
            }
        } else {
            const Rsrc rq = make_rsrc(Qg, q_bytes);
#pragma unroll
            for (int it = 0; it < Q_LD; ++it) {
                const int cidx = tid + it * kThreads;
                const int r = rt * kRowsPerTile + cidx / QCH;
                int hh_ = 0, ipos = 0;
                row_split(min(r, R - 1), hh_, ipos);
                const int off = r < R ? ((hh_ * S + ipos) * D) * 2 + qoff[it] : q_bytes;
                qreg[it] = bload16(rq, off);
            }
            if (tid < kRowsPerTile) {
                const int r = rt * kRowsPerTile + tid;
                int hh_ = 0, ipos = 0;
                row_split(min(r, R - 1), hh_, ipos);
                lraw = __float_as_uint(Lg[hh_ * S + ipos]);
                lvalid = r < R;
            }
        }
    };
    auto lstore = [&](int which) {
#pragma unroll
        for (int it = 0; it < Q_LD; ++it) {
            const int cidx = tid + it * kThreads;
            *reinterpret_cast<u32x4*>(&sQ[which][(cidx / QCH) * QROW + (cidx % QCH) * 8]) =
                qreg[it];
        }
        if (tid < kRowsPerTile) sL[which][tid] = lvalid ? __uint_as_float(lraw) * kLog2e : INFINITY;
    };

    const float c = a.sm_scale * kLog2e;
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    // S^T (this wave's 32 keys x 32 query rows of sub-tile `sub`) from buffer `buf`.
    auto mma = [&](int buf, int sub) {
        f32x16 r = f32x16{};
        const u16* qp = &sQ[buf][(sub * 32 + lq) * QROW + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) r = mfma32(kf[ks], as_bf16x8(ld16(qp + 16 * ks)), r);
        return r;
    };
    auto first_pos = [&](int rt, int sub) {
        const int rf = min(rt * kRowsPerTile + sub * 32, R - 1);
        return a.P + (G == 1 ? rf : (int)__umulhi((uint32_t)rf, g_magic));
    };
    auto lane_pos = [&](int rt, int sub) {
        const int rq = min(rt * kRowsPerTile + sub * 32 + lq, R - 1);
        return a.P + (G == 1 ? rq : (int)__umulhi((uint32_t)rq, g_magic));
    };
    auto exp_full = [&](const f32x16& sv, float lse2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += fast_exp2(fmaf(sv[r], c, -lse2));
    };
    // Masked tiles (chunk keys near the diagonal, or empty-slot markers) re-read
    // the positions of this lane's 16 keys instead of keeping them live.
    auto exp_masked = [&](const f32x16& sv, float lse2, int qpos) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kp = key_pos(first + 8 * (r >> 2) + 4 * hh + (r & 3));
            const float p = fast_exp2(fmaf(sv[r], c, -lse2));
            acc[r] += (kp >= 0 && kp <= qpos) ? p : 0.f;
        }
    };
    // Interleave the 8 MFMAs of one sub-tile with the exp/accumulate VALU work
    // of the other, so the matrix pipe and the vector ALU run together.
#define H2O_INTERLEAVE(VALU_PER_MFMA)                                  \
    do {                                                             \
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);           \
        _Pragma("unroll") for (int i_ = 0; i_ < KS; ++i_) {          \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       \
            __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER_MFMA, 0); \
            if (i_ + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); \
        }                                                            \
    } while (0)

    // Two-stage pipeline over row tiles.  Buffer (rt - tile0) & 1 holds tile rt.
    // Step rt: store tile rt+1 (loaded during the previous step), load tile
    // rt+2; stage A = MFMAs of sub-tile 1 with the exps of sub-tile 0; barrier;
    // stage B = MFMAs of sub-tile 0 of tile rt+1 with the exps of sub-tile 1.
    // A buffer is refilled only after the barrier that follows its last read.
    gload(tile0);
    lstore(0);
    if (tile0 + 1 < ntile) gload(tile0 + 1);
    __syncthreads();
    const bool keys_ok = kmin >= 0;
    f32x16 s0 = mma(0, 0);
    for (int rt = tile0; rt < ntile; ++rt) {
        const int cur = (rt - tile0) & 1;
        const bool has_next = rt + 1 < ntile;
        const float l0 = sL[cur][lq], l1 = sL[cur][32 + lq];
        if (has_next) lstore(cur ^ 1);
        if (rt + 2 < ntile) gload(rt + 2);
        f32x16 s1;
        if (keys_ok && kmax <= first_pos(rt, 0)) {
            s1 = mma(cur, 1);
            exp_full(s0, l0);
            H2O_INTERLEAVE(6);
        } else {
            s1 = mma(cur, 1);
            exp_masked(s0, l0, lane_pos(rt, 0));
        }
        __syncthreads();
        const bool full1 = keys_ok && kmax <= first_pos(rt, 1);
        if (has_next && full1) {
            s0 = mma(cur ^ 1, 0);
            exp_full(s1, l1);
            H2O_INTERLEAVE(6);
        } else {
            if (has_next) s0 = mma(cur ^ 1, 0);
            if (full1) exp_full(s1, l1);
            else exp_masked(s1, l1, lane_pos(rt, 1));
        }
    }
#undef H2O_INTERLEAVE

#pragma unroll
    for (int r = 0; r < 16; ++r) sRed[wave][8 * (r >> 2) + 4 * hh + (r & 3)][lq] = acc[r];
    __syncthreads();
    if (lane < 32) {
        float sum = 0.f;
#pragma unroll 8
        for (int j = 0; j < 32; ++j) sum += sRed[wave][lane][j];
        const int idx = first + lane;
        if (idx < limit) {
            if (is_cache) a.cs_cache[(size_t)bg * a.NC + idx] = sum;
            else a.cs_new[(size_t)bg * S + idx] = sum;
        }
    }
}

}  // namespace

template <int D>
hipError_t launch_attn_d(const ChunkArgs& a, hipStream_t s) {
    // More than 64 KB of LDS per workgroup must be requested explicitly, once per device.
    static unsigned configured = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned bit = 1u << (dev & 31);
    if (!(configured & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_kernel<D>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, AttnSmem<D>::BYTES);
        if (e != hipSuccess) return e;
        configured |= bit;
    }
    const int R = a.G * a.S;
    const int total = ((R + kRowsPerBlock - 1) / kRowsPerBlock) * a.B * a.Hkv;
    hipLaunchKernelGGL(attn_bf16_kernel<D>, dim3(xcd_grid(total)), dim3(kAttnThreads),
                       AttnSmem<D>::BYTES, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const ChunkArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_attn_d<128>(a, s) : launch_attn_d<64>(a, s);
}

hipError_t launch_colsum_bf16(const ChunkArgs& a, hipStream_t s) {
    const int blocks = (a.n + kKeysPerBlock - 1) / kKeysPerBlock +
                       (a.S + kKeysPerBlock - 1) / kKeysPerBlock;
    const int total = blocks * a.B * a.Hkv;
    // floor(r / G) = umulhi(r, ceil(2^32 / G)) for r * G < 2^32 (checked by the caller)
    const uint32_t magic = a.G > 1 ? (uint32_t)((0x100000000ull + a.G - 1) / a.G) : 0u;
    const dim3 grid(xcd_grid(total)), block(kThreads);
    const bool even = kRowsPerTile % a.G == 0;
    if (a.D == 128) {
        if (even) hipLaunchKernelGGL((colsum_bf16_kernel<128, true>), grid, block, 0, s, a, magic);
        else hipLaunchKernelGGL((colsum_bf16_kernel<128, false>), grid, block, 0, s, a, magic);
    } else {
        if (even) hipLaunchKernelGGL((colsum_bf16_kernel<64, true>), grid, block, 0, s, a, magic);
        else hipLaunchKernelGGL((colsum_bf16_kernel<64, false>), grid, block, 0, s, a, magic);
    }
    return hipGetLastError();
}

}  // namespace h2o
