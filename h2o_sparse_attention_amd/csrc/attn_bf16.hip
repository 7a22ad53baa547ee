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
// shuffle) and V^T from LDS through transposing reads, and the O^T
// accumulator keeps the lane's own query row, so the softmax rescale needs no
// cross-lane traffic.
#include "h2o_internal.h"
#include "device_common.h"

#include <climits>
#include <cmath>
#include <type_traits>

namespace h2o {
namespace {

using namespace dev;


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 32 * kWaves;   // attention pass: 32 query rows per wave
constexpr int kKeysPerTile = 64;             // attention pass: keys staged per step
constexpr int kColsumKB = 1;                 // colsum pass: 32-key blocks per wave
constexpr int kKeysPerBlock = 32 * kColsumKB * kWaves;   // colsum pass: keys per workgroup
constexpr int kRowsPerTile = 64;             // colsum pass: query rows staged per step
constexpr int kColsumMaxParts = 4;           // colsum pass: row ranges per key block

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

// ---------------------------------------------------------------------------
// Attention pass: O and LSE for 128 query rows of one (b, kv head).
// Rows of a KV head are ordered position-major: row r = i*G + hl is query
// head g*G + hl at chunk position i.  Eight waves: waves 0-3 and 4-7 (the two
// halves) own the same four 32-row groups and split the key tiles between
// them (tiles 0, 2, 4, ... and 1, 3, 5, ...); the two partial softmax states
// are merged through LDS at the end.  When the blocks tile the rows exactly,
// a block's four groups are two from the front of the chunk and their mirror
// images from the back, which evens out the blocks' work: with contiguous
// groups the last block of a 1k chunk sees 1024 more chunk keys than the
// first, and a launch of one round of blocks lasts as long as its slowest.
//
// Staging.  K and V tiles go from global memory straight into LDS (buffer
// loads with the LDS destination, 16 bytes per lane, lane-linear in LDS), so
// no registers hold tiles in flight.  Rows are stored unpadded with their
// 16-byte chunks XOR-swizzled by row: the lane that fills LDS chunk c of row r
// fetches global chunk c ^ swz(r).  The swizzles keep the MFMA operand reads
// free of bank conflicts.  V stays row-major and is read transposed by
// ds_read_b64_tr_b16: a 16-lane group addresses four rows of four consecutive
// bf16 and lane j receives column j%4 of rows j/4, j/4+4, j/4+8, j/4+12, i.e.
// four keys of one d, which are the k-slots of the V^T operand.
//
// Pipeline.  Each half has two K buffers and two V buffers.  Iteration j of a
// half starts the loads of K(j+2) and V(j+1), then computes S(j+1) = K Q^T by
// MFMA while the exponentials of tile j run on the VALU, then O += V(j)^T P(j)^T,
// then waits for its loads and meets the other waves at one barrier.
// ---------------------------------------------------------------------------
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;

template <int D>
struct AttnTile {
    static constexpr int RB = 2 * D;                    // bytes per K / V row
    static constexpr int U16 = kKeysPerTile * D;        // u16 per tile
    static constexpr int LOADS = kKeysPerTile * RB / 1024 / 4;   // 1 KB loads per wave per tile
};


typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Loads that write LDS are counted by vmcnt; the compiler only tracks them as
// this wave's own writes, so before a barrier that publishes them to the other
// waves each wave waits for all of its own (s_waitcnt vmcnt(0); expcnt and
// lgkmcnt left at their maximum in the gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;
__device__ __forceinline__ void publish_lds_loads() {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
}

__device__ __forceinline__ void load_lds16(Rsrc r, void* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void load_lds4(Rsrc r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}
// Eight bf16 of the V^T operand: two transposing reads, four rows apart.
__device__ __forceinline__ bf16x8 ld_vt(const unsigned char* p, int row_bytes4) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + row_bytes4));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_bf16_kernel(ChunkArgs a) {
    using T = AttnTile<D>;
    constexpr int KS = D / 16;                    // MFMA k-steps over head_dim
    constexpr int DT = D / 32;                    // 32-row tiles of O^T
    constexpr int RB = T::RB;
    // Stage s of half h: sK<s>[h], sV<s>[h].
    // Separate objects per stage let the compiler see that loads into one stage
    // never alias reads of the other.
    __shared__ __attribute__((aligned(1024))) u16 sK0[2][T::U16];
    __shared__ __attribute__((aligned(1024))) u16 sK1[2][T::U16];
    __shared__ __attribute__((aligned(1024))) u16 sV0[2][T::U16];
    __shared__ __attribute__((aligned(1024))) u16 sV1[2][T::U16];
    // Positions t(j) of the cache tile in each K stage, [stage][half][key].
    __shared__ __attribute__((aligned(256))) int sPos[2][2][kKeysPerTile];

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
    // Row-group slot rw: the second half takes the slots in the order 2, 3, 0, 1,
    // so waves w and w + 4, which share a SIMD, hold one front and one back row
    // group (with both halves in slot order the balanced rows gained nothing).
    const int kh = wave >> 2, rw = (wave & 3) ^ (2 * kh);
    const int lq = lane & 31, hh = lane >> 5;
    const int g16 = lane >> 4, j16 = lane & 15;
    // Row group (32 packed rows) of slot rw.  When the blocks tile the rows
    // exactly, block rb takes groups 2rb, 2rb+1 from the front of the chunk and
    // their mirror images from the back.  A chunk key is visible to the rows at
    // or after its position, so a block's front groups see few chunk tiles and
    // its back groups many; the front groups' waves skip the tiles they cannot
    // see, and their SIMD partners run those alone.
    const int nrg = (R + 31) / 32;
    const bool mirror = R % kRowsPerBlock == 0;
    auto group_of = [&](int slot) {
        if (!mirror) return rb * 4 + slot;
        return slot < 2 ? 2 * rb + slot : nrg - 4 + slot - 2 * rb;
    };
    const int row = group_of(rw) * 32 + lq;
    const bool row_ok = row < R;
    const int i = row_ok ? row / a.G : a.S - 1;
    const int h = g * a.G + (row_ok ? row % a.G : 0);

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
    // Key tiles of the block (what its last row sees; group_of(3) holds it) and
    // of this wave's own rows.  A half loads tiles kh, kh+2, ... of the block's
    // range; a wave computes those within its own range (the rest are masked
    // in full for its rows and would add nothing).
    const int last_row = min(R - 1, group_of(3) * 32 + 31);
    const int ntiles = cache_tiles + (last_row / a.G) / kKeysPerTile + 1;
    const int steps = (ntiles + 1) / 2;
    const int mine = (ntiles - kh + 1) / 2;       // tiles of this half: kh, kh+2, ...
    const int wave_row0 = min(R - 1, group_of(rw) * 32);
    const int wave_last = min(R - 1, group_of(rw) * 32 + 31);
    const int mine_c = (cache_tiles + (wave_last / a.G) / kKeysPerTile + 1 - kh + 1) / 2;
    const int qpos_wave_min = a.P + wave_row0 / a.G;

    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D;
    const u16* Vc = static_cast<const u16*>(a.vc) + (size_t)bg * a.NC * D;
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
    const u16* Vn = static_cast<const u16*>(a.vn) + (size_t)bg * S * D;

    // Global byte offset (within a tile) of this lane's 16-byte load `it`:
    // LDS chunk cp of row r is filled from global chunk cp ^ swz(r).
    auto goff = [&](int it, bool is_v) {
        const int off = (it * 4 + rw) * 1024 + 16 * lane;
        const int r = off / RB, cp = (off % RB) / 16;
        return r * RB + 16 * (cp ^ (is_v ? swz_v<D>(r) : swz_k<D>(r)));
    };
    // K tile jt of this half into stage st; a cache tile's positions go with it
    // (one 4-byte load per lane of the half's first wave).
    const int32_t* posg = a.pos + (size_t)bg * a.NC;
    auto issue_k = [&](int st, int jt) {
        const TileRef tr = tile_ref(2 * jt + kh, cache_tiles, n, S, D, Kc, Vc, Kn, Vn);
        const Rsrc rk = make_rsrc(tr.k, tr.valid * RB);
        unsigned char* d = reinterpret_cast<unsigned char*>(st ? sK1[kh] : sK0[kh]) + rw * 1024;
#pragma unroll
        for (int it = 0; it < T::LOADS; ++it) load_lds16(rk, d + it * 4096, goff(it, false), 0);
        if (tr.cache && rw == 0) load_lds4(make_rsrc(posg + tr.first, tr.valid * 4),
                                           &sPos[st][kh][0], 4 * lane);
    };
    auto issue_v = [&](u16* dst, int jt) {
        const TileRef tr = tile_ref(2 * jt + kh, cache_tiles, n, S, D, Kc, Vc, Kn, Vn);
        const Rsrc rv = make_rsrc(tr.v, tr.valid * RB);
        unsigned char* d = reinterpret_cast<unsigned char*>(dst) + rw * 1024;
#pragma unroll
        for (int it = 0; it < T::LOADS; ++it) load_lds16(rv, d + it * 4096, goff(it, true), 0);
    };

    // Operand offsets: K row perm_key(lq) (+32 per sub-tile), k-step ks at
    // kb ^ 32*ks; V^T rows 8*hh + j16/4 (+16*s2, +32*sub, +4 for the second
    // read), d block dt at vb ^ 64*dt.
    const int prow = perm_key(lq);
    const int kb = prow * RB + 16 * (hh ^ swz_k<D>(prow));
    const int vrow = 8 * hh + (j16 >> 2);
    const int vb = vrow * RB + 16 * ((2 * (g16 & 1) + ((j16 & 3) >> 1)) ^ swz_v<D>(vrow)) +
                   8 * (j16 & 1);

    const float c = a.sm_scale * kLog2e;          // logits -> log2 units
    const float tau_raw = kRescaleLog2 / c;
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // S^T = K Q^T of the tile in sKt.
    auto qk = [&](const u16* sKt, f32x16 (&sd)[2]) {
        const unsigned char* base = reinterpret_cast<const unsigned char*>(sKt);
        sd[0] = f32x16{};
        sd[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
                sd[sub] = mfma32(as_bf16x8(ld16(base + ((kb ^ (32 * ks)) + sub * 32 * RB))),
                                 qf[ks], sd[sub]);
    };
    // Visibility: key j is visible to row i iff 0 <= t(j) <= P + i.  Chunk key
    // i' sits at P + i', so it is visible iff i' <= i.  A filled cache slot
    // normally holds an earlier token, 0 <= t(j) < P, visible to every row:
    // within tile jt, key k is then visible to this lane's row iff k <= lim(jt).
    // Tiles whose keys are all visible to every row of the wave skip the mask;
    // cache slots outside [0, P) take the positional mask below.
    auto tile_lim = [&](int jt) {
        const TileRef tr = tile_ref(2 * jt + kh, cache_tiles, n, S, D, Kc, Vc, Kn, Vn);
        return tr.cache ? tr.valid - 1 : min(tr.valid - 1, i - tr.first);
    };
    auto tile_all_visible = [&](int jt) {
        const TileRef tr = tile_ref(2 * jt + kh, cache_tiles, n, S, D, Kc, Vc, Kn, Vn);
        return tr.valid == kKeysPerTile &&
               (tr.cache || tr.first + kKeysPerTile - 1 <= qpos_wave_min - a.P);
    };
    // Buffer form: bits of the tile's slots that the chunk overwrites (cache
    // tiles only; those slots are not keys).
    const uint64_t* exrow = a.excl ? a.excl + (size_t)bg * excl_tiles(a.NC) : nullptr;
    auto tile_excl = [&](int jt) -> uint64_t {
        const int tile = 2 * jt + kh;
        return (exrow != nullptr && tile < cache_tiles) ? exrow[tile] : 0ull;
    };
    // -inf for this lane's keys k > lim and for excluded slots (the lane holds
    // keys 32*sub + 16*(r/8) + 8*hh + r%8 of the tile: bytes 4*sub + 2*(r/8) +
    // hh of the tile's bits, gathered by one byte permute into bit 16*sub + r).
    auto apply_mask = [&](f32x16 (&sv)[2], int lim, uint64_t ex) {
        const int d = lim - 8 * hh;
        const uint32_t lb = __builtin_amdgcn_perm((uint32_t)(ex >> 32), (uint32_t)ex,
                                                  hh ? 0x07050301u : 0x06040200u);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (sub * 32 + 16 * (r >> 3) + (r & 7) > d || ((lb >> (16 * sub + r)) & 1u))
                    sv[sub][r] = -INFINITY;
    };
    // Bits of the cache tile's keys (in stage st) whose position lies outside
    // [0, P): a filled slot marked empty (never visible) or holding a token at
    // or after the chunk start (visible from that position on).  A cache built
    // by this library's insertions has none; the test costs one LDS read and a
    // ballot per tile.
    auto tile_irregular = [&](int jt, int st) -> uint64_t {
        const TileRef tr = tile_ref(2 * jt + kh, cache_tiles, n, S, D, Kc, Vc, Kn, Vn);
        if (!tr.cache) return 0ull;
        const int tp = sPos[st][kh][lane];
        return __ballot(lane < tr.valid && (tp < 0 || tp >= a.P));
    };
    // -inf for this lane's cache keys with t < 0 or t > P + i (the lane holds keys
    // 32*sub + 16*(r/8) + 8*hh + r%8 of the tile).
    auto apply_pos_mask = [&](f32x16 (&sv)[2], int st) {
        const int qpos = a.P + i;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tp = sPos[st][kh][32 * sub + 16 * (r >> 3) + 8 * hh + (r & 7)];
                if (tp < 0 || tp > qpos) sv[sub][r] = -INFINITY;
            }
    };
    // Row max over both lane halves, running-max update and (rarely) the
    // rescale of O and l; returns m_run * c for the exponentials.
    auto rescale_for = [&](float mt) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                         __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
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
        return (m_run == -INFINITY) ? 0.f : m_run * c;
    };
    auto rowmax = [&](const f32x16 (&sv)[2]) {
        float m4[4] = {sv[0][0], sv[0][1], sv[0][2], sv[0][3]};
#pragma unroll
        for (int idx = 4; idx < 32; ++idx) m4[idx & 3] = fmaxf(m4[idx & 3], sv[idx >> 4][idx & 15]);
        return fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    };

    // O^T += V^T P^T for the tile in sVt, operands read two MFMAs ahead,
    // interleaved with the running max of the next tile's scores (sn).
    // The MFMAs of the first 32 keys (sub-tile 0, whose P is complete) also carry
    // the last 8 exponentials of each lane (keys 48..63 of this tile), the ones
    // of sub-tile 1 the maxima of the next tile, so both phases of an iteration
    // hold VALU work under their MFMAs.
    auto pv_max = [&](const u16* sVt, bf16x8 (&pb)[2][2], const f32x16 (&sc)[2],
                      const f32x16 (&sn)[2], float mcv, float& lsum) {
        const unsigned char* base = reinterpret_cast<const unsigned char*>(sVt);
        auto vread = [&](int x) {
            const int dt = x % DT, s2 = (x / DT) & 1, sub = x / (2 * DT);
            return ld_vt(base + (vb ^ (64 * dt)) + (sub * 32 + 16 * s2) * RB, 4 * RB);
        };
        constexpr int NX = 4 * DT;
        constexpr int HX = 2 * DT;                // MFMAs of one sub-tile
        constexpr int AHEAD = 2;
        float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        float p[8];
        bf16x8 va[AHEAD + 1];
#pragma unroll
        for (int x = 0; x < AHEAD; ++x) va[x] = vread(x);
#pragma unroll
        for (int x = 0; x < NX; ++x) {
            if (x + AHEAD < NX) va[(x + AHEAD) % (AHEAD + 1)] = vread(x + AHEAD);
            const int dt = x % DT, s2 = (x / DT) & 1, sub = x / (2 * DT);
            o[dt] = mfma32(va[x % (AHEAD + 1)], pb[sub][s2], o[dt]);
            if (x < HX) {
#pragma unroll
                for (int e = 8 * x / HX; e < 8 * (x + 1) / HX; ++e) {
                    p[e] = fast_exp2(fmaf(sc[1][8 + e], c, -mcv));
                    lsum += p[e];
                }
                if (x == HX - 1)
                    pb[1][1] = as_bf16x8(u32x4{pack2(p[0], p[1]), pack2(p[2], p[3]),
                                               pack2(p[4], p[5]), pack2(p[6], p[7])});
            } else {
#pragma unroll
                for (int idx = 32 * (x - HX) / HX; idx < 32 * (x - HX + 1) / HX; ++idx)
                    m4[idx & 3] = fmaxf(m4[idx & 3], sn[idx >> 4][idx & 15]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        return fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    };

    // Prologue: K(0), V(0), K(1) of this half; S(0), its mask, max and
    // exponent offset.
    f32x16 sA[2], sB[2];
    float mc = 0.f;
    if (mine > 0) {
        issue_k(0, 0);
        issue_v(sV0[kh], 0);
    }
    if (mine > 1) issue_k(1, 1);
    publish_lds_loads();
    if (mine_c > 0) {
        qk(sK0[kh], sA);
        const uint64_t ex0 = tile_excl(0);
        if (!tile_all_visible(0) || ex0 != 0) apply_mask(sA, tile_lim(0), ex0);
        if (tile_irregular(0, 0) != 0) apply_pos_mask(sA, 0);
        mc = rescale_for(rowmax(sA));
    }
    // Iteration 0 loads K(2) into K(0)'s buffer: every wave must be done
    // reading K(0) first.  (The reads have completed once their MFMAs issued.)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // Iteration jt: S(jt) is masked and mc is its exponent offset; K stage
    // jt&1 is free (K(jt) was consumed), K stage (jt+1)&1 holds K(jt+1), V
    // stage jt&1 holds V(jt).
    auto iter = [&](auto odd_c, int jt, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
        constexpr bool odd = decltype(odd_c)::value;
        constexpr int st_free = odd ? 1 : 0;      // K stage of tile jt (consumed)
        constexpr int st_next = odd ? 0 : 1;      // K stage of tile jt+1
        const u16* knext = odd ? sK0[kh] : sK1[kh];
        const u16* vcur = odd ? sV1[kh] : sV0[kh];
        u16* vnext = odd ? sV0[kh] : sV1[kh];
        if (jt + 2 < mine) issue_k(st_free, jt + 2);
        if (jt + 1 < mine) issue_v(vnext, jt + 1);
        if (jt < mine_c) {
            const bool has_next = jt + 1 < mine_c;
            bf16x8 pb[2][2];
            float lsum = 0.f;
            // Phase A: QK^T of the next tile interleaved with this tile's
            // exponentials, in source order (each k-step: read the next K
            // fragments, two MFMAs, a slice of the exponentials).  On the
            // half's last tile the next buffer holds stale data (in bounds)
            // and the result is unused.
            const unsigned char* kbase = reinterpret_cast<const unsigned char*>(knext);
            auto kread = [&](int ks, int sub) {
                return as_bf16x8(ld16(kbase + ((kb ^ (32 * ks)) + sub * 32 * RB)));
            };
            constexpr int NEA = 24;               // exponentials in this phase (of 32)
            // K fragments are read two k-steps ahead of their MFMAs (one ahead:
            // 147.2 against 146.4 us per steady chunk).
            bf16x8 kr[3][2];
            kr[0][0] = kread(0, 0);
            kr[0][1] = kread(0, 1);
            kr[1][0] = kread(1, 0);
            kr[1][1] = kread(1, 1);
            snext[0] = f32x16{};
            snext[1] = f32x16{};
            float p[8];
            // Raised wave priority in this phase: the two waves of a SIMD run in
            // lockstep, and favouring the one in its QK^T phase keeps the MFMA
            // pipe fed (140 -> 138 us; the same in the P V phase: no change).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 2 < KS) {
                    kr[(ks + 2) % 3][0] = kread(ks + 2, 0);
                    kr[(ks + 2) % 3][1] = kread(ks + 2, 1);
                }
                snext[0] = mfma32(kr[ks % 3][0], qf[ks], snext[0]);
                snext[1] = mfma32(kr[ks % 3][1], qf[ks], snext[1]);
#pragma unroll
                for (int idx = ks * NEA / KS; idx < (ks + 1) * NEA / KS; ++idx) {
                    const int q4 = idx >> 3, ee = idx & 7;
                    p[ee] = fast_exp2(fmaf(scur[q4 >> 1][8 * (q4 & 1) + ee], c, -mc));
                    lsum += p[ee];
                    if (ee == 7)
                        pb[q4 >> 1][q4 & 1] =
                            as_bf16x8(u32x4{pack2(p[0], p[1]), pack2(p[2], p[3]),
                                            pack2(p[4], p[5]), pack2(p[6], p[7])});
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
            // Keep the exponentials here: their only uses come after a branch
            // and would otherwise be sunk past it, out of the MFMA stream.
#pragma unroll
            for (int q4 = 0; q4 < 3; ++q4)
                asm volatile("" : : "v"(__builtin_bit_cast(u32x4, pb[q4 >> 1][q4 & 1])));
            asm volatile("" : : "v"(lsum));
            // The next tile's mask (rare: partial or diagonal tiles).
            if (has_next) {
                const uint64_t exn = tile_excl(jt + 1);
                if (!tile_all_visible(jt + 1) || exn != 0) apply_mask(snext, tile_lim(jt + 1), exn);
                if (tile_irregular(jt + 1, st_next) != 0) apply_pos_mask(snext, st_next);
            }
            // Phase B: P V of this tile with the next tile's row max.
            const float mt = pv_max(vcur, pb, scur, snext, mc, lsum);
            asm volatile("" : : "v"(mt));         // keep the maxima under the MFMAs
            l_run += lsum;
            if (has_next) mc = rescale_for(mt);
        }
        publish_lds_loads();
    };
    for (int jt = 0; jt < steps; jt += 2) {
        iter(std::false_type{}, jt, sA, sB);
        if (jt + 1 < steps) iter(std::true_type{}, jt + 1, sB, sA);
    }

    // Merge the two halves' (m, l, O) for each row; the tile buffers are free
    // (the loop ended on a barrier with no loads in flight).
    auto mo = [&](int dt, int r) -> float& {
        float* reg = reinterpret_cast<float*>(dt < DT / 2 ? &sK0[0][0] : &sK1[0][0]);
        return reg[((rw * (DT / 2) + dt % (DT / 2)) * 16 + r) * 64 + lane];
    };
    float* ml = reinterpret_cast<float*>(&sV0[0][0]) + rw * 128;
    if (kh == 1) {
        ml[lane] = m_run;
        ml[64 + lane] = l_run;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mo(dt, r) = o[dt][r];
    }
    __syncthreads();
    if (kh == 1) return;
    {
        const float m1 = ml[lane], l1 = ml[64 + lane];
        const float m = fmaxf(m_run, m1);
        const float a0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m) * c);
        const float a1 = m1 == -INFINITY ? 0.f : fast_exp2((m1 - m) * c);
        l_run = l_run * a0 + l1 * a1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * a0 + mo(dt, r) * a1;
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
// query row of the group (G heads x S positions).  Each wave holds kColsumKB
// blocks of 32 keys (one: at two, each Q fragment read from LDS feeds two
// MFMAs, but the 2 waves per SIMD that the registers then allow ran slower
// than 3 or 4 waves with one block).  K stays in registers; Q and
// LSE tiles of 64 packed rows (row r = i*G + head) go from global memory
// straight into double-buffered LDS, Q rows XOR-swizzled like the attention
// pass's K.  Each lane accumulates its 16 keys over its query column, and the
// 32 columns are added in a fixed order at the end, so the result is
// deterministic (no atomics).  Key blocks follow the same cache / chunk split
// as the attention tiles.  A filled cache slot normally holds an earlier token
// (0 <= t(j) < P), visible to every row; a chunk key is visible to the rows at
// or after its own position, which only blocks near the diagonal have to test.
// A wave whose cache keys include a slot outside [0, P) tests every row tile
// against the positions (visible iff 0 <= t(j) <= P + i).
//
// Load balance: a key block's work is every row tile after its first visible
// one; with few blocks per CU, whole blocks leave CUs idle at the end (576
// blocks on 768 resident slots at chunk 1k / 8192 slots).  The row tiles are
// then split into `parts` contiguous ranges, one workgroup each, whose fp32
// partial sums go to the workspace and are added in part order by
// colsum_reduce_kernel, so the result does not depend on timing.
//
// Pipeline, per row tile rt (stage buffer (rt - t_lo) & 1):
//   A: MFMAs of sub-tile 1 of tile rt, exponentials of sub-tile 0 of tile rt;
//   barrier (tile rt+1 has landed; tile rt's buffer is free);
//   B: start the loads of tile rt+2; MFMAs of sub-tile 0 of tile rt+1,
//      exponentials of sub-tile 1 of tile rt.
// ---------------------------------------------------------------------------
template <int D, bool EVEN_ROWS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kColsumKB == 1 ? 4 : 2)))
void colsum_bf16_kernel(ChunkArgs a, uint32_t g_magic, int parts, float* __restrict__ part_ws) {
    constexpr int KS = D / 16;
    constexpr int RB = 2 * D;                          // bytes per Q row
    constexpr int QT = kRowsPerTile * RB;              // bytes per Q tile
    constexpr int QLOADS = QT / 1024 / kWaves;         // 1 KB loads per wave per tile
    static_assert(QLOADS >= 1, "tile shape");
    // Two separate Q tile buffers (as slices of one array the compiler could not
    // tell a tile load into one from a read of the other, and waited for the load).
    // After the loop their bytes hold the per-wave key sums -- waves 0 and 1 in
    // sQ0, 2 and 3 in sQ1 -- which keeps a workgroup at 33 KB of LDS: four fit on
    // a CU, and at 126 VGPRs so do their 16 waves.
    __shared__ __attribute__((aligned(1024))) unsigned char sQ0[QT];
    __shared__ __attribute__((aligned(1024))) unsigned char sQ1[QT];
    constexpr int RED_WAVE = 32 * kColsumKB * 33;       // floats of one wave's key sums
    constexpr bool RED_IN_Q = 2 * RED_WAVE * (int)sizeof(float) <= QT;
    __shared__ float sRedOwn[RED_IN_Q ? 1 : kWaves * RED_WAVE];
    __shared__ __attribute__((aligned(16))) float sL0[kRowsPerTile];
    __shared__ __attribute__((aligned(16))) float sL1[kRowsPerTile];
    constexpr int KB = kColsumKB;

    const int n = a.n, S = a.S, G = a.G;
    const int cache_blocks = (n + kKeysPerBlock - 1) / kKeysPerBlock;
    const int nkb = cache_blocks + (S + kKeysPerBlock - 1) / kKeysPerBlock;
    const int total = nkb * a.B * a.Hkv * parts;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    // Consecutive tiles: key blocks of one (b, g, part), which read the same Q rows.
    const int kb = t % nkb, part = (t / nkb) % parts, bg = t / nkb / parts;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const bool is_cache = kb < cache_blocks;
    const int block_first = (is_cache ? kb : kb - cache_blocks) * kKeysPerBlock;
    const int limit = is_cache ? n : S;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int first = block_first + wave * 32 * KB;    // this wave's first key in its source

    const u16* Ksrc = is_cache ? static_cast<const u16*>(a.kc) + (size_t)bg * a.NC * D
                               : static_cast<const u16*>(a.kn) + (size_t)bg * S * D;
    bf16x8 kf[KB][KS];
#pragma unroll
    for (int kbl = 0; kbl < KB; ++kbl) {
        const int idx = first + 32 * kbl + lq;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (idx < limit) v = ld16(Ksrc + (size_t)idx * D + 16 * ks + 8 * hh);
            kf[kbl][ks] = as_bf16x8(v);
        }
    }

    // Positions of this wave's cache keys; irr: some lie outside [0, P) (none in a
    // cache built by this library's insertions).
    int tpos[KB];
    bool irr_lane = false;
#pragma unroll
    for (int kbl = 0; kbl < KB; ++kbl) {
        const int idx = first + 32 * kbl + lq;
        tpos[kbl] = (is_cache && idx < limit) ? a.pos[(size_t)bg * a.NC + idx] : 0;
        irr_lane |= tpos[kbl] < 0 || tpos[kbl] >= a.P;
    }
    const bool irr = __ballot(irr_lane) != 0;

    const int R = G * S;
    const int ntile = (R + kRowsPerTile - 1) / kRowsPerTile;
    // Chunk keys are invisible to the rows before their own position.
    const int tile0 = is_cache ? 0 : (block_first * G) / kRowsPerTile;
    // This workgroup's row tiles [t_lo, t_hi).
    const int per_part = (ntile + parts - 1) / parts;
    const int t_lo = max(tile0, part * per_part), t_hi = min(ntile, (part + 1) * per_part);
    // Where this wave's 32 sums go: the output, or this part's workspace row.
    float* dst = parts == 1
        ? (is_cache ? a.cs_cache + (size_t)bg * a.NC : a.cs_new + (size_t)bg * S)
        : part_ws + ((size_t)part * a.B * a.Hkv + bg) * (a.NC + S) + (is_cache ? 0 : a.NC);
    if (t_lo >= t_hi) {                    // no visible row in this range
        if (lane < 32 * KB && first + lane < limit) dst[first + lane] = 0.f;
        return;
    }

    // The G query heads of KV head g are contiguous in Q and in LSE.
    const u16* Qg = static_cast<const u16*>(a.q) + (size_t)(b * a.Hq + g * G) * S * D;
    const float* Lg = a.lse + (size_t)(b * a.Hq + g * G) * S;
    const int q_bytes = G * S * D * 2;
    // Packed row r of the group -> byte offset of its Q row / LSE entry, or
    // past the end for r >= R (the loads then return zeros).
    auto row_split = [&](int r, int& hl, int& ipos) {
        ipos = G == 1 ? r : (int)__umulhi((uint32_t)r, g_magic);
        hl = r - ipos * G;
    };
    // This lane's 16-byte Q loads: load `it` fills LDS bytes
    // (it*4 + wave)*1024 + 16*lane = row rl, chunk cp, from global chunk
    // cp ^ swz(rl) of that row.
    const int rl_base = (wave * 1024 + 16 * lane) / RB;
    const int cp = (16 * lane % RB) / 16;
    constexpr int ROWS_PER_LOAD = 4096 / RB;           // rows between loads it and it+1
    int qoff[QLOADS];
#pragma unroll
    for (int it = 0; it < QLOADS; ++it) {
        const int rl = rl_base + it * ROWS_PER_LOAD;
        const int sw = D == 128 ? (rl & 15) : ((rl >> 1) & 7);
        int hl = 0, il = 0;
        if (EVEN_ROWS) {
            hl = rl % G;
            il = rl / G;
        }
        qoff[it] = ((hl * S + il) * D) * 2 + 16 * (cp ^ sw);
    }
    const int ppt = EVEN_ROWS ? kRowsPerTile / G : 0;  // positions per tile (EVEN_ROWS)
    auto issue = [&](unsigned char* dq, float* dl, int rt) {
        if (EVEN_ROWS) {
            const int p0 = rt * ppt;
            const Rsrc rq = make_rsrc(Qg + (size_t)p0 * D, max(0, q_bytes - p0 * D * 2));
            unsigned char* d = dq + wave * 1024;
#pragma unroll
            for (int it = 0; it < QLOADS; ++it) load_lds16(rq, d + it * 4096, qoff[it], 0);
        } else {
            const Rsrc rq = make_rsrc(Qg, q_bytes);
            unsigned char* d = dq + wave * 1024;
#pragma unroll
            for (int it = 0; it < QLOADS; ++it) {
                const int r = rt * kRowsPerTile + rl_base + it * ROWS_PER_LOAD;
                const int rl = rl_base + it * ROWS_PER_LOAD;
                const int sw = D == 128 ? (rl & 15) : ((rl >> 1) & 7);
                int hl = 0, ipos = 0;
                row_split(min(r, R - 1), hl, ipos);
                const int off = r < R ? ((hl * S + ipos) * D) * 2 + 16 * (cp ^ sw) : q_bytes;
                load_lds16(rq, d + it * 4096, off, 0);
            }
        }
        if (wave == 0) {
            const int r = rt * kRowsPerTile + lane;
            int hl = 0, ipos = 0;
            row_split(min(r, R - 1), hl, ipos);
            const Rsrc rl = make_rsrc(Lg, G * S * 4);
            load_lds4(rl, dl, r < R ? (hl * S + ipos) * 4 : G * S * 4);
        }
    };

    const float c = a.sm_scale * kLog2e;
    float acc[KB][16];
#pragma unroll
    for (int kbl = 0; kbl < KB; ++kbl)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kbl][r] = 0.f;

    // Q operand of query row lq of sub-tile `sub`, k-step ks: chunk 2*ks + hh
    // of that row, swizzled.
    const int qb = lq * RB + 16 * (hh ^ (D == 128 ? (lq & 15) : ((lq >> 1) & 7)));
    auto qread = [&](const unsigned char* sQt, int sub, int ks) {
        return as_bf16x8(ld16(sQt + ((qb ^ (32 * ks)) + sub * 32 * RB)));
    };
    // log2-scaled LSE of this lane's query row (+inf past the last row, which
    // makes its weights zero).
    auto lse2_of = [&](const float* sLt, int rt, int sub) {
        const int r = rt * kRowsPerTile + sub * 32 + lq;
        const float v = sLt[sub * 32 + lq];            // in bounds for every lane
        return r < R ? v * kLog2e : INFINITY;
    };
    // Chunk key blocks near the diagonal: is every key of this wave visible
    // to every row of sub-tile (rt, sub)?
    const int kmax = min(first + 32 * KB - 1, limit - 1);   // largest key index of the wave
    auto full_tile = [&](int rt, int sub) {
        if (is_cache) return !irr;
        const int r0 = min(rt * kRowsPerTile + sub * 32, R - 1);
        const int i0 = G == 1 ? r0 : (int)__umulhi((uint32_t)r0, g_magic);
        return kmax <= i0;
    };
    // Exponentials of sub-tile values sv (lse2 of this lane's row) into acc,
    // with the causal test when the tile is not fully visible.
    auto exp_masked = [&](const f32x16 (&sv)[KB], float lse2, int rt, int sub)
        __attribute__((always_inline)) {
        const int r = min(rt * kRowsPerTile + sub * 32 + lq, R - 1);
        const int ipos = G == 1 ? r : (int)__umulhi((uint32_t)r, g_magic);
        if (is_cache) {
            // Cache keys with positions outside [0, P): the lane's key
            // 8*(e/4) + 4*hh + e%4 of each block has its position in lane
            // (that key) of tpos.
            const int qpos = a.P + ipos;
#pragma unroll
            for (int kbl = 0; kbl < KB; ++kbl)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int tk = __shfl(tpos[kbl], 8 * (e >> 2) + 4 * hh + (e & 3));
                    const float p = fast_exp2(fmaf(sv[kbl][e], c, -lse2));
                    acc[kbl][e] += (tk >= 0 && tk <= qpos) ? p : 0.f;
                }
            return;
        }
        // key first + 4*hh + off is visible iff off <= dlim
        const int dlim = ipos - first - 4 * hh;
#pragma unroll
        for (int kbl = 0; kbl < KB; ++kbl)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(fmaf(sv[kbl][e], c, -lse2));
                acc[kbl][e] += 32 * kbl + 8 * (e >> 2) + (e & 3) <= dlim ? p : 0.f;
            }
    };

    // One stage: 8 MFMAs of (sQm, subm) into the result, interleaved with the
    // exponentials of sv (fully visible) or followed by the masked form.
    // Each Q fragment read from LDS feeds KB MFMAs, one per 32-key block.
    auto stage = [&](auto mfma_c, const unsigned char* sQm, int subm, const f32x16 (&sv)[KB],
                     float lse2, bool full, int rt_e, int sub_e, f32x16 (&r)[KB])
        __attribute__((always_inline)) {
        constexpr bool do_mfma = decltype(mfma_c)::value;
        constexpr int PER = 16 * KB / KS;                 // exponentials per k-step
#pragma unroll
        for (int kbl = 0; kbl < KB; ++kbl) r[kbl] = f32x16{};
        if (full) {
            // Q fragments are read two k-steps ahead of their MFMA (one ahead
            // left the LDS latency exposed: 89 us against 87 us per chunk).
            constexpr int QA = 2;
            bf16x8 qr[QA + 1];
            if (do_mfma) {
#pragma unroll
                for (int j = 0; j < QA; ++j) qr[j] = qread(sQm, subm, j);
            }
            // Each exponential is added one k-step later, off its latency (the
            // same additions in the same order: 87.1 -> 85.8 us per steady chunk).
            float pend[PER];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (do_mfma) {
                    if (ks + QA < KS) qr[(ks + QA) % (QA + 1)] = qread(sQm, subm, ks + QA);
#pragma unroll
                    for (int kbl = 0; kbl < KB; ++kbl)
                        r[kbl] = mfma32(kf[kbl][ks], qr[ks % (QA + 1)], r[kbl]);
                }
#pragma unroll
                for (int e = 0; e < PER; ++e) {
                    const int x = ks * PER + e;
                    const float p = fast_exp2(fmaf(sv[x >> 4][x & 15], c, -lse2));
                    if (ks > 0) {
                        const int xp = x - PER;
                        acc[xp >> 4][xp & 15] += pend[e];
                    }
                    pend[e] = p;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int xp = (KS - 1) * PER + e;
                acc[xp >> 4][xp & 15] += pend[e];
            }
        } else {
            if (do_mfma) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 q = qread(sQm, subm, ks);
#pragma unroll
                    for (int kbl = 0; kbl < KB; ++kbl) r[kbl] = mfma32(kf[kbl][ks], q, r[kbl]);
                }
            }
            exp_masked(sv, lse2, rt_e, sub_e);
        }
    };

    // Prologue: tiles t_lo and t_lo+1; S of (t_lo, sub 0).
    issue(sQ0, sL0, t_lo);
    if (t_lo + 1 < t_hi) issue(sQ1, sL1, t_lo + 1);
    publish_lds_loads();
    f32x16 s0[KB], s1[KB];
#pragma unroll
    for (int kbl = 0; kbl < KB; ++kbl) s0[kbl] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 q = qread(sQ0, 0, ks);
#pragma unroll
        for (int kbl = 0; kbl < KB; ++kbl) s0[kbl] = mfma32(kf[kbl][ks], q, s0[kbl]);
    }

    auto step = [&](auto odd_c, int rt) __attribute__((always_inline)) {
        constexpr bool odd = decltype(odd_c)::value;      // (rt - t_lo) & 1
        unsigned char* qc = odd ? sQ1 : sQ0;              // tile rt
        unsigned char* qn = odd ? sQ0 : sQ1;              // tile rt+1
        float* lc = odd ? sL1 : sL0;
        float* ln = odd ? sL0 : sL1;
        const bool has_next = rt + 1 < t_hi;
        const float l0 = lse2_of(lc, rt, 0), l1 = lse2_of(lc, rt, 1);
        // A: MFMAs of (rt, 1) with the exponentials of (rt, 0), at raised wave
        // priority (81.7 -> 81.1 us).
        __builtin_amdgcn_s_setprio(1);
        stage(std::true_type{}, qc, 1, s0, l0, full_tile(rt, 0), rt, 0, s1);
        __builtin_amdgcn_s_setprio(0);
        publish_lds_loads();
        // B: loads of tile rt+2 into tile rt's buffer; MFMAs of (rt+1, 0) with
        // the exponentials of (rt, 1).
        if (rt + 2 < t_hi) issue(qc, lc, rt + 2);
        // (the MFMA flag is a template argument: as a runtime flag it split the
        // MFMAs into conditional blocks ahead of all the exponentials)
        if (has_next) stage(std::true_type{}, qn, 0, s1, l1, full_tile(rt, 1), rt, 1, s0);
        else stage(std::false_type{}, qn, 0, s1, l1, full_tile(rt, 1), rt, 1, s0);
        (void)ln;
    };
    for (int rt = t_lo; rt < t_hi; rt += 2) {
        step(std::false_type{}, rt);
        if (rt + 1 < t_hi) step(std::true_type{}, rt + 1);
    }
    publish_lds_loads();

    float* const red = RED_IN_Q ? reinterpret_cast<float*>((wave < 2 ? sQ0 : sQ1) +
                                                          (wave & 1) * RED_WAVE * sizeof(float))
                                : sRedOwn + wave * RED_WAVE;
#pragma unroll
    for (int kbl = 0; kbl < KB; ++kbl)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            red[(32 * kbl + 8 * (r >> 2) + 4 * hh + (r & 3)) * 33 + lq] = acc[kbl][r];
    __syncthreads();
    if (lane < 32 * KB) {
        float sum = 0.f;
#pragma unroll 8
        for (int j = 0; j < 32; ++j) sum += red[lane * 33 + j];
        const int idx = first + lane;
        // Buffer form: a slot the chunk overwrites is not a key (weight 0).
        if (idx < limit) {
            const bool ex = is_cache && a.excl != nullptr &&
                            ((a.excl[(size_t)bg * excl_tiles(a.NC) + idx / 64] >> (idx % 64)) & 1);
            dst[idx] = ex ? 0.f : sum;
        }
    }
}

// Sum of the parts' partial column sums, in part order; zero for the empty
// slots [n, N_C).  One (b, kv head) row of N_C + S entries per blockIdx.y.
__global__ __launch_bounds__(256) void colsum_reduce_kernel(ChunkArgs a, int parts,
                                                            const float* __restrict__ part_ws) {
    const int bg = blockIdx.y;
    const int row = a.NC + a.S;
    const size_t part_stride = (size_t)a.B * a.Hkv * row;
    const float* src = part_ws + (size_t)bg * row;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < row; j += gridDim.x * blockDim.x) {
        const bool empty = j >= a.n && j < a.NC;
        float sum = 0.f;
        if (!empty) {
            sum = src[j];
            for (int p = 1; p < parts; ++p) sum += src[p * part_stride + j];
        }
        if (j < a.NC) a.cs_cache[(size_t)bg * a.NC + j] = sum;
        else a.cs_new[(size_t)bg * a.S + (j - a.NC)] = sum;
    }
}

}  // namespace

template <int D>
hipError_t launch_attn_d(const ChunkArgs& a, hipStream_t s) {
    const int R = a.G * a.S;
    const int total = ((R + kRowsPerBlock - 1) / kRowsPerBlock) * a.B * a.Hkv;
    hipLaunchKernelGGL(attn_bf16_kernel<D>, dim3(xcd_grid(total)), dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attn_bf16(const ChunkArgs& a, hipStream_t s) {
    return a.D == 128 ? launch_attn_d<128>(a, s) : launch_attn_d<64>(a, s);
}

size_t colsum_workspace_bytes(int B, int Hkv, int NC, int S) {
    return (size_t)kColsumMaxParts * B * Hkv * (NC + S) * sizeof(float);
}

int colsum_parts(const ChunkArgs& a, int cus) {
    // Key blocks as whole units of work; 4 workgroups fit on a CU (2 with two key
    // blocks per wave).  Take the
    // split that needs the fewest rounds of resident workgroups, counted in
    // whole-block units (ties: the smaller split).
    const long long units = (long long)((a.n + kKeysPerBlock - 1) / kKeysPerBlock +
                                        (a.S + kKeysPerBlock - 1) / kKeysPerBlock) * a.B * a.Hkv;
    const long long slots = (kColsumKB == 1 ? 4LL : 2LL) * cus;
    int best = 1;
    double best_t = 1e30;
    for (int p = 1; p <= kColsumMaxParts; p *= 2) {
        const double rounds = (double)((units * p + slots - 1) / slots) / p;
        if (rounds < best_t - 1e-9) {
            best_t = rounds;
            best = p;
        }
    }
    return best;
}

hipError_t launch_colsum_bf16(const ChunkArgs& a, int parts, float* part_ws, hipStream_t s) {
    const int blocks = (a.n + kKeysPerBlock - 1) / kKeysPerBlock +
                       (a.S + kKeysPerBlock - 1) / kKeysPerBlock;
    const int total = blocks * a.B * a.Hkv * parts;
    // floor(r / G) = umulhi(r, ceil(2^32 / G)) for r * G < 2^32 (checked by the caller)
    const uint32_t magic = a.G > 1 ? (uint32_t)((0x100000000ull + a.G - 1) / a.G) : 0u;
    const dim3 grid(xcd_grid(total)), block(kThreads);
    const bool even = kRowsPerTile % a.G == 0;
    if (a.D == 128) {
        if (even) hipLaunchKernelGGL((colsum_bf16_kernel<128, true>), grid, block, 0, s, a, magic, parts, part_ws);
        else hipLaunchKernelGGL((colsum_bf16_kernel<128, false>), grid, block, 0, s, a, magic, parts, part_ws);
    } else {
        if (even) hipLaunchKernelGGL((colsum_bf16_kernel<64, true>), grid, block, 0, s, a, magic, parts, part_ws);
        else hipLaunchKernelGGL((colsum_bf16_kernel<64, false>), grid, block, 0, s, a, magic, parts, part_ws);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || parts == 1) return e;
    const int row = a.NC + a.S;
    int bx = (row + 255) / 256;
    if (bx > 256) bx = 256;
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3(bx, a.B * a.Hkv), dim3(256), 0, s, a, parts,
                       part_ws);
    return hipGetLastError();
}

}  // namespace h2o
