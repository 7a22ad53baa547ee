// Decode (S = 1) chunk attention for gfx950: split over cache slots.
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention",
// montaan paper page, "Kernel Support Needs" (summed attention weights and
// the implicit positional mask) specialised to one query token per sequence,
// the generation setting of the metallab summary's Table 7.  With one query
// row per head the pass is bound by reading the cache once.  One workgroup
// takes one (b, kv head, 4096-slot range); each of its 4 waves streams
// 32-slot tiles through a private LDS region (no workgroup barriers in the
// loop) and keeps an online-softmax state (m, l, O); the waves merge and the
// workgroup writes one partial per split.
//
//  decode_attn4_kernel  (at most four query heads per KV head) 4x4x4 MFMA
//      blocks put one slot per lane, so a wave holds the logits of all its
//      tiles in registers.  With summed weights and a grid that the device
//      holds at once, the splits of a (b, kv head) exchange (m, l) within
//      the launch, and each workgroup turns its held logits into summed
//      weights -- and, for a whole step (h2o_chunk_step), the score update,
//      the eviction keys and its (key, slot) minimum.  decode_merge_kernel
//      then forms O and LSE and inserts the new token.  Otherwise the held
//      logits go to the workspace in one burst after the loads.
//  decode_attn_kernel  (more heads per KV head) the G query heads are the
//      columns of 32x32x16 MFMAs; the logits go to the workspace tile by tile.
//  decode_finish_kernel  after either of the logit-writing forms: merges the
//      partials with the new token (its own key and value) into O and LSE,
//      turns the stored logits into summed weights, and for a whole step
//      adds them to the scores and reduces the eviction keys to one minimum
//      per range; decode_insert_kernel (one wave per (b, kv head)) takes the
//      minimum of those, the victim, and writes the new token into it.
//  (A hand-over inside one finishing kernel -- a device-scope fence per
//  finishing workgroup so that the last one could insert -- writes back its
//  XCD's L2 and measured 61 us against 22 us for the separate launches.)
//
// P V uses ds_read_b64_tr_b16: a 16-lane group addresses four rows of four
// consecutive bf16 (one key, four d each) and lane j receives column j%4 of
// the pieces addressed by lanes j/4, j/4+4, j/4+8, j/4+12, i.e. four keys of
// one d -- the k-slots of the MFMA operand V^T -- so V stays row-major in LDS.
#include "h2o_internal.h"
#include "device_common.h"

#include <hip/hip_bf16.h>

#include <climits>
#include <cmath>

namespace h2o {
namespace {

using namespace dev;

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecSub = 32;                 // slots per wave step
constexpr int kDecSplit = 4096;             // slots per workgroup
constexpr int kFinishKeys = 2048;           // slots per finishing workgroup

template <int D>
struct DecSmem {
    // K and V tiles are unpadded with XOR-swizzled 16-byte chunks (swz_k,
    // swz_v), which keeps two workgroups per CU.
    static constexpr int RB = 2 * D;        // bytes per K / V row
    static constexpr int K_BYTES = kDecSub * RB;
    static constexpr int V_BYTES = kDecSub * RB;
    static constexpr int WAVE_BYTES = K_BYTES + V_BYTES + kDecSub * 4;
    static constexpr int QROW = D + 8;      // Q^T operand rows (32 columns)
    static constexpr int Q_BYTES = 32 * QROW * 2;
    static constexpr int MERGE_FLOATS = 2 + (D / 32) * 16;
    static constexpr int MERGE_BYTES = kDecWaves * MERGE_FLOATS * 64 * 4;
    static constexpr int TILE_BYTES = kDecWaves * WAVE_BYTES + Q_BYTES;
    static constexpr int BYTES = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
};

struct DecodeWs {
    float* logits;      // [B*Hkv][G][NCP]  log2-unit logits, -inf where masked
    float* partial;     // [B*Hkv][nsplit][G][D + 2]  (m, l, O unnormalised)
    uint64_t* part_min; // [B*Hkv][nfin]  eviction: (key, slot) minimum per finish workgroup (split)
    uint64_t* xch;      // [B*Hkv][nsplit][4]  LSE exchange words of the fused kernel
    int nsplit;         // workgroups per (b, kv head) at full capacity
    int ncp;            // logit row length (capacity rounded up to kDecSub)
    int nfin;           // finish workgroups per (b, kv head) at full capacity
};

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

template <int D>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_attn_kernel(ChunkArgs a, DecodeWs ws, int nsplit_rt) {
    using L = DecSmem<D>;
    constexpr int KS = D / 16, DT = D / 32, RB = L::RB;
    constexpr int CH = D / 8;                              // 16-byte chunks per row
    constexpr int LD = kDecSub * CH / 64;                  // 16-byte loads per lane
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int total = nsplit_rt * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nsplit_rt, split = t % nsplit_rt;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.G, n = a.n, NC = a.NC;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int j16 = lane & 15, g16 = lane >> 4;

    // B operand: Q^T with the group's G heads as columns (zero beyond G), kept in
    // LDS (32 columns x D) and read per sub-tile rather than held in registers.
    const u16* Q = static_cast<const u16*>(a.q);
    u16* sQ = reinterpret_cast<u16*>(smem + kDecWaves * L::WAVE_BYTES);
    for (int idx = tid; idx < 32 * (D / 8); idx += kDecThreads) {
        const int col = idx / (D / 8), ch = (idx % (D / 8)) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (col < G) v = ld16(Q + (size_t)(b * a.Hq + g * G + col) * D + ch);
        *reinterpret_cast<u32x4*>(&sQ[col * L::QROW + ch]) = v;
    }
    __syncthreads();

    unsigned char* wbase = smem + wave * L::WAVE_BYTES;
    unsigned char* sK = wbase;
    unsigned char* sV = wbase + L::K_BYTES;
    int* sPos = reinterpret_cast<int*>(wbase + L::K_BYTES + L::V_BYTES);

    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * NC * D;
    const u16* Vc = static_cast<const u16*>(a.vc) + (size_t)bg * NC * D;
    const int32_t* posg = a.pos + (size_t)bg * NC;
    const int victim = a.freed != nullptr ? a.freed[bg] : -1;   // S = 1: one target
    const int k_begin = split * kDecSplit;
    const int k_end = min(n, k_begin + kDecSplit);
    const int nsub = (k_end - k_begin + kDecSub - 1) / kDecSub;

    // Lane offsets: load `it` covers rows it*(64/CH) + lane/CH, 16-byte chunk lane%CH.
    constexpr int RPL = 64 / CH;                            // rows per load instruction
    const int row0 = lane / CH, col0 = (lane % CH) * 8;
    const int goff0 = (row0 * D + col0) * 2;
    u32x4 kreg[LD], vreg[LD];
    int preg = 0;
    bool pvalid = false;
    auto gload = [&](int sub) {
        const int k0 = k_begin + sub * kDecSub;
        const int valid = min(kDecSub, k_end - k0);
        const Rsrc rk = make_rsrc(Kc + (size_t)k0 * D, valid * D * 2);
        const Rsrc rv = make_rsrc(Vc + (size_t)k0 * D, valid * D * 2);
#pragma unroll
        for (int it = 0; it < LD; ++it) {
            kreg[it] = bload16_stream(rk, goff0 + it * RPL * D * 2);
            vreg[it] = bload16_stream(rv, goff0 + it * RPL * D * 2);
        }
        if (lane < kDecSub) {
            const Rsrc rp = make_rsrc(posg + k0, valid * 4);
            preg = (int)bload4(rp, lane * 4);
            pvalid = lane < valid;
            if (k0 + lane == victim) preg = -1;   // buffer form: the slot being overwritten
        }
    };
    // LDS byte offsets of this lane's chunks (row row0 + it*RPL, chunk lane%CH);
    // RPL is a multiple of 4, so swz_v is the same for every `it`.
    const int cg = lane % CH;
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < LD; ++it) {
            const int r = row0 + it * RPL;
            *reinterpret_cast<u32x4*>(sK + r * RB + 16 * (cg ^ swz_k<D>(r))) = kreg[it];
            *reinterpret_cast<u32x4*>(sV + r * RB + 16 * (cg ^ swz_v<D>(r))) = vreg[it];
        }
        if (lane < kDecSub) sPos[lane] = pvalid ? preg : INT_MAX;
    };

    const float c = a.sm_scale * kLog2e;
    const float tau_raw = kRescaleLog2 / c;
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int prow = perm_key(lq);
    // K operand: row prow, chunk 2*ks + hh at kb ^ 32*ks; V^T operand rows
    // 8*hh + j16/4 (+16*s2, +4 for the second read), d block dt at vb ^ 64*dt.
    const int kb = prow * RB + 16 * (hh ^ swz_k<D>(prow));
    const int vrow = 8 * hh + (j16 >> 2);
    const int vb = vrow * RB + 16 * ((2 * (g16 & 1) + ((j16 & 3) >> 1)) ^ swz_v<D>(vrow)) +
                   8 * (j16 & 1);
    const int qpos = a.P;
    float* logit_row = ws.logits + ((size_t)bg * G + min(lq, G - 1)) * ws.ncp;
    const bool want_logits = a.cs_cache != nullptr;     // only the summed weights read them

    // Wave w owns sub-tiles w, w+4, ...; the LDS region is private to the wave,
    // whose LDS operations complete in order, so no workgroup barrier is needed.
    int sub = wave;
    if (sub < nsub) {
        gload(sub);
        lstore();
    }
    for (; sub < nsub; sub += kDecWaves) {
        const int next = sub + kDecWaves;
        // The next tile's loads go out at raised wave priority: waves that are
        // issuing loads win the arbitration against waves in their MFMA / softmax
        // work, which keeps more of the cache stream in flight (199 -> 193 us).
        __builtin_amdgcn_s_setprio(1);
        if (next < nsub) gload(next);
        __builtin_amdgcn_s_setprio(0);
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = mfma32(as_bf16x8(ld16(sK + (kb ^ (32 * ks)))),
                       as_bf16x8(ld16(&sQ[lq * L::QROW + 16 * ks + 8 * hh])), s);
        // key of C register r: 16*(r/8) + 8*hh + r%8 within the sub-tile
        const int kp_lane = sPos[lane & 31];
        if (!__all(kp_lane >= 0 && kp_lane <= qpos)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kpv = sPos[16 * (r >> 3) + 8 * hh + (r & 7)];
                if (!(kpv >= 0 && kpv <= qpos)) s[r] = -INFINITY;
            }
        }
        // The logits are stored after this iteration's wait for the next tile:
        // vmcnt counts stores too, so stores issued before that wait would be
        // waited for as well.
        const f32x16 s_log = s;
        float mt = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
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
        bf16x8 pb[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(fmaf(s[8 * s2 + e], c, -mc));
                l_run += p[e];
            }
            u32x4 w = {pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7])};
            pb[s2] = as_bf16x8(w);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const unsigned char* vp = sV + (vb ^ (64 * dt)) + 16 * s2 * RB;
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vp));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vp + 4 * RB));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 av = {l2[0], l2[1], h2[0], h2[1]};
                o[dt] = mfma32(as_bf16x8(av), pb[s2], o[dt]);
            }
        if (next < nsub) lstore();
        if (want_logits && lq < G) {
            const int k0 = k_begin + sub * kDecSub;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float4 w0, w1;
                w0.x = s_log[8 * half + 0] * c; w0.y = s_log[8 * half + 1] * c;
                w0.z = s_log[8 * half + 2] * c; w0.w = s_log[8 * half + 3] * c;
                w1.x = s_log[8 * half + 4] * c; w1.y = s_log[8 * half + 5] * c;
                w1.z = s_log[8 * half + 6] * c; w1.w = s_log[8 * half + 7] * c;
                float* dst = logit_row + k0 + 16 * half + 8 * hh;
                *reinterpret_cast<float4*>(dst) = w0;
                *reinterpret_cast<float4*>(dst + 4) = w1;
            }
        }
    }

    // Merge the four waves' states, then write this split's partial.
    __syncthreads();
    constexpr int MF = L::MERGE_FLOATS;
    float* mb = reinterpret_cast<float*>(smem) + wave * MF * 64;
    if (wave != 0) {
    mb[lane] = m_run;
    mb[64 + lane] = l_run;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb[(2 + dt * 16 + r) * 64 + lane] = o[dt][r];
    }
    __syncthreads();
    if (wave != 0) return;
    // Wave 0 folds the other waves' states into its own, in wave order.
    float m = m_run;
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w)
        m = fmaxf(m, reinterpret_cast<float*>(smem)[w * MF * 64 + lane]);
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m) * c);
    float l = l_run * a0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= a0;
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) {
        const float* src = reinterpret_cast<float*>(smem) + w * MF * 64;
        const float mw = src[lane];
        const float aw = mw == -INFINITY ? 0.f : fast_exp2((mw - m) * c);
        l += src[64 + lane] * aw;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] += src[(2 + dt * 16 + r) * 64 + lane] * aw;
    }
    l += __shfl_xor(l, 32);
    if (lq < G) {
        float* rec = ws.partial + (((size_t)bg * ws.nsplit + split) * G + lq) * (D + 2);
        if (hh == 0) {
            rec[0] = m == -INFINITY ? -INFINITY : m * c;    // log2 units
            rec[1] = l;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) rec[2 + dt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3)] = o[dt][r];
    }
}

// decode_attn_kernel for groups of at most four query heads, built on the
// 4x4x4 MFMA (16 blocks of 4 x 4 x 4 per instruction).  Its products put one
// slot in each lane: S = Q K^T with the heads as the four rows and the 32
// slots of a sub-tile as the block columns (lanes 32..63 take the upper half
// of d; one v_permlane32_swap adds the halves and leaves lane l holding heads
// 2*(l/32) and 2*(l/32)+1 of slot l%32), and O = P V with the heads as rows
// and 64 d columns per instruction.  O takes 8 registers instead of 64, so a
// wave can keep the logits of all its sub-tiles in 64 registers and write
// them in one burst once its loads are done: logit stores mixed into the
// cache read stream slow that stream far more than their 3% of the bytes.
constexpr int kDec4MaxSub = kDecSplit / (kDecSub * kDecWaves);   // sub-tiles per wave

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// What decode_attn4_kernel does with the logits.
enum Dec4Mode {
    kDec4NoWeights = 0,   // no summed weights: the logits are not kept
    kDec4Logits = 1,      // logits to the workspace; decode_finish_kernel forms the weights
    kDec4Fused = 2,       // summed weights formed in the kernel (LSE exchange)
    kDec4FusedEvict = 3,  // and the score update, eviction keys and per-split minimum
};

// LSE exchange between the workgroups (splits) of one (b, kv head): one 64-bit
// word per (split, head), (m log2 units) << 32 | l, all ones while unwritten.
constexpr uint64_t kXchEmpty = ~0ull;
constexpr int kXchMaxSplits = 16;          // one lane per (split, head) in the polling wave
// Bound on the polls of a missing word (a memory round trip and s_sleep 1
// each, well under 0.2 s in all): the launch keeps every workgroup resident at
// once, so the wait ends as soon as the siblings publish, within microseconds;
// the bound only guarantees that the kernel ends otherwise.
constexpr int kXchSpinLimit = 1 << 16;

// The new token's logit q.k * c (log2 units) for one head, in one wave:
// lane-strided products, then a butterfly sum.
template <int D>
__device__ __forceinline__ float new_token_logit2(const u16* q, const u16* k, float c, int lane) {
    auto bf = [](u16 x) { return __uint_as_float((uint32_t)x << 16); };
    float dot = 0.f;
#pragma unroll
    for (int d = lane; d < D; d += 64) dot = fmaf(bf(q[d]), bf(k[d]), dot);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    return dot * c;
}

// One head's log-sum-exp (log2 units) over the split states (lane sp holds
// split sp's (m, l), -inf / 0 beyond the splits) and the new token, in one
// wave; m_out is the merged maximum.
__device__ __forceinline__ float merge_lse2(float mrec, float lrec, float s_new, int lane,
                                            float& m_out) {
    float m = fmaxf(s_new, mrec);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float l = lane == 0 ? fast_exp2(s_new - m) : 0.f;
    if (mrec != -INFINITY) l += lrec * fast_exp2(mrec - m);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    m_out = m;
    return m + log2f(l);
}

template <int D>
struct Dec4Smem {
    static constexpr int RB = 2 * D;                  // bytes per K / V row
    static constexpr int K_BYTES = kDecSub * RB;
    static constexpr int V_BYTES = kDecSub * RB;
    static constexpr int P_BYTES = 4 * kDecSub * 2;   // P tile [4 heads][32 slots] bf16
    static constexpr int WAVE_BYTES = K_BYTES + V_BYTES + P_BYTES;
    // Q rows padded by 16 bytes: the four heads' reads of one instruction fall
    // in different banks.
    static constexpr int QROWB = 2 * D + 16;
    static constexpr int Q_BYTES = 4 * QROWB;
    static constexpr int MERGE_FLOATS = 8 + (D / 64) * 4 * 64;   // m[4], l[4], O
    static constexpr int MERGE_BYTES = kDecWaves * MERGE_FLOATS * 4;
    static constexpr int TILE_BYTES = kDecWaves * WAVE_BYTES + Q_BYTES;
    static constexpr int BYTES = TILE_BYTES > MERGE_BYTES ? TILE_BYTES : MERGE_BYTES;
};

template <int D, int MODE>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_attn4_kernel(ChunkArgs a, DecodeWs ws, int nsplit_rt, EvictArgs ev) {
    constexpr bool HOLD = MODE != kDec4NoWeights;
    using L = Dec4Smem<D>;
    constexpr int RB = L::RB;
    constexpr int CH = D / 8;                              // 16-byte chunks per row
    constexpr int LD = kDecSub * CH / 64;                  // 16-byte loads per lane
    constexpr int KH = D / 8;                              // QK^T k-steps over half of d
    constexpr int NO = D / 64;                             // PV products per 4 slots
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int total = nsplit_rt * a.B * a.Hkv;
    const int t = xcd_tile(blockIdx.x, total);
    if (t >= total) return;
    const int bg = t / nsplit_rt, split = t % nsplit_rt;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.G, n = a.n, NC = a.NC;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int key = lane & 31, hi = lane >> 5;    // slot within a sub-tile; d half / head pair

    // The group's Q rows (zero rows for heads >= G).
    unsigned char* sQ = smem + kDecWaves * L::WAVE_BYTES;
    const u16* Q = static_cast<const u16*>(a.q);
    for (int idx = tid; idx < 4 * CH; idx += kDecThreads) {
        const int h = idx / CH, ch = idx % CH;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < G) v = ld16(Q + (size_t)(b * a.Hq + g * G + h) * D + ch * 8);
        *reinterpret_cast<u32x4*>(sQ + h * L::QROWB + 16 * ch) = v;
    }
    __syncthreads();

    unsigned char* wbase = smem + wave * L::WAVE_BYTES;
    unsigned char* sK = wbase;
    unsigned char* sV = wbase + L::K_BYTES;
    unsigned char* sP = wbase + L::K_BYTES + L::V_BYTES;

    const u16* Kc = static_cast<const u16*>(a.kc) + (size_t)bg * NC * D;
    const u16* Vc = static_cast<const u16*>(a.vc) + (size_t)bg * NC * D;
    const int32_t* posg = a.pos + (size_t)bg * NC;
    const int victim = a.freed != nullptr ? a.freed[bg] : -1;   // S = 1: one target
    const int k_begin = split * kDecSplit;
    const int k_end = min(n, k_begin + kDecSplit);
    const int nsub = (k_end - k_begin + kDecSub - 1) / kDecSub;

    // Staging: load `it` covers rows it*(64/CH) + lane/CH, 16-byte chunk lane%CH;
    // every lane also loads the position of its own slot.
    constexpr int RPL = 64 / CH;
    const int row0 = lane / CH, cg = lane % CH;
    const int goff0 = (row0 * D + cg * 8) * 2;
    u32x4 kreg[LD], vreg[LD];
    int pnext = 0, pcur = INT_MAX;
    bool pvalid = false;
    auto gload = [&](int sub) {
        const int k0 = k_begin + sub * kDecSub;
        // Scalar on purpose: compared with the lane's slot below, it would
        // otherwise sit in a vector register and the buffer descriptors built
        // from it would need waterfall loops.
        const int valid = __builtin_amdgcn_readfirstlane(min(kDecSub, k_end - k0));
        const Rsrc rk = make_rsrc(Kc + (size_t)k0 * D, valid * D * 2);
        const Rsrc rv = make_rsrc(Vc + (size_t)k0 * D, valid * D * 2);
#pragma unroll
        for (int it = 0; it < LD; ++it) {
            kreg[it] = bload16_stream(rk, goff0 + it * RPL * D * 2);
            vreg[it] = bload16_stream(rv, goff0 + it * RPL * D * 2);
        }
        const Rsrc rp = make_rsrc(posg + k0, valid * 4);
        pnext = (int)bload4(rp, key * 4);
        pvalid = key < valid;
        if (k0 + key == victim) pnext = -1;       // buffer form: the slot being overwritten
    };
    auto lstore = [&]() {
#pragma unroll
        for (int it = 0; it < LD; ++it) {
            const int r = row0 + it * RPL;
            *reinterpret_cast<u32x4*>(sK + r * RB + 16 * (cg ^ swz_k<D>(r))) = kreg[it];
            *reinterpret_cast<u32x4*>(sV + r * RB + 16 * (cg ^ swz_v<D>(r))) = vreg[it];
        }
        pcur = pvalid ? pnext : INT_MAX;
    };

    // Operand addresses.  K^T (B of S): row `key`, d = hi*D/2 + 4*step, i.e.
    // 16-byte chunk hi*D/16 + step/2 (no carry into the half bit), half step%2.
    const int krow = key * RB;
    const int ksw = (hi * (D / 16)) ^ swz_k<D>(key);
    // Q (A of S): head lane%4, same d.
    const int qoff = (lane & 3) * L::QROWB + hi * D;
    // V (B of O) through ds_read_b64_tr_b16: 16-lane group q4, lane j addresses
    // slot 4*t4 + j/4, d 16*q4 + 4*(j%4) (+64 per product) and receives slots
    // 4*t4 .. 4*t4+3 of d = lane (+64).
    const int q4 = lane >> 4, j16 = lane & 15;
    int voff[NO];
#pragma unroll
    for (int nn = 0; nn < NO; ++nn)
        voff[nn] = (j16 >> 2) * RB +
                   16 * ((2 * q4 + ((j16 & 3) >> 1) + 8 * nn) ^ swz_v<D>(j16 >> 2)) +
                   8 * (j16 & 1);
    // P (A of O): head lane%4, slots 4*t4 .. 4*t4+3.
    const int poff = (lane & 3) * (2 * kDecSub);

    const float c = a.sm_scale * kLog2e;
    const float tau_raw = kRescaleLog2 / c;
    const int qpos = a.P;
    // Online-softmax state of this lane's two heads (2*hi, 2*hi+1): running max
    // (the same in every lane of a half), this lane's share of the sum, and O
    // (lane l, register r: head r, d = l + 64*nn) for all four heads.
    float mA = -INFINITY, mB = -INFINITY, lA = 0.f, lB = 0.f;
    f32x4 o[NO];
#pragma unroll
    for (int nn = 0; nn < NO; ++nn) o[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lg[HOLD ? 2 * kDec4MaxSub : 1];
    uint32_t elig = 0;
    const int elig_thr = a.P - ev.W;
#pragma unroll
    for (int i = 0; i < (HOLD ? 2 * kDec4MaxSub : 1); ++i) lg[i] = 0.f;

    // Wave w owns sub-tiles w, w+4, ...; the LDS region is private to the wave,
    // whose LDS operations complete in order, so no workgroup barrier is needed.
    int sub = wave;
    if (sub < nsub) {
        gload(sub);
        lstore();
    }
    for (; sub < nsub; sub += kDecWaves) {
        const int next = sub + kDecWaves;
        __builtin_amdgcn_s_setprio(1);
        if (next < nsub) gload(next);
        __builtin_amdgcn_s_setprio(0);
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KH; ++st) {
            const s16x4 qa = *reinterpret_cast<const s16x4*>(sQ + qoff + 8 * st);
            const s16x4 kb = *reinterpret_cast<const s16x4*>(
                sK + krow + 16 * ((st >> 1) ^ ksw) + 8 * (st & 1));
            if (st & 1) acc1 = mfma4(qa, kb, acc1);
            else acc0 = mfma4(qa, kb, acc0);
        }
        const f32x4 sp = acc0 + acc1;
        const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sp[0]),
                                                          __float_as_uint(sp[2]), false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sp[1]),
                                                          __float_as_uint(sp[3]), false, false);
        const bool vis = pcur >= 0 && pcur <= qpos;
        const float sa = vis ? __uint_as_float(x02[0]) + __uint_as_float(x02[1]) : -INFINITY;
        const float sb = vis ? __uint_as_float(x13[0]) + __uint_as_float(x13[1]) : -INFINITY;
        if constexpr (HOLD) {
#pragma unroll
            for (int i = 0; i < 2 * kDec4MaxSub - 2; ++i) lg[i] = lg[i + 2];
            lg[2 * kDec4MaxSub - 2] = sa * c;
            lg[2 * kDec4MaxSub - 1] = sb * c;
        }
        // Eviction eligibility of this lane's slot, t(j) < P - W, shifted in like
        // the logits (h2o keys need nothing else of the position).
        if constexpr (MODE == kDec4FusedEvict)
            elig = (elig >> 1) | ((uint32_t)(pcur < elig_thr) << 31);
        if (__any(sa > mA + tau_raw || sb > mB + tau_raw)) {
            float ta = sa, tb = sb;
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                ta = fmaxf(ta, __shfl_xor(ta, off));
                tb = fmaxf(tb, __shfl_xor(tb, off));
            }
            const float nA = fmaxf(mA, ta), nB = fmaxf(mB, tb);
            const float mA2 = nA > mA + tau_raw ? nA : mA;
            const float mB2 = nB > mB + tau_raw ? nB : mB;
            const float alA = mA2 == mA ? 1.f : fast_exp2((mA - mA2) * c);
            const float alB = mB2 == mB ? 1.f : fast_exp2((mB - mB2) * c);
            lA *= alA;
            lB *= alB;
            mA = mA2;
            mB = mB2;
            const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alA), 0));
            const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alB), 0));
            const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alA), 32));
            const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alB), 32));
#pragma unroll
            for (int nn = 0; nn < NO; ++nn) {
                o[nn][0] *= r0;
                o[nn][1] *= r1;
                o[nn][2] *= r2;
                o[nn][3] *= r3;
            }
        }
        const float mcA = mA == -INFINITY ? 0.f : mA * c;
        const float mcB = mB == -INFINITY ? 0.f : mB * c;
        const float pa = fast_exp2(fmaf(sa, c, -mcA));
        const float pb = fast_exp2(fmaf(sb, c, -mcB));
        lA += pa;
        lB += pb;
        const uint32_t pp = pack2(pa, pb);
        u16* sPh = reinterpret_cast<u16*>(sP);
        sPh[(2 * hi) * kDecSub + key] = (u16)(pp & 0xFFFFu);
        sPh[(2 * hi + 1) * kDecSub + key] = (u16)(pp >> 16);
#pragma unroll
        for (int t4 = 0; t4 < kDecSub / 4; ++t4) {
            const s16x4 pa4 = *reinterpret_cast<const s16x4*>(sP + poff + 8 * t4);
#pragma unroll
            for (int nn = 0; nn < NO; ++nn) {
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const s16x4 vb4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(sV + voff[nn] + 4 * t4 * RB));
                o[nn] = mfma4(pa4, vb4, o[nn]);
            }
        }
        if (next < nsub) lstore();
    }

    // This wave's logits, oldest sub-tile first: sub-tile `it` sits in lg[2*j],
    // j = it + 32 - niter.
    const int niter = nsub > wave ? (nsub - wave + kDecWaves - 1) / kDecWaves : 0;
    if constexpr (MODE == kDec4Logits) {
        float* rowA = ws.logits + ((size_t)bg * G + 2 * hi) * ws.ncp;
        const bool wA = 2 * hi < G, wB = 2 * hi + 1 < G;
#pragma unroll
        for (int j = 0; j < kDec4MaxSub; ++j) {
            const int it = niter - kDec4MaxSub + j;
            if (it >= 0) {
                const int k0 = k_begin + (wave + kDecWaves * it) * kDecSub;
                if (wA) rowA[k0 + key] = lg[2 * j];
                if (wB) rowA[ws.ncp + k0 + key] = lg[2 * j + 1];
            }
        }
    }
    // Fused: after the halves combine, lane (key, hi) holds the summed weight
    // of sub-tile j = 2*i + hi for i < NT; its score and position are loaded
    // now so that they arrive during the merge and the exchange.
    constexpr int NT = kDec4MaxSub / 2;
    auto slot_of = [&](int i, bool& ok) {
        const int it = niter - kDec4MaxSub + 2 * i + hi;
        const int slot = k_begin + (wave + kDecWaves * it) * kDecSub + key;
        ok = it >= 0 && slot < k_end;
        return ok ? slot : k_begin;
    };
    // Under h2o-norm the keys also need each slot's age, so its position is read
    // again; h2o keys use the eligibility bits kept during the loop.
    const bool norm = ev.score_mode == H2O_SCORE_H2O_NORM;
    uint32_t phr[MODE == kDec4FusedEvict ? NT : 1], psr[MODE == kDec4FusedEvict ? NT : 1];
    if constexpr (MODE == kDec4FusedEvict) {
        const Rsrc rs = make_rsrc(ev.score + (size_t)bg * NC, n * 4);
        const Rsrc rp = make_rsrc(ev.pos + (size_t)bg * NC, norm ? n * 4 : 0);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            bool ok;
            const int slot = slot_of(i, ok);
            phr[i] = bload4(rs, slot * 4);
            psr[i] = norm ? bload4(rp, slot * 4) : 0u;
        }
    }

    // Sums over the 32 slots of each half; then the four waves' states merge.
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
        lA += __shfl_xor(lA, off);
        lB += __shfl_xor(lB, off);
    }
    float mh[4], lh[4];
    mh[0] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mA), 0));
    mh[1] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mB), 0));
    mh[2] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mA), 32));
    mh[3] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mB), 32));
    lh[0] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lA), 0));
    lh[1] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lB), 0));
    lh[2] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lA), 32));
    lh[3] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(lB), 32));
    __shared__ float sL2[4];
    __syncthreads();
    constexpr int MF = L::MERGE_FLOATS;
    float* mb = reinterpret_cast<float*>(smem) + wave * MF;
    if (wave != 0) {
        if (lane < 4) {
            mb[lane] = mh[lane];
            mb[4 + lane] = lh[lane];
        }
#pragma unroll
        for (int nn = 0; nn < NO; ++nn)
#pragma unroll
            for (int r = 0; r < 4; ++r) mb[8 + (nn * 4 + r) * 64 + lane] = o[nn][r];
    }
    __syncthreads();
    if (wave == 0) {
        // Wave 0 folds the other waves' states into its own, in wave order.
        const float* mall = reinterpret_cast<const float*>(smem);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = mh[r];
#pragma unroll
            for (int w = 1; w < kDecWaves; ++w) m = fmaxf(m, mall[w * MF + r]);
            const float a0 = mh[r] == -INFINITY ? 0.f : fast_exp2((mh[r] - m) * c);
            float l = lh[r] * a0;
#pragma unroll
            for (int nn = 0; nn < NO; ++nn) o[nn][r] *= a0;
#pragma unroll
            for (int w = 1; w < kDecWaves; ++w) {
                const float mw = mall[w * MF + r];
                const float aw = mw == -INFINITY ? 0.f : fast_exp2((mw - m) * c);
                l += mall[w * MF + 4 + r] * aw;
#pragma unroll
                for (int nn = 0; nn < NO; ++nn)
                    o[nn][r] += mall[w * MF + 8 + (nn * 4 + r) * 64 + lane] * aw;
            }
            mh[r] = m == -INFINITY ? -INFINITY : m * c;    // log2 units from here on
            lh[r] = l;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r >= G) break;
            float* rec = ws.partial + (((size_t)bg * ws.nsplit + split) * G + r) * (D + 2);
            if (lane == 0) {
                rec[0] = mh[r];
                rec[1] = lh[r];
            }
#pragma unroll
            for (int nn = 0; nn < NO; ++nn) rec[2 + lane + 64 * nn] = o[nn][r];
        }
        if constexpr (MODE >= kDec4Fused) {
            // Publish this split's (m, l) per head, form the new token's logits,
            // then wait for every split of the (b, kv head) and merge the LSE.
            uint64_t* xw = ws.xch + ((size_t)bg * ws.nsplit + split) * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (lane == r && r < G)
                    __hip_atomic_store(xw + r,
                                       ((uint64_t)__float_as_uint(mh[r]) << 32) |
                                           __float_as_uint(lh[r]),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * D;
            float snew[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                snew[r] = r < G ? new_token_logit2<D>(Q + (size_t)(b * a.Hq + g * G + r) * D, Kn,
                                                      c, lane)
                                : 0.f;
            const int sp = lane >> 2, hq = lane & 3;
            const bool need = sp < nsplit_rt && hq < G;
            const uint64_t* xr = ws.xch + ((size_t)bg * ws.nsplit + min(sp, nsplit_rt - 1)) * 4 + hq;
            uint64_t w = kXchEmpty;
            for (int spin = 0; spin < kXchSpinLimit; ++spin) {
                if (need && w == kXchEmpty)
                    w = __hip_atomic_load(xr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (__all(!need || w != kXchEmpty)) break;
                __builtin_amdgcn_s_sleep(1);
            }
            const int whi = (int)(uint32_t)(w >> 32), wlo = (int)(uint32_t)w;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int src = min(lane, kXchMaxSplits - 1) * 4 + r;
                const float m0 = __int_as_float(__shfl(whi, src));
                const float l0 = __int_as_float(__shfl(wlo, src));
                const bool has = lane < nsplit_rt;
                float mm;
                const float l2 = merge_lse2(has ? m0 : -INFINITY, has ? l0 : 0.f, snew[r], lane, mm);
                if (lane == 0) sL2[r] = r < G ? l2 : INFINITY;   // heads >= G add nothing
            }
        }
    }
    if constexpr (MODE >= kDec4Fused) {
        __syncthreads();
        // Summed weights sum_h exp2(s_h - LSE_h) of this lane's slots: its two heads
        // per sub-tile, then the other half's two heads through one swap per pair
        // of sub-tiles (heads 0+1, then 2+3 added, in every slot).
        const float La = sL2[2 * hi], Lb = sL2[2 * hi + 1];
        float tot[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const float wa = fast_exp2(lg[4 * i] - La) + fast_exp2(lg[4 * i + 1] - Lb);
            const float wb = fast_exp2(lg[4 * i + 2] - La) + fast_exp2(lg[4 * i + 3] - Lb);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(wa),
                                                             __float_as_uint(wb), false, false);
            tot[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        float* csr = a.cs_cache + (size_t)bg * NC;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            bool ok;
            const int slot = slot_of(i, ok);
            if (ok) csr[slot] = tot[i];
        }
        if constexpr (MODE == kDec4FusedEvict) {
            // Score update phi += summed weight, and the eviction key of every filled
            // slot: eligible iff t(j) < P - W; h2o-norm divides by the age t - t(j),
            // t = P + 1.  The same operations as the separate update and selection.
            __shared__ uint64_t sBest[kDecWaves];
            const bool full = n == NC;                    // one victim (k = n + 1 - N_C)
            const int thr = a.P - ev.W, t_now = a.P + 1;
            float* scw = ev.score + (size_t)bg * NC;
            uint64_t best = ~0ull;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                bool ok;
                const int slot = slot_of(i, ok);
                const float v = __uint_as_float(phr[i]) + tot[i];
                if (ok) scw[slot] = v;
                uint32_t k;
                if (norm) {
                    const int pj = (int)psr[i];
                    k = pj < thr ? order_key(v / (float)(t_now - pj)) : kIneligible;
                } else {
                    k = ((elig >> (2 * i + hi)) & 1u) ? order_key(v) : kIneligible;
                }
                const uint64_t kv = ((uint64_t)k << 32) | (uint32_t)slot;
                if (ok && kv < best) best = kv;
            }
            if (!full) return;                            // filling: the token goes to slot n
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const uint64_t ot = __shfl_xor(best, off);
                best = ot < best ? ot : best;
            }
            if (lane == 0) sBest[wave] = best;
            __syncthreads();
            if (tid == 0) {
                uint64_t m = sBest[0];
#pragma unroll
                for (int w = 1; w < kDecWaves; ++w) m = sBest[w] < m ? sBest[w] : m;
                ws.part_min[(size_t)bg * ws.nfin + split] = m;
            }
        }
    }
}

// After the fused decode_attn4_kernel: one workgroup per (b, kv head) merges
// the split partials with the new token into O and LSE (the same LSE
// arithmetic as the fused kernel), writes the new token's own summed weight,
// and (EVICT) takes the smallest (key, slot) of the splits' minima (full
// cache) or slot n (filling) and writes the new token there: K and V rows,
// t = P, score = its summed weight, freed_slots.
template <int D, bool EVICT>
__global__ __launch_bounds__(kDecThreads) void decode_merge_kernel(ChunkArgs a, DecodeWs ws,
                                                                   int nsplit_rt, EvictArgs ev) {
    constexpr int PER = 4 * D / kDecThreads;           // (head, d) outputs per thread (G <= 4)
    constexpr int units = D * 2 / 16;                  // 16-byte units of a bf16 row
    static_assert(2 * units <= 64, "one lane per row unit");
    __shared__ float sLse2[4], sNew[4], sM[4];
    const int bg = blockIdx.x;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float c = a.sm_scale * kLog2e;
    const u16* Q = static_cast<const u16*>(a.q);
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * D;
    const u16* Vn = static_cast<const u16*>(a.vn) + (size_t)bg * D;
    const size_t stride = (size_t)G * (D + 2);
    const float* rec_bg = ws.partial + (size_t)bg * ws.nsplit * stride;
    auto bf = [](u16 x) { return __uint_as_float((uint32_t)x << 16); };

    // Every global read first, so that they are in flight together: wave hh's
    // split records of head hh; each thread's partial outputs of its (head, d)
    // pairs; the new value row; (EVICT) the splits' minima and the new K and V rows.
    const int hh = wave;
    const bool has = hh < G && lane < nsplit_rt;
    const float mrec = has ? rec_bg[lane * stride + hh * (D + 2)] : -INFINITY;
    const float lrec = has ? rec_bg[lane * stride + hh * (D + 2) + 1] : 0.f;
    float pm[PER][kXchMaxSplits], po[PER][kXchMaxSplits], vn[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = min(tid + i * kDecThreads, G * D - 1);
        const int h = idx / D, d = idx % D;
        vn[i] = bf(Vn[d]);
#pragma unroll
        for (int sp = 0; sp < kXchMaxSplits; ++sp) {
            const float* rec = rec_bg + min(sp, nsplit_rt - 1) * stride + h * (D + 2);
            pm[i][sp] = sp < nsplit_rt ? rec[0] : -INFINITY;
            po[i][sp] = sp < nsplit_rt ? rec[2 + d] : 0.f;
        }
    }
    uint64_t mn = ~0ull;
    u32x4 row = {0u, 0u, 0u, 0u};
    if (EVICT && wave == 0) {
        if (a.n == a.NC && lane < nsplit_rt) mn = ws.part_min[(size_t)bg * ws.nfin + lane];
        if (lane < 2 * units)
            row = static_cast<const u32x4*>(lane >= units ? a.vn : a.kn)[(size_t)bg * units +
                                                                       lane % units];
    }

    if (hh < G) {
        const float s_new =
            new_token_logit2<D>(Q + (size_t)(b * a.Hq + g * G + hh) * D, Kn, c, lane);
        float m;
        const float l2 = merge_lse2(mrec, lrec, s_new, lane, m);
        if (lane == 0) {
            sLse2[hh] = l2;
            sNew[hh] = s_new;
            sM[hh] = m;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = tid + i * kDecThreads;
        if (idx >= G * D) break;
        const int h = idx / D, d = idx % D;
        const float m = sM[h];
        float acc = vn[i] * fast_exp2(sNew[h] - m);
#pragma unroll
        for (int sp = 0; sp < kXchMaxSplits; ++sp)
            if (pm[i][sp] != -INFINITY) acc += po[i][sp] * fast_exp2(pm[i][sp] - m);
        const float inv = fast_exp2(m - sLse2[h]);         // 1 / l
        const size_t oi = (size_t)(b * a.Hq + g * G + h) * D + d;
        static_cast<__hip_bfloat16*>(a.out)[oi] = __float2bfloat16(acc * inv);
        if (d == 0) a.lse[(size_t)(b * a.Hq + g * G + h)] = sLse2[h] * 0.6931471805599453f;
    }
    if (wave != 0) return;
    float cs = 0.f;
    for (int h = 0; h < G; ++h) cs += fast_exp2(sNew[h] - sLse2[h]);
    if (lane == 0) a.cs_new[bg] = cs;
    if constexpr (EVICT) {
        int slot = a.n;
        if (a.n == a.NC) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const uint64_t o = __shfl_xor(mn, off);
                mn = o < mn ? o : mn;
            }
            slot = (int)(uint32_t)mn;
        }
        if (lane < 2 * units)
            static_cast<u32x4*>(lane >= units ? ev.vc : ev.kc)[((size_t)bg * a.NC + slot) * units +
                                                              lane % units] = row;
        if (lane == 0) {
            ev.freed[bg] = slot;
            ev.pos[(size_t)bg * a.NC + slot] = a.P;
            ev.score[(size_t)bg * a.NC + slot] = cs;
        }
    }
}

__global__ void decode_clear_kernel(uint64_t* x, int count) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x)
        x[i] = kXchEmpty;
}

// Merge the splits and the new token, write O / LSE (first workgroup of each
// (b, g)), and form the summed weights of a range of slots.  EVICT: also the
// score update, the eviction keys and this range's (key, slot) minimum (a full
// cache: one victim), which decode_insert_kernel reduces.
template <int D, bool EVICT>
__global__ __launch_bounds__(kDecThreads) void decode_finish_kernel(ChunkArgs a, DecodeWs ws,
                                                                    int nsplit_rt, int kchunks,
                                                                    EvictArgs ev) {
    __shared__ float sLse2[64];
    __shared__ float sNew[64];
    __shared__ float sM[64];
    __shared__ uint64_t sBest[kDecWaves];
    const int bg = blockIdx.y, kc = blockIdx.x;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int G = a.G, n = a.n;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float c = a.sm_scale * kLog2e;
    const u16* Q = static_cast<const u16*>(a.q);
    const u16* Kn = static_cast<const u16*>(a.kn) + (size_t)bg * D;
    const u16* Vn = static_cast<const u16*>(a.vn) + (size_t)bg * D;
    auto bf = [](u16 x) { return __uint_as_float((uint32_t)x << 16); };

    // The logits of this workgroup's slots for the first kPre heads do not
    // depend on the merged LSE: start their loads before computing it.
    // Slots past n read zeros and are never stored.
    const int j0 = kc * kFinishKeys, j1 = min(n, j0 + kFinishKeys);
    // Slots j0 + 4*tid + 4*kDecThreads*u + e (e < 4): 16-byte loads and stores.
    constexpr int U = kFinishKeys / (4 * kDecThreads);     // 4-slot groups per thread
    static_assert(kFinishKeys % (4 * kDecThreads) == 0, "finish tiling");
    constexpr int kPre = 4;
    const Rsrc rlog = make_rsrc(ws.logits + (size_t)bg * G * ws.ncp, G * ws.ncp * 4);
    auto lload = [&](int hh, int u) {
        return __builtin_bit_cast(float4, bload16_stream(
            rlog, (hh * ws.ncp + j0 + 4 * tid + 4 * kDecThreads * u) * 4));
    };
    const bool want_cs = a.cs_cache != nullptr;
    float4 vpre[kPre][U];
#pragma unroll
    for (int hh = 0; hh < kPre; ++hh)
#pragma unroll
        for (int u = 0; u < U; ++u)
            vpre[hh][u] = (want_cs && hh < G) ? lload(hh, u) : float4{0.f, 0.f, 0.f, 0.f};
    // EVICT: this range's scores and positions go out with the logits (zeros past n).
    u32x4 sc4[U], ps4[U];
    if constexpr (EVICT) {
        const Rsrc rs = make_rsrc(ev.score + (size_t)bg * a.NC, n * 4);
        const Rsrc rp = make_rsrc(ev.pos + (size_t)bg * a.NC, n * 4);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int off = (j0 + 4 * tid + 4 * kDecThreads * u) * 4;
            sc4[u] = bload16(rs, off);
            ps4[u] = bload16(rp, off);
        }
    }

    // The output merge's loads (workgroup kc == 0) go out now too, so that every
    // global read of this kernel is in flight at once: each thread's (head, d)
    // pairs idx = tid, tid + 256 (G*D <= 512, at most kMaxSplits splits).
    constexpr int kMaxSplits = 8;
    const size_t stride = (size_t)G * (D + 2);
    const bool pre_out = kc == 0 && G * D <= 2 * kDecThreads && nsplit_rt <= kMaxSplits;
    float pm[2][kMaxSplits], po[2][kMaxSplits];
    if (pre_out) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = min(tid + i * kDecThreads, G * D - 1);
            const float* rec0 = ws.partial + ((size_t)bg * ws.nsplit * G + idx / D) * (D + 2);
#pragma unroll
            for (int sp = 0; sp < kMaxSplits; ++sp) {
                const int spc = min(sp, nsplit_rt - 1);
                pm[i][sp] = rec0[spc * stride];
                po[i][sp] = rec0[spc * stride + 2 + idx % D];
            }
        }
    }

    // Per head: the new token's logit and the merged log-sum-exp (log2 units).
    for (int hh = wave; hh < G; hh += kDecWaves) {
        const u16* q = Q + (size_t)(b * a.Hq + g * G + hh) * D;
        const float* rec0 = ws.partial + ((size_t)bg * ws.nsplit * G + hh) * (D + 2);
        // the split records first (one per lane), then the dot product
        const bool has_rec = lane < nsplit_rt;
        const float mrec = has_rec ? rec0[lane * stride] : -INFINITY;
        const float lrec = has_rec ? rec0[lane * stride + 1] : 0.f;
        float dot = 0.f;
        for (int d = lane; d < D; d += 64) dot = fmaf(bf(q[d]), bf(Kn[d]), dot);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
        const float s_new = dot * c;
        float m = fmaxf(s_new, mrec);
        for (int sp = lane + 64; sp < nsplit_rt; sp += 64) m = fmaxf(m, rec0[sp * stride]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float l = lane == 0 ? fast_exp2(s_new - m) : 0.f;
        if (mrec != -INFINITY) l += lrec * fast_exp2(mrec - m);
        for (int sp = lane + 64; sp < nsplit_rt; sp += 64) {
            const float ms = rec0[sp * stride];
            if (ms != -INFINITY) l += rec0[sp * stride + 1] * fast_exp2(ms - m);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
        if (lane == 0) {
            sLse2[hh] = m + log2f(l);
            sNew[hh] = s_new;
            sM[hh] = m;
        }
    }
    __syncthreads();

    if (pre_out) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + i * kDecThreads;
            if (idx >= G * D) break;
            const int hh = idx / D, d = idx % D;
            const float m = sM[hh];
            float acc = bf(Vn[d]) * fast_exp2(sNew[hh] - m);
#pragma unroll
            for (int sp = 0; sp < kMaxSplits; ++sp)
                if (sp < nsplit_rt && pm[i][sp] != -INFINITY)
                    acc += po[i][sp] * fast_exp2(pm[i][sp] - m);
            const float inv = fast_exp2(m - sLse2[hh]);       // 1 / l
            const size_t oi = (size_t)(b * a.Hq + g * G + hh) * D + d;
            static_cast<__hip_bfloat16*>(a.out)[oi] = __float2bfloat16(acc * inv);
            if (d == 0) a.lse[(size_t)(b * a.Hq + g * G + hh)] = sLse2[hh] * 0.6931471805599453f;
        }
        if (want_cs && tid == 0) {
            float cs = 0.f;
            for (int hh = 0; hh < G; ++hh) cs += fast_exp2(sNew[hh] - sLse2[hh]);
            a.cs_new[bg] = cs;
        }
    } else if (kc == 0) {
        for (int idx = tid; idx < G * D; idx += kDecThreads) {
            const int hh = idx / D, d = idx % D;
            const float m = sM[hh];
            const float* rec0 = ws.partial + ((size_t)bg * ws.nsplit * G + hh) * (D + 2);
            const size_t stride = (size_t)G * (D + 2);
            float acc = bf(Vn[d]) * fast_exp2(sNew[hh] - m);
            // Issue the split loads in batches of 8 so they are in flight together.
            for (int sp0 = 0; sp0 < nsplit_rt; sp0 += 8) {
                float ms[8], ov[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int sp = min(sp0 + u, nsplit_rt - 1);
                    ms[u] = rec0[sp * stride];
                    ov[u] = rec0[sp * stride + 2 + d];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (sp0 + u < nsplit_rt && ms[u] != -INFINITY)
                        acc += ov[u] * fast_exp2(ms[u] - m);
            }
            const float inv = fast_exp2(m - sLse2[hh]);       // 1 / l
            const size_t oi = (size_t)(b * a.Hq + g * G + hh) * D + d;
            static_cast<__hip_bfloat16*>(a.out)[oi] = __float2bfloat16(acc * inv);
            if (d == 0) a.lse[(size_t)(b * a.Hq + g * G + hh)] = sLse2[hh] * 0.6931471805599453f;
        }
        if (want_cs && tid == 0) {
            float cs = 0.f;
            for (int hh = 0; hh < G; ++hh) cs += fast_exp2(sNew[hh] - sLse2[hh]);
            a.cs_new[bg] = cs;
        }
    }
    if (!want_cs) return;
    float4 cs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cs[u] = float4{0.f, 0.f, 0.f, 0.f};
    auto add_head = [&](const float4 (&v)[U], float l2) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            cs[u].x += fast_exp2(v[u].x - l2);
            cs[u].y += fast_exp2(v[u].y - l2);
            cs[u].z += fast_exp2(v[u].z - l2);
            cs[u].w += fast_exp2(v[u].w - l2);
        }
    };
#pragma unroll
    for (int hh = 0; hh < kPre; ++hh)
        if (hh < G) add_head(vpre[hh], sLse2[hh]);
    for (int hh = kPre; hh < G; ++hh) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = lload(hh, u);
        add_head(v, sLse2[hh]);
    }
    float* csr = a.cs_cache + (size_t)bg * a.NC;
    const bool vec = ((reinterpret_cast<uintptr_t>(csr) & 15u) | (uintptr_t)(a.NC & 3)) == 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = j0 + 4 * tid + 4 * kDecThreads * u;
        if (vec && j + 3 < j1) {
            *reinterpret_cast<float4*>(csr + j) = cs[u];
        } else {
            const float w[4] = {cs[u].x, cs[u].y, cs[u].z, cs[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < j1) csr[j + e] = w[e];
        }
    }
    if constexpr (EVICT) {
        // Score update phi += summed weight (written back), and the eviction key of
        // every filled slot: eligible iff t(j) < P - W; h2o-norm divides by the
        // age t - t(j), t = P + 1.  Same operations as the separate update and
        // selection, so the same bits.
        const bool full = n == a.NC;                  // one victim (k = n + 1 - N_C)
        const int thr = a.P - ev.W, t_now = a.P + 1;
        float* scw = ev.score + (size_t)bg * a.NC;
        uint64_t best = ~0ull;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + 4 * tid + 4 * kDecThreads * u;
            const float c4[4] = {cs[u].x, cs[u].y, cs[u].z, cs[u].w};
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(sc4[u][e]) + c4[e];
            if (vec && j + 3 < j1) {
                *reinterpret_cast<float4*>(scw + j) = float4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < j1) scw[j + e] = v[e];
            }
            if (full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pj = (int)ps4[u][e];
                    float r = v[e];
                    if (ev.score_mode == H2O_SCORE_H2O_NORM) r = r / (float)(t_now - pj);
                    const uint32_t key = pj < thr ? order_key(r) : kIneligible;
                    const uint64_t kv = ((uint64_t)key << 32) | (uint32_t)(j + e);
                    if (j + e < j1 && kv < best) best = kv;
                }
            }
        }
        if (!full) return;                            // filling: the token goes to slot n
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off);
            best = o < best ? o : best;
        }
        if (lane == 0) sBest[wave] = best;
        __syncthreads();
        if (tid == 0) {
            uint64_t m = sBest[0];
#pragma unroll
            for (int w = 1; w < kDecWaves; ++w) m = sBest[w] < m ? sBest[w] : m;
            ws.part_min[(size_t)bg * ws.nfin + kc] = m;
        }
    }
}

// After decode_finish_kernel<EVICT>: one wave per (b, kv head) takes the
// smallest (key, slot) of the finishing workgroups' minima (full cache) or slot
// n (filling) and writes the new token there: K and V rows, t = P, score = the
// token's own summed weight, freed_slots.  Same victim and contents as the
// one-victim selection and insertion of h2o_update_evict_and_insert.
__global__ __launch_bounds__(64) void decode_insert_kernel(ChunkArgs a, DecodeWs ws,
                                                           int kchunks, EvictArgs ev) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const int bg = blockIdx.x, lane = threadIdx.x;
    int slot = a.n;
    if (a.n == a.NC) {
        uint64_t m = lane < kchunks ? ws.part_min[(size_t)bg * ws.nfin + lane] : ~0ull;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(m, off);
            m = o < m ? o : m;
        }
        slot = (int)(uint32_t)m;
    }
    const int units = a.D * 2 / 16;                   // 16-byte units of a bf16 row
    if (lane < 2 * units) {
        const bool is_v = lane >= units;
        const int part = lane % units;
        const u32x4_t* src = static_cast<const u32x4_t*>(is_v ? a.vn : a.kn) + (size_t)bg * units;
        u32x4_t* dst = static_cast<u32x4_t*>(is_v ? ev.vc : ev.kc) +
                       ((size_t)bg * a.NC + slot) * units;
        dst[part] = src[part];
    }
    if (lane == 0) {
        ev.freed[bg] = slot;
        ev.pos[(size_t)bg * a.NC + slot] = a.P;
        ev.score[(size_t)bg * a.NC + slot] = a.cs_new[bg];
    }
}

// Workspace: logits, split partials, then (8-byte aligned) the finish
// workgroups' minima and the LSE exchange words.
struct WsSizes {
    size_t logits, partial, part_min, xch;
};
WsSizes ws_sizes(int B, int Hq, int Hkv, int NC) {
    const int G = Hq / Hkv;
    const size_t ncp = round_up(NC, kDecSub);
    const size_t nsplit = (NC + kDecSplit - 1) / kDecSplit;
    const size_t nfin = (NC + kFinishKeys - 1) / kFinishKeys;
    const size_t D = 128;
    WsSizes w;
    w.logits = (size_t)B * Hkv * G * ncp * 4;
    w.partial = (size_t)B * Hkv * nsplit * G * (D + 2) * 4;
    w.part_min = (size_t)B * Hkv * nfin * 8;
    w.xch = (size_t)B * Hkv * nsplit * 4 * 8;
    return w;
}

DecodeWs ws_layout(void* base, int B, int Hq, int Hkv, int NC, int D) {
    DecodeWs w;
    const WsSizes z = ws_sizes(B, Hq, Hkv, NC);
    w.ncp = round_up(NC, kDecSub);
    w.nsplit = (NC + kDecSplit - 1) / kDecSplit;
    w.nfin = (NC + kFinishKeys - 1) / kFinishKeys;
    char* p = static_cast<char*>(base);
    w.logits = reinterpret_cast<float*>(p);
    w.partial = reinterpret_cast<float*>(p + z.logits);
    const size_t mins = (z.logits + z.partial + 7) / 8 * 8;
    w.part_min = reinterpret_cast<uint64_t*>(p + mins);
    w.xch = reinterpret_cast<uint64_t*>(p + mins + z.part_min);
    (void)D;
    return w;
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int NC) {
    const WsSizes z = ws_sizes(B, Hq, Hkv, NC);
    return (z.logits + z.partial + 7) / 8 * 8 + z.part_min + z.xch;
}

namespace {

template <int MODE>
const void* dec4_fn() {
    return reinterpret_cast<const void*>(&decode_attn4_kernel<128, MODE>);
}

// Once per device: the LDS limit of the decode kernels, and how many
// workgroups of each fused variant the device holds at once.
hipError_t configure_decode(int* cap_fused, int* cap_evict) {
    static unsigned configured = 0;
    static int cap[2][32] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 32) return hipErrorInvalidDevice;
    const unsigned bit = 1u << dev;
    if (!(configured & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_attn_kernel<128>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, DecSmem<128>::BYTES);
        const void* fns[4] = {dec4_fn<kDec4NoWeights>(), dec4_fn<kDec4Logits>(),
                              dec4_fn<kDec4Fused>(), dec4_fn<kDec4FusedEvict>()};
        for (int m = 0; m < 4 && e == hipSuccess; ++m)
            e = hipFuncSetAttribute(fns[m], hipFuncAttributeMaxDynamicSharedMemorySize,
                                    Dec4Smem<128>::BYTES);
        int cus = 0;
        if (e == hipSuccess) e = cu_count(&cus);
        for (int m = 0; m < 2 && e == hipSuccess; ++m) {
            int nb = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fns[2 + m], kDecThreads,
                                                             Dec4Smem<128>::BYTES);
            cap[m][dev] = nb * cus;
        }
        if (e != hipSuccess) return e;
        configured |= bit;
    }
    *cap_fused = cap[0][dev];
    *cap_evict = cap[1][dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode(const ChunkArgs& a, void* workspace, hipStream_t s,
                         const EvictArgs* ev) {
    if (a.D != 128) return hipErrorNotSupported;
    const DecodeWs ws = ws_layout(workspace, a.B, a.Hq, a.Hkv, a.NC, a.D);
    const int nsplit_rt = (a.n + kDecSplit - 1) / kDecSplit;
    int cap_fused = 0, cap_evict = 0;
    hipError_t e = configure_decode(&cap_fused, &cap_evict);
    if (e != hipSuccess) return e;
    const int total = nsplit_rt * a.B * a.Hkv;
    const int grid = xcd_grid(total);

    // Summed weights inside the attention kernel: its workgroups wait for their
    // siblings' (m, l), so every workgroup of the launch must be resident at once.
    // Our workgroups never hold up another kernel's, so a grid within the
    // device's capacity for this kernel always becomes fully resident.
    if (nsplit_rt > 0 && a.cs_cache != nullptr && a.G <= 4 && nsplit_rt <= kXchMaxSplits &&
        grid <= (ev != nullptr ? cap_evict : cap_fused)) {
        const int words = a.B * a.Hkv * ws.nsplit * 4;
        hipLaunchKernelGGL(decode_clear_kernel, dim3((words + kDecThreads - 1) / kDecThreads),
                           dim3(kDecThreads), 0, s, ws.xch, words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        timer_begin(H2O_KERNEL_DECODE, s);
        if (ev != nullptr)
            hipLaunchKernelGGL((decode_attn4_kernel<128, kDec4FusedEvict>), dim3(grid),
                               dim3(kDecThreads), Dec4Smem<128>::BYTES, s, a, ws, nsplit_rt, *ev);
        else
            hipLaunchKernelGGL((decode_attn4_kernel<128, kDec4Fused>), dim3(grid),
                               dim3(kDecThreads), Dec4Smem<128>::BYTES, s, a, ws, nsplit_rt,
                               EvictArgs{});
        timer_end(H2O_KERNEL_DECODE, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        timer_begin(H2O_KERNEL_DECODE_FINISH, s);
        if (ev != nullptr)
            hipLaunchKernelGGL((decode_merge_kernel<128, true>), dim3(a.B * a.Hkv),
                               dim3(kDecThreads), 0, s, a, ws, nsplit_rt, *ev);
        else
            hipLaunchKernelGGL((decode_merge_kernel<128, false>), dim3(a.B * a.Hkv),
                               dim3(kDecThreads), 0, s, a, ws, nsplit_rt, EvictArgs{});
        timer_end(H2O_KERNEL_DECODE_FINISH, s);
        return hipGetLastError();
    }

    if (nsplit_rt > 0) {
        timer_begin(H2O_KERNEL_DECODE, s);
        if (a.G > 4)
            hipLaunchKernelGGL(decode_attn_kernel<128>, dim3(grid), dim3(kDecThreads),
                               DecSmem<128>::BYTES, s, a, ws, nsplit_rt);
        else if (a.cs_cache != nullptr)
            hipLaunchKernelGGL((decode_attn4_kernel<128, kDec4Logits>), dim3(grid),
                               dim3(kDecThreads), Dec4Smem<128>::BYTES, s, a, ws, nsplit_rt,
                               EvictArgs{});
        else
            hipLaunchKernelGGL((decode_attn4_kernel<128, kDec4NoWeights>), dim3(grid),
                               dim3(kDecThreads), Dec4Smem<128>::BYTES, s, a, ws, nsplit_rt,
                               EvictArgs{});
        timer_end(H2O_KERNEL_DECODE, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // Without summed weights only the first workgroup of each (b, g) has work.
    const int kchunks = (a.n > 0 && a.cs_cache) ? (a.n + kFinishKeys - 1) / kFinishKeys : 1;
    timer_begin(H2O_KERNEL_DECODE_FINISH, s);
    if (ev != nullptr)
        hipLaunchKernelGGL((decode_finish_kernel<128, true>), dim3(kchunks, a.B * a.Hkv),
                           dim3(kDecThreads), 0, s, a, ws, nsplit_rt, kchunks, *ev);
    else
        hipLaunchKernelGGL((decode_finish_kernel<128, false>), dim3(kchunks, a.B * a.Hkv),
                           dim3(kDecThreads), 0, s, a, ws, nsplit_rt, kchunks, EvictArgs{});
    timer_end(H2O_KERNEL_DECODE_FINISH, s);
    e = hipGetLastError();
    if (e != hipSuccess || ev == nullptr) return e;
    timer_begin(H2O_KERNEL_INSERT, s);
    hipLaunchKernelGGL(decode_insert_kernel, dim3(a.B * a.Hkv), dim3(64), 0, s, a, ws, kchunks,
                       *ev);
    timer_end(H2O_KERNEL_INSERT, s);
    return hipGetLastError();
}

}  // namespace h2o
