// Decode (S = 1) chunk attention for gfx950: split over cache slots.
//
// "Learning how to Forget: Fine-tuning for Long-Context Sparse Attention",
// montaan paper page, "Kernel Support Needs" (summed attention weights and
// the implicit positional mask) specialised to one query token per sequence,
// the generation setting of the metallab summary's Table 7.  With one query
// row per head the pass is bound by reading the cache once, so:
//
//  decode_attn_kernel  one workgroup per (b, kv head, 4096-slot range).  Each
//      of its 4 waves streams 32-slot tiles through a private LDS region (no
//      workgroup barriers), forms S^T = K Q^T with the G query heads of the
//      group as MFMA columns, writes the scaled logits (log2 units) of every
//      slot to the workspace, and keeps an online-softmax state (m, l, O);
//      the waves merge and the workgroup writes one partial per split.
//  decode_finish_kernel  merges the partials with the new token (its own key
//      and value) into O and LSE, then turns the stored logits into the summed
//      weights sum_{h in g} exp(s - LSE_h) per slot.
//  When the caller asks for no summed weights, the logits are not stored and
//  the finish kernel runs one workgroup per (b, kv head) for O and LSE only.
//
// P V uses ds_read_b64_tr_b16: a 16-lane group addresses four rows of four
// consecutive bf16 (one key, four d each) and lane j receives column j%4 of
// rows j/4, j/4+4, j/4+8, j/4+12, i.e. four keys of one d -- exactly the
// k-slots of the MFMA A operand V^T -- so V stays row-major in LDS.
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
    int nsplit;         // workgroups per (b, kv head) at full capacity
    int ncp;            // logit row length (capacity rounded up to kDecSub)
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

// Merge the splits and the new token, write O / LSE (first workgroup of each
// (b, g)), and form the summed weights of a range of slots.
template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_finish_kernel(ChunkArgs a, DecodeWs ws,
                                                                    int nsplit_rt, int kchunks) {
    __shared__ float sLse2[64];
    __shared__ float sNew[64];
    __shared__ float sM[64];
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
}

DecodeWs ws_layout(void* base, int B, int Hq, int Hkv, int NC, int D) {
    DecodeWs w;
    const int G = Hq / Hkv;
    w.ncp = round_up(NC, kDecSub);
    w.nsplit = (NC + kDecSplit - 1) / kDecSplit;
    const size_t logits = (size_t)B * Hkv * G * w.ncp * 4;
    w.logits = static_cast<float*>(base);
    w.partial = reinterpret_cast<float*>(static_cast<char*>(base) + logits);
    (void)D;
    return w;
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int NC) {
    const int G = Hq / Hkv;
    const size_t ncp = round_up(NC, kDecSub);
    const size_t nsplit = (NC + kDecSplit - 1) / kDecSplit;
    const size_t D = 128;
    return (size_t)B * Hkv * G * ncp * 4 + (size_t)B * Hkv * nsplit * G * (D + 2) * 4;
}

hipError_t launch_decode(const ChunkArgs& a, void* workspace, hipStream_t s) {
    if (a.D != 128) return hipErrorNotSupported;
    const DecodeWs ws = ws_layout(workspace, a.B, a.Hq, a.Hkv, a.NC, a.D);
    const int nsplit_rt = (a.n + kDecSplit - 1) / kDecSplit;
    if (nsplit_rt > 0) {
        static unsigned configured = 0;
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const unsigned bit = 1u << (dev & 31);
        if (!(configured & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_attn_kernel<128>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    DecSmem<128>::BYTES);
            if (e != hipSuccess) return e;
            configured |= bit;
        }
        const int total = nsplit_rt * a.B * a.Hkv;
        timer_begin(H2O_KERNEL_DECODE, s);
        hipLaunchKernelGGL(decode_attn_kernel<128>, dim3(xcd_grid(total)), dim3(kDecThreads),
                           DecSmem<128>::BYTES, s, a, ws, nsplit_rt);
        timer_end(H2O_KERNEL_DECODE, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // Without summed weights only the first workgroup of each (b, g) has work.
    const int kchunks = (a.n > 0 && a.cs_cache) ? (a.n + kFinishKeys - 1) / kFinishKeys : 1;
    timer_begin(H2O_KERNEL_DECODE_FINISH, s);
    hipLaunchKernelGGL(decode_finish_kernel<128>, dim3(kchunks, a.B * a.Hkv), dim3(kDecThreads), 0,
                       s, a, ws, nsplit_rt, kchunks);
    timer_end(H2O_KERNEL_DECODE_FINISH, s);
    return hipGetLastError();
}

}  // namespace h2o
