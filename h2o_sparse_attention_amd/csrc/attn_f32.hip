// fp32 chunk attention: a plain VALU path for float32 caches (small shapes).
//
// Same computation as the bf16 kernels ("Kernel Support Needs", montaan paper
// page: SDPA returning sum_i m_{b,h,i,j} under the implicit positional mask),
// in float32 throughout: four lanes share one query row (or one key), each
// holding a quarter of head_dim, and the partial dot products are combined
// with two lane shuffles.  Softmax is exact online softmax with expf/logf.
#include "h2o_internal.h"

#include <climits>
#include <cmath>

namespace h2o {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerItem = 4;
constexpr int kItemsPerBlock = kThreads / kLanesPerItem;   // 64 rows or keys

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(ChunkArgs a) {
    constexpr int DL = D / kLanesPerItem;
    const int R = a.G * a.S;
    const int nrb = (R + kItemsPerBlock - 1) / kItemsPerBlock;
    const int bg = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    if (bg >= a.B * a.Hkv) return;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int part = threadIdx.x % kLanesPerItem;
    const int row = rb * kItemsPerBlock + threadIdx.x / kLanesPerItem;
    const bool row_ok = row < R;
    const int i = row_ok ? row / a.G : a.S - 1;
    const int h = g * a.G + (row_ok ? row % a.G : 0);
    const int qpos = a.P + i;

    const float* Q = static_cast<const float*>(a.q) + ((size_t)(b * a.Hq + h) * a.S + i) * D;
    const float* Kc = static_cast<const float*>(a.kc) + (size_t)bg * a.NC * D;
    const float* Vc = static_cast<const float*>(a.vc) + (size_t)bg * a.NC * D;
    const float* Kn = static_cast<const float*>(a.kn) + (size_t)bg * a.S * D;
    const float* Vn = static_cast<const float*>(a.vn) + (size_t)bg * a.S * D;
    const int32_t* posg = a.pos + (size_t)bg * a.NC;

    float qv[DL], o[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) {
        qv[e] = Q[part * DL + e];
        o[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int nkeys = a.n + a.S;
    for (int kk = 0; kk < nkeys; ++kk) {
        const bool cached = kk < a.n;
        const int kp = cached ? posg[kk] : a.P + (kk - a.n);
        const float* kr = cached ? Kc + (size_t)kk * D : Kn + (size_t)(kk - a.n) * D;
        const float* vr = cached ? Vc + (size_t)kk * D : Vn + (size_t)(kk - a.n) * D;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) s = fmaf(qv[e], kr[part * DL + e], s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (!(kp >= 0 && kp <= qpos)) continue;
        if (cached && a.excl && ((a.excl[(size_t)bg * excl_tiles(a.NC) + kk / 64] >> (kk % 64)) & 1))
            continue;                              // a slot the chunk overwrites
        s *= a.sm_scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);       // m = -inf gives 0
        const float p = expf(s - m_new);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < DL; ++e) o[e] = fmaf(p, vr[part * DL + e], o[e] * alpha);
        m = m_new;
    }
    if (!row_ok) return;
    float* O = static_cast<float*>(a.out) + ((size_t)(b * a.Hq + h) * a.S + i) * D;
#pragma unroll
    for (int e = 0; e < DL; ++e) O[part * DL + e] = o[e] / l;
    if (part == 0) a.lse[(size_t)(b * a.Hq + h) * a.S + i] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(kThreads) void colsum_f32_kernel(ChunkArgs a) {
    constexpr int DL = D / kLanesPerItem;
    const int nkeys = a.n + a.S;
    const int nkb = (nkeys + kItemsPerBlock - 1) / kItemsPerBlock;
    const int bg = blockIdx.x / nkb, kb = blockIdx.x % nkb;
    if (bg >= a.B * a.Hkv) return;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int part = threadIdx.x % kLanesPerItem;
    const int kk = kb * kItemsPerBlock + threadIdx.x / kLanesPerItem;
    const bool key_ok = kk < nkeys;
    const int kc = key_ok ? kk : 0;
    const bool cached = kc < a.n;
    const int kp = !key_ok ? INT_MAX : (cached ? a.pos[(size_t)bg * a.NC + kc] : a.P + (kc - a.n));
    const float* kr = cached ? static_cast<const float*>(a.kc) + ((size_t)bg * a.NC + kc) * D
                             : static_cast<const float*>(a.kn) + ((size_t)bg * a.S + (kc - a.n)) * D;
    float kv[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) kv[e] = kr[part * DL + e];

    const float* Q = static_cast<const float*>(a.q);
    const int R = a.G * a.S;
    float acc = 0.f;
    for (int r = 0; r < R; ++r) {
        const int h = g * a.G + r % a.G, i = r / a.G;
        const size_t qi = (size_t)(b * a.Hq + h) * a.S + i;
        const float* qr = Q + qi * D;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) s = fmaf(qr[part * DL + e], kv[e], s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (kp >= 0 && kp <= a.P + i) acc += expf(s * a.sm_scale - a.lse[qi]);
    }
    if (!key_ok || part != 0) return;
    if (cached && a.excl && ((a.excl[(size_t)bg * excl_tiles(a.NC) + kk / 64] >> (kk % 64)) & 1))
        acc = 0.f;                                 // not a key in the buffer form
    if (kk < a.n) a.cs_cache[(size_t)bg * a.NC + kk] = acc;
    else a.cs_new[(size_t)bg * a.S + (kk - a.n)] = acc;
}

}  // namespace

hipError_t launch_attn_f32(const ChunkArgs& a, hipStream_t s) {
    const int nrb = (a.G * a.S + kItemsPerBlock - 1) / kItemsPerBlock;
    const dim3 grid(nrb * a.B * a.Hkv), block(kThreads);
    if (a.D == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_colsum_f32(const ChunkArgs& a, hipStream_t s) {
    const int nkb = (a.n + a.S + kItemsPerBlock - 1) / kItemsPerBlock;
    const dim3 grid(nkb * a.B * a.Hkv), block(kThreads);
    if (a.D == 128) hipLaunchKernelGGL(colsum_f32_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(colsum_f32_kernel<64>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace h2o
