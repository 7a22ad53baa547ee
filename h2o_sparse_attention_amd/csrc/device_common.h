// Device helpers shared by the bf16 HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

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

// Raw buffer descriptors: a wave-uniform base and byte count in scalar
// registers, a loop-invariant per-lane byte offset in a vector register.
// Loads past `bytes` return zero, which is how partial tiles are padded.
constexpr int kBufferFlags = 0x00020000;
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}
__device__ __forceinline__ u32x4 bload16(Rsrc r, int voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(Rsrc r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
// Streaming loads of data read exactly once: cache-policy operand 2, the `nt`
// (non-temporal) bit on gfx950 (1 is sc0, 16 is sc1).  For the decode cache
// stream it measured faster than the default policy, sc1 or nt sc1.
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ uint32_t bload4_stream(Rsrc r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, kStreamPolicy);
}
__device__ __forceinline__ u32x4 bload16_stream(Rsrc r, int voff) {
    return __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kStreamPolicy));
}

// Workgroup ids are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles that share K/V (or Q) share an L2.
__device__ __forceinline__ int xcd_tile(int lin, int total) {
    const int per = (total + 7) >> 3;
    return (lin & 7) * per + (lin >> 3);
}

__host__ __device__ inline int xcd_grid(int total) { return ((total + 7) >> 3) << 3; }

// Unpadded LDS tiles of D-element bf16 rows hold their 16-byte chunks
// XOR-swizzled: LDS chunk c of row r holds logical chunk c ^ swz(r).  swz_k
// keeps the MFMA operand reads (row r of 16 or 32 consecutive rows, one chunk)
// free of bank conflicts; swz_v does the same for ds_read_b64_tr_b16 reads
// (four consecutive rows, two 8-byte halves of neighbouring chunks).
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
// For tiles read both ways (the backward's Q, dO and K): swz_k ^ swz_v.  Over
// 16 consecutive rows it still takes every value once (x = 4a + b maps to
// 4(a ^ b) + b), as the row reads need; and over 4 consecutive rows its bits
// 2-3 (D = 128; bit 2 over rows two apart, D = 64) still differ, as the
// transposed reads need.
template <int D>
__device__ __forceinline__ int swz_kt(int r) { return swz_k<D>(r) ^ swz_v<D>(r); }

// Eviction order keys: scores map to uint32 keys whose unsigned order is the
// float order; slots that may not be evicted take the top two codes.
constexpr uint32_t kIneligible = 0xFFFFFFFEu;   // filled slot inside the recent window
constexpr uint32_t kAbsent = 0xFFFFFFFFu;       // slot >= n: never a victim
constexpr uint32_t kMaxEligible = 0xFF800001u;  // just above +inf: NaN scores rank here

// Monotone map float -> uint32 (a < b  =>  key(a) < key(b); -0 == +0).
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return u < kMaxEligible ? u : kMaxEligible;
}

// A-operand row m of the QK^T product reads physical key perm_key(m).
__device__ __forceinline__ int perm_key(int m) {
    return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}


}  // namespace dev
}  // namespace h2o
