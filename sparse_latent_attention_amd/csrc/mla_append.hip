// Cache append: the step that fills the caches the attention reads.  Per new
// position, the joint down-projection's 576 outputs split into the latent
// (512, RMS-normalised with learned gains) and the rotary key (64, rotated
// pair by pair), both written at the position's cache row.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive values as float (one 16-byte load for bf16, two for float).
__device__ __forceinline__ void load8(const __bf16* p, float (&x)[8]) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = b[e];
    }
}
__device__ __forceinline__ void store8(__bf16* p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// One wave per new position (b, s), four per workgroup.  Lane l normalises
// latent values 8l .. 8l+7 (the mean square is a wave-wide sum); lanes 0..31
// each rotate one pair (2l, 2l+1) of the rotary key: re' = re c - im s,
// im' = re s + im c.  Arithmetic in float32; stores round to the cache type.
template <typename T>
__global__ __launch_bounds__(256) void cache_append_kernel(const T* __restrict__ a, const T* __restrict__ w,
                                                           const float* __restrict__ cos_sin,
                                                           T* __restrict__ kv, T* __restrict__ pe, int B, int S,
                                                           int start_pos, long long ld_T, float eps) {
    const int lane = threadIdx.x & 63;
    const long long p = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // b * S + s
    if (p >= (long long)B * S) return;
    const long long b = p / S;
    const int s = (int)(p % S);
    const T* row = a + p * kQRow;
    const long long dst = b * ld_T + start_pos + s;

    float x[8], g[8];
    load8(row + 8 * lane, x);
    load8(w + 8 * lane, g);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.f / sqrtf(ss * (1.f / kLatent) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * g[e];
    store8(kv + dst * kLatent + 8 * lane, x);

    if (lane < kRope / 2) {
        const float re = (float)row[kLatent + 2 * lane], im = (float)row[kLatent + 2 * lane + 1];
        const float c = cos_sin[((long long)s * (kRope / 2) + lane) * 2];
        const float sn = cos_sin[((long long)s * (kRope / 2) + lane) * 2 + 1];
        pe[dst * kRope + 2 * lane] = (T)(re * c - im * sn);
        pe[dst * kRope + 2 * lane + 1] = (T)(re * sn + im * c);
    }
}

}  // namespace

hipError_t launch_cache_append(const void* kv_a_out, const void* norm_weight, const float* cos_sin, void* kv_cache,
                               void* pe_cache, int B, int S, int start_pos, int ld_T, float eps, bool bf16,
                               hipStream_t s) {
    const long long n = (long long)B * S;
    const unsigned blocks = (unsigned)((n + 3) / 4);
    if (bf16)
        hipLaunchKernelGGL(cache_append_kernel<__bf16>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const __bf16*>(kv_a_out), static_cast<const __bf16*>(norm_weight), cos_sin,
                           static_cast<__bf16*>(kv_cache), static_cast<__bf16*>(pe_cache), B, S, start_pos,
                           (long long)ld_T, eps);
    else
        hipLaunchKernelGGL(cache_append_kernel<float>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const float*>(kv_a_out), static_cast<const float*>(norm_weight), cos_sin,
                           static_cast<float*>(kv_cache), static_cast<float*>(pe_cache), B, S, start_pos,
                           (long long)ld_T, eps);
    return hipGetLastError();
}

}  // namespace mla
