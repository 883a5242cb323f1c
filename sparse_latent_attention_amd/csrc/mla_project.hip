// Output projection: out[b, n] = sum_k o[b, k] W_O[n, k], with o the 128 head
// outputs flattened head by head (16,384 features) and W_O in its
// [7168 out, 16384 in] storage.  A weight-streaming product: at decode batch
// sizes the 235 MB of bf16 weights are the whole cost.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kOutRows = 32;                 // output features per workgroup
constexpr int kChunk = 4;                    // k-steps per load batch
constexpr int kWaves = 8;                    // waves per workgroup, one k range each
constexpr int kRange = kProjIn / kWaves;     // k range of one wave
static_assert(kProjOut % kOutRows == 0 && kRange % (16 * kChunk) == 0, "projection tiling");

// bf16: workgroup = 32 output features for every batch row; its eight waves
// (two per SIMD, 177 registers each) take eight ranges of k and their partial
// products are added in LDS.
// Out^T[n][b] = sum_k W[n][k] o[b][k] on v_mfma_f32_32x32x16_bf16: W rows
// are the A operand and o rows the B operand, both read straight from memory
// (lane l: row l % 32, k = 16 ks + 8 (l / 32) .. +7), the next eight k-steps'
// operands in flight while the current eight are multiplied.  64 batch rows
// (two B blocks) per pass over the weights.
__global__ __launch_bounds__(64 * kWaves) void project_bf16(const __bf16* __restrict__ o,
                                                            const __bf16* __restrict__ w,
                                                            __bf16* __restrict__ out, int B) {
    __shared__ float red[kWaves][2][16][65];   // [wave][block][element][lane] (+1 spreads banks)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 31, half = lane >> 5;
    const int n0 = blockIdx.x * kOutRows;
    const __bf16* wrow = w + (size_t)(n0 + j) * kProjIn + wave * kRange + 8 * half;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int r0 = b0 + j, r1 = b0 + 32 + j;
        const __bf16* x0 = o + (size_t)min(r0, B - 1) * kProjIn + wave * kRange + 8 * half;
        const __bf16* x1 = o + (size_t)min(r1, B - 1) * kProjIn + wave * kRange + 8 * half;
        f32x16 acc0 = {}, acc1 = {};
        bf16x8 A[kChunk], X0[kChunk], X1[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            A[u] = *reinterpret_cast<const bf16x8*>(wrow + 16 * u);
            X0[u] = *reinterpret_cast<const bf16x8*>(x0 + 16 * u);
            X1[u] = *reinterpret_cast<const bf16x8*>(x1 + 16 * u);
        }
        for (int c = 0; c < kRange / 16; c += kChunk) {
            bf16x8 nA[kChunk], nX0[kChunk], nX1[kChunk];
            const bool more = c + kChunk < kRange / 16;
            if (more) {
#pragma unroll
                for (int u = 0; u < kChunk; ++u) {
                    const int ks = c + kChunk + u;
                    nA[u] = *reinterpret_cast<const bf16x8*>(wrow + 16 * ks);
                    nX0[u] = *reinterpret_cast<const bf16x8*>(x0 + 16 * ks);
                    nX1[u] = *reinterpret_cast<const bf16x8*>(x1 + 16 * ks);
                }
            }
#pragma unroll
            for (int u = 0; u < kChunk; ++u) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u], X0[u], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[u], X1[u], acc1, 0, 0, 0);
            }
            if (more) {
#pragma unroll
                for (int u = 0; u < kChunk; ++u) {
                    A[u] = nA[u];
                    X0[u] = nX0[u];
                    X1[u] = nX1[u];
                }
            }
        }
        // rows past B read row B-1 and are dropped here
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            red[wave][0][i][lane] = acc0[i];
            red[wave][1][i][lane] = acc1[i];
        }
        __syncthreads();
        if (wave < 2) {
            // block `wave`: lane (b = lane % 32, g = lane / 32) holds features
            // n0 + 8 (i / 4) + 4 g + i % 4 of batch row b0 + 32 wave + b
            const int r = b0 + 32 * wave + j;
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float t = 0.f;
#pragma unroll
                for (int q = 0; q < kWaves; ++q) t += red[q][wave][i][lane];
                v[i] = t;
            }
            if (r < B) {
                __bf16* dst = out + (size_t)r * kProjOut + n0 + 4 * half;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 q;
#pragma unroll
                    for (int e = 0; e < 4; ++e) q[e] = (__bf16)v[4 * g + e];
                    *reinterpret_cast<bf16x4*>(dst + 8 * g) = q;
                }
            }
        }
        __syncthreads();
    }
}

// float32: one thread per (batch row, output feature), a plain dot product
// over the 16,384 inputs in float32 (the path for the float32 parity checks).
__global__ __launch_bounds__(256) void project_f32(const float* __restrict__ o, const float* __restrict__ w,
                                                   float* __restrict__ out, int B) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)B * kProjOut) return;
    const int n = (int)(e % kProjOut);
    const long long b = e / kProjOut;
    const f32x4* x = reinterpret_cast<const f32x4*>(o + b * kProjIn);
    const f32x4* wr = reinterpret_cast<const f32x4*>(w + (size_t)n * kProjIn);
    float acc = 0.f;
    for (int k = 0; k < kProjIn / 4; ++k) {
        const f32x4 a = x[k], c = wr[k];
        acc = fmaf(a[0], c[0], acc);
        acc = fmaf(a[1], c[1], acc);
        acc = fmaf(a[2], c[2], acc);
        acc = fmaf(a[3], c[3], acc);
    }
    out[e] = acc;
}

}  // namespace

hipError_t launch_project(const void* o, const void* w_o, void* out, int B, bool bf16, hipStream_t s) {
    if (bf16) {
        hipLaunchKernelGGL(project_bf16, dim3(kProjOut / kOutRows), dim3(64 * kWaves), 0, s, static_cast<const __bf16*>(o),
                           static_cast<const __bf16*>(w_o), static_cast<__bf16*>(out), B);
    } else {
        const long long n = (long long)B * kProjOut;
        hipLaunchKernelGGL(project_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(o), static_cast<const float*>(w_o), static_cast<float*>(out), B);
    }
    return hipGetLastError();
}

}  // namespace mla
