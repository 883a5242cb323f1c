// FP8 wkv_b dequantisation: the decode branch dequantises the stored wkv_b once
// when it carries a scale, then views it [heads, 256, 512] and takes the first
// 128 rows of each head as W_UK and the rest as W_UV ("Mix and project",
// Explanation, decode-branch code; FP8 block scales: "Key heads", Parameters,
// the note under the table).  Format (not on the pages): OCP E4M3 codes, one
// float32 scale per 128 x 128 block.  Elementwise and bound by HBM: 1 byte in,
// 2 bytes out per weight.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;                       // rows and columns per scale
constexpr int kRows = kHeads * (kNope + kValue);  // 32768 stacked rows

// Value of one E4M3 byte as float32 (exact): sign, 4 exponent bits (bias 7),
// 3 mantissa bits; exponent 0 holds m * 2^-9; S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_value(unsigned b) {
    const unsigned sign = (b & 0x80u) << 24;
    const unsigned e = (b >> 3) & 15u, m = b & 7u;
    const unsigned normal = sign | ((e + 120u) << 23) | (m << 20);       // (1 + m/8) 2^(e - 7)
    const unsigned sub = sign | __builtin_bit_cast(unsigned, (float)m * 0x1p-9f);
    const unsigned bits = e == 0 ? sub : (e == 15 && m == 7 ? (sign | 0x7FC00000u) : normal);
    return __builtin_bit_cast(float, bits);
}

// Thread i converts codes 16 i .. 16 i + 15 (one 16-byte load, two 16-byte
// stores): stacked row r = 16 i / 512 of head r / 256, columns c .. c + 15.
__global__ __launch_bounds__(256) void wkv_b_dequant_kernel(const unsigned char* __restrict__ codes,
                                                            const float* __restrict__ scales,
                                                            __bf16* __restrict__ w_uk, __bf16* __restrict__ w_uv) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int r = i / (kLatent / 16), c = (i % (kLatent / 16)) * 16;
    const float sc = scales[(r / kBlock) * (kLatent / kBlock) + c / kBlock];
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes + (size_t)i * 16);
    bf16x8 out[2];
#pragma unroll
    for (int k = 0; k < 16; ++k) out[k >> 3][k & 7] = (__bf16)(e4m3_value((v[k >> 2] >> (8 * (k & 3))) & 0xFFu) * sc);
    const int h = r / (kNope + kValue), j = r % (kNope + kValue);
    __bf16* dst = (j < kNope ? w_uk + ((size_t)h * kNope + j) * kLatent
                             : w_uv + ((size_t)h * kValue + j - kNope) * kLatent) + c;
    *reinterpret_cast<bf16x8*>(dst) = out[0];
    *reinterpret_cast<bf16x8*>(dst + 8) = out[1];
}

}  // namespace

hipError_t launch_wkv_b_dequant(const void* codes, const float* scales, void* w_uk, void* w_uv, hipStream_t s) {
    constexpr int kThreads = kRows * (kLatent / 16);
    static_assert(kThreads % 256 == 0, "whole workgroups");
    hipLaunchKernelGGL(wkv_b_dequant_kernel, dim3(kThreads / 256), dim3(256), 0, s,
                       static_cast<const unsigned char*>(codes), scales, static_cast<__bf16*>(w_uk),
                       static_cast<__bf16*>(w_uv));
    return hipGetLastError();
}

}  // namespace mla
