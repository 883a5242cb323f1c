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

// bf16: split-K GEMM.  Workgroup = (256 output features, one eighth of the
// 16,384 inputs), eight waves of 32 features each: 28 x 8 = 224 workgroups.
// Out^T[n][b] = sum_k W[n][k] o[b][k] on v_mfma_f32_32x32x16_bf16 with W rows
// as the A operand and o rows as the B operand, 64 batch rows per pass.
// Memory is read as whole 128-byte lines: 64 inputs at a time, each wave
// loads its 32 weight rows and one eighth of the 64 o rows (16 bytes per
// lane, eight lanes per row), and the chunk goes through LDS (rows padded to
// 144 bytes, so the 16-byte operand reads are conflict-free); the o rows are
// shared by the eight waves.  Loading 32 bytes of each of 32 rows per
// instruction, as the MFMA operand layout would have it, ran at half this
// rate.  Two LDS stages and two register sets: a chunk is loaded two chunks
// before it is multiplied.  Each workgroup writes its 64 x 256 float32
// partial sums (through LDS, whole rows) to the workspace; project_reduce
// adds the eight splits and rounds to bf16.
constexpr int kPSplits = 8;                       // input ranges (workgroups per feature block)
constexpr int kPWaves = 8;
constexpr int kPRows = 32 * kPWaves;              // output features per workgroup
constexpr int kPRange = kProjIn / kPSplits;       // 2048 inputs per workgroup
constexpr int kPC = 64;                           // inputs per chunk
constexpr int kPChunks = kPRange / kPC;           // 32
constexpr int kPStride = kPC + 8;                 // bf16 per staged row
constexpr int kPWBytes = kPRows * kPStride * 2;
constexpr int kPStage = kPWBytes + 64 * kPStride * 2;
constexpr int kPOutStride = kPRows + 4;           // floats per staged output row
static_assert(kProjOut % kPRows == 0 && kPRange % kPC == 0 && kPChunks % 2 == 0, "projection tiling");
static_assert(64 * kPOutStride * 4 <= 2 * kPStage, "output staging fits in the operand stages");

__global__ __launch_bounds__(64 * kPWaves, 1) void project_bf16(const __bf16* __restrict__ o,
                                                               const __bf16* __restrict__ w,
                                                               float* __restrict__ part, int B) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kPStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 31, half = lane >> 5;
    const int n0 = blockIdx.x * kPRows, sp = blockIdx.y;
    const int k0 = sp * kPRange;
    // staging: lane l takes 16 bytes at column 8 (l % 8) of rows l / 8 + 8 i (i < 4) of the
    // wave's weight rows, and of o row 8 wave + l / 8
    const int srow = lane >> 3, scol = 8 * (lane & 7);
    const __bf16* wsrc = w + (size_t)(n0 + 32 * wave + srow) * kProjIn + k0 + scol;
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    struct Set {
        u32x4 w[4], x;
    };
    for (int b0 = 0; b0 < B; b0 += 64) {
        const __bf16* xsrc = o + (size_t)min(b0 + 8 * wave + srow, B - 1) * kProjIn + k0 + scol;
        auto gload = [&](int c, Set& st) {
            const int kk = min(c, kPChunks - 1) * kPC;
#pragma unroll
            for (int i = 0; i < 4; ++i) st.w[i] = *reinterpret_cast<const u32x4*>(wsrc + (size_t)8 * i * kProjIn + kk);
            st.x = *reinterpret_cast<const u32x4*>(xsrc + kk);
        };
        auto sstore = [&](int stage, const Set& st) {
            unsigned char* base = lds + stage * kPStage;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(base + ((32 * wave + srow + 8 * i) * kPStride + scol) * 2) = st.w[i];
            *reinterpret_cast<u32x4*>(base + kPWBytes + ((8 * wave + srow) * kPStride + scol) * 2) = st.x;
        };
        f32x16 acc0 = {}, acc1 = {};
        auto compute = [&](int stage) {
            const __bf16* wl = reinterpret_cast<const __bf16*>(lds + stage * kPStage) + (32 * wave + j) * kPStride + 8 * half;
            const __bf16* xl = reinterpret_cast<const __bf16*>(lds + stage * kPStage + kPWBytes) + j * kPStride + 8 * half;
#pragma unroll
            for (int ks = 0; ks < kPC / 16; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(wl + 16 * ks);
                const bf16x8 x0 = *reinterpret_cast<const bf16x8*>(xl + 16 * ks);
                const bf16x8 x1 = *reinterpret_cast<const bf16x8*>(xl + 32 * kPStride + 16 * ks);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, x0, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, x1, acc1, 0, 0, 0);
            }
        };
        // chunk c: staged at the top of step c - 1 from the register set it was loaded into at
        // step c - 3 (c - 2 for the first ones); branch-free, past the end the last chunk is
        // loaded again into a stage nobody reads
        Set s0, s1;
        gload(0, s0);
        sstore(0, s0);
        gload(1, s1);
        __builtin_amdgcn_sched_barrier(0);
        gload(2, s0);
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < kPChunks; c += 2) {
            sstore(1, s1);
            gload(min(c + 3, kPChunks - 1), s1);
            __builtin_amdgcn_sched_barrier(0);
            compute(0);
            __syncthreads();
            sstore(0, s0);
            gload(min(c + 4, kPChunks - 1), s0);
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            __syncthreads();
        }
        // partial sums through LDS: lane (b = j, g) holds features 32 wave + 8 (i / 4) + 4 g + i % 4
        // of batch rows b and 32 + b; then each row's 256 floats go out as 16-byte stores
        float* ostage = reinterpret_cast<float*>(lds);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 v0, v1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v0[e] = acc0[4 * g + e];
                v1[e] = acc1[4 * g + e];
            }
            *reinterpret_cast<f32x4*>(ostage + j * kPOutStride + 32 * wave + 8 * g + 4 * half) = v0;
            *reinterpret_cast<f32x4*>(ostage + (32 + j) * kPOutStride + 32 * wave + 8 * g + 4 * half) = v1;
        }
        __syncthreads();
#pragma unroll
        for (int pass = 0; pass < 64 * kPRows / 4 / (64 * kPWaves); ++pass) {
            const int e = pass * 64 * kPWaves + tid;            // float4 index in the 64 x 256 tile
            const int r = e / (kPRows / 4), c4 = e % (kPRows / 4);
            if (b0 + r < B)
                *reinterpret_cast<f32x4*>(part + ((size_t)sp * B + b0 + r) * kProjOut + n0 + 4 * c4) =
                    *reinterpret_cast<const f32x4*>(ostage + r * kPOutStride + 4 * c4);
        }
        __syncthreads();
    }
}

// out[b][n] = bf16(sum over the splits of part[s][b][n]), four outputs per thread.
__global__ __launch_bounds__(256) void project_reduce(const float* __restrict__ part, __bf16* __restrict__ out,
                                                     int B) {
    const long long e = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= (long long)B * kProjOut) return;
    f32x4 t = *reinterpret_cast<const f32x4*>(part + e);
#pragma unroll
    for (int s = 1; s < kPSplits; ++s) t += *reinterpret_cast<const f32x4*>(part + (size_t)s * B * kProjOut + e);
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (__bf16)t[i];
    *reinterpret_cast<bf16x4*>(out + e) = q;
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

size_t project_workspace_bytes(int B, bool bf16) {
    return bf16 ? (size_t)kPSplits * B * kProjOut * sizeof(float) : 0;
}

hipError_t launch_project(const void* o, const void* w_o, void* out, int B, bool bf16, void* ws, hipStream_t s) {
    if (bf16) {
        float* part = static_cast<float*>(ws);
        hipLaunchKernelGGL(project_bf16, dim3(kProjOut / kPRows, kPSplits), dim3(64 * kPWaves), 0, s,
                           static_cast<const __bf16*>(o), static_cast<const __bf16*>(w_o), part, B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const long long n4 = (long long)B * kProjOut / 4;
        hipLaunchKernelGGL(project_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, part,
                           static_cast<__bf16*>(out), B);
    } else {
        const long long n = (long long)B * kProjOut;
        hipLaunchKernelGGL(project_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(o), static_cast<const float*>(w_o), static_cast<float*>(out), B);
    }
    return hipGetLastError();
}

}  // namespace mla
