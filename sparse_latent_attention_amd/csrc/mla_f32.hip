// float32 kernels: the same five steps in plain float32 vector arithmetic
// (no reduced-precision operands anywhere), plus the index-list validator.
#include <hip/hip_ext.h>

#include "mla_internal.h"

namespace mla {
namespace {

// Step 1: q_c[r,h,c] = sum_d q_nope[r,h,d] W_UK[h,d,c]; columns 512..575 copy q_pe.
__global__ __launch_bounds__(256) void absorb_q_f32(const float* __restrict__ q_nope,
                                                    const float* __restrict__ q_pe,
                                                    const float* __restrict__ w_uk,
                                                    float* __restrict__ q_out, long long total,
                                                    int* stats) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < 2) stats[e] = 0;  // the call's diagnostics (this path never reruns a split)
    if (e >= total) return;
    const int c = (int)(e % kQRow);
    const long long rh = e / kQRow;
    const int h = (int)(rh % kHeads);
    if (c >= kLatent) {
        q_out[e] = q_pe[rh * kRope + (c - kLatent)];
        return;
    }
    const float* q = q_nope + rh * kNope;
    const float* w = w_uk + (size_t)h * kNope * kLatent + c;
    float acc = 0.f;
    for (int d = 0; d < kNope; ++d) acc = fmaf(q[d], w[(size_t)d * kLatent], acc);
    q_out[e] = acc;
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, w) : v + w;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

// Steps 2-4 for one (query row, head, split): scores of up to 256 selected
// rows at a time (one per thread), online softmax, then each thread
// accumulates two latent columns over those rows.  Writes unnormalised
// partials with their running max (log2 domain) and sum.
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
    __shared__ float q[kQRow];
    __shared__ float p[256];
    __shared__ int pos[256];
    __shared__ float red[4];

    const int h = blockIdx.x;
    const int split = blockIdx.y;
    const int r = blockIdx.z;
    const int tid = threadIdx.x;

    const float* qrow = reinterpret_cast<const float*>(a.q) + ((size_t)r * kHeads + h) * kQRow;
    for (int c = tid; c < kQRow; c += 256) q[c] = qrow[c];

    const int slot_begin = split * a.slots_per_split;
    const int slot_end = min(a.k, slot_begin + a.slots_per_split);
    const int limit = a.causal_base < 0 ? 0x7fffffff : a.causal_base + r;
    const int32_t* idx_row = a.idx + (size_t)r * a.k;
    const float* kv = reinterpret_cast<const float*>(a.kv) + (size_t)r * a.cache_rows_per_query * kLatent;
    const float* pe = reinterpret_cast<const float*>(a.pe) + (size_t)r * a.cache_rows_per_query * kRope;

    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    __syncthreads();
    for (int base = slot_begin; base < slot_end; base += 256) {
        const int slot = base + tid;
        int t = -1;
        if (slot < slot_end) {
            const int cand = idx_row[slot];
            if (cand >= 0 && cand < a.T && cand <= limit) t = cand;
        }
        float s = -INFINITY;
        if (t >= 0) {
            const float* row = kv + (size_t)t * kLatent;
            const float* rrow = pe + (size_t)t * kRope;
            float dot = 0.f;
            for (int c = 0; c < kLatent; ++c) dot = fmaf(q[c], row[c], dot);
            for (int c = 0; c < kRope; ++c) dot = fmaf(q[kLatent + c], rrow[c], dot);
            s = dot * a.scale_log2;
        }
        const float tmax = block_reduce(s, red, true);
        const float m_new = fmaxf(m, tmax);
        const float alpha = (m == -INFINITY) ? 1.f : exp2f(m - m_new);
        const float pv = (t >= 0) ? exp2f(s - m_new) : 0.f;
        const float psum = block_reduce(pv, red, false);
        l = l * alpha + psum;
        acc0 *= alpha;
        acc1 *= alpha;
        m = m_new;
        p[tid] = pv;
        pos[tid] = t;
        __syncthreads();
        const int n = min(256, slot_end - base);
        for (int j = 0; j < n; ++j) {
            const int tj = pos[j];
            if (tj < 0) continue;
            const float* row = kv + (size_t)tj * kLatent;
            acc0 = fmaf(p[j], row[tid], acc0);
            acc1 = fmaf(p[j], row[tid + 256], acc1);
        }
        __syncthreads();
    }
    const size_t o = ((size_t)split * a.R + r) * kHeads + h;
    float* dst = reinterpret_cast<float*>(a.o) + o * kLatent;
    dst[tid] = acc0;
    dst[tid + 256] = acc1;
    if (tid == 0) {
        a.m_part[o] = m;
        a.l_part[o] = l;
    }
}

// Step 4 merge + step 5 for one (query row, head).
__global__ __launch_bounds__(256) void uv_f32(const float* __restrict__ o_part,
                                              const float* __restrict__ m_part,
                                              const float* __restrict__ l_part,
                                              const float* __restrict__ w_uv,
                                              float* __restrict__ out, int R, int n_split) {
    __shared__ float ot[kLatent];
    const int h = blockIdx.x;
    const int r = blockIdx.y;
    const int tid = threadIdx.x;
    float mmax = -INFINITY;
    for (int sp = 0; sp < n_split; ++sp) mmax = fmaxf(mmax, m_part[((size_t)sp * R + r) * kHeads + h]);
    float L = 0.f, x0 = 0.f, x1 = 0.f;
    if (mmax != -INFINITY) {
        for (int sp = 0; sp < n_split; ++sp) {
            const size_t o = ((size_t)sp * R + r) * kHeads + h;
            if (m_part[o] == -INFINITY) continue;
            const float wgt = exp2f(m_part[o] - mmax);
            L += wgt * l_part[o];
            x0 = fmaf(wgt, o_part[o * kLatent + tid], x0);
            x1 = fmaf(wgt, o_part[o * kLatent + tid + 256], x1);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    ot[tid] = x0 * inv;
    ot[tid + 256] = x1 * inv;
    __syncthreads();
    // 2 threads per output value d, each summing half of the 512 columns
    const int d = tid >> 1;
    const int half = tid & 1;
    const float* w = w_uv + ((size_t)h * kValue + d) * kLatent + half * 256;
    float acc = 0.f;
    for (int c = 0; c < 256; ++c) acc = fmaf(ot[half * 256 + c], w[c], acc);
    acc += __shfl_xor(acc, 1);
    if (half == 0) out[((size_t)r * kHeads + h) * kValue + d] = acc;
}

__global__ void zero_flag(int* flag) { *flag = 0; }

// One workgroup per index list: range check and pairwise distinctness.
__global__ __launch_bounds__(256) void validate_idx(const int32_t* __restrict__ idx, int k, int T,
                                                    int allow_pad, int* flag) {
    const int32_t* row = idx + (size_t)blockIdx.x * k;
    int bits = 0;
    for (int i = threadIdx.x; i < k; i += 256) {
        const int v = row[i];
        if (v < 0) {
            if (!allow_pad) bits |= 1;
            continue;
        }
        if (v >= T) bits |= 1;
        for (int j = i + 1; j < k; ++j)
            if (row[j] == v) {
                bits |= 2;
                break;
            }
    }
    if (bits) atomicOr(flag, bits);
}

}  // namespace

hipError_t launch_absorb_f32(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                             int R, int* stats, hipStream_t s) {
    const long long total = (long long)R * kHeads * kQRow;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(absorb_q_f32, dim3(blocks), dim3(256), 0, s, static_cast<const float*>(q_nope),
                       static_cast<const float*>(q_pe), static_cast<const float*>(w_uk),
                       static_cast<float*>(q_out), total, stats);
    return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    hipExtLaunchKernelGGL(attn_f32, dim3(kHeads, a.n_split, a.R), dim3(256), 0, s, start, stop, 0, a);
    return hipGetLastError();
}

hipError_t launch_uv_f32(const float* o_part, const float* m_part, const float* l_part,
                         const void* w_uv, void* out, int R, int n_split, hipStream_t s) {
    hipLaunchKernelGGL(uv_f32, dim3(kHeads, R), dim3(256), 0, s, o_part, m_part, l_part,
                       static_cast<const float*>(w_uv), static_cast<float*>(out), R, n_split);
    return hipGetLastError();
}

hipError_t launch_validate(const int32_t* idx, int rows, int k, int T, int allow_pad, int* flag,
                           hipStream_t s) {
    hipLaunchKernelGGL(zero_flag, dim3(1), dim3(1), 0, s, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(validate_idx, dim3(rows), dim3(256), 0, s, idx, k, T, allow_pad, flag);
    return hipGetLastError();
}

}  // namespace mla
