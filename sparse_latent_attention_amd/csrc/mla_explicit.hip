// Explicit-form sparse prefill: the prefill branch the pages print ("Key heads"
// page, Explanation: the prefill-branch code), on bf16 MFMA.
//
//   1. up-projection: kv[t, h, 0:128] = c_t . W_UK[h]^T (content key), kv[t, h,
//      128:256] = c_t . W_UV[h]^T (value), for every position a query of the
//      chunk can see;
//   2. selection bitmap: bit t of query s is set iff t is in its index list
//      and t <= start_pos + s (the index mask and the causal mask together);
//   3. attention per (block of 128 queries, head): keys [k_nope ; k_R] (192)
//      and values (128) of 32 positions at a time in LDS, scores on MFMA,
//      positions whose bit is clear masked to -inf, online softmax, values
//      mixed on MFMA.
// Positions are shared by all queries of a block, so a key/value tile is read
// once per block rather than once per (query, position); the price is that
// the attention visits every position up to the block's last one, selected
// or not (the dense causal region and half of the rest at the chunk shape).
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// --------------------------------------------------------------------------
// 1. Up-projection.  Workgroup = (block of 64 positions, head h); output
// [64 t x 256 j] computed transposed, D[j][t] = sum_c W[j][c] c_t[c], with
// the head's stacked weights (j < 128: W_UK[h][j], else W_UV[h][j - 128]) as
// the A operand and the latent rows as the B operand, both read straight
// from memory (16 bytes per lane and k-step).  Wave w takes positions
// 32 (w % 2) .. +31 and rows j = 128 (w / 2) .. +127 (four 32-row blocks);
// the next four k-steps' operands are in flight while four are multiplied.
// --------------------------------------------------------------------------
constexpr int kUpChunk = 4;

__global__ __launch_bounds__(256) void upproject_bf16(const __bf16* __restrict__ kv, const __bf16* __restrict__ w_uk,
                                                      const __bf16* __restrict__ w_uv, __bf16* __restrict__ up,
                                                      int Tv) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = blockIdx.y;
    const int t0 = blockIdx.x * 64 + 32 * (wave & 1);
    const int jhalf = wave >> 1;                          // 0: W_UK rows, 1: W_UV rows
    const int r = lane & 31, half = lane >> 5;
    const int t = min(t0 + r, Tv - 1);
    const __bf16* xrow = kv + (size_t)t * kLatent + 8 * half;
    const __bf16* wbase = (jhalf ? w_uv : w_uk) + ((size_t)h * kNope + r) * kLatent + 8 * half;
    f32x16 acc[4] = {};
    bf16x8 A[kUpChunk][4], X[kUpChunk];
    auto load = [&](int ks, bf16x8 (&a)[4], bf16x8& x) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) a[jb] = *reinterpret_cast<const bf16x8*>(wbase + (size_t)32 * jb * kLatent + 16 * ks);
        x = *reinterpret_cast<const bf16x8*>(xrow + 16 * ks);
    };
#pragma unroll
    for (int u = 0; u < kUpChunk; ++u) load(u, A[u], X[u]);
    for (int c = 0; c < kLatent / 16; c += kUpChunk) {
        bf16x8 nA[kUpChunk][4], nX[kUpChunk];
        const bool more = c + kUpChunk < kLatent / 16;
        if (more) {
#pragma unroll
            for (int u = 0; u < kUpChunk; ++u) load(c + kUpChunk + u, nA[u], nX[u]);
        }
#pragma unroll
        for (int u = 0; u < kUpChunk; ++u)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) acc[jb] = mfma(A[u][jb], X[u], acc[jb]);
        if (more) {
#pragma unroll
            for (int u = 0; u < kUpChunk; ++u) {
                X[u] = nX[u];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) A[u][jb] = nA[u][jb];
            }
        }
    }
    // lane (t = lane % 32, g = lane / 32) holds j = 32 jb + 8 (i / 4) + 4 g + i % 4
    if (t0 + r < Tv) {
        __bf16* dst = up + ((size_t)(t0 + r) * kHeads + h) * (2 * kNope) + 128 * jhalf + 4 * half;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[jb][4 * g + e];
                *reinterpret_cast<bf16x4*>(dst + 32 * jb + 8 * g) = v;
            }
    }
}

// --------------------------------------------------------------------------
// 2. Selection bitmap [S][words], words = ceil(Tv / 32).
// --------------------------------------------------------------------------
__global__ void bitmap_clear(unsigned* bm, long long n) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
        bm[i] = 0u;
}

__global__ void bitmap_set(const int32_t* __restrict__ idx, unsigned* bm, int S, int k, int words, int Tv,
                           int start_pos) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)S * k) return;
    const int s = (int)(e / k);
    const int t = idx[e];
    if (t < 0 || t >= Tv || t > start_pos + s) return;    // empty slot, past the cache or after the query
    atomicOr(&bm[(size_t)s * words + (t >> 5)], 1u << (t & 31));
}

// --------------------------------------------------------------------------
// 3. Attention.  Workgroup = (block of 128 queries, head h); wave w owns
// queries 32w .. 32w+31 of the block.  Per tile of 32 positions:
//   scores  S^T[t][q] = sum_d K[t][d] Q[q][d] (12 MFMAs, k = 192): K from LDS
//           as the A operand, the wave's queries in registers as B; lane
//           (q, g) ends up with rows t = 8 (i / 4) + 4 g + i % 4;
//   mask    bit clear -> -inf (queries past S have no bits);
//   softmax per query, online: running maximum m and sum l, the accumulator
//           and l scaled by 2^(m_old - m_new) on every tile (64 multiplies);
//   mix     O^T[v][q] += sum_t V^T[v][t] P^T[t][q] (8 MFMAs): the
//           probabilities, packed to bf16 where the scores are, are the B
//           operand once k slot 8 g' + e stands for row 4 g' + e (e < 4) or
//           8 + 4 g' + e - 4 (e >= 4) of the k-step's 16; V is stored
//           transposed in LDS, so each lane reads those rows of its value
//           column as two 8-byte pieces.
// K/V tiles are staged through LDS by all 256 threads, three in flight.
// --------------------------------------------------------------------------
constexpr int kQb = 128;                  // queries per workgroup
constexpr int kKStride = 200;             // bf16 per staged key row (192 + pad)
constexpr int kVStride = 40;              // bf16 per staged transposed value row (32 + pad)
constexpr int kKBytes = 32 * kKStride * 2;
constexpr int kVBytes = 128 * kVStride * 2;
constexpr int kStage = kKBytes + kVBytes;
constexpr int kStages = 3;

__global__ __launch_bounds__(256) void explicit_attn_bf16(const __bf16* __restrict__ q_nope,
                                                          const __bf16* __restrict__ q_pe,
                                                          const __bf16* __restrict__ up,
                                                          const __bf16* __restrict__ pe,
                                                          const unsigned* __restrict__ bm, __bf16* __restrict__ out,
                                                          int S, int Tv, int words, int start_pos, float scale_log2) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kStages * kStage];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = lane & 31, g = lane >> 5;
    const int h = blockIdx.y;
    const int qb0 = blockIdx.x * kQb;
    const int qs = qb0 + 32 * wave + q;                   // this lane's query
    const bool qvalid = qs < S;
    // positions any query of the block can see: 0 .. start_pos + last query
    const int last_q = min(qb0 + kQb, S) - 1;
    const int ntiles = (min(start_pos + last_q + 1, Tv) + 31) / 32;

    // query fragments: Q[q][16 ks + 8 g .. +7], ks < 8 from q_nope, else q_pe
    bf16x8 qf[12];
    {
        const int qq = qvalid ? qs : 0;
        const __bf16* qn = q_nope + ((size_t)qq * kHeads + h) * kNope + 8 * g;
        const __bf16* qp = q_pe + ((size_t)qq * kHeads + h) * kRope + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qn + 16 * ks);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[8 + ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
    }

    // Stage tile kt: thread tid takes row tid / 8 and 16-byte chunks tid % 8 + 8 i of its
    // 40 (16 key-content, 8 rotary, 16 value).
    auto load_tile = [&](int kt, u32x4 (&v)[5]) {
        const int row = tid >> 3, c0 = tid & 7;
        const int t = min(kt * 32 + row, Tv - 1);
        const __bf16* kvrow = up + ((size_t)t * kHeads + h) * (2 * kNope);
        const __bf16* perow = pe + (size_t)t * kRope;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int c = c0 + 8 * i;                     // 0..15 key, 16..23 rotary, 24..39 value
            const __bf16* src = c < 16 ? kvrow + 8 * c : c < 24 ? perow + 8 * (c - 16) : kvrow + kNope + 8 * (c - 24);
            v[i] = *reinterpret_cast<const u32x4*>(src);
        }
    };
    auto store_tile = [&](int stage, const u32x4 (&v)[5]) {
        unsigned char* kb = lds + stage * kStage;
        __bf16* vt = reinterpret_cast<__bf16*>(kb + kKBytes);
        const int row = tid >> 3, c0 = tid & 7;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int c = c0 + 8 * i;
            if (c < 24) {
                *reinterpret_cast<u32x4*>(kb + (row * kKStride + 8 * c) * 2) = v[i];
            } else {
                const bf16x8 x = __builtin_bit_cast(bf16x8, v[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) vt[(8 * (c - 24) + e) * kVStride + row] = x[e];
            }
        }
    };

    f32x16 acc[4] = {};
    float m_run = -INFINITY, l_run = 0.f;
    // One tile: stage tile kt+1 (held in `nxt`) to LDS, start loading tile kt+2 into `fut`,
    // then score, mask, softmax and mix tile kt.  The two register sets alternate, so the
    // loop runs two tiles per trip and every array index is a constant.
    auto step = [&](int kt, const u32x4 (&nxt)[5], u32x4 (&fut)[5]) {
        const int stage = kt % kStages;
        if (kt + 1 < ntiles) store_tile((kt + 1) % kStages, nxt);
        if (kt + 2 < ntiles) load_tile(kt + 2, fut);
        const unsigned char* kb = lds + stage * kStage;
        const __bf16* vt = reinterpret_cast<const __bf16*>(kb + kKBytes);

        // scores: A = K[t][16 ks + 8 g' .. +7] for t = lane % 32
        f32x16 s = {};
        const __bf16* krow = reinterpret_cast<const __bf16*>(kb) + q * kKStride + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) s = mfma(*reinterpret_cast<const bf16x8*>(krow + 16 * ks), qf[ks], s);

        // mask, maximum, probabilities
        const unsigned bits = qvalid ? bm[(size_t)qs * words + kt] : 0u;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 8 * (i >> 2) + 4 * g + (i & 3);
            s[i] = (bits >> t) & 1u ? s[i] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float f = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float neg = m_new == -INFINITY ? 0.f : -m_new;
        bf16x8 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[i] + neg);
            psum += p;
            pb[i >> 3][i & 7] = (__bf16)p;
        }
        l_run = l_run * f + psum;
        m_run = m_new;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) acc[vb] *= f;

        // mix: A = V^T[v][rows of slots 8 g' + e] for v = 32 vb + lane % 32
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) {
                const __bf16* vrow = vt + (32 * vb + q) * kVStride + 16 * kc + 4 * g;
                const bf16x8 a = cat(*reinterpret_cast<const bf16x4*>(vrow), *reinterpret_cast<const bf16x4*>(vrow + 8));
                acc[vb] = mfma(a, pb[kc], acc[vb]);
            }
        __syncthreads();                                  // stage kt free; stage kt+1 complete
    };
    u32x4 pa[5], pb2[5];
    load_tile(0, pa);
    if (ntiles > 1) load_tile(1, pb2);
    store_tile(0, pa);
    __syncthreads();
    for (int kt = 0; kt < ntiles; kt += 2) {
        step(kt, pb2, pa);                                // tile kt+1 from pb2, tile kt+2 into pa
        if (kt + 1 < ntiles) step(kt + 1, pa, pb2);       // tile kt+2 from pa, tile kt+3 into pb2
    }

    // normalise and store: lane (q, g) holds v = 32 vb + 8 (i / 4) + 4 g + i % 4
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qvalid) {
        __bf16* dst = out + ((size_t)qs * kHeads + h) * kValue + 4 * g;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[vb][4 * gq + e] * inv);
                *reinterpret_cast<bf16x4*>(dst + 32 * vb + 8 * gq) = v;
            }
    }
}

}  // namespace

ExplicitPlan plan_explicit(int S, int T, int start_pos) {
    ExplicitPlan p{};
    const long long tv = (long long)start_pos + S;
    p.Tv = (int)(tv < T ? tv : T);
    p.words = (p.Tv + 31) / 32;
    p.up_bytes = (size_t)p.Tv * kHeads * 2 * kNope * 2;
    p.bm_off = (p.up_bytes + 255) / 256 * 256;
    p.total = p.bm_off + ((size_t)S * p.words * 4 + 255) / 256 * 256;
    return p;
}

hipError_t launch_explicit_prefill(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                                   const int32_t* idx, const void* w_uk, const void* w_uv, void* out, int S, int k,
                                   int start_pos, float scale_log2, const ExplicitPlan& p, void* ws, hipStream_t s) {
    __bf16* up = static_cast<__bf16*>(ws);
    unsigned* bm = reinterpret_cast<unsigned*>(static_cast<unsigned char*>(ws) + p.bm_off);
    hipLaunchKernelGGL(upproject_bf16, dim3((p.Tv + 63) / 64, kHeads), dim3(256), 0, s,
                       static_cast<const __bf16*>(kv), static_cast<const __bf16*>(w_uk),
                       static_cast<const __bf16*>(w_uv), up, p.Tv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long nbm = (long long)S * p.words;
    const long long clear_blocks = (nbm + 255) / 256;
    hipLaunchKernelGGL(bitmap_clear, dim3((unsigned)(clear_blocks < 4096 ? clear_blocks : 4096)), dim3(256), 0, s,
                       bm, nbm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long nidx = (long long)S * k;
    hipLaunchKernelGGL(bitmap_set, dim3((unsigned)((nidx + 255) / 256)), dim3(256), 0, s, idx, bm, S, k, p.words, p.Tv,
                       start_pos);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(explicit_attn_bf16, dim3((S + kQb - 1) / kQb, kHeads), dim3(256), 0, s,
                       static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_pe), up,
                       static_cast<const __bf16*>(pe), bm, static_cast<__bf16*>(out), S, p.Tv, p.words, start_pos,
                       scale_log2);
    return hipGetLastError();
}

}  // namespace mla
